// Fused RMSNorm -> online Walsh-Hadamard rotation -> per-token quantisation.
//
// QbitAI article on BitNet v2, section 引入H-BitLinear模块, and 新智元 article
// "微软再放LLM量化大招", section H-BitLinear模块: the layer normalises the
// activations, applies an orthogonal +-1 Hadamard transform computed by the
// fast O(n log n) algorithm, then quantises each token (INT8 absmax or INT4
// absmean) before the ternary matmul.
//
// The transform's dealing of index bits over threads and registers is in
// fwht.h.
//
// RMSNorm's 1/r and the 1/sqrt(K) scale are per-token scalars that commute
// with the transform, so the transform runs on x*g and both scalars are
// applied once, folded into the quantiser multiplier.
#include "fwht.h"

namespace hbl {

// MODE 0: write codes + scales.  MODE 1: write the rotated activations (fp32).
// MODE 3: rotate rows without normalising (the weight rotation of the
// weight + activation variant, 新智元 article, section 实验效果, table 5):
// xt = H_K x / sqrt(K), fp32.
// ROT = false leaves the transform out (BitLinear for the layers whose inputs
// are already close to Gaussian, 新智元 article, section H-BitLinear模块): the
// quantiser then sees RMSNorm(x) = x / r in the load's own dealing.
// NORM = false (with ROT = false, fp32 input, MODE 0 or 2) leaves RMSNorm out
// too: the quantiser sees x as given, for callers that hold the rotated
// activations xt already (the second of the layer's two stages on its own).
// MODE 2 (INT4 only): write the codes as the fp6 (e2m3) operand of the
// fp6 x fp4 matrix instruction, plus the scales.  One 24-byte group per token
// and 32 consecutive k (k0 = 32c) holds q/2 for the 32 codes as six-bit
// fields, field p at bits 6p, where field p = h + 2b + 8d0 + 16d1 carries
// k = k0 + b + 4d0 + 8h + 16d1 (b < 4): the order in which the matmul unpacks
// a pair of packed ternary words into fp4 operands.  The groups are blocked
// by 128 k: block kb = c / 4 is a [M][96-byte] array at byte kb * M * 96, so
// the matmul's 128-k stage of 256 tokens is one contiguous 24 KiB run.
HBL_DEV constexpr int fp6_pos(int k) {
  return (k & ~31) | ((k >> 3) & 1) | ((k & 3) << 1) | (((k >> 2) & 1) << 3) | (k & 16);
}
constexpr int prep_wg(int logk, int loge) { return (1 << (logk - loge)) < 64 ? 64 : (1 << (logk - loge)); }

// Persistent: a workgroup walks tokens blockIdx.x*TPB + tok, then + gridDim.x*TPB,
// ...; the next token's activations are requested right after the current
// ones have been unpacked, so their HBM latency hides behind the transform.
// With a gain, its slice is requested once the activations are unpacked and
// applied before the next token's prefetch is issued: loads return in issue
// order, so a gain load queued behind the prefetch would wait for that whole
// HBM round trip (and holding the slice across the unpack costs registers
// and occupancy).
template <int LOGK, int LOGE, int P2, int BITS, bool XBF16, int MODE, bool ROT, bool NORM = true>
__global__ __launch_bounds__(prep_wg(LOGK, LOGE)) void prep_kernel(
    const void* __restrict__ x, const float* __restrict__ gain, int M,
    uint8_t* __restrict__ codes, float* __restrict__ dscale, float* __restrict__ xt,
    uint32_t* __restrict__ zero, int nzero, int blocked) {
  using C = PrepCfg<LOGK, LOGE, P2>;
  static_assert(ROT || (MODE == 0 || MODE == 2), "only the quantising modes run without the transform");
  static_assert(NORM || (!ROT && !XBF16 && (MODE == 0 || MODE == 2)), "quantising fp32 rows as given only");
  using P0 = Pass<LOGK, LOGE, 0>;
  using PL = Pass<LOGK, LOGE, ROT ? C::NP - 1 : 0>;
  constexpr int K = C::K, E = C::E, T = C::T;
  __shared__ __attribute__((aligned(16))) float lds[C::REGION * C::TPB];
  __shared__ float red[32];

  const int tok = threadIdx.x / T;
  const int tau = threadIdx.x % T;
  float* region = lds + tok * C::REGION;
  const int stride = gridDim.x * C::TPB;
  const int first = blockIdx.x * C::TPB;
  const int iters = first < M ? (M - first + stride - 1) / stride : 0;   // uniform over the workgroup
  const int base0 = P0::thr_idx(tau);
  const int baseL = PL::thr_idx(tau);

  // pass-0 dealing: 8 contiguous features per 16-byte (bf16) or 2x16-byte (fp32) load
  RawX<E, XBF16> raw;
  auto load = [&](int m) {
    const bool ok = m < M;
    const int mm = ok ? m : M - 1;
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      const int idx = base0 + P0::reg_idx(8 * gi);
      if constexpr (XBF16) {
        raw.u[gi] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)mm * K + idx);
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + (size_t)mm * K + idx);
        raw.u[2 * gi] = p[0];
        raw.u[2 * gi + 1] = p[1];
      }
    }
  };
  if (iters > 0) load(first + tok);
  // the following matmul's split-K counters start at zero (here, behind the
  // first activation load, whose latency covers it)
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0u;

  for (int it = 0; it < iters; ++it) {
    const int m = first + tok + it * stride;
    const bool valid = m < M;
    float v[E];
    // ---- RMSNorm statistic (of x, before the gain); bf16 pairs go through
    // the packed dot product.  It is reduced over the token together with
    // the quantisation statistic after the transform, which does not need it
    // (1/r is applied after, as a scalar).
    float ss = 0.f;
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      if constexpr (XBF16) {
        const uint4 w = raw.u[gi];
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.x), __builtin_bit_cast(bf2, w.x), ss, false);
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.y), __builtin_bit_cast(bf2, w.y), ss, false);
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.z), __builtin_bit_cast(bf2, w.z), ss, false);
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.w), __builtin_bit_cast(bf2, w.w), ss, false);
        v[8 * gi + 0] = bf16_lo(w.x); v[8 * gi + 1] = bf16_hi(w.x);
        v[8 * gi + 2] = bf16_lo(w.y); v[8 * gi + 3] = bf16_hi(w.y);
        v[8 * gi + 4] = bf16_lo(w.z); v[8 * gi + 5] = bf16_hi(w.z);
        v[8 * gi + 6] = bf16_lo(w.w); v[8 * gi + 7] = bf16_hi(w.w);
      } else {
        const uint4 a = raw.u[2 * gi], b = raw.u[2 * gi + 1];
        v[8 * gi + 0] = __uint_as_float(a.x); v[8 * gi + 1] = __uint_as_float(a.y);
        v[8 * gi + 2] = __uint_as_float(a.z); v[8 * gi + 3] = __uint_as_float(a.w);
        v[8 * gi + 4] = __uint_as_float(b.x); v[8 * gi + 5] = __uint_as_float(b.y);
        v[8 * gi + 6] = __uint_as_float(b.z); v[8 * gi + 7] = __uint_as_float(b.w);
      }
    }
    // (with one token per workgroup every token the loop visits exists)
    if (C::TPB > 1 && !valid) {
#pragma unroll
      for (int r = 0; r < E; ++r) v[r] = 0.f;
    }

    if constexpr (!XBF16) {
#pragma unroll
      for (int r = 0; r < E; ++r) ss = __builtin_fmaf(v[r], v[r], ss);
    }
    if (gain != nullptr) {
#pragma unroll
      for (int gi = 0; gi < E / 8; ++gi) {
        const float4* p = reinterpret_cast<const float4*>(gain + base0 + P0::reg_idx(8 * gi));
        const float4 a = p[0], b = p[1];
        v[8 * gi + 0] *= a.x; v[8 * gi + 1] *= a.y; v[8 * gi + 2] *= a.z; v[8 * gi + 3] *= a.w;
        v[8 * gi + 4] *= b.x; v[8 * gi + 5] *= b.y; v[8 * gi + 6] *= b.z; v[8 * gi + 7] *= b.w;
      }
    }
    // the squares are summed before the prefetch is issued (an empty asm
    // consumes ss): otherwise they are sunk below it, the raw registers stay
    // live across the load, and the loop-carried buffer gets copied twice
    __asm__ volatile("" : : "v"(ss));
    if (it + 1 < iters) load(m + stride);
    // ---- Walsh-Hadamard transform (unnormalised) of x*g
    if constexpr (ROT) run_passes<LOGK, LOGE, P2, 0>(v, region, tau);

    // c = 1 / (r * sqrt(K)) (1 / r without the transform), r = sqrt(mean x^2 + eps)
    auto scale_c = [&](float sst) {
      if constexpr (!NORM) return 1.0f;
      const float r = sqrtf(sst * (1.0f / K) + kEpsNorm);
      return ROT ? 1.0f / (r * sqrtf((float)K)) : 1.0f / r;
    };
    if constexpr (MODE == 1 || MODE == 3) {
      float c;
      if constexpr (MODE == 3) {
        c = 1.0f / sqrtf((float)K);
      } else {
        float unused = 0.f;
        token_reduce2<T, false>(ss, unused, red);
        c = scale_c(ss);
      }
      if (valid) {
#pragma unroll
        for (int r = 0; r < E; ++r) xt[(size_t)m * K + baseL + PL::reg_idx(r)] = v[r] * c;
      }
    } else {
      // ---- per-token statistic of the rotated token xt = v * c
      float st = 0.f;
      if constexpr (BITS == 8) {
#pragma unroll
        for (int r = 0; r < E; ++r) st = fmaxf(st, fabsf(v[r]));
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) st += fabsf(v[r]);
      }
      token_reduce2<T, BITS == 8>(ss, st, red);
      const float c = scale_c(ss);
      st = BITS == 8 ? st * c : (st * (1.0f / K)) * c;
      const float Q = BITS == 8 ? kQ8 : kQ4;
      // MODE 2 keeps q + 8 (0..15) in the low byte; the extra 8 is even, so
      // the ties of the rounding fall the same way.
      constexpr float RM = MODE == 2 ? kRoundMagic + 8.0f : kRoundMagic;
      const float G = fmaxf(st, kEpsQ);
      const float s = Q / G;
      const float cs = c * s;
      if (valid && tau == 0) dscale[m] = G / Q;

      // ---- round to codes: fma(v, cs, 1.5*2^23) rounds v*cs to the nearest
      // integer (ties to even) and leaves it in the low mantissa bits; INT4
      // clamps in that representation.  Codes are gathered through LDS for
      // coalesced stores.
      uint8_t* bytes = reinterpret_cast<uint8_t*>(region);
      // MODE 2 stores code k at LDS byte fp6_pos(k): the bit permutation acts
      // on the low five index bits, which split between thread and register
      // bits, so the address is a per-thread base plus a constant.
      const int wb = MODE == 2 ? padb(fp6_pos(baseL)) : padb(baseL);
#pragma unroll
      for (int r = 0; r < E; ++r) {
        float t = __builtin_fmaf(v[r], cs, RM);
        if constexpr (BITS == 4) t = fminf(fmaxf(t, RM - 8.0f), RM + 7.0f);
        const int ri = PL::reg_idx(r);
        bytes[wb + (MODE == 2 ? padb(fp6_pos(ri)) : padb(ri))] = (uint8_t)__float_as_uint(t);
      }
      __syncthreads();
      if (valid) {
        if constexpr (MODE == 2) {
          // 32 codes (one 32-k group) per step -> 24 bytes.  Byte pairs
          // become f16 pairs 1024 + n (byte permute next to the constant
          // 0x64), then q/2 = 0.5 * (1024 + n) - 516 exactly, then one packed
          // conversion turns 32 halves into 32 fp6 fields (exact: every q/2
          // in [-4, 3.5] is an e2m3 value).
          uint8_t* out = codes + (size_t)m * 96;
          const size_t kb_stride = (size_t)M * 96;
          // one 32-k group (24 output bytes) per thread and step: K/32 groups
          // keep every thread of the token busy (K/64 pairs left half idle)
          for (int u = tau; u < K / 32; u += T) {
            const uint32_t* s4 = reinterpret_cast<const uint32_t*>(bytes + padb(32 * u));
            h32 hv;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const uint32_t pr = __builtin_amdgcn_perm(0x64646464u, s4[e >> 1], (e & 1) ? 0x04030402u : 0x04010400u);
              const h2 x = __builtin_elementwise_fma(__builtin_bit_cast(h2, pr), h2{(_Float16)0.5f, (_Float16)0.5f},
                                                     h2{(_Float16)-516.0f, (_Float16)-516.0f});
              hv[2 * e] = x[0];
              hv[2 * e + 1] = x[1];
            }
            const u6 f = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(hv, 1.0f);
            // group u: block u/4 of 128 k, 24 bytes at 24 (u % 4) of the token's 96
            uint2* dst = reinterpret_cast<uint2*>(out + (size_t)(u >> 2) * kb_stride + 24 * (u & 3));
            dst[0] = make_uint2(f[0], f[1]);
            dst[1] = make_uint2(f[2], f[3]);
            dst[2] = make_uint2(f[4], f[5]);
          }
        } else if constexpr (BITS == 8) {
          // int8 codes: thread tau stores 16-byte chunks j*T + tau (row-major,
          // or each chunk at its place in the decode-blocked layout)
          uint8_t* out = codes + (size_t)m * K;
          const int mbt = (M + 15) >> 4;
#pragma unroll
          for (int j = 0; j < E / 16; ++j) {
            const int ch = j * T + tau;
            const uint32_t* s4 = reinterpret_cast<const uint32_t*>(bytes + padb(16 * ch));
            uint8_t* dst = blocked ? codes + dblk_offset(8, mbt, m, 16 * ch) : out + 16 * ch;
            *reinterpret_cast<uint4*>(dst) = make_uint4(s4[0], s4[1], s4[2], s4[3]);
          }
        } else {
          // int4 codes: 8 consecutive codes per 32-bit word, code k0+4j+i at bits 8i+4j
          uint8_t* out = codes + (size_t)m * (K / 2);
          const int mbt = (M + 15) >> 4;
          constexpr int OB = E / 2;  // output bytes per thread
          if constexpr (OB >= 16) {
#pragma unroll
            for (int j = 0; j < OB / 16; ++j) {
              const int ch = j * T + tau;  // 16 output bytes = 32 codes
              const uint32_t* s4 = reinterpret_cast<const uint32_t*>(bytes + padb(32 * ch));
              uint32_t w[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                w[i] = (s4[2 * i] & 0x0F0F0F0Fu) | ((s4[2 * i + 1] & 0x0F0F0F0Fu) << 4);
              uint8_t* dst = blocked ? codes + dblk_offset(4, mbt, m, 32 * ch) : out + 16 * ch;
              *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
            }
          } else {
            static_assert(OB == 8, "E >= 16");
            const int ch = tau;  // 8 output bytes = 16 codes
            const uint32_t* s4 = reinterpret_cast<const uint32_t*>(bytes + padb(16 * ch));
            uint32_t w0 = (s4[0] & 0x0F0F0F0Fu) | ((s4[1] & 0x0F0F0F0Fu) << 4);
            uint32_t w1 = (s4[2] & 0x0F0F0F0Fu) | ((s4[3] & 0x0F0F0F0Fu) << 4);
            uint8_t* dst = blocked ? codes + dblk_offset(4, mbt, m, 16 * ch) : out + 8 * ch;
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
          }
        }
      }
    }
    __syncthreads();   // the region is rewritten by the next token
  }
}

}  // namespace hbl

// ---------------------------------------------------------------------------
// Host-side launchers (called from the C ABI layer).
#include "launch.h"

namespace hbl {

template <int LOGK, int LOGE, int P2>
static hipError_t launch_prep_t(const PrepArgs& a) {
  using C = PrepCfg<LOGK, LOGE, P2>;
  // persistent grid: about 24 waves per CU (six per SIMD) where the LDS
  // footprint allows -- the transform's exchanges, barriers and reductions
  // stall a wave often, and only other resident waves hide that
  const int fit = (160 * 1024) / (int)(sizeof(float) * C::REGION * C::TPB + 64);
  const int waves = C::WG / 64;
  int per_cu = (24 + waves - 1) / waves;
  if (per_cu > fit) per_cu = fit;
  if (per_cu < 1) per_cu = 1;
  const int want = (a.M + C::TPB - 1) / C::TPB;
  const int grid = want < a.cus * per_cu ? want : a.cus * per_cu;
  if (grid == 0) return hipSuccess;   // (M == 0: no matmul follows either)
#define HBL_PREP(BITS, BF, MODE, ROT)                                                           \
  hipLaunchKernelGGL((prep_kernel<LOGK, LOGE, P2, BITS, BF, MODE, ROT>), dim3(grid), dim3(C::WG), 0, \
                     a.stream, a.x, a.gain, a.M, a.codes, a.dscale, a.xt, a.zero, a.zero ? a.nzero : 0, \
                     a.blocked ? 1 : 0)
#define HBL_PREP_R(BITS, BF, MODE) \
  if (a.rotate) HBL_PREP(BITS, BF, MODE, true); else HBL_PREP(BITS, BF, MODE, false)
#define HBL_PREP_G(BITS, MODE)                                                                            \
  hipLaunchKernelGGL((prep_kernel<LOGK, LOGE, P2, BITS, false, MODE, false, false>), dim3(grid), dim3(C::WG), 0, \
                     a.stream, a.x, nullptr, a.M, a.codes, a.dscale, nullptr, a.zero, a.zero ? a.nzero : 0, 0)
  if (a.as_given) {
    if (a.x_bf16 || a.rotate || (a.mode != 0 && a.mode != 2)) return hipErrorInvalidValue;
    if (a.mode == 2) HBL_PREP_G(4, 2); else if (a.bits == 8) HBL_PREP_G(8, 0); else HBL_PREP_G(4, 0);
  } else if (a.mode == 1) {
    if (a.x_bf16) HBL_PREP(8, true, 1, true); else HBL_PREP(8, false, 1, true);
  } else if (a.mode == 3) {
    HBL_PREP(8, false, 3, true);
  } else if (a.mode == 2) {
    if (a.x_bf16) { HBL_PREP_R(4, true, 2); } else { HBL_PREP_R(4, false, 2); }
  } else if (a.bits == 8) {
    if (a.x_bf16) { HBL_PREP_R(8, true, 0); } else { HBL_PREP_R(8, false, 0); }
  } else {
    if (a.x_bf16) { HBL_PREP_R(4, true, 0); } else { HBL_PREP_R(4, false, 0); }
  }
#undef HBL_PREP_G
#undef HBL_PREP_R
#undef HBL_PREP
  return hipGetLastError();
}

// Dealing per K.  Few values per thread (16 or 32) and many resident waves
// beat fewer LDS exchanges: at 8192 tokens, 128 values per thread (one
// exchange, one wave per SIMD) took 125 / 104 / 57 us at K = 16384 / 8192 /
// 4096 against 108 / 50 / 27 us here.  At K = 8192 small M takes 16 values
// per thread (no measurable difference); at K = 16384 32 values per thread
// also serve 8 to 64 tokens best (4.8 us instead of 5.4 us with 16).
hipError_t launch_prep(const PrepArgs& a) {
  const bool small = a.M <= 64;
  switch (a.logk) {
    case 6:  return launch_prep_t<6, 4, 6>(a);
    case 7:  return launch_prep_t<7, 4, 6>(a);
    case 8:  return launch_prep_t<8, 4, 6>(a);
    case 9:  return launch_prep_t<9, 5, 6>(a);
    case 10: return launch_prep_t<10, 5, 7>(a);
    case 11: return launch_prep_t<11, 4, 6>(a);
    case 12: return launch_prep_t<12, 4, 6>(a);
    case 13: return small ? launch_prep_t<13, 4, 6>(a) : launch_prep_t<13, 5, 7>(a);
    case 14: return launch_prep_t<14, 5, 7>(a);
    // one token per 1024-thread workgroup, 148 KiB of LDS: one workgroup per CU
    case 15: return launch_prep_t<15, 5, 7>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hbl
