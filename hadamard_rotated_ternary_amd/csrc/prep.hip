// Fused RMSNorm -> online Walsh-Hadamard rotation -> per-token quantisation.
//
// QbitAI article on BitNet v2, section 引入H-BitLinear模块, and 新智元 article
// "微软再放LLM量化大招", section H-BitLinear模块: the layer normalises the
// activations, applies an orthogonal +-1 Hadamard transform computed by the
// fast O(n log n) algorithm, then quantises each token (INT8 absmax or INT4
// absmean) before the ternary matmul.
//
// One token of K = 2^LOGK features is spread over T = 2^(LOGK-LOGE) threads
// holding E = 2^LOGE values each.  The Walsh-Hadamard transform is a product
// of independent radix-2 butterflies, one per index bit, that may be applied
// in any order; each "pass" applies the butterflies of the index bits that a
// thread currently holds in registers, and an LDS exchange between passes
// re-deals the index bits so that the not-yet-transformed ones land in
// registers.  No shuffles are needed: every add/sub is register to register.
//
// RMSNorm's 1/r and the 1/sqrt(K) scale are per-token scalars that commute
// with the transform, so the transform runs on x*g and both scalars are
// applied once, folded into the quantiser multiplier.
#include "common.h"

namespace hbl {

// ---------------------------------------------------------------------------
// Compile-time bit dealing.
struct PassBits {
  int reg[8];   // index bit held by register-number bit i
  int thr[16];  // index bit held by thread-number bit j
  int fresh;    // register-number bits whose butterflies run in this pass
};

constexpr int num_passes(int logk, int loge) {
  return 1 + ((logk - loge) + loge - 1) / loge;
}

// Pass 0 holds index bits {0,1,2} (8 contiguous features = one 16-byte load)
// plus the top LOGE-3 bits; later passes take the middle bits upward, LOGE at
// a time, padding the last one with the lowest already-transformed bits.
constexpr PassBits pass_bits(int logk, int loge, int p) {
  PassBits b{};
  bool inreg[32] = {};
  bool fresh[32] = {};
  if (p == 0) {
    for (int k = 0; k < 3; ++k) inreg[k] = fresh[k] = true;
    for (int k = logk - (loge - 3); k < logk; ++k) inreg[k] = fresh[k] = true;
  } else {
    const int lo = 3 + (p - 1) * loge, hi = logk - (loge - 3);
    int n = 0;
    for (int k = lo; k < hi && n < loge; ++k) { inreg[k] = fresh[k] = true; ++n; }
    for (int k = 0; k < logk && n < loge; ++k)
      if (!inreg[k]) { inreg[k] = true; ++n; }
  }
  int i = 0, j = 0;
  b.fresh = 0;
  for (int k = 0; k < logk; ++k) {
    if (inreg[k]) { if (fresh[k]) b.fresh |= 1 << i; b.reg[i++] = k; }
    else b.thr[j++] = k;
  }
  return b;
}

template <int LOGK, int LOGE, int P>
struct Pass {
  static constexpr PassBits B = pass_bits(LOGK, LOGE, P);
  static constexpr int LOGT = LOGK - LOGE;
  // Register part of the feature index of register r (compile-time).
  static constexpr int reg_idx(int r) {
    int v = 0;
    for (int i = 0; i < LOGE; ++i) if ((r >> i) & 1) v |= 1 << B.reg[i];
    return v;
  }
  // Thread part of the feature index of thread tau.
  static HBL_DEV int thr_idx(int tau) {
    int v = 0;
#pragma unroll
    for (int j = 0; j < LOGT; ++j) v |= ((tau >> j) & 1) << B.thr[j];
    return v;
  }
  static constexpr bool vec4 = B.reg[0] == 0 && B.reg[1] == 1;
};

// Padded LDS position of feature index i; thread and register parts of i
// occupy disjoint bits, so pad(thr | reg) == pad(thr) + pad(reg).  The
// padding makes every exchange of the shipped configurations free of bank
// conflicts and keeps groups of 4 consecutive features 16-byte aligned.
template <int P2>
HBL_DEV constexpr int pad(int i) { return i + 4 * (i >> 5) + 4 * (i >> P2); }
// Byte buffer used to gather the codes before the coalesced store.
HBL_DEV constexpr int padb(int i) { return i + 16 * (i >> 10); }

template <int LOGE, int FRESH>
HBL_DEV void butterflies(float (&v)[1 << LOGE]) {
#pragma unroll
  for (int i = 0; i < LOGE; ++i) {
    if (!((FRESH >> i) & 1)) continue;
#pragma unroll
    for (int r = 0; r < (1 << LOGE); ++r) {
      if (r & (1 << i)) continue;
      const float a = v[r], b = v[r | (1 << i)];
      v[r] = a + b;
      v[r | (1 << i)] = a - b;
    }
  }
}

template <int LOGK, int LOGE, int P2>
struct PrepCfg {
  static constexpr int K = 1 << LOGK, E = 1 << LOGE, LOGT = LOGK - LOGE, T = 1 << LOGT;
  static constexpr int WG = T < 64 ? 64 : T;     // threads per workgroup
  static constexpr int TPB = WG / T;             // tokens per workgroup
  static constexpr int NP = num_passes(LOGK, LOGE);
  static constexpr int REGION = pad<P2>(K - 1) + 1;  // floats per token
  static_assert(LOGE >= 4 && LOGE <= 7, "4..7 register bits");
  static_assert(REGION * 4 >= K + 16 * (K >> 10), "byte buffer must fit");
};

// Reduction over W consecutive lanes (W a power of two up to 64), result in
// every lane of the group.  Within a row of 16 lanes it uses DPP moves (swap
// neighbours, swap pairs, mirror 8, mirror 16: after each step every lane
// holds the reduction of its 2, 4, 8, 16 lanes); across rows, lane reads.
template <int CTRL>
HBL_DEV float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <bool MAX>
HBL_DEV float rop(float a, float b) { return MAX ? fmaxf(a, b) : a + b; }
template <int W, bool MAX>
HBL_DEV float lane_reduce(float v) {
  if constexpr (W >= 2) v = rop<MAX>(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v = rop<MAX>(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v = rop<MAX>(v, dpp<0x141>(v));   // row_half_mirror
  if constexpr (W >= 16) v = rop<MAX>(v, dpp<0x140>(v));  // row_mirror
  if constexpr (W == 32) v = rop<MAX>(v, __shfl_xor(v, 16, 64));
  if constexpr (W == 64) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    v = rop<MAX>(rop<MAX>(r0, r1), rop<MAX>(r2, r3));
  }
  return v;
}

// Token-wide reductions of two statistics at once (a: sum; b: sum or max):
// the T threads of a token are contiguous lanes of one wave (T <= 64) or
// whole waves of a one-token workgroup (T > 64).
template <int T, bool MAXB>
HBL_DEV void token_reduce2(float& a, float& b, float* red) {
  constexpr int W = T < 64 ? T : 64;
  a = lane_reduce<W, false>(a);
  b = lane_reduce<W, MAXB>(b);
  if constexpr (T > 64) {
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    constexpr int NW = T / 64;   // waves of the token; red holds 2 * NW floats
    static_assert(2 * NW <= 32, "reduction scratch");
    if ((threadIdx.x & 63) == 0) { red[wave] = a; red[NW + wave] = b; }
    __syncthreads();
    float sa = red[0], sb = red[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) { sa += red[w]; sb = rop<MAXB>(sb, red[NW + w]); }
    a = sa; b = sb;
  }
}

// Exchange: registers dealt as pass P -> registers dealt as pass P+1.
template <int LOGK, int LOGE, int P2, int P>
HBL_DEV void exchange(float (&v)[1 << LOGE], float* region, int tau) {
  using A = Pass<LOGK, LOGE, P>;
  using Bn = Pass<LOGK, LOGE, P + 1>;
  constexpr int E = 1 << LOGE;
  const int wbase = pad<P2>(A::thr_idx(tau));
  if constexpr (A::vec4) {
#pragma unroll
    for (int r = 0; r < E; r += 4)
      *reinterpret_cast<float4*>(region + wbase + pad<P2>(A::reg_idx(r))) =
          make_float4(v[r], v[r + 1], v[r + 2], v[r + 3]);
  } else {
#pragma unroll
    for (int r = 0; r < E; ++r) region[wbase + pad<P2>(A::reg_idx(r))] = v[r];
  }
  __syncthreads();
  const int rbase = pad<P2>(Bn::thr_idx(tau));
  if constexpr (Bn::vec4) {
#pragma unroll
    for (int r = 0; r < E; r += 4) {
      const float4 f = *reinterpret_cast<const float4*>(region + rbase + pad<P2>(Bn::reg_idx(r)));
      v[r] = f.x; v[r + 1] = f.y; v[r + 2] = f.z; v[r + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < E; ++r) v[r] = region[rbase + pad<P2>(Bn::reg_idx(r))];
  }
  __syncthreads();
}

template <int LOGK, int LOGE, int P2, int P>
HBL_DEV void run_passes(float (&v)[1 << LOGE], float* region, int tau) {
  using C = PrepCfg<LOGK, LOGE, P2>;
  butterflies<LOGE, Pass<LOGK, LOGE, P>::B.fresh>(v);
  if constexpr (P + 1 < C::NP) {
    exchange<LOGK, LOGE, P2, P>(v, region, tau);
    run_passes<LOGK, LOGE, P2, P + 1>(v, region, tau);
  }
}

// Raw activations of one thread for one token: E values, 16-byte units.
template <int E, bool XBF16>
struct RawX {
  static constexpr int U = XBF16 ? E / 8 : E / 4;
  uint4 u[U];
};

// MODE 0: write codes + scales.  MODE 1: write the rotated activations (fp32).
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
template <int LOGK, int LOGE, int P2, int BITS, bool XBF16, int MODE>
__global__ __launch_bounds__(prep_wg(LOGK, LOGE)) void prep_kernel(
    const void* __restrict__ x, const float* __restrict__ gain, int M,
    uint8_t* __restrict__ codes, float* __restrict__ dscale, float* __restrict__ xt) {
  using C = PrepCfg<LOGK, LOGE, P2>;
  using P0 = Pass<LOGK, LOGE, 0>;
  using PL = Pass<LOGK, LOGE, C::NP - 1>;
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
    if (it + 1 < iters) load(m + stride);
    if (!valid) {
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
        const int idx = base0 + P0::reg_idx(8 * gi);
        const float4* p = reinterpret_cast<const float4*>(gain + idx);
        const float4 a = p[0], b = p[1];
        v[8 * gi + 0] *= a.x; v[8 * gi + 1] *= a.y; v[8 * gi + 2] *= a.z; v[8 * gi + 3] *= a.w;
        v[8 * gi + 4] *= b.x; v[8 * gi + 5] *= b.y; v[8 * gi + 6] *= b.z; v[8 * gi + 7] *= b.w;
      }
    }
    // ---- Walsh-Hadamard transform (unnormalised) of x*g
    run_passes<LOGK, LOGE, P2, 0>(v, region, tau);

    // c = 1 / (r * sqrt(K)), r = sqrt(mean x^2 + eps)
    auto scale_c = [&](float sst) { return 1.0f / (sqrtf(sst * (1.0f / K) + kEpsNorm) * sqrtf((float)K)); };
    if constexpr (MODE == 1) {
      float unused = 0.f;
      token_reduce2<T, false>(ss, unused, red);
      const float c = scale_c(ss);
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
          // 64 codes (two 32-k groups) per step -> 48 bytes.  Byte pairs
          // become f16 pairs 1024 + n (byte permute next to the constant
          // 0x64), then q/2 = 0.5 * (1024 + n) - 516 exactly, then one packed
          // conversion turns 32 halves into 32 fp6 fields (exact: every q/2
          // in [-4, 3.5] is an e2m3 value).
          uint8_t* out = codes + (size_t)m * 96;
          const size_t kb_stride = (size_t)M * 96;
          for (int cp = tau; cp < K / 64; cp += T) {
            uint32_t o[12];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const uint32_t* s4 = reinterpret_cast<const uint32_t*>(bytes + padb(64 * cp + 32 * c));
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
#pragma unroll
              for (int i = 0; i < 6; ++i) o[6 * c + i] = f[i];
            }
            uint4* dst = reinterpret_cast<uint4*>(out + (size_t)(cp >> 1) * kb_stride + 48 * (cp & 1));
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
            dst[2] = make_uint4(o[8], o[9], o[10], o[11]);
          }
        } else if constexpr (BITS == 8) {
          // int8 codes: thread tau stores 16-byte chunks j*T + tau
          uint8_t* out = codes + (size_t)m * K;
#pragma unroll
          for (int j = 0; j < E / 16; ++j) {
            const int ch = j * T + tau;
            const uint32_t* s4 = reinterpret_cast<const uint32_t*>(bytes + padb(16 * ch));
            *reinterpret_cast<uint4*>(out + 16 * ch) = make_uint4(s4[0], s4[1], s4[2], s4[3]);
          }
        } else {
          // int4 codes: 8 consecutive codes per 32-bit word, code k0+4j+i at bits 8i+4j
          uint8_t* out = codes + (size_t)m * (K / 2);
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
              *reinterpret_cast<uint4*>(out + 16 * ch) = make_uint4(w[0], w[1], w[2], w[3]);
            }
          } else {
            static_assert(OB == 8, "E >= 16");
            const int ch = tau;  // 8 output bytes = 16 codes
            const uint32_t* s4 = reinterpret_cast<const uint32_t*>(bytes + padb(16 * ch));
            uint32_t w0 = (s4[0] & 0x0F0F0F0Fu) | ((s4[1] & 0x0F0F0F0Fu) << 4);
            uint32_t w1 = (s4[2] & 0x0F0F0F0Fu) | ((s4[3] & 0x0F0F0F0Fu) << 4);
            *reinterpret_cast<uint2*>(out + 8 * ch) = make_uint2(w0, w1);
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
  // persistent grid: enough workgroups to fill every CU at the occupancy the
  // LDS footprint allows (two workgroups per CU for the prefill dealings)
  const int per_cu = (160 * 1024) / (int)(sizeof(float) * C::REGION * C::TPB + 64) >= 2 ? 2 : 1;
  const int want = (a.M + C::TPB - 1) / C::TPB;
  const int grid = want < a.cus * per_cu ? want : a.cus * per_cu;
  if (grid == 0) return hipSuccess;
#define HBL_PREP(BITS, BF, MODE)                                                           \
  hipLaunchKernelGGL((prep_kernel<LOGK, LOGE, P2, BITS, BF, MODE>), dim3(grid), dim3(C::WG), 0, \
                     a.stream, a.x, a.gain, a.M, a.codes, a.dscale, a.xt)
  if (a.mode == 1) {
    if (a.x_bf16) HBL_PREP(8, true, 1); else HBL_PREP(8, false, 1);
  } else if (a.mode == 2) {
    if (a.x_bf16) HBL_PREP(4, true, 2); else HBL_PREP(4, false, 2);
  } else if (a.bits == 8) {
    if (a.x_bf16) HBL_PREP(8, true, 0); else HBL_PREP(8, false, 0);
  } else {
    if (a.x_bf16) HBL_PREP(4, true, 0); else HBL_PREP(4, false, 0);
  }
#undef HBL_PREP
  return hipGetLastError();
}

// Dealing per K: one LDS exchange for the prefill shapes (E >= T), more
// threads per token for small M so a single token is not latency bound.
hipError_t launch_prep(const PrepArgs& a) {
  const bool small = a.M <= 64;
  switch (a.logk) {
    case 8:  return launch_prep_t<8, 4, 6>(a);
    case 9:  return launch_prep_t<9, 5, 6>(a);
    case 10: return launch_prep_t<10, 5, 7>(a);
    case 11: return launch_prep_t<11, 6, 7>(a);
    case 12: return small ? launch_prep_t<12, 4, 6>(a) : launch_prep_t<12, 6, 8>(a);
    case 13: return small ? launch_prep_t<13, 4, 6>(a) : launch_prep_t<13, 7, 8>(a);
    case 14: return small ? launch_prep_t<14, 4, 6>(a) : launch_prep_t<14, 7, 9>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hbl
