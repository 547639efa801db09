// Single-launch forward for a few tokens (decode): RMSNorm -> Hadamard
// rotation -> per-token quantisation -> ternary matmul -> dequant in one
// kernel.
//
// QbitAI article on BitNet v2, section 引入H-BitLinear模块: the layer is
// normalisation, the online Hadamard transform, activation quantisation, the
// ternary matmul and dequantisation; 新智元 article "微软再放LLM量化大招",
// section H-BitLinear模块, for the transform applied to the activations ahead
// of the quantiser.  For a single token the matmul streams the packed weights
// once (16 MiB at the 7B down-projection shape) and the activation side is
// tiny; run as two kernels, the quantiser's latency chain adds a second
// launch and ~3 us in front of the weight stream.
//
// Here every workgroup owns 16 output channels (N/16 workgroups, one per CU
// at N = 4096).  It first requests its whole slice of the weight stream
// (16 bytes per lane per 256-k block, straight into registers), then computes
// the quantised activations of the M tokens itself -- the same transform as
// the prep kernel, T = 512 threads per token -- while the weights are in
// flight, and keeps them in LDS in int8 operand form.  That transform runs on
// every CU and is VALU- and LDS-bound (~4.5 us per token at K = 16384), so
// the kernel's time grows with M: at K = 16384 it takes 8.4 / 12.6 / 17.2 /
// 21.6 us for 1-4 tokens where prep + matmul take 11.4 / 11.7 / 12.1 /
// 12.6 us (at K = 8192: 5.0 / 7.2 / 10.2 us against 8.3 / 8.8 / 8.9 us).
// The forward uses it while M * K <= 16384 (49152 without the transform).
// The matmul part is the few-token decode kernel's: v_mfma_i32_16x16x64_i8
// with channels on the instruction's M side and the tokens on its N side,
// integer partials of the 8 waves combined with LDS atomics, then the
// dequant epilogue.
#include <mutex>

#include "fwht.h"
#include "mma.h"

namespace hbl {

constexpr int FD_NW = 8, FD_MAXM = 4, FD_DKB = 256;

// ROT = false: BitLinear without the transform (quantiser input x / r).
template <int LOGK, int LOGE, int P2, int BITS, bool XBF16, int OUT, bool ROT>
__global__ __launch_bounds__(64 * FD_NW) void decode_fused_kernel(
    const void* __restrict__ x, const float* __restrict__ gain, const uint8_t* __restrict__ W,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N) {
  using C = PrepCfg<LOGK, LOGE, P2>;
  static_assert(C::T == 64 * FD_NW, "one token per pass of the whole workgroup");
  using P0 = Pass<LOGK, LOGE, 0>;
  using PL = Pass<LOGK, LOGE, ROT ? C::NP - 1 : 0>;
  constexpr int K = C::K, E = C::E;
  constexpr int NBLK = K / FD_DKB;
  constexpr int MAXB = NBLK / FD_NW;
  static_assert(MAXB * FD_NW == NBLK, "256-k blocks dealt evenly over the waves");
  constexpr int REGION_BYTES = (C::REGION * 4 + 15) & ~15;

  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  float* region = reinterpret_cast<float*>(dyn);               // transform exchange
  uint8_t* slab = dyn + REGION_BYTES;                          // [M][K] operand bytes, then a zero row
  __shared__ float red[32];
  __shared__ int part[16 * 16];
  __shared__ float dtok[FD_MAXM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ch0 = blockIdx.x * 16;

  // ---- the tokens (bf16) and the gain are requested before the weights:
  // loads complete in issue order, so anything requested after the weight
  // stream could only be used once the whole stream had arrived
  const int base0 = P0::thr_idx(tid);
  const int baseL = PL::thr_idx(tid);
  // (only the M tokens present: every load instruction costs the CU's
  // address unit 16 cycles, and at M = 1 three redundant tokens would delay
  // the weight requests queued behind them)
  uint4 xr[XBF16 ? FD_MAXM : 1][E / 8];
  if constexpr (XBF16) {
#pragma unroll
    for (int t = 0; t < FD_MAXM; ++t) {
      if (t >= M) break;                                   // uniform
#pragma unroll
      for (int gi = 0; gi < E / 8; ++gi)
        xr[t][gi] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)t * K + base0 +
                                                    P0::reg_idx(8 * gi));
    }
  }
  float gv[E];
  if (gain != nullptr) {
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      const float4* p = reinterpret_cast<const float4*>(gain + base0 + P0::reg_idx(8 * gi));
      const float4 a = p[0], b = p[1];
      gv[8 * gi + 0] = a.x; gv[8 * gi + 1] = a.y; gv[8 * gi + 2] = a.z; gv[8 * gi + 3] = a.w;
      gv[8 * gi + 4] = b.x; gv[8 * gi + 5] = b.y; gv[8 * gi + 6] = b.z; gv[8 * gi + 7] = b.w;
    }
  }

  // ---- weight stream: block b = wave + FD_NW * i, 16 bytes per lane
  uint4 wq[MAXB];
  const int n = min(ch0 + c, N - 1);
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = wave + FD_NW * i;
    wq[i] = *reinterpret_cast<const uint4*>(W + wrow_base(n, K) + (size_t)b * 1024 + 16 * g);
  }

  // ---- quantised activations of the M tokens, into LDS
  const float Q = BITS == 8 ? kQ8 : kQ4;
#pragma unroll
  for (int t = 0; t < FD_MAXM; ++t) {
    if (t >= M) break;                                     // uniform
    float v[E];
    float ss = 0.f;
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      const int idx = base0 + P0::reg_idx(8 * gi);
      if constexpr (XBF16) {
        const uint4 w = xr[t][gi];
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.x), __builtin_bit_cast(bf2, w.x), ss, false);
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.y), __builtin_bit_cast(bf2, w.y), ss, false);
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.z), __builtin_bit_cast(bf2, w.z), ss, false);
        ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w.w), __builtin_bit_cast(bf2, w.w), ss, false);
        v[8 * gi + 0] = bf16_lo(w.x); v[8 * gi + 1] = bf16_hi(w.x);
        v[8 * gi + 2] = bf16_lo(w.y); v[8 * gi + 3] = bf16_hi(w.y);
        v[8 * gi + 4] = bf16_lo(w.z); v[8 * gi + 5] = bf16_hi(w.z);
        v[8 * gi + 6] = bf16_lo(w.w); v[8 * gi + 7] = bf16_hi(w.w);
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + (size_t)t * K + idx);
        const uint4 a = p[0], b = p[1];
        v[8 * gi + 0] = __uint_as_float(a.x); v[8 * gi + 1] = __uint_as_float(a.y);
        v[8 * gi + 2] = __uint_as_float(a.z); v[8 * gi + 3] = __uint_as_float(a.w);
        v[8 * gi + 4] = __uint_as_float(b.x); v[8 * gi + 5] = __uint_as_float(b.y);
        v[8 * gi + 6] = __uint_as_float(b.z); v[8 * gi + 7] = __uint_as_float(b.w);
#pragma unroll
        for (int r = 8 * gi; r < 8 * gi + 8; ++r) ss = __builtin_fmaf(v[r], v[r], ss);
      }
    }
    if (gain != nullptr) {
#pragma unroll
      for (int r = 0; r < E; ++r) v[r] *= gv[r];
    }
    if constexpr (ROT) run_passes<LOGK, LOGE, P2, 0>(v, region, tid);
    float st = 0.f;
    if constexpr (BITS == 8) {
#pragma unroll
      for (int r = 0; r < E; ++r) st = fmaxf(st, fabsf(v[r]));
    } else {
#pragma unroll
      for (int r = 0; r < E; ++r) st += fabsf(v[r]);
    }
    token_reduce2<C::T, BITS == 8>(ss, st, red);
    // c = 1 / (r * sqrt(K)) (1 / r without the transform), r = sqrt(mean x^2 + eps);
    // statistic of xt = v * c
    const float rr = sqrtf(ss * (1.0f / K) + kEpsNorm);
    const float cc = ROT ? 1.0f / (rr * sqrtf((float)K)) : 1.0f / rr;
    st = BITS == 8 ? st * cc : (st * (1.0f / K)) * cc;
    const float G = fmaxf(st, kEpsQ);
    const float cs = cc * (Q / G);
    if (tid == 0) dtok[t] = G / Q;
    // round to nearest even in the adder (fma with 1.5 * 2^23), clamp INT4,
    // keep the low byte: the operand byte is q itself for both widths (the
    // codes never take the packed nibble form here), so the accumulators
    // hold 64 * acc either way
    uint8_t* row = slab + t * K;
#pragma unroll
    for (int r = 0; r < E; ++r) {
      float q = __builtin_fmaf(v[r], cs, kRoundMagic);
      if constexpr (BITS == 4) q = fminf(fmaxf(q, kRoundMagic - 8.0f), kRoundMagic + 7.0f);
      row[baseL + PL::reg_idx(r)] = (uint8_t)__float_as_uint(q);
    }
  }
  if (tid < 4) reinterpret_cast<uint4*>(slab + M * K)[tid] = make_uint4(0, 0, 0, 0);
  if (tid < 256) part[tid] = 0;
  __syncthreads();

  // ---- matmul: 16 channels x up to 4 tokens, k blocks dealt over the waves
  v4i acc = v4i{};
  const uint8_t* arow = c < M ? slab + c * K + 64 * g : slab + M * K;
  const int astep = c < M ? 1 : 0;                         // padding lanes keep reading the zero row
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = wave + FD_NW * i;
    const uint4* ap = reinterpret_cast<const uint4*>(arow + astep * b * FD_DKB);
    const uint4 p = wq[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4i wop = wstep(u4get(p, j));
      const v4i aop = as_v4i(ap[j]);                       // codes 16j .. 16j+15 of the lane's 64
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, aop, acc, 0, 0, 0);
    }
  }
  // 16x16 accumulator layout: lane l, register r -> channel 4*(l/16) + r, token l%16
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (c < M) atomicAdd(&part[c * 16 + 4 * g + r], acc[r]);
  __syncthreads();
  if (tid < M * 16) {
    const int t = tid / 16, nn = ch0 + tid % 16;
    if (nn < N) store_out<OUT>(Y, (size_t)t * N + nn, unscale<8>(part[tid]), dtok[t] * fmaxf(walpha[0], kEpsQ));
  }
}

// ---------------------------------------------------------------------------
// Short rows (K = 64, 128, 256) and up to 64 tokens: the whole layer in one
// launch.  Every workgroup (4 waves, 64 output channels) first computes the
// codes of all M tokens itself -- one wave per token, K / 64 values per lane,
// the butterflies of the lane's own index bits in registers and those of the
// six lane bits by lane exchanges -- with the same arithmetic as the prep
// kernel (unnormalised transform of x * g, 1/r and 1/sqrt(K) folded into the
// quantiser multiplier, rounding by the 1.5 * 2^23 adder, INT4 clamped to
// [-8, 7]); codes go to LDS as int8 (an INT4 code is its own int8 value, so
// both widths take the INT8 matmul: weights expanded to 64 w, sums shifted
// back by 6).  Then each wave multiplies 16 channels by the M tokens on
// v_mfma_i32_16x16x64_i8 (channels on the M side, as in the short-row
// matmul) and stores the dequantised outputs.  At these sizes the work is
// a few microseconds of launch and latency; one launch instead of two halves
// that.
constexpr int SF_MAXM = 64;
template <int LOGK, int BITS, bool XBF16, int OUT, bool ROT>
__global__ __launch_bounds__(256) void forward_short_kernel(const void* __restrict__ x, const float* __restrict__ gain,
                                                            const uint8_t* __restrict__ W,
                                                            const float* __restrict__ walpha, void* __restrict__ Y,
                                                            int M, int N) {
  constexpr int K = 1 << LOGK, E = K / 64, LOGE = LOGK - 6;
  static_assert(LOGK >= 6 && LOGK <= 8, "short rows only");
  __shared__ __attribute__((aligned(16))) int8_t codes[SF_MAXM][K];
  __shared__ float dtok[SF_MAXM];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ---- codes of every token, one wave per token (the loop is wave-uniform)
  for (int t = wave; t < M; t += 4) {
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const size_t i = (size_t)t * K + lane * E + e;
      v[e] = XBF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[i] << 16)
                   : static_cast<const float*>(x)[i];
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
    if (gain != nullptr) {
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] *= gain[lane * E + e];
    }
    if constexpr (ROT) {
      // index k = E * lane + e: the low LOGE bits are the register's, the
      // next six the lane's
#pragma unroll
      for (int bb = 0; bb < LOGE; ++bb)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (!(e & (1 << bb))) {
            const float p = v[e], q = v[e | (1 << bb)];
            v[e] = p + q;
            v[e | (1 << bb)] = p - q;
          }
#pragma unroll
      for (int bb = 0; bb < 6; ++bb) {
        const bool upper = (lane >> bb) & 1;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float other = __shfl_xor(v[e], 1 << bb, 64);
          v[e] = upper ? other - v[e] : v[e] + other;
        }
      }
    }
    float st = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) st = BITS == 8 ? fmaxf(st, fabsf(v[e])) : st + fabsf(v[e]);
    ss = lane_reduce<64, false>(ss);
    st = lane_reduce<64, BITS == 8>(st);
    const float r = sqrtf(ss * (1.0f / K) + kEpsNorm);
    const float cc = ROT ? 1.0f / (r * sqrtf((float)K)) : 1.0f / r;
    st = BITS == 8 ? st * cc : (st * (1.0f / K)) * cc;
    const float Q = BITS == 8 ? kQ8 : kQ4;
    const float G = fmaxf(st, kEpsQ);
    const float cs = cc * (Q / G);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float q = __builtin_fmaf(v[e], cs, kRoundMagic);
      if constexpr (BITS == 4) q = fminf(fmaxf(q, kRoundMagic - 8.0f), kRoundMagic + 7.0f);
      codes[t][lane * E + e] = (int8_t)(__float_as_uint(q) & 0xFFu);
    }
    if (lane == 0) dtok[t] = G / Q;
  }
  __syncthreads();

  // ---- 16 channels x up to 64 tokens per wave
  const int ch0 = blockIdx.x * 64 + 16 * wave;
  if (ch0 >= N) return;                          // whole wave past the last channel (N % 16 == 0)
  const int c = lane & 15, g = lane >> 4;
  constexpr int STEPS = K / 64;
  const uint32_t* wrow = reinterpret_cast<const uint32_t*>(W + (size_t)(ch0 + c) * (K / 4));
  const float aw = fmaxf(walpha[0], kEpsQ);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (16 * mb >= M) break;                     // wave-uniform
    const int tt = min(16 * mb + c, M - 1);      // tokens past M repeat the last; never stored
    v4i acc = v4i{};
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      const uint4 a4 = *reinterpret_cast<const uint4*>(&codes[tt][64 * j + 16 * g]);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wstep(wrow[4 * j + g]), as_v4i(a4), acc, 0, 0, 0);
    }
    const int t = 16 * mb + c;
    // lane l / register r hold channel 4*(l/16)+r, token l%16
    if (t < M) store_out4<OUT>(Y, (size_t)t * N + ch0 + 4 * g, unscale4<8>(acc), dtok[t] * aw);
  }
}

template <int LOGK, bool ROT>
static hipError_t launch_short_k(const FusedDecodeArgs& a) {
#define HBL_SF(BITS, BF, OUT)                                                                                   \
  hipLaunchKernelGGL((forward_short_kernel<LOGK, BITS, BF, OUT, ROT>), dim3((a.N + 63) / 64), dim3(256), 0,    \
                     a.stream, a.x, a.gain, a.wpack, a.walpha, a.out, a.M, a.N);                               \
  return hipGetLastError()
  if (a.bits == 8) {
    if (a.x_bf16) { if (a.out_kind == OUT_BF16) { HBL_SF(8, true, OUT_BF16); } HBL_SF(8, true, OUT_F32); }
    if (a.out_kind == OUT_BF16) { HBL_SF(8, false, OUT_BF16); }
    HBL_SF(8, false, OUT_F32);
  }
  if (a.x_bf16) { if (a.out_kind == OUT_BF16) { HBL_SF(4, true, OUT_BF16); } HBL_SF(4, true, OUT_F32); }
  if (a.out_kind == OUT_BF16) { HBL_SF(4, false, OUT_BF16); }
  HBL_SF(4, false, OUT_F32);
#undef HBL_SF
}

template <int LOGK, int LOGE, int P2, int BITS, bool XBF16, int OUT, bool ROT>
static hipError_t launch_fd_t(const FusedDecodeArgs& a) {
  using C = PrepCfg<LOGK, LOGE, P2>;
  const size_t lds = (size_t)((C::REGION * 4 + 15) & ~15) + (size_t)a.M * C::K + 64;
  auto kern = &decode_fused_kernel<LOGK, LOGE, P2, BITS, XBF16, OUT, ROT>;
  // more than 64 KiB of dynamic LDS needs the per-function limit raised,
  // once per device and instantiation (thread-safe)
  static std::once_flag once[64];
  static hipError_t set_err[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev, kern] {
    set_err[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 146 * 1024);
  });
  if (set_err[dev] != hipSuccess) return set_err[dev];
  hipLaunchKernelGGL(kern, dim3((a.N + 15) / 16), dim3(64 * FD_NW), lds, a.stream, a.x, a.gain, a.wpack, a.walpha,
                     a.out, a.M, a.N);
  return hipGetLastError();
}

template <int LOGK, int LOGE, int P2, bool ROT>
static hipError_t launch_fd_k(const FusedDecodeArgs& a) {
#define HBL_FD(BITS, BF, OUT) return launch_fd_t<LOGK, LOGE, P2, BITS, BF, OUT, ROT>(a)
  if (a.bits == 8) {
    if (a.x_bf16) { if (a.out_kind == OUT_BF16) HBL_FD(8, true, OUT_BF16); HBL_FD(8, true, OUT_F32); }
    if (a.out_kind == OUT_BF16) HBL_FD(8, false, OUT_BF16);
    HBL_FD(8, false, OUT_F32);
  }
  if (a.x_bf16) { if (a.out_kind == OUT_BF16) HBL_FD(4, true, OUT_BF16); HBL_FD(4, true, OUT_F32); }
  if (a.out_kind == OUT_BF16) HBL_FD(4, false, OUT_BF16);
  HBL_FD(4, false, OUT_F32);
#undef HBL_FD
}

bool decode_fused_supported(int M, int logk, bool rotate) {
  // short rows: up to 64 tokens (forward_short_kernel)
  if (logk <= 8) return M >= 1 && M <= SF_MAXM && logk >= 6;
  // without the transform the per-token work on each CU is smaller: one
  // kernel wins while M * K <= 49152 (at K = 16384, 6.5 / 8.0 / 10.0 / 11.7 us
  // for 1-4 tokens against 9.6 / 9.8 / 10.2 / 10.7 us for prep + matmul)
  return M >= 1 && M <= FD_MAXM && (logk == 13 || logk == 14) &&
         ((int64_t)M << logk) <= (rotate ? 16384 : 49152);
}

hipError_t launch_decode_fused(const FusedDecodeArgs& a) {
  if (!decode_fused_supported(a.M, a.logk, a.rotate)) return hipErrorInvalidValue;
  if (a.logk == 6) return a.rotate ? launch_short_k<6, true>(a) : launch_short_k<6, false>(a);
  if (a.logk == 7) return a.rotate ? launch_short_k<7, true>(a) : launch_short_k<7, false>(a);
  if (a.logk == 8) return a.rotate ? launch_short_k<8, true>(a) : launch_short_k<8, false>(a);
  // T = 512 threads per token: E = K / 512 values per thread
  if (a.logk == 14) return a.rotate ? launch_fd_k<14, 5, 8, true>(a) : launch_fd_k<14, 5, 8, false>(a);
  return a.rotate ? launch_fd_k<13, 4, 6, true>(a) : launch_fd_k<13, 4, 6, false>(a);
}

}  // namespace hbl
