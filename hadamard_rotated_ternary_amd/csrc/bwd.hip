// Backward pass of H-BitLinear with the straight-through estimator.
//
// QbitAI article on BitNet v2, section 引入H-BitLinear模块 (training): the
// quantisers' non-differentiable functions are bypassed and the gradient is
// transformed with the Hadamard matrix, whose orthogonality makes the
// transposed transform the transform itself.  With the forward
// y = xh . Wh^T (xh = q * d per token, Wh = W_t * a):
//   dxh = dy . Wh                      (bf16 MFMA on exact ternary values)
//   du  = H_K dxh / sqrt(K)             (the forward's FWHT machinery)
//   dx  = RMSNorm backward of du        (fused with the transform)
//   dg  = sum over tokens of du * x / r
//   dW  = dy^T . xh                     (bf16 MFMA over the tokens)
// Both products run as one bf16 "NT" kernel (both operands stored with the
// contraction index contiguous): the weights once per update as W_t^T in
// bf16, and dy and xh transposed token-last for the weight gradient.
#include "fwht.h"
#include "launch.h"
#include "mma.h"

namespace hbl {
namespace {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Ternary weights -> W_t^T as bf16 [K][N] (values -1, 0, +1; the scale a is
// applied in the product's epilogue).  One thread per 8 consecutive n of one
// k: the packed code of (n, k) is field (k % 16) / 4 of byte k % 4 of word
// k / 16 of row n (word position: wword).
__global__ __launch_bounds__(256) void wbt_kernel(const uint8_t* __restrict__ wpack, int N, int K,
                                                  uint16_t* __restrict__ wbt) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int ng = N / 8;
  if (t >= (int64_t)K * ng) return;
  const int k = (int)(t / ng), n0 = (int)(t % ng) * 8;
  const int sh = 2 * ((k & 15) >> 2);
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t c = (wpack[wword(n0 + 2 * p + e, k >> 4, K) * 4 + (k & 3)] >> sh) & 3u;
      const uint32_t bf = (c & 1u) ? (0x3F80u | ((c & 2u) << 14)) : 0u;   // 01 -> +1, 11 -> -1, 00 -> 0
      h |= bf << (16 * e);
    }
    o[p] = h;
  }
  *reinterpret_cast<uint4*>(wbt + (size_t)k * N + n0) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------
// Token-last copies for the weight gradient, through 64 x 64 LDS tiles:
//   dyT[n][m] = dy[m][n]               (bf16)
//   xhT[k][m] = bf16(q[m][k] * d[m])    (codes INT8 [M][K] or INT4 [M][K/2])
// m runs to Mp (a multiple of 64); columns past M are zero.  C % 8 == 0 (C
// is N or K here).
//
// The tile is held transposed, as token pairs: LDS row c holds 32 dwords,
// dword p = tokens 2p (low half) and 2p+1 (high half) of column c, so the
// transpose itself happens in registers and every LDS access is a whole
// dword or a 16-byte chunk (a first version moved single bf16 values down
// LDS columns and spent 40-50 % of its cycles on bank conflicts).  Rows are
// 36 dwords apart (8 rows = 288 dwords = 32 banks apart) and row r's 16-byte
// chunks are rotated by 2 * ((r >> 4) & 3), which makes both phases
// conflict-free: a dword write instruction covers rows 8j + e (j = 0..7) at
// 8 consecutive pair columns, 64 distinct banks; a chunk read instruction
// gives 8 lanes the 8 chunks of one row and the next 8 lanes those of the
// row 8 further on, the other half of the banks.
// Load: lane L of wave w takes columns 8 (L % 8) .. +7 of tokens
// 2 (L / 8 + 8 w) and the next (16 contiguous bytes of bf16 per lane,
// coalesced along the source row).  Store: 16 bytes (8 tokens) per lane
// along a destination row.
template <int KIND>   // 0: dy (bf16), 8: INT8 codes, 4: INT4 codes
__global__ __launch_bounds__(256) void tr_kernel(const void* __restrict__ src, const float* __restrict__ dscale,
                                                 int M, int C, int Mp, uint16_t* __restrict__ dst) {
  constexpr int P = 36;                       // dwords per LDS row
  __shared__ __attribute__((aligned(16))) uint32_t tile[64 * P];
  const int c0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto rot = [](int r) { return 8 * ((r >> 4) & 3); };   // dword rotation of row r (two chunks per step)
  // ---- load one token pair x 8 columns
  const int cg = lane & 7, pp = (lane >> 3) + 8 * wave;   // column group, token pair
  const int cc = c0 + 8 * cg;
  uint16_t v[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int m = m0 + 2 * pp + h;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[h][e] = 0;
    if (m < M && cc < C) {
      if constexpr (KIND == 0) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + (size_t)m * C + cc);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[h][2 * e] = (uint16_t)w[e]; v[h][2 * e + 1] = (uint16_t)(w[e] >> 16); }
      } else {
        const float dm = dscale[m];
        int q[8];
        if constexpr (KIND == 8) {
          const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(src) + (size_t)m * C + cc);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            q[e] = (int)(int8_t)(u.x >> (8 * e));
            q[4 + e] = (int)(int8_t)(u.y >> (8 * e));
          }
        } else {
          // INT4: one LE word per 8 k; code of k0 + 4j + i at bits 8i + 4j
          const uint32_t u = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(src) +
                                                                (size_t)m * (C / 2) + cc / 2);
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = ((int)(((u >> (8 * (e & 3) + 4 * (e >> 2))) & 15u) << 28)) >> 28;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[h][e] = f32_to_bf16((float)q[e] * dm);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = 8 * cg + e;
    tile[r * P + ((pp + rot(r)) & 31)] = (uint32_t)v[0][e] | ((uint32_t)v[1][e] << 16);
  }
  __syncthreads();
  // ---- store: instruction j of wave w covers rows b, b+8, b+1, b+9, ..., b+3, b+11
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = wave + 4 * j;
    const int b = 16 * (idx >> 1) + 4 * (idx & 1);
    const int g = lane >> 3;                              // 0..7
    const int r = b + (g >> 1) + 8 * (g & 1);
    const int k = lane & 7;                               // chunk: tokens 8k .. 8k+7
    const int c = c0 + r;
    const uint4 val = *reinterpret_cast<const uint4*>(&tile[r * P + ((4 * k + rot(r)) & 31)]);
    if (c < C) *reinterpret_cast<uint4*>(dst + (size_t)c * Mp + m0 + 8 * k) = val;
  }
}

// ---------------------------------------------------------------------------
// bf16 NT product: out[i][j] = s * sum_c A[i][c] B[j][c], fp32 out.
// 256 x 256 tile per workgroup (8 waves of 64 x 128, each 2 x 4
// v_mfma_f32_32x32x16_bf16 tiles; 4 waves of 128 x 128 also build), 32 c per stage in a three-deep LDS ring
// filled by global_load_lds_dwordx4 (each stage requested two ahead).  Rows
// of 64 bytes, 16-byte units XOR-swizzled by row bits 2-3, which the
// bank-conflict counter shows conflict-free for the fragment reads (rows
// r..r+31 of one unit column, both k halves); a swizzle by row bits 1 and 3
// spent 100 M conflict cycles per 1 ms product (20 % of its LDS cycles).
#ifndef HBL_BF16_NW
#define HBL_BF16_NW 8   // waves per workgroup of the bf16 product (4 or 8)
#endif
constexpr int GT = 256, GBK = 32, GROW = GBK * 2, GUNITS = GROW / 16;
constexpr int G_A_STAGE = GT * GROW, G_STAGE = 2 * G_A_STAGE;
HBL_DEV int gswz(int row) { return (row >> 2) & 3; }

// NW = 4: 2 x 2 waves of 128 x 128 (one wave per SIMD); NW = 8: 4 x 2 waves
// of 64 x 128, whose accumulators take half the registers, so two waves
// share a SIMD and one's MFMAs cover the other's waits.
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_bf16_nt_kernel(const uint16_t* __restrict__ A,
                                                                  const uint16_t* __restrict__ B,
                                                                  const float* __restrict__ sptr,
                                                                  float* __restrict__ out, int I, int J, int Cn,
                                                                  int tiles_i, int tiles_j) {
  constexpr int WI = NW / 2;                  // wave rows
  constexpr int RB = GT / WI / 32;            // 32-row blocks per wave
  constexpr int CP = 16 / NW;                 // 1 KiB copies per wave per operand per stage
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * G_STAGE];
  const int bid = blockIdx.x, total = tiles_i * tiles_j;
  // XCD-aware order (8 consecutive ids go to 8 XCDs): contiguous runs of
  // logical tiles per XCD, walked 4 tile-rows at a time.
  const int logical = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  constexpr int GM = 4;
  const int per_group = GM * tiles_j;
  const int first_i = (logical / per_group) * GM;
  const int gm = min(tiles_i - first_i, GM);
  const int in_g = logical % per_group;
  const int i0 = (first_i + in_g % gm) * GT;
  const int j0 = (in_g / gm) * GT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;

  // Per stage: A 16 KiB + B 16 KiB = 32 copies of 1 KiB; CP of each per wave.
  const uint16_t* a_src[CP];
  const uint16_t* b_src[CP];
#pragma unroll
  for (int j = 0; j < CP; ++j) {
    const int P = (j * NW + wave) * 64 + lane, row = P / GUNITS, u = (P % GUNITS) ^ gswz(row);
    a_src[j] = A + (size_t)min(i0 + row, I - 1) * Cn + 8 * u;
    b_src[j] = B + (size_t)min(j0 + row, J - 1) * Cn + 8 * u;
  }
  auto dma = [&](int kt, int buf) {
    uint8_t* base = smem + buf * G_STAGE;
#pragma unroll
    for (int j = 0; j < CP; ++j) lds_copy16(a_src[j] + (size_t)kt * GBK, base + (j * NW + wave) * 1024);
#pragma unroll
    for (int j = 0; j < CP; ++j) lds_copy16(b_src[j] + (size_t)kt * GBK, base + G_A_STAGE + (j * NW + wave) * 1024);
  };

  v16f acc[RB][4];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  // Fragments of one 16-wide k-step: RB A row blocks and 4 B column blocks.
  struct GFrag {
    bf8v a[RB], b[4];
  };
  auto read_frag = [&](GFrag& f, int buf, int ks) __attribute__((always_inline)) {
    const uint8_t* sa = smem + buf * G_STAGE;
    const uint8_t* sb = sa + G_A_STAGE;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = wi * (32 * RB) + rb * 32 + l32;
      f.a[rb] = *reinterpret_cast<const bf8v*>(sa + row * GROW + 16 * ((2 * ks + g) ^ gswz(row)));
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int row = wj * 128 + cb * 32 + l32;
      f.b[cb] = *reinterpret_cast<const bf8v*>(sb + row * GROW + 16 * ((2 * ks + g) ^ gswz(row)));
    }
  };
  auto mfmas = [&](const GFrag& f) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[rb], f.b[cb], acc[rb][cb], 0, 0, 0);
  };

  // Stage kt lives in LDS buffer kt % 3.  Within stage kt the fragments of
  // k-step 1 are read while the k-step 0 MFMAs run; then this wave waits for
  // its copies of stage kt+1 (stage kt+2's may still be in flight) and the
  // barrier makes every wave's copies visible and guarantees that every wave
  // has read all of stage kt (its reads completed before the barrier), so
  // stage kt+3 is requested into that buffer; the fragments of stage kt+1's
  // k-step 0 are read while the k-step 1 MFMAs run.  Copies are thus issued
  // two stages ahead of their use.
  constexpr int NL = 2 * CP;   // copy instructions per wave per stage
  const int KT = Cn / GBK;
  GFrag f0, f1;
  dma(0, 0);
  if (KT > 1) dma(1, 1);
  if (KT > 2) dma(2, 2);
  if (KT > 2) wait_vmcnt<2 * NL>(); else if (KT > 1) wait_vmcnt<NL>(); else wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
  read_frag(f0, 0, 0);
  auto phase = [&](int kt, int buf) __attribute__((always_inline)) {
    read_frag(f1, buf, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < KT) {
      if (kt + 2 < KT) wait_vmcnt<NL>(); else wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
      if (kt + 3 < KT) dma(kt + 3, buf);
      read_frag(f0, buf == 2 ? 0 : buf + 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f1);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < KT; kt += 3) {
    phase(kt, 0);
    if (kt + 1 < KT) phase(kt + 1, 1);
    if (kt + 2 < KT) phase(kt + 2, 2);
  }

  // Epilogue: lane l / register r of a 32 x 32 block hold row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32.
  const float s = sptr ? fmaxf(sptr[0], kEpsQ) : 1.0f;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + wi * (32 * RB) + rb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        const int col = j0 + wj * 128 + cb * 32 + l32;
        if (row < I && col < J) out[(size_t)row * J + col] = acc[rb][cb][r] * s;
      }
}

// The same product with 64 c per stage (contraction length a multiple of
// 64): rows of 128 bytes whose 16-byte units are xor-swizzled by
// (row >> 1) & 7 (conflict-free for the fragment reads, by the bank-conflict
// counter), two stage buffers (128 KiB), stage kt+2 requested once every
// wave is done with stage kt, so one barrier per 64 c instead of per 32.
// Waiting at the per-stage barrier was about a fifth of the 32-c kernel's
// loop time; with half the barriers the backward step took 2.24 instead of
// 2.35 ms.  The MFMA sequence per output is the same, so the results are
// identical.
constexpr int G2BK = 64, G2ROW = G2BK * 2, G2UNITS = G2ROW / 16;
constexpr int G2_A_STAGE = GT * G2ROW, G2_STAGE = 2 * G2_A_STAGE;
HBL_DEV int gswz2(int row) { return (row >> 1) & 7; }
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_bf16_nt64_kernel(const uint16_t* __restrict__ A,
                                                                   const uint16_t* __restrict__ B,
                                                                   const float* __restrict__ sptr,
                                                                   float* __restrict__ out, int I, int J, int Cn,
                                                                   int tiles_i, int tiles_j) {
  constexpr int WI = NW / 2;
  constexpr int RB = GT / WI / 32;
  constexpr int CP = 32 / NW;                 // 1 KiB copies per wave per operand per stage
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * G2_STAGE];
  const int bid = blockIdx.x, total = tiles_i * tiles_j;
  const int logical = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  constexpr int GM = 4;
  const int per_group = GM * tiles_j;
  const int first_i = (logical / per_group) * GM;
  const int gm = min(tiles_i - first_i, GM);
  const int in_g = logical % per_group;
  const int i0 = (first_i + in_g % gm) * GT;
  const int j0 = (in_g / gm) * GT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;
  const uint16_t* a_src[CP];
  const uint16_t* b_src[CP];
#pragma unroll
  for (int j = 0; j < CP; ++j) {
    const int P = (j * NW + wave) * 64 + lane, row = P / G2UNITS, u = (P % G2UNITS) ^ gswz2(row);
    a_src[j] = A + (size_t)min(i0 + row, I - 1) * Cn + 8 * u;
    b_src[j] = B + (size_t)min(j0 + row, J - 1) * Cn + 8 * u;
  }
  auto dma = [&](int kt, int buf) {
    uint8_t* base = smem + buf * G2_STAGE;
#pragma unroll
    for (int j = 0; j < CP; ++j) lds_copy16(a_src[j] + (size_t)kt * G2BK, base + (j * NW + wave) * 1024);
#pragma unroll
    for (int j = 0; j < CP; ++j) lds_copy16(b_src[j] + (size_t)kt * G2BK, base + G2_A_STAGE + (j * NW + wave) * 1024);
  };
  v16f acc[RB][4];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  struct GFrag {
    bf8v a[RB], b[4];
  };
  auto read_frag = [&](GFrag& f, int buf, int ks) __attribute__((always_inline)) {
    const uint8_t* sa = smem + buf * G2_STAGE;
    const uint8_t* sb = sa + G2_A_STAGE;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = wi * (32 * RB) + rb * 32 + l32;
      f.a[rb] = *reinterpret_cast<const bf8v*>(sa + row * G2ROW + 16 * ((2 * ks + g) ^ gswz2(row)));
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int row = wj * 128 + cb * 32 + l32;
      f.b[cb] = *reinterpret_cast<const bf8v*>(sb + row * G2ROW + 16 * ((2 * ks + g) ^ gswz2(row)));
    }
  };
  auto mfmas = [&](const GFrag& f) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[rb], f.b[cb], acc[rb][cb], 0, 0, 0);
  };
  constexpr int NL = 2 * CP;
  const int KT = Cn / G2BK;
  GFrag f0, f1;
  dma(0, 0);
  if (KT > 1) dma(1, 1);
  if (KT > 1) wait_vmcnt<NL>(); else wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
  read_frag(f0, 0, 0);
  // stage kt in buffer kt & 1: k-steps 0..3; each k-step's MFMAs run while the
  // next k-step's fragments are read.  Before the last k-step's MFMAs: wait
  // for stage kt+1 (the only copies in flight), barrier (every wave has read
  // all of stage kt), request stage kt+2 into this buffer, read stage kt+1's
  // first fragments.
  auto stage = [&](int kt, int buf) __attribute__((always_inline)) {
    read_frag(f1, buf, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0);
    __builtin_amdgcn_sched_barrier(0);
    read_frag(f0, buf, 2);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f1);
    __builtin_amdgcn_sched_barrier(0);
    read_frag(f1, buf, 3);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f0);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < KT) {
      wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
      if (kt + 2 < KT) dma(kt + 2, buf);
      read_frag(f0, buf ^ 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfmas(f1);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < KT; kt += 2) {
    stage(kt, 0);
    if (kt + 1 < KT) stage(kt + 1, 1);
  }
  const float s = sptr ? fmaxf(sptr[0], kEpsQ) : 1.0f;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + wi * (32 * RB) + rb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        const int col = j0 + wj * 128 + cb * 32 + l32;
        if (row < I && col < J) out[(size_t)row * J + col] = acc[rb][cb][r] * s;
      }
}

// ---------------------------------------------------------------------------
// Fused transform + RMSNorm backward, one token per T threads (persistent
// over tokens like the forward's prep): dxh (fp32, pass-0 dealing: 8
// contiguous features per group) -> FWHT -> back to the pass-0 dealing ->
// du = (.) / sqrt(K); with x and g in the same dealing:
//   r = sqrt(mean x^2 + eps), S = sum du g x,
//   dx = g du / r - x S / (K r^3),   dg partial += du x / r.
// Without the rotation du = dxh.  dg partials: one row of K per (workgroup,
// token slot), summed by dg_reduce_kernel in a fixed order.
template <int LOGK, int LOGE, int P2, int PA, int PB>
HBL_DEV void exchange_to(float (&v)[1 << LOGE], float* region, int tau) {
  using A = Pass<LOGK, LOGE, PA>;
  using Bn = Pass<LOGK, LOGE, PB>;
  constexpr int E = 1 << LOGE;
  const int wbase = pad<P2>(A::thr_idx(tau));
#pragma unroll
  for (int r = 0; r < E; ++r) region[wbase + pad<P2>(A::reg_idx(r))] = v[r];
  __syncthreads();
  const int rbase = pad<P2>(Bn::thr_idx(tau));
#pragma unroll
  for (int r = 0; r < E; ++r) v[r] = region[rbase + pad<P2>(Bn::reg_idx(r))];
  __syncthreads();
}

constexpr int bwd_wg(int logk, int loge) { return (1 << (logk - loge)) < 64 ? 64 : (1 << (logk - loge)); }

template <int LOGK, int LOGE, int P2, bool XBF16, bool DXBF16, bool ROT>
__global__ __launch_bounds__(bwd_wg(LOGK, LOGE)) void bwd_prep_kernel(
    const float* __restrict__ dxh, const void* __restrict__ x, const float* __restrict__ gain, int M,
    void* __restrict__ dx, float* __restrict__ dgpart) {
  using C = PrepCfg<LOGK, LOGE, P2>;
  using P0 = Pass<LOGK, LOGE, 0>;
  constexpr int K = C::K, E = C::E, T = C::T;
  __shared__ __attribute__((aligned(16))) float lds[C::REGION * C::TPB];
  __shared__ float red[32];
  const int tok = threadIdx.x / T, tau = threadIdx.x % T;
  float* region = lds + tok * C::REGION;
  const int stride = gridDim.x * C::TPB;
  const int first = blockIdx.x * C::TPB;
  const int iters = first < M ? (M - first + stride - 1) / stride : 0;   // uniform over the workgroup
  const int base0 = P0::thr_idx(tau);

  // gain in the pass-0 dealing, read from L1/L2 where needed
  auto gain8 = [&](int gi, float (&gg)[8]) {
    if (gain) {
      const float4* p = reinterpret_cast<const float4*>(gain + base0 + P0::reg_idx(8 * gi));
      const float4 a = p[0], b = p[1];
      gg[0] = a.x; gg[1] = a.y; gg[2] = a.z; gg[3] = a.w; gg[4] = b.x; gg[5] = b.y; gg[6] = b.z; gg[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gg[e] = 1.0f;
    }
  };
  float dg[E];
#pragma unroll
  for (int r = 0; r < E; ++r) dg[r] = 0.0f;

  for (int it = 0; it < iters; ++it) {
    const int m = first + tok + it * stride;
    const bool valid = m < M;
    const int mm = valid ? m : M - 1;
    float v[E];
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      const int idx = base0 + P0::reg_idx(8 * gi);
      const float4* p = reinterpret_cast<const float4*>(dxh + (size_t)mm * K + idx);
      const float4 a = p[0], b = p[1];
      v[8 * gi + 0] = a.x; v[8 * gi + 1] = a.y; v[8 * gi + 2] = a.z; v[8 * gi + 3] = a.w;
      v[8 * gi + 4] = b.x; v[8 * gi + 5] = b.y; v[8 * gi + 6] = b.z; v[8 * gi + 7] = b.w;
    }
    if constexpr (ROT) {
      run_passes<LOGK, LOGE, P2, 0>(v, region, tau);
      if constexpr (C::NP > 1) exchange_to<LOGK, LOGE, P2, C::NP - 1, 0>(v, region, tau);
      const float rs = 1.0f / sqrtf((float)K);
#pragma unroll
      for (int r = 0; r < E; ++r) v[r] *= rs;
    }
    // x of this token in the same dealing (bf16 kept packed: E/2 registers)
    RawX<E, XBF16> raw;
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      const int idx = base0 + P0::reg_idx(8 * gi);
      if constexpr (XBF16) {
        raw.u[gi] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)mm * K + idx);
      } else {
        const uint4* q = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + (size_t)mm * K + idx);
        raw.u[2 * gi] = q[0];
        raw.u[2 * gi + 1] = q[1];
      }
    }
    auto x8 = [&](int gi, float (&xx)[8]) {
      if constexpr (XBF16) {
        const uint4 w = raw.u[gi];
        xx[0] = bf16_lo(w.x); xx[1] = bf16_hi(w.x); xx[2] = bf16_lo(w.y); xx[3] = bf16_hi(w.y);
        xx[4] = bf16_lo(w.z); xx[5] = bf16_hi(w.z); xx[6] = bf16_lo(w.w); xx[7] = bf16_hi(w.w);
      } else {
        const uint4 a = raw.u[2 * gi], b = raw.u[2 * gi + 1];
        xx[0] = __uint_as_float(a.x); xx[1] = __uint_as_float(a.y); xx[2] = __uint_as_float(a.z);
        xx[3] = __uint_as_float(a.w); xx[4] = __uint_as_float(b.x); xx[5] = __uint_as_float(b.y);
        xx[6] = __uint_as_float(b.z); xx[7] = __uint_as_float(b.w);
      }
    };
    float ss = 0.0f, sd = 0.0f;
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      float xx[8], gg[8];
      x8(gi, xx);
      gain8(gi, gg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = __builtin_fmaf(xx[e], xx[e], ss);
        sd = __builtin_fmaf(v[8 * gi + e] * gg[e], xx[e], sd);
      }
    }
    token_reduce2<T, false>(ss, sd, red);
    const float rr = sqrtf(ss * (1.0f / K) + kEpsNorm);
    const float ir = 1.0f / rr;
    const float cx = sd * ir * ir * ir * (1.0f / K);
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      float xx[8], gg[8], o[8];
      x8(gi, xx);
      gain8(gi, gg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = gg[e] * v[8 * gi + e] * ir - xx[e] * cx;
        if (valid) dg[8 * gi + e] = __builtin_fmaf(v[8 * gi + e] * xx[e], ir, dg[8 * gi + e]);
      }
      if (valid) {
        const int idx = base0 + P0::reg_idx(8 * gi);
        if constexpr (DXBF16) {
          uint4 w;
          w.x = f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
          w.y = f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
          w.z = f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
          w.w = f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(dx) + (size_t)m * K + idx) = w;
        } else {
          float4* q = reinterpret_cast<float4*>(static_cast<float*>(dx) + (size_t)m * K + idx);
          q[0] = make_float4(o[0], o[1], o[2], o[3]);
          q[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
      }
    }
  }
  if (dgpart) {
    float* row = dgpart + ((size_t)blockIdx.x * C::TPB + tok) * K;
#pragma unroll
    for (int gi = 0; gi < E / 8; ++gi) {
      const int idx = base0 + P0::reg_idx(8 * gi);
      float4* q = reinterpret_cast<float4*>(row + idx);
      q[0] = make_float4(dg[8 * gi + 0], dg[8 * gi + 1], dg[8 * gi + 2], dg[8 * gi + 3]);
      q[1] = make_float4(dg[8 * gi + 4], dg[8 * gi + 5], dg[8 * gi + 6], dg[8 * gi + 7]);
    }
  }
}

// dg[k] = sum of the partial rows in a fixed order: a workgroup owns 64
// columns; its 4 waves sum interleaved row sets (8 independent loads in
// flight per lane) and the 4 partial sums are added in wave order.
__global__ __launch_bounds__(256) void dg_reduce_kernel(const float* __restrict__ part, int rows, int K,
                                                        float* __restrict__ dg) {
  __shared__ float ps[4][64];
  const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k = blockIdx.x * 64 + c;
  float s = 0.0f;
  if (k < K) {
    int i = w;
    for (; i + 28 < rows; i += 32) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(i + 4 * u) * K + k];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; i < rows; i += 4) s += part[(size_t)i * K + k];
  }
  ps[w][c] = s;
  __syncthreads();
  if (w == 0 && k < K) dg[k] = ((ps[0][c] + ps[1][c]) + ps[2][c]) + ps[3][c];
}

// Transform configurations: one token of K features over T threads x E
// registers.  The backward keeps more per feature live (gradient, x, gain
// sums) than the forward, so from K = 4096 it uses 16 registers per thread
// and more exchanges: 315 us instead of 378 us (64 registers) at K = 16384,
// M = 8192.
template <bool XBF16, bool DXBF16, bool ROT>
hipError_t launch_bwd_prep_t(const BwdArgs& a, int grid, float* dgpart) {
#define HBL_BP(LK, LE, P2)                                                                                   \
  case LK:                                                                                                   \
    hipLaunchKernelGGL((bwd_prep_kernel<LK, LE, P2, XBF16, DXBF16, ROT>), dim3(grid),                       \
                       dim3(PrepCfg<LK, LE, P2>::WG), 0, a.stream, a.dxh, a.x, a.gain, a.M, a.dx, dgpart); \
    break;
  switch (a.logk) {
    HBL_BP(6, 4, 6) HBL_BP(7, 4, 6) HBL_BP(8, 4, 6) HBL_BP(9, 5, 6) HBL_BP(10, 5, 7) HBL_BP(11, 6, 7)
    HBL_BP(12, 4, 6) HBL_BP(13, 4, 6) HBL_BP(14, 4, 6) HBL_BP(15, 5, 7)
    default: return hipErrorInvalidValue;
  }
#undef HBL_BP
  return hipGetLastError();
}

}  // namespace

int bwd_prep_tpb(int logk) {
  switch (logk) {
    case 6: return PrepCfg<6, 4, 6>::TPB;
    case 7: return PrepCfg<7, 4, 6>::TPB;
    case 8: return PrepCfg<8, 4, 6>::TPB;
    case 9: return PrepCfg<9, 5, 6>::TPB;
    case 10: return PrepCfg<10, 5, 7>::TPB;
    case 11: return PrepCfg<11, 6, 7>::TPB;
    case 12: return PrepCfg<12, 4, 6>::TPB;
    case 13: return PrepCfg<13, 4, 6>::TPB;
    case 14: return PrepCfg<14, 4, 6>::TPB;
    case 15: return PrepCfg<15, 5, 7>::TPB;
    default: return 0;
  }
}

hipError_t launch_wbt(const uint8_t* wpack, int N, int K, uint16_t* wbt, hipStream_t stream) {
  const int64_t threads = (int64_t)K * (N / 8);
  hipLaunchKernelGGL(wbt_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, wpack, N, K, wbt);
  return hipGetLastError();
}

hipError_t launch_transpose_tokens(int kind, const void* src, const float* dscale, int M, int C, int Mp,
                                   uint16_t* dst, hipStream_t stream) {
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)(Mp / 64));
  if (kind == 0) hipLaunchKernelGGL(tr_kernel<0>, grid, dim3(256), 0, stream, src, dscale, M, C, Mp, dst);
  else if (kind == 8) hipLaunchKernelGGL(tr_kernel<8>, grid, dim3(256), 0, stream, src, dscale, M, C, Mp, dst);
  else hipLaunchKernelGGL(tr_kernel<4>, grid, dim3(256), 0, stream, src, dscale, M, C, Mp, dst);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_nt(const uint16_t* A, const uint16_t* B, const float* scale, float* out, int I, int J,
                               int Cn, hipStream_t stream) {
  const int ti = (I + GT - 1) / GT, tj = (J + GT - 1) / GT;
  if (Cn % G2BK == 0) {
    hipLaunchKernelGGL(gemm_bf16_nt64_kernel<HBL_BF16_NW>, dim3(ti * tj), dim3(64 * HBL_BF16_NW), 0, stream, A, B,
                       scale, out, I, J, Cn, ti, tj);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gemm_bf16_nt_kernel<HBL_BF16_NW>, dim3(ti * tj), dim3(64 * HBL_BF16_NW), 0, stream, A, B, scale,
                     out, I, J, Cn, ti, tj);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdArgs& a, int grid, float* dgpart) {
#define HBL_BPX(XB, DB, R) \
  if (a.x_bf16 == XB && a.dx_bf16 == DB && a.rotate == R) return launch_bwd_prep_t<XB, DB, R>(a, grid, dgpart);
  HBL_BPX(true, true, true) HBL_BPX(true, false, true) HBL_BPX(false, true, true) HBL_BPX(false, false, true)
  HBL_BPX(true, true, false) HBL_BPX(true, false, false) HBL_BPX(false, true, false) HBL_BPX(false, false, false)
#undef HBL_BPX
  return hipErrorInvalidValue;
}

hipError_t launch_dg_reduce(const float* part, int rows, int K, float* dg, hipStream_t stream) {
  hipLaunchKernelGGL(dg_reduce_kernel, dim3((unsigned)((K + 63) / 64)), dim3(256), 0, stream, part, rows, K, dg);
  return hipGetLastError();
}

}  // namespace hbl
