// Ternary integer matmul with dequant epilogue on gfx950 int8 MFMA.
//
// acc[m][n] = sum_k q[m][k] * W_t[n][k]   (exact, int32)
// y[m][n]   = acc[m][n] * (d[m] * max(alpha, 1e-5))
// QbitAI article on BitNet v2, section 引入H-BitLinear模块: the layer is a
// matmul of the quantised activations with the ternary weights, followed by
// dequantisation; 新智元 article, section 原生4比特盘算: dense compute suits
// batched inference.
//
// Two kernels:
//  * prefill (large M): 256x256 output tile per 256-thread workgroup, 2x2
//    waves of 128x128, v_mfma_i32_32x32x32_i8, K staged 128 at a time through
//    double-buffered LDS.  Packed 2-bit weights stay packed in LDS (a quarter
//    of the bytes) and are expanded to int8 in registers right before the
//    MFMA with one byte-permute lookup per dword; INT4 activation codes are
//    likewise kept packed and sign-extended in registers.
//  * decode (M <= 64): weight streaming.  Every wave owns 16 output channels
//    and one K slab, loads its packed weights with 16-byte loads straight into
//    registers (each weight byte is read from HBM once), and runs
//    v_mfma_i32_16x16x64_i8 with the channels on the MFMA's M side and up to
//    16 tokens on its N side.  The K slabs of one channel block are reduced
//    exactly in int32 by the last workgroup to finish, which also dequantises.
//
// Inside one MFMA the pairing of A and B bytes is what matters: lane group g
// (lanes 32g..32g+31, or 16g.. for 16x16x64) byte b of A meets byte b of B.
// Both operands are therefore fed the same k for every (group, byte), and the
// k order across the K loop is free.  Per 128-k stage, lane group g of the
// 32x32x32 MFMA covers k-chunks 4g..4g+3 (16 k each), one chunk per MFMA step;
// that makes every weight fragment one contiguous 16-byte read.
#include "common.h"
#include "launch.h"

namespace hbl {

// Operand expansion without lookups.
//
// A packed weight word holds the 2-bit two's complement codes of 16
// consecutive k, the code of k0+4j+i in bits 8i+2j (field j of byte i).
// Shifting field j to the top of its byte and masking gives, byte by byte,
// exactly 64*w as a signed int8 (0x40 = +64, 0xC0 = -64).  MFMA step j of a
// 64-k group takes field j of four packed words, so its operand covers codes
// 16d + 4j + i (d = word, i = byte): 1-2 VALU ops per operand dword.
HBL_DEV uint32_t wfield(uint32_t p, int j) {
  return (j == 3 ? p : (p << (6 - 2 * j))) & 0xC0C0C0C0u;
}
// INT4 activation words hold codes 8 at a time, the code of k0+4j+i in bits
// 8i+4j.  Moving a nibble to the top of its byte gives 16*q as a signed int8.
// For the same code set 16d + 4j + i, step j takes the low (j even) or high
// (j odd) nibbles of word 2d + j/2.
HBL_DEV uint32_t a4field(uint32_t w, int j) {
  return ((j & 1) ? w : (w << 4)) & 0xF0F0F0F0u;
}
// The accumulators therefore hold 64 * acc (INT8 path) or 1024 * acc (INT4),
// exact multiples whose magnitude stays below 2^27 for K <= 16384 (|q| <= 128
// after scaling, |w| = 64): an arithmetic shift recovers acc exactly.
template <int BITS>
HBL_DEV int unscale(int v) { return BITS == 8 ? (v >> 6) : (v >> 10); }
HBL_DEV uint32_t u4get(const uint4& u, int j) { return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w; }

template <int OUT>
HBL_DEV void store_out(void* Y, size_t off, int acc, float t) {
  if constexpr (OUT == OUT_ACC_I32) {
    static_cast<int32_t*>(Y)[off] = acc;
  } else if constexpr (OUT == OUT_F32) {
    static_cast<float*>(Y)[off] = (float)acc * t;
  } else {
    static_cast<uint16_t*>(Y)[off] = f32_to_bf16((float)acc * t);
  }
}

// ===========================================================================
// Prefill
constexpr int PBM = 256, PBN = 256, PBK = 128;

template <int BITS>
struct PCfg {
  static constexpr int ABYTES = BITS == 8 ? PBK : PBK / 2;  // A bytes per row per stage
  static constexpr int AUNITS = ABYTES / 16;
  static constexpr int A_STAGE = PBM * ABYTES;
  static constexpr int B_STAGE = PBN * (PBK / 4);
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int A_LOADS = A_STAGE / 16 / 256;
  static constexpr int B_LOADS = B_STAGE / 16 / 256;
};

// XOR swizzles of the 16-byte units of an LDS row, chosen so the MFMA
// fragment reads (8 or 16 lanes per LDS cycle, rows r..r+7 / r+15 of one
// unit column) and the staging writes hit distinct banks.
template <int BITS>
HBL_DEV int swz_a(int row) {
  if constexpr (BITS == 8) return (row ^ (row >> 3)) & 7;
  else return ((row >> 1) ^ (row >> 3)) & 3;
}
HBL_DEV int swz_b(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

template <int BITS, int OUT>
__global__ __launch_bounds__(256, 1) void gemm_prefill_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K, int tiles_m, int tiles_n) {
  using C = PCfg<BITS>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  // Tile order: consecutive workgroups go to different XCDs, so give each XCD
  // a contiguous run of logical tiles, and walk them in groups of 4 tile-rows
  // so the tiles resident on one XCD share A rows and weight columns in its L2.
  const int bid = blockIdx.x, total = tiles_m * tiles_n;
  const int logical = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  constexpr int GM = 4;
  const int per_group = GM * tiles_n;
  const int first_m = (logical / per_group) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_g = logical % per_group;
  const int m0 = (first_m + in_g % gm) * PBM;
  const int n0 = (in_g / gm) * PBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;
  const size_t arow = BITS == 8 ? (size_t)K : (size_t)K / 2;
  const size_t wrow = (size_t)K / 4;

  uint4 ra[C::A_LOADS], rb[C::B_LOADS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < C::A_LOADS; ++j) {
      const int q = j * 256 + tid, row = q / C::AUNITS, u = q % C::AUNITS, m = m0 + row;
      ra[j] = m < M ? *reinterpret_cast<const uint4*>(A + (size_t)m * arow + (size_t)kt * C::ABYTES + 16 * u)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j) {
      const int q = j * 256 + tid, row = q >> 1, u = q & 1, n = n0 + row;
      rb[j] = n < N ? *reinterpret_cast<const uint4*>(W + (size_t)n * wrow + (size_t)kt * (PBK / 4) + 16 * u)
                    : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* sa = smem + buf * C::STAGE;
    uint8_t* sb = sa + C::A_STAGE;
#pragma unroll
    for (int j = 0; j < C::A_LOADS; ++j) {
      const int q = j * 256 + tid, row = q / C::AUNITS, u = q % C::AUNITS;
      *reinterpret_cast<uint4*>(sa + row * C::ABYTES + 16 * (u ^ swz_a<BITS>(row))) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j) {
      const int q = j * 256 + tid, row = q >> 1, u = q & 1;
      *reinterpret_cast<uint4*>(sb + row * 32 + 16 * (u ^ swz_b(row))) = rb[j];
    }
  };

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};

  const int KT = K / PBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t* sa = smem + buf * C::STAGE;
    const uint8_t* sb = sa + C::A_STAGE;
    // weight fragments: 4 packed words = k-chunks 4g..4g+3 of channel n
    uint4 bq[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int n = wn * 128 + cb * 32 + l32;
      bq[cb] = *reinterpret_cast<const uint4*>(sb + n * 32 + 16 * (g ^ swz_b(n)));
    }
    // activation fragments: k-chunks 4g..4g+3 of row m (64 codes)
    uint4 aq[4][4];
#pragma unroll
    for (int rbk = 0; rbk < 4; ++rbk) {
      const int row = wm * 128 + rbk * 32 + l32;
      if constexpr (BITS == 8) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          aq[rbk][d] = *reinterpret_cast<const uint4*>(sa + row * 128 + 16 * ((4 * g + d) ^ swz_a<8>(row)));
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          aq[rbk][h] = *reinterpret_cast<const uint4*>(sa + row * 64 + 16 * ((2 * g + h) ^ swz_a<4>(row)));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4i bf[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        bf[cb] = v4i{(int)wfield(bq[cb].x, j), (int)wfield(bq[cb].y, j), (int)wfield(bq[cb].z, j),
                     (int)wfield(bq[cb].w, j)};
#pragma unroll
      for (int rbk = 0; rbk < 4; ++rbk) {
        v4i af;
        if constexpr (BITS == 8) {
          // dword j of chunks 4g..4g+3: codes 16d + 4j .. +3
          af = v4i{(int)u4get(aq[rbk][0], j), (int)u4get(aq[rbk][1], j), (int)u4get(aq[rbk][2], j),
                   (int)u4get(aq[rbk][3], j)};
        } else {
          // chunk d = words 2d, 2d+1 of the 32 bytes; step j uses word 2d + j/2
          const uint32_t w[8] = {aq[rbk][0].x, aq[rbk][0].y, aq[rbk][0].z, aq[rbk][0].w,
                                 aq[rbk][1].x, aq[rbk][1].y, aq[rbk][1].z, aq[rbk][1].w};
          af = v4i{(int)a4field(w[0 + (j >> 1)], j), (int)a4field(w[2 + (j >> 1)], j),
                   (int)a4field(w[4 + (j >> 1)], j), (int)a4field(w[6 + (j >> 1)], j)};
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[rbk][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf[cb], acc[rbk][cb], 0, 0, 0);
      }
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 32x32 accumulator layout, lane l / register r hold
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
#pragma unroll
  for (int rbk = 0; rbk < 4; ++rbk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 128 + rbk * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (m >= M) continue;
      const float t = OUT == OUT_ACC_I32 ? 0.f : dscale[m] * aw;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int n = n0 + wn * 128 + cb * 32 + l32;
        if (n < N) store_out<OUT>(Y, (size_t)m * N + n, unscale<BITS>(acc[rbk][cb][r]), t);
      }
    }
  }
}

// ===========================================================================
// Decode (M <= 64): weight streaming.
//
// A workgroup of 4 waves owns 16*CPW output channels and one of S equal K
// ranges.  The range is cut into 256-k blocks dealt round-robin to the waves;
// each wave issues all its packed-weight loads (16 bytes per lane per block)
// up front, so every weight byte is read from HBM once with the whole stream
// in flight, and reads the (small, L2-resident) activation codes per block.
// v_mfma_i32_16x16x64_i8 runs with channels on the MFMA's M side and up to 16
// tokens on its N side.  The waves' int32 partials meet in LDS through integer
// atomics (exact, order free).  With S > 1 a second small kernel sums the S
// partials in order and dequantises; integer sums are exact, so the result is
// the same for every S.
constexpr int DKB = 256;

struct DecodePlan { int cpw, S, mb; };
static DecodePlan decode_plan(int M, int K) {
  DecodePlan p = M <= 4 ? DecodePlan{1, 1, 1} : M <= 16 ? DecodePlan{2, 2, 1} : DecodePlan{4, 4, 4};
  while (p.S > 1 && K / p.S < DKB) p.S /= 2;
  return p;
}
// Weight blocks a wave may hold in registers (MAXB * CPW uint4 <= 16).
constexpr int decode_maxb(int cpw) { return 16 / cpw; }

template <int BITS, int MB, int CPW, int OUT>
__global__ __launch_bounds__(256) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K, int S,
    int32_t* __restrict__ partial) {
  constexpr int MAXB = decode_maxb(CPW);
  constexpr int CH = 16 * CPW;
  __shared__ int red[CH * MB * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ch0 = blockIdx.x * CH, s = blockIdx.y;
  const int Kr = K / S, kbeg = s * Kr;
  const int nblk = Kr / DKB;                       // 256-k blocks in this range
  const int nb = nblk > wave ? (nblk - wave + 3) / 4 : 0;   // blocks of this wave: wave, wave+4, ...
  const size_t arow = (size_t)K * BITS / 8;

  for (int i = tid; i < CH * MB * 16; i += 256) red[i] = 0;

  // ---- all weight loads of this wave: block b = wave + 4i, channel ch0 + 16cp + c, k [64g, 64g+64)
  uint4 wq[MAXB][CPW];
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
#pragma unroll
    for (int cp = 0; cp < CPW; ++cp) {
      const int n = ch0 + 16 * cp + c;
      const int kb = kbeg + (wave + 4 * i) * DKB;
      wq[i][cp] = (i < nb && n < N) ? *reinterpret_cast<const uint4*>(W + (size_t)n * (K / 4) + kb / 4 + 16 * g)
                                    : make_uint4(0, 0, 0, 0);
    }
  }
  v4i acc[CPW][MB];
#pragma unroll
  for (int cp = 0; cp < CPW; ++cp)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[cp][mb] = v4i{};

#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    if (i >= nb) continue;   // wave-uniform; keeps the loop fully unrolled (wq stays in registers)
    const int kb = kbeg + (wave + 4 * i) * DKB + 64 * g;   // this lane's 64 codes
    uint4 aq[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int t = 16 * mb + c;
      const uint8_t* ap = A + (size_t)t * arow + (size_t)kb * BITS / 8;
#pragma unroll
      for (int d = 0; d < BITS / 2; ++d)
        aq[mb][d] = t < M ? reinterpret_cast<const uint4*>(ap)[d] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int cp = 0; cp < CPW; ++cp) {
        const uint4 p = wq[i][cp];
        const v4i wop = v4i{(int)wfield(p.x, j), (int)wfield(p.y, j), (int)wfield(p.z, j), (int)wfield(p.w, j)};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          v4i aop;
          if constexpr (BITS == 8) {
            aop = v4i{(int)u4get(aq[mb][0], j), (int)u4get(aq[mb][1], j), (int)u4get(aq[mb][2], j),
                      (int)u4get(aq[mb][3], j)};
          } else {
            const uint32_t w[8] = {aq[mb][0].x, aq[mb][0].y, aq[mb][0].z, aq[mb][0].w,
                                   aq[mb][1].x, aq[mb][1].y, aq[mb][1].z, aq[mb][1].w};
            aop = v4i{(int)a4field(w[0 + (j >> 1)], j), (int)a4field(w[2 + (j >> 1)], j),
                      (int)a4field(w[4 + (j >> 1)], j), (int)a4field(w[6 + (j >> 1)], j)};
          }
          acc[cp][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, aop, acc[cp][mb], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();
  // 16x16 accumulator layout: lane l / register r hold channel 4*(l/16)+r, token l%16
#pragma unroll
  for (int cp = 0; cp < CPW; ++cp)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        atomicAdd(&red[(16 * mb + c) * CH + 16 * cp + 4 * g + r], acc[cp][mb][r]);
  __syncthreads();

  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
  for (int e = tid; e < M * CH && e < MB * 16 * CH; e += 256) {
    const int t = e / CH, n = ch0 + e % CH;
    if (n >= N) continue;
    const int v = red[e];
    if (S == 1) {
      const float tt = OUT == OUT_ACC_I32 ? 0.f : dscale[t] * aw;
      store_out<OUT>(Y, (size_t)t * N + n, unscale<BITS>(v), tt);
    } else {
      partial[((size_t)s * M + t) * N + n] = v;
    }
  }
}

// Sum of the S partials in slab order, then unscale and dequantise.
template <int BITS, int OUT>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const int32_t* __restrict__ partial, int S, int M, int N,
                                                           const float* __restrict__ dscale,
                                                           const float* __restrict__ walpha, void* __restrict__ Y) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= M * N) return;
  int v = 0;
  for (int s = 0; s < S; ++s) v += partial[(size_t)s * M * N + e];
  const int t = e / N;
  const float tt = OUT == OUT_ACC_I32 ? 0.f : dscale[t] * fmaxf(walpha[0], kEpsQ);
  store_out<OUT>(Y, (size_t)e, unscale<BITS>(v), tt);
}

// ===========================================================================
// Host side

size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M > 64 || M <= 0) return 0;
  const DecodePlan p = decode_plan((int)M, (int)K);
  return p.S > 1 ? (((size_t)p.S * M * N * 4 + 255) & ~(size_t)255) : 0;
}

template <int BITS, int MB, int CPW, int OUT>
static void launch_decode_p(const GemmArgs& a, int S) {
  constexpr int CH = 16 * CPW;
  dim3 grid((a.N + CH - 1) / CH, S);
  int32_t* part = static_cast<int32_t*>(a.ws);
  hipLaunchKernelGGL((gemm_decode_kernel<BITS, MB, CPW, OUT>), grid, dim3(256), 0, a.stream, a.codes, a.wpack,
                     a.dscale, a.walpha, a.out, a.M, a.N, a.K, S, part);
  if (S > 1)
    hipLaunchKernelGGL((decode_reduce_kernel<BITS, OUT>), dim3((a.M * a.N + 255) / 256), dim3(256), 0, a.stream,
                       part, S, a.M, a.N, a.dscale, a.walpha, a.out);
}

template <int BITS, int OUT>
static void launch_decode_t(const GemmArgs& a) {
  const DecodePlan p = decode_plan(a.M, a.K);
  if (p.cpw == 1) launch_decode_p<BITS, 1, 1, OUT>(a, p.S);
  else if (p.cpw == 2) launch_decode_p<BITS, 1, 2, OUT>(a, p.S);
  else launch_decode_p<BITS, 4, 4, OUT>(a, p.S);
}

template <int BITS, int OUT>
static void launch_prefill_t(const GemmArgs& a) {
  const int tm = (a.M + PBM - 1) / PBM, tn = (a.N + PBN - 1) / PBN;
  hipLaunchKernelGGL((gemm_prefill_kernel<BITS, OUT>), dim3(tm * tn), dim3(256), 0, a.stream, a.codes, a.wpack,
                     a.dscale, a.walpha, a.out, a.M, a.N, a.K, tm, tn);
}

template <int BITS, int OUT>
static void launch_t(const GemmArgs& a) {
  if (a.M <= 64) launch_decode_t<BITS, OUT>(a);
  else launch_prefill_t<BITS, OUT>(a);
}

hipError_t launch_gemm(const GemmArgs& a) {
  if (a.M == 0) return hipSuccess;
#define HBL_G(BITS)                                              \
  switch (a.out_kind) {                                          \
    case OUT_ACC_I32: launch_t<BITS, OUT_ACC_I32>(a); break;     \
    case OUT_F32: launch_t<BITS, OUT_F32>(a); break;             \
    default: launch_t<BITS, OUT_BF16>(a); break;                 \
  }
  if (a.bits == 8) { HBL_G(8) } else { HBL_G(4) }
#undef HBL_G
  return hipGetLastError();
}

}  // namespace hbl
