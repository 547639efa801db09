// Ternary integer matmul with dequant epilogue on gfx950 int8 MFMA.
//
// acc[m][n] = sum_k q[m][k] * W_t[n][k]   (exact, int32)
// y[m][n]   = acc[m][n] * (d[m] * max(alpha, 1e-5))
// QbitAI article on BitNet v2, section 引入H-BitLinear模块: the layer is a
// matmul of the quantised activations with the ternary weights, followed by
// dequantisation; 新智元 article, section 原生4比特盘算: dense compute suits
// batched inference.
//
// Three kernel families:
//  * prefill on the int8 instruction (INT8 codes; INT4 codes in format 4):
//    256x256 output tile per workgroup, v_mfma_i32_32x32x32_i8, 4 waves of
//    128x128 (INT8) or 8 waves of 128x64 (INT4).  K is staged BK = 128 (INT8)
//    or 256 (INT4) codes at a time through a ring of three LDS stages filled
//    by direct global-to-LDS copies.  Packed 2-bit weights stay packed in LDS
//    (a quarter of the bytes) and are expanded to int8 in registers right
//    before the MFMA with shifts and masks (wstep / wfield); INT4 activation
//    codes likewise stay packed and each nibble is moved to the top of its
//    byte (a4field).
//  * prefill on the fp6 x fp4 instruction (INT4 codes in format 6, more than
//    64 tokens): described with gemm_fp6_kernel below.
//  * decode (M <= 64): weight streaming.  Every wave owns 16 output channels
//    (64 per workgroup above 32 tokens when the codes are row-major) and a
//    share of the 256-k blocks of its K range; its packed weights are loaded with 16-byte loads straight into
//    registers (each weight byte is read from HBM once), and
//    v_mfma_i32_16x16x64_i8 runs with the channels on the MFMA's M side and 16
//    tokens on its N side per token group.  When K is split, the partials of
//    one channel tile are summed exactly in int32 by the last workgroup to
//    finish, which also dequantises.  Up to 4 tokens, gemm_decode_few_kernel
//    stages the codes once per workgroup in LDS instead.
//
// Inside one MFMA the pairing of A and B bytes is what matters: lane group g
// (lanes 32g..32g+31, or 16g.. for 16x16x64) byte b of A meets byte b of B.
// Both operands are therefore fed the same k for every (group, byte), and the
// k order across the K loop is free.  Per 128-k half-stage, lane group g of
// the 32x32x32 MFMA covers k-chunks 4g..4g+3 (16 k each), one chunk per MFMA
// step; that makes every weight fragment one contiguous 16-byte read.
#include <mutex>
#include <type_traits>

#include "copy_schedule.h"
#include "mma.h"

namespace hbl {

// ===========================================================================
// Prefill
constexpr int PBM = 256, PBN = 256;

// Stage geometry: BK codes of K per stage (128 or 256).
template <int BITS, int BK>
struct PCfg {
  static constexpr int ABYTES = BK * BITS / 8;        // A bytes per row per stage
  static constexpr int AUNITS = ABYTES / 16;          // 16-byte units per A row
  static constexpr int BBYTES = BK / 4;               // packed weight bytes per row per stage
  static constexpr int BUNITS = BBYTES / 16;
  static constexpr int A_STAGE = PBM * ABYTES;
  static constexpr int B_STAGE = PBN * BBYTES;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int A_COPIES = A_STAGE / 16;        // 16-byte copies per stage
  static constexpr int B_COPIES = B_STAGE / 16;
  static constexpr int HALVES = BK / 128;             // 128-k sub-steps per stage
  static_assert(AUNITS == 4 || AUNITS == 8, "row of 4 or 8 units");
  static_assert(BUNITS == 2 || BUNITS == 4, "row of 2 or 4 units");
};

// XOR swizzles of the 16-byte units of an LDS row (U units per row), chosen
// so that the MFMA fragment reads (rows r..r+31 of one unit column) and the
// copies hit distinct banks.  Rows of 4 units swizzle by row bits 2-3: the
// bank-conflict counter shows that conflict-free, while bits 1 and 3 (the
// former choice) conflicted on every read.
template <int U>
HBL_DEV int swz(int row) {
  if constexpr (U == 8) return (row ^ (row >> 3)) & 7;
  else if constexpr (U == 4) return (row >> 2) & 3;
  else return ((row >> 2) ^ (row >> 3)) & 1;
}

// NWV waves: 2 along M (128 rows each) and NWV/2 along N (256/(NWV/2) columns).
template <int BITS, int BK, int NWV, int OUT>
__global__ __launch_bounds__(64 * NWV, 1) void gemm_prefill_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K, int tiles_m, int tiles_n) {
  using C = PCfg<BITS, BK>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * C::STAGE];
  constexpr int A_LOADS = C::A_COPIES / (64 * NWV), B_LOADS = C::B_COPIES / (64 * NWV);
  static_assert(A_LOADS * 64 * NWV == C::A_COPIES && B_LOADS * 64 * NWV == C::B_COPIES, "copies per thread");

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
  __shared__ __attribute__((aligned(16))) float srow[PBM];   // epilogue row scales (row_scale_copy)

  constexpr int NT = 64 * NWV;                 // threads
  constexpr int WNW = NWV / 2;                 // waves along N
  constexpr int CB = 256 / (WNW * 32);         // 32-column blocks per wave (4 or 2)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const int l32 = lane & 31, g = lane >> 5;
  const size_t arow = BITS == 8 ? (size_t)K : (size_t)K / 2;

  // Global -> LDS directly (global_load_lds_dwordx4: no staging registers),
  // three LDS stages in a ring so every stage is requested two stages before
  // it is consumed.  One wave instruction fills 1 KiB of LDS, lane L writing
  // bytes 16L..16L+15; each lane therefore fetches the global 16-byte unit
  // that the swizzled layout places at its LDS position.  Rows past M and
  // channels past N are clamped to the last valid one (never stored), so the
  // loads are unconditional.
  const uint8_t* a_src[A_LOADS];
  const uint8_t* b_src[B_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int P = (j * NWV + wave) * 64 + lane, row = P / C::AUNITS, u = (P % C::AUNITS) ^ swz<C::AUNITS>(row);
    a_src[j] = A + (size_t)min(m0 + row, M - 1) * arow + 16 * u;
  }
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int P = (j * NWV + wave) * 64 + lane, row = P / C::BUNITS, u = (P % C::BUNITS) ^ swz<C::BUNITS>(row);
    b_src[j] = W + wrow_base(min(n0 + row, N - 1), K) + 16 * u;
  }
  // packed weights of stage kt: BK = 256 is one 64-byte segment per row
  // (tiles 1 KiB apart), BK = 128 half of one
  auto bstage = [](int kt) -> size_t {
    return BK == 256 ? (size_t)kt * 1024 : (size_t)(kt >> 1) * 1024 + (size_t)(kt & 1) * 32;
  };
  auto dma = [&](int kt, int buf) {
    uint8_t* base = smem + buf * C::STAGE;
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j)
      lds_copy16(a_src[j] + (size_t)kt * C::ABYTES, base + (j * NWV + wave) * 1024);
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j)
      lds_copy16(b_src[j] + bstage(kt), base + C::A_STAGE + (j * NWV + wave) * 1024);
  };

  v16i acc[4][CB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = v16i{};

  auto compute = [&](int buf) {
    const uint8_t* sa = smem + buf * C::STAGE;
    const uint8_t* sb = sa + C::A_STAGE;
#pragma unroll
    for (int hh = 0; hh < C::HALVES; ++hh) {
      // weight fragments: 4 packed words = k-chunks 4g..4g+3 (of this 128-k half) of channel n
      uint4 bq[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = wn * (32 * CB) + cb * 32 + l32;
        bq[cb] = *reinterpret_cast<const uint4*>(sb + n * C::BBYTES + 16 * ((2 * hh + g) ^ swz<C::BUNITS>(n)));
      }
      // activation fragments: k-chunks 4g..4g+3 of row m (64 codes)
      uint4 aq[4][4];
#pragma unroll
      for (int rbk = 0; rbk < 4; ++rbk) {
        const int row = wm * 128 + rbk * 32 + l32;
        if constexpr (BITS == 8) {
#pragma unroll
          for (int d = 0; d < 4; ++d)
            aq[rbk][d] = *reinterpret_cast<const uint4*>(
                sa + row * C::ABYTES + 16 * ((8 * hh + 4 * g + d) ^ swz<C::AUNITS>(row)));
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            aq[rbk][h] = *reinterpret_cast<const uint4*>(
                sa + row * C::ABYTES + 16 * ((4 * hh + 2 * g + h) ^ swz<C::AUNITS>(row)));
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // INT8: step j = weight word j (k-chunk 4g+j) against that chunk's 16
        // codes as loaded; INT4: field j of the four weight words against the
        // matching nibbles of the four activation words (the pairing the INT4
        // decode kernel measured faster with; 1 op per operand dword)
        v4i bf[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          if constexpr (BITS == 8)
            bf[cb] = wstep(u4get(bq[cb], j));
          else
            bf[cb] = v4i{(int)wfield(bq[cb].x, j), (int)wfield(bq[cb].y, j), (int)wfield(bq[cb].z, j),
                         (int)wfield(bq[cb].w, j)};
        }
#pragma unroll
        for (int rbk = 0; rbk < 4; ++rbk) {
          v4i af;
          if constexpr (BITS == 8) {
            af = as_v4i(aq[rbk][j]);
          } else {
            // chunk d = words 2d, 2d+1 of the 32 bytes; step j uses word 2d + j/2
            const uint32_t w[8] = {aq[rbk][0].x, aq[rbk][0].y, aq[rbk][0].z, aq[rbk][0].w,
                                   aq[rbk][1].x, aq[rbk][1].y, aq[rbk][1].z, aq[rbk][1].w};
            af = v4i{(int)a4field(w[0 + (j >> 1)], j), (int)a4field(w[2 + (j >> 1)], j),
                     (int)a4field(w[4 + (j >> 1)], j), (int)a4field(w[6 + (j >> 1)], j)};
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[rbk][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf[cb], acc[rbk][cb], 0, 0, 0);
        }
      }
    }
  };

  // Stage kt lives in LDS buffer kt % 3.  Before consuming stage kt a wave
  // waits for its own copies of that stage (only the next stage's may still
  // be in flight), then the barrier makes every wave's copies visible and
  // guarantees that all waves are done with stage kt-1, whose buffer is then
  // refilled with stage kt+2.
  constexpr int NL = A_LOADS + B_LOADS;   // copy instructions per wave per stage
  using R = sched::Ring3;
  static_assert(R::NBUF == 3 && R::AHEAD == 2, "the loop below unrolls a ring of three, two stages ahead");
  static_assert(sched::ring_ok<R>(1, NL) && sched::ring_ok<R>(2, NL) && sched::ring_ok<R>(3, NL) &&
                    sched::ring_ok<R>(4, NL) && sched::ring_ok<R>(7, NL) && sched::ring_ok<R>(256, NL),
                "copy schedule: a wait leaves a needed copy in flight or a copy targets a buffer in use");
  const int KT = K / BK;
  auto phase = [&](int kt, int buf) {
    if (kt + 1 < KT) wait_vmcnt<R::wait_steady(NL)>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + R::AHEAD < KT) dma(kt + R::AHEAD, R::write_buf(buf));
    compute(buf);
  };
  if (OUT != OUT_ACC_I32) row_scale_copy(dscale, m0, M, srow, wave, lane);
  dma(0, 0);
  if (KT > 1) dma(1, 1);
  for (int kt = 0; kt < KT; kt += 3) {
    phase(kt, 0);
    if (kt + 1 < KT) phase(kt + 1, 1);
    if (kt + 2 < KT) phase(kt + 2, 2);
  }

  // ---- epilogue: 32x32 accumulator layout, lane l / register r hold
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
  if constexpr (OUT == OUT_BF16) {
    static_assert(NWV * 64 * (CB * 64 + 32) <= 3 * C::STAGE, "staging fits the ring");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");   // every wave is done with the ring
    store_bf16_staged<CB>(smem + wave * (64 * (CB * 64 + 32)), static_cast<uint16_t*>(Y), srow + wm * 128, aw, M, N,
                          m0 + wm * 128, n0 + wn * (32 * CB), lane,
                          [&](int rb, int cb, int r) { return (float)unscale<BITS>(acc[rb][cb][r]); });
    return;
  }
  __syncthreads();
#pragma unroll
  for (int rbk = 0; rbk < 4; ++rbk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * 128 + rbk * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      const int m = m0 + rl;
      if (m >= M) continue;
      const float t = OUT == OUT_ACC_I32 ? 0.f : srow[rl] * aw;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = n0 + wn * (32 * CB) + cb * 32 + l32;
        if (n < N) store_out<OUT>(Y, (size_t)m * N + n, unscale<BITS>(acc[rbk][cb][r]), t);
      }
    }
  }
}

// ===========================================================================
// INT4 prefill on the fp6 x fp4 matrix instruction
// (v_mfma_scale_f32_32x32x64_f8f6f4, A in e2m3, B in e2m1, unit scales).
//
// gfx950 runs this instruction at twice the int8 rate.  Every INT4 code q is
// an e2m3 value once halved (q/2 in [-4, 3.5]); a ternary weight w doubled
// is an e2m1 value (2w in {-2, 0, 2}).  Each product is the integer q*w and
// every partial sum is an integer below 2^24 in magnitude, so the fp32
// accumulator holds the exact integer dot product whatever the order of
// accumulation.
//
// A comes from prep mode 2: per token one 24-byte group per 32 k, six-bit
// fields in the operand order, blocked by 128 k ([K/128][M][96 bytes]).
// B stays the packed 2-bit format: masking
// bits 2-3 and 6-7 of every byte of a packed word (after a left shift by 2
// for fields 0 and 2) leaves, nibble by nibble, the e2m1 code of 2w
// (code 01 -> 0100 = +2, 11 -> 1100 = -2).  Word w0 (k0..k0+15) gives operand
// dwords 0 and 1, word w1 (k0+16..k0+31) dwords 2 and 3; the fp6 field order
// matches that nibble order.
//
// 256x256 tile per workgroup of 4 waves (2x2, 128x128 each), 128 k per
// stage.  A: 96 bytes per row per stage, 4 stage buffers in a ring, copies
// issued 3-4 stages ahead.  B: fetched for two stages at once (64 bytes per
// column, so each column costs one cache-line request per two stages), 2
// pair slots.  Lane group g of the 64-k instruction takes 32-k group 2g+s
// of the stage in step s, so every lane reads 48 contiguous A bytes and 16
// contiguous B bytes per stage.  The global memory requests are what bounds
// this kernel, so both operands are fetched as whole, contiguous runs.
constexpr int F6_BK = 128, F6_NBUF = 4;
constexpr int F6_AROW = F6_BK / 4 * 3;             // 96 bytes of fp6 codes per row per stage
constexpr int F6_A_STAGE = PBM * F6_AROW;          // 24 KiB
constexpr int F6_BPROW = 2 * F6_BK / 4;            // 64 bytes of packed weights per column per stage pair
constexpr int F6_B_PAIR = PBN * F6_BPROW;          // 16 KiB
constexpr int F6_B_BASE = F6_NBUF * F6_A_STAGE;    // B slots after the A ring
constexpr int F6_LDS = F6_B_BASE + 2 * F6_B_PAIR;  // 128 KiB
// The same pipeline on T x TN tiles: T = TN = 256 above; T = TN = 128 (four
// waves of 64 x 64) for problems with fewer 256 x 256 tiles than compute
// units; T = 256, TN = 192 (four waves of 128 x 96) where N is cut in 192s
// more evenly than in 256s -- N = 3072 at M = 4096 is 256 such tiles, one
// per compute unit, against 192 tiles of 256 x 256 (a quarter of the chip
// idle) or 768 of 128 x 128 (one and a half rounds of two per CU).
template <int T, int TN = T>
struct F6Geo {
  static constexpr int RBM = T / 64;                 // 32-row blocks per wave
  static constexpr int RBN = TN / 64;                // 32-column blocks per wave
  static constexpr int A_STAGE = T * F6_AROW;        // bytes of one A stage
  static constexpr int B_PAIR = TN * F6_BPROW;       // bytes of one B stage pair
  static constexpr int B_BASE = F6_NBUF * A_STAGE;
  static constexpr int LDS = B_BASE + 2 * B_PAIR;
  static constexpr int A_LOADS = A_STAGE / 1024 / 4, B_LOADS = B_PAIR / 1024 / 4;
  static constexpr int READS = RBN + 3 * RBM;        // LDS reads per stage: B blocks, then A units
};
static_assert(F6Geo<256>::LDS == F6_LDS && F6Geo<256>::A_STAGE == F6_A_STAGE && F6Geo<256>::B_PAIR == F6_B_PAIR,
              "256-tile geometry");
static_assert(F6Geo<256, 192>::LDS == 120 * 1024 && F6Geo<256, 192>::B_LOADS == 3 && F6Geo<256, 192>::READS == 15,
              "256 x 192 geometry");

// gfx950 LDS: 64 banks of 4 bytes; a 16-byte read serves 16 consecutive
// lanes per cycle, so 16 consecutive rows reading the same logical unit must
// hit 16 distinct 16-byte bank groups.  A rows hold 6 units of 16 bytes
// (96 bytes: 6*row mod 16 repeats after 8 rows); rows with bit 3 set are
// rotated by one unit.  B columns hold 4 units (stage parity, lane group) of
// 64-byte rows (repeating after 4 columns), xor-swizzled by column bits 2-3.
HBL_DEV int f6_arot(int row) { return (row >> 3) & 1; }
HBL_DEV int f6_bswz(int col) { return (col >> 2) & 3; }

// Copy 16 bytes per lane from global memory (scalar base + 32-bit per-lane
// offset) straight into LDS at lds_base + 16 * lane (wave-uniform base).
HBL_DEV void lds_copy16s(const void* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(lds_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

// US: stages per loop trip (4; 2 when K = 256), so that LDS buffer numbers are
// compile-time constants.  T x TN: tile rows x columns (256 x 256 or 256 x 192,
// one workgroup per CU; 128 x 128 with two).
template <int OUT, int US, int T = 256, int TN = T>
__global__ __launch_bounds__(256, T == 256 ? 1 : 2) void gemm_fp6_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K, int tiles_m, int tiles_n) {
  using G = F6Geo<T, TN>;
  constexpr int RBM = G::RBM, RBN = G::RBN;          // 32 x 32 blocks per wave: RBM x RBN
  constexpr int WT = T / 2, WTN = TN / 2;            // wave tile
  static_assert((T == 256 && (TN == 256 || TN == 192)) || (T == 128 && TN == 128), "shipped tile shapes");
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];
  constexpr int A_LOADS = G::A_LOADS, B_LOADS = G::B_LOADS;   // 6 and 4 (256 x 256), 6 and 3 (256 x 192), 3 and 2
  using S6 = std::conditional_t<T == 256, std::conditional_t<TN == 256, sched::Fp6, sched::Fp6Wide>, sched::Fp6Small>;
  static_assert(S6::NBUF == F6_NBUF && S6::WAVES == 4 && S6::A_COPIES == A_LOADS && S6::B_COPIES == B_LOADS &&
                    S6::MFMAS == (T == 256 ? RBM * RBN : 8),
                "schedule model and kernel geometry agree");
  static_assert(sched::fp6_ok<S6>(2) && sched::fp6_ok<S6>(4) && sched::fp6_ok<S6>(8) && sched::fp6_ok<S6>(20) &&
                    sched::fp6_ok<S6>(256),
                "copy schedule: a wait leaves a needed copy in flight or a copy targets a buffer in use");

  const int bid = blockIdx.x, total = tiles_m * tiles_n;
  const int logical = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  constexpr int GM = 4;
  const int per_group = GM * tiles_n;
  const int first_m = (logical / per_group) * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_g = logical % per_group;
  const int m0 = (first_m + in_g % gm) * T;
  const int n0 = (in_g / gm) * TN;
  __shared__ __attribute__((aligned(16))) float srow[T];   // epilogue row scales (row_scale_copy)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;
  // A is blocked by 128 k: stage kt of the tile is the contiguous run of
  // T x 96 bytes at (kt * M + m0) * 96.
  const size_t a_stage = (size_t)M * F6_AROW;
  const uint8_t* a_tile = A + (size_t)m0 * F6_AROW;
  const uint8_t* b_tile = W + wrow_base(n0, K);     // n0 is a multiple of 16
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  // copy P of a stage fills LDS bytes 16P..16P+15 (wave instruction = 1 KiB);
  // per-lane source offsets inside the tile (rows past M / channels past N
  // repeat the last one and are never stored) fit 32 bits: < 256 rows.
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int P = (j * 4 + wave) * 64 + lane, row = P / 6, pu = P % 6;
    int u = pu - f6_arot(row);
    if (u < 0) u += 6;
    a_off[j] = (uint32_t)(min(m0 + row, M - 1) - m0) * F6_AROW + 16 * u;
  }
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int P = (j * 4 + wave) * 64 + lane, col = P >> 2, u = (P & 3) ^ f6_bswz(col);   // col < TN
    const int nr = min(n0 + col, N - 1) - n0;       // tiled: 16-row blocks of 4K bytes, 64-byte row segments
    b_off[j] = (uint32_t)(nr >> 4) * (uint32_t)K * 4u + (uint32_t)(nr & 15) * 64u + 16u * u;
  }
  // A copy j (0..5) of stage kt into A buffer buf; B copy j (0..3) of stage
  // pair p into B slot sl
  auto dmaA = [&](int j, int kt, int buf) __attribute__((always_inline)) {
    lds_copy16s(a_tile + (size_t)kt * a_stage, a_off[j], lds0 + buf * G::A_STAGE + (j * 4 + wave_s) * 1024);
  };
  auto dmaB = [&](int j, int p, int sl) __attribute__((always_inline)) {
    lds_copy16s(b_tile + (size_t)p * 1024, b_off[j], lds0 + G::B_BASE + sl * G::B_PAIR + (j * 4 + wave_s) * 1024);
  };

  v16f acc[RBM][RBN];
#pragma unroll
  for (int i = 0; i < RBM; ++i)
#pragma unroll
    for (int j = 0; j < RBN; ++j) acc[i][j] = v16f{};

  // Register fragments of one stage: per lane 48 A bytes (32-k groups 2g and
  // 2g+1 of four 32-row blocks), kept as one 12-dword vector per block so the
  // two 6-dword MFMA operands (8-dword vectors, the last two unused) are
  // sub-ranges of it, and 16 packed B bytes
  // (the same groups of the 32-column blocks).  Read r of a stage: r < RBN
  // the B block r, else A block (r-RBN)/3, unit (r-RBN)%3.
  struct Frag {
    v16i a[RBM];
    v4i b[RBN];
  };
  // read r of stage kt (A buffer kt % 4, B slot (kt / 2) % 2, half kt % 2)
  auto read1 = [&](Frag& f, int r, int kt) __attribute__((always_inline)) {
    const uint8_t* sa = smem + (kt & (F6_NBUF - 1)) * G::A_STAGE;
    if (r < RBN) {
      const int n = wn * WTN + r * 32 + l32;
      const uint8_t* sb = smem + G::B_BASE + ((kt >> 1) & 1) * G::B_PAIR;
      f.b[r] = *reinterpret_cast<const v4i*>(sb + n * F6_BPROW + 16 * ((2 * (kt & 1) + g) ^ f6_bswz(n)));
    } else {
      const int rb = (r - RBN) / 3, t = (r - RBN) % 3;
      const int row = wm * WT + rb * 32 + l32;
      int pu = 3 * g + t + f6_arot(row);
      if (pu >= 6) pu -= 6;
      const v4i x = *reinterpret_cast<const v4i*>(sa + row * F6_AROW + 16 * pu);
      const v16i xe = __builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1);
      if (t == 0)
        f.a[rb] = __builtin_shufflevector(f.a[rb], xe, 16, 17, 18, 19, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      else if (t == 1)
        f.a[rb] = __builtin_shufflevector(f.a[rb], xe, 0, 1, 2, 3, 16, 17, 18, 19, 8, 9, 10, 11, 12, 13, 14, 15);
      else
        f.a[rb] = __builtin_shufflevector(f.a[rb], xe, 0, 1, 2, 3, 4, 5, 6, 7, 16, 17, 18, 19, 12, 13, 14, 15);
    }
  };
  // fp4 operand of MFMA step st for 32-column block cb: 2w per nibble
  auto bexp1 = [&](const Frag& f, int st, int cb) __attribute__((always_inline)) {
    const uint32_t w0 = (uint32_t)f.b[cb][2 * st], w1 = (uint32_t)f.b[cb][2 * st + 1];
    return v8i{(int)((w0 << 2) & 0xCCCCCCCCu), (int)(w0 & 0xCCCCCCCCu), (int)((w1 << 2) & 0xCCCCCCCCu),
               (int)(w1 & 0xCCCCCCCCu), 0, 0, 0, 0};
  };
  // dwords 6st .. 6st+5 of the block's 12 A dwords (the instruction reads six
  // registers for fp6; the last two lanes of the vector are not used)
  auto aop = [&](const Frag& f, int st, int rb) __attribute__((always_inline)) {
    return st == 0 ? __builtin_shufflevector(f.a[rb], f.a[rb], 0, 1, 2, 3, 4, 5, 6, 7)
                   : __builtin_shufflevector(f.a[rb], f.a[rb], 6, 7, 8, 9, 10, 11, 12, 13);
  };
  auto mfma = [&](const v8i& af, const v8i& bf, v16f& c) __attribute__((always_inline)) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, c, 2, 4, 0, 127, 0, 127);
  };

  // Software pipeline, one wave per SIMD.  Stage kt lives in buffer kt % 4
  // and its fragments are in registers (cur) when it starts.  First MFMA
  // step of cur; then wait for this wave's copies of stage kt+1 and barrier
  // (every wave's copies of kt+1 have landed, every wave's reads of stage kt
  // are complete); then the second MFMA step, with one LDS read of stage
  // kt+1's fragments (nxt) after every MFMA and one copy of stage kt+4 into
  // stage kt's buffer after every other MFMA, so the memory instructions
  // issue in the shadow of the matrix instructions instead of in bursts.
  // Past the last stage the copies repeat stage KT-1 and the reads fetch an
  // unused buffer (both harmless), which keeps the loop free of branches and
  // the copy count per stage constant.
  // The operand expansion is pipelined too: during step 0 the B operands of
  // step 1 (bf1) are expanded, during step 1 those of the next stage's step 0
  // (bf0, from nxt, a few MFMAs after their LDS reads were issued).  All the
  // VALU work then issues between MFMAs.  sched_barrier(0) fixes the order
  // of these groups.
  // Copy issue order (each A stage 6 instructions per wave, each B pair 4):
  // prologue A0 B0 A1 A2 B1 A3; at the boundary of stage kt, B pair
  // (kt+3)/2 if kt is odd, then A stage kt+4.  Before reading stage kt+1
  // this wave waits until A kt+1 and B pair (kt+1)/2 have landed, which
  // leaves 16 instructions (A, B, A) in flight after an even stage and 12
  // (A, A) after an odd one.  Past the end, copies repeat the last stage or
  // pair into the buffer just freed, which keeps the counts constant.
  const int KT = K / F6_BK;                 // a multiple of US
  const int KP = KT / 2;
  auto stage = [&](int kt, int u, const Frag& cur, Frag& nxt, v8i* bf0, v8i* bf1) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < RBM; ++rb) {
      const v8i af = aop(cur, 0, rb);
#pragma unroll
      for (int cb = 0; cb < RBN; ++cb) {
        mfma(af, bf0[cb], acc[rb][cb]);
        if (cb == 1 && rb < RBN) bf1[rb] = bexp1(cur, 1, rb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (u & 1) wait_vmcnt<S6::wait(true)>(); else wait_vmcnt<S6::wait(false)>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
    const int akt = S6::a_stage(kt, KT);
    const int bp = S6::b_pair(kt, KT);
#pragma unroll
    for (int rb = 0; rb < RBM; ++rb) {
      const v8i af = aop(cur, 1, rb);
#pragma unroll
      for (int cb = 0; cb < RBN; ++cb) {
        const int i = rb * RBN + cb;
        mfma(af, bf1[cb], acc[rb][cb]);
        if constexpr (T == 256) {
          // MF = RBM * RBN MFMAs (16, or 12 with 192 columns) and READS LDS
          // reads (16, or 15): read i after MFMA i, and the reads past MF
          // (the last A block's units) after the last MFMAs
          constexpr int MF = RBM * RBN, XR = G::READS - MF;
          static_assert(XR >= 0 && XR <= MF, "reads per stage");
          read1(nxt, i, u + 1);
          if (i >= MF - XR) read1(nxt, i + XR, u + 1);
          // odd stage: B pair into the slot this pair of stages used, then A;
          // even stage: the A copies of stage kt+4 after MFMAs 1, 3, ..., 11
          // (u is kt modulo a multiple of 4, or kt itself when K = 256)
          const sched::Copy cp = S6::after(i, u & 1);
          if (cp.kind == 2) dmaB(cp.j, bp, S6::b_slot(u));
          else if (cp.kind == 1) dmaA(cp.j, akt, S6::a_buf(u));
          // the next stage's B operands, expanded after every other one of
          // the last 2 * RBN MFMAs (their reads were the first RBN)
          constexpr int E0 = MF - 2 * RBN;
          if (i >= E0 && !((i - E0) & 1)) bf0[(i - E0) >> 1] = bexp1(nxt, 0, (i - E0) >> 1);
        } else {
          // four MFMAs: two reads and two copy slots after each; the next
          // stage's B expansion after the last two (its B reads came first)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            read1(nxt, 2 * i + h, u + 1);
            const sched::Copy cp = S6::after(2 * i + h, u & 1);
            if (cp.kind == 2) dmaB(cp.j, bp, S6::b_slot(u));
            else if (cp.kind == 1) dmaA(cp.j, akt, S6::a_buf(u));
          }
          if (i >= 2) bf0[i - 2] = bexp1(nxt, 0, i - 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  Frag f0, f1;
  // prologue: A0 B0 A1 A2 B1 A3
  auto dmaA_all = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) dmaA(j, min(kt, KT - 1), kt);
  };
  auto dmaB_all = [&](int p) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) dmaB(j, min(p, KP - 1), p);
  };
  if (OUT != OUT_ACC_I32) row_scale_copy<T>(dscale, m0, M, srow, wave, lane);
#pragma unroll
  for (int p = 0; p < S6::PROLOGUE; ++p) {    // A0 B0 A1 A2 B1 A3
    const sched::Copy cp = S6::prologue(p);
    if (cp.kind == 1) dmaA_all(cp.j); else dmaB_all(cp.j);
  }
  wait_vmcnt<S6::wait_prologue()>();       // A0 and B0 have landed
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
#pragma unroll
  for (int r = 0; r < G::READS; ++r) read1(f0, r, 0);
  v8i bf0[RBN], bf1[RBN];
#pragma unroll
  for (int cb = 0; cb < RBN; ++cb) bf0[cb] = bexp1(f0, 0, cb);
  for (int kt = 0; kt < KT; kt += US) {
#pragma unroll
    for (int u = 0; u < US; u += 2) {
      stage(kt + u, u, f0, f1, bf0, bf1);
      stage(kt + u + 1, u + 1, f1, f0, bf0, bf1);
    }
  }
  // no copy may still be writing LDS when the workgroup exits
  wait_vmcnt<0>();

  // epilogue: 32x32 accumulator layout, lane l / register r hold
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.  The accumulators are exact
  // integers below 2^24.
  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
  if constexpr (OUT == OUT_BF16) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");   // every wave is done with the ring
    static_assert(4 * 64 * (RBN * 64 + 32) <= G::LDS, "staging fits the ring");
    store_bf16_staged<RBN, RBM / 2>(smem + wave * (64 * (RBN * 64 + 32)), static_cast<uint16_t*>(Y), srow + wm * WT,
                                    aw, M, N, m0 + wm * WT, n0 + wn * WTN, lane,
                                  [&](int rb, int cb, int r) { return acc[rb][cb][r]; });
  } else {
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RBM; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * WT + rb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        const int m = m0 + rl;
        if (m >= M) continue;
        const float t = OUT == OUT_ACC_I32 ? 0.f : srow[rl] * aw;
#pragma unroll
        for (int cb = 0; cb < RBN; ++cb) {
          const int n = n0 + wn * WTN + cb * 32 + l32;
          if (n < N) store_out<OUT>(Y, (size_t)m * N + n, (int)acc[rb][cb][r], t);
        }
      }
    }
  }
}

// ===========================================================================
// Decode (M <= 64): weight streaming.
//
// A workgroup of NW waves owns 16*CPW output channels and one of S equal K
// ranges.  The range is cut into 256-k blocks dealt round-robin to the waves;
// each block's packed weights (16 bytes per lane per 16 channels) and
// activation codes are loaded straight into registers, and every weight byte
// is read from HBM once.  With one channel group (CPW == 1) a wave keeps a
// ring of a few blocks requested ahead (decode_plan and the kernel below say
// how many); with four groups it requests two blocks at a time.
// v_mfma_i32_16x16x64_i8 runs with channels on the MFMA's M side and up to 16
// tokens on its N side.  The waves' int32 partials meet in LDS: per-wave
// slices summed in a fixed order (CPW == 1) or integer atomics into one tile
// (CPW == 4); both exact.  With S > 1 the S partials of a channel tile are
// summed by the last workgroup of the tile to finish (when the launch passes
// arrival counters: the forward) or by decode_reduce_kernel (stage calls);
// integer sums are exact, so the result is the same for every S.
constexpr int DKB = 256;

struct DecodePlan { int cpw, S, mb, nw; };
constexpr int kDecodeMaxSplit = 4;   // split-K ways the in-kernel reduction handles
// Up to 32 tokens: 16 channels per workgroup over the whole K, one or two
// token groups.  33..64: 64 channels per workgroup and K split four ways, so
// each INT4 activation operand expanded in registers feeds four channel
// groups (with one group per workgroup the expansion was repeated for every
// 16 channels: 64 tokens took 18.0 us unsplit against 13.5 us split), at the
// price of the cross-workgroup reduction.  Measured at K = 16384, N = 4096:
// 17 / 32 tokens 8.2 / 10.8 us unsplit against ~12.5 us split.
// Codes in the decode-blocked layout (blocked, the forward's) make the code
// stream cheap enough that 33..64 tokens also run unsplit on 16 channels
// per workgroup (four token groups) up to K = 16384: the 64-token matmul
// inside the forward 13.0 us against 14.6 us split, 40 tokens 11.7 against
// 13.3 us.
static DecodePlan decode_plan(int64_t M, int64_t K, int64_t N, bool blocked) {
  DecodePlan p = M <= 16                    ? DecodePlan{1, 1, 1, 8}
                 : M <= 32                  ? DecodePlan{1, 1, 2, 8}
                 : (blocked && K <= 16384) ? DecodePlan{1, 1, 4, 8}
                                            : DecodePlan{4, 4, 4, 8};
  while (p.S > 1 && K / p.S < DKB) p.S /= 2;
  // split-K partials are addressed with 32-bit byte offsets
  if (p.S > 1 && (int64_t)p.S * M * N * 4 >= (int64_t(1) << 31)) p.S = 1;
  return p;
}

// With S > 1 the S workgroups of a channel tile write int32 partial sums.
// tile_count == nullptr: decode_reduce_kernel sums them.  Otherwise (the
// counters zeroed before the launch) each workgroup stores its partial rows,
// waits until those stores have completed, and counts itself in; the one
// that arrives last sums the S partials, dequantises and stores, then leaves
// its counter zero.  Nothing waits on another workgroup.  Partials are
// stored and re-read as device-scope atomics, which write through and bypass
// the per-XCD L2s, so no cache-wide fence is needed (a device-scope fence
// writes back and invalidates the whole L2 of the XCD, which cost the
// 64-token forward 55 us instead of 21 us: every workgroup threw away the
// activation codes the others were still reading).
// BLK: the codes are in the decode-blocked layout (dblk_offset: each
// activation fragment load one contiguous KiB; with the row-major codes a
// fragment load touches 16 token rows, and at 32 tokens the matmul took
// 11.2 us instead of 8.4 us); bits 8 and 4 only.
template <int BITS, int MB, int CPW, int NW, int OUT, int KB1 = 8, bool BLK = false>
__global__ __launch_bounds__(64 * NW) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K, int S,
    int32_t* __restrict__ partial, uint32_t* __restrict__ tile_count) {
  // Blocks held per wave per round: their loads need MAXB * (CPW + MB*BITS/2)
  // uint4 registers, kept near 48 (192 VGPRs).
  // (two with four token groups: 8 waves of 184 registers, two per SIMD, so
  // one wave's MFMAs cover another's waits)
  // One 16-channel group (CPW == 1, K unsplit): blocks stream through a ring
  // (below), at most KB1 per wave (8: K <= 16384 with 8 waves; 16 up to
  // 32768; only the unrolled loop grows, not the registers).  Four groups
  // (CPW == 4, K split four ways): two blocks per wave per round, all
  // requested at once (8 waves of ~160 registers, two per SIMD, so one wave's
  // MFMAs cover another's waits).
  constexpr int MAXB = CPW == 1 ? KB1 : 2;
  constexpr int CH = 16 * CPW;
  // Reduction over the waves (which split K): each wave stores its
  // accumulators, 16 bytes per lane per 16x16 block, into its own LDS slice,
  // then every thread sums the NW slices of GPT groups of four outputs (four
  // consecutive channels of one token), 16 bytes per slice.  Integer atomics
  // into one shared tile (64 per lane at 64 tokens) took 2.2 us of a 12 us
  // launch.  Group p is token p / Q, channel quad p % Q (Q = 4 CPW quads per
  // token), so the threads of a wave cover whole rows of the partials and the
  // output (a first numbering in the accumulator order put 16 token rows
  // under each 16-byte access, and the split-K hand-off took 1 us longer).
  // Slice rows of Q + 1 quads keep both the accumulator stores (16 tokens x
  // 4 quads per instruction) and the row reads free of bank conflicts.
  constexpr int Q = 4 * CPW;
  constexpr int GROUPS = MB * 16 * Q;
  constexpr int GPT = (GROUPS + 64 * NW - 1) / (64 * NW);
  __shared__ v4i slices[CPW == 1 ? NW : 1][CPW == 1 ? MB * 16 * (Q + 1) : 1];
  // The split configuration (CPW == 4) reduces over the waves with integer
  // atomics into one tile of rows of RL ints instead (measured faster there
  // with its partials handed over element by element: 64 tokens 19.5 against
  // 20.1 us forward): inside each block of 16 channels column 4r + q holds
  // channel 4q + r, and RL = 4 (mod 64), so the 64 lanes of one accumulate
  // (token c, channel 4g + r) hit 64 distinct banks (4c + g).
  constexpr int RL = CH + 4;
  constexpr int NQ = (MB * 16 * CH + 64 * NW - 1) / (64 * NW);   // outputs per thread, split configuration
  __shared__ int red[CPW == 1 ? 1 : MB * 16 * RL];
  auto red_col = [](int nl) { return (nl & ~15) | ((nl & 3) << 2) | ((nl >> 2) & 3); };
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ch0 = blockIdx.x * CH, s = blockIdx.y;
  const int Kr = K / S, kbeg = s * Kr;
  const int nblk = Kr / DKB;                                   // 256-k blocks in this range
  const size_t arow = (size_t)K * BITS / 8;
  auto group_token = [](int p) { return p / Q; };
  auto group_channel = [](int p) { return 4 * (p % Q); };

  // epilogue scales fetched up front (their latency is not paid at the end)
  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
  constexpr int NPRE = CPW == 1 ? GPT : NQ;
  float ds_pre[NPRE];
#pragma unroll
  for (int h = 0; h < NPRE; ++h) {
    const int t = CPW == 1 ? group_token(min(h * 64 * NW + tid, GROUPS - 1)) : (h * 64 * NW + tid) / CH;
    ds_pre[h] = OUT == OUT_ACC_I32 ? 0.f : dscale[min(t, M - 1)];
  }
  if constexpr (CPW != 1)
    for (int i = tid; i < MB * 16 * RL; i += 64 * NW) red[i] = 0;

  v4i acc[CPW][MB];
#pragma unroll
  for (int cp = 0; cp < CPW; ++cp)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[cp][mb] = v4i{};

  if constexpr (CPW == 1) {
    // Blocks b = wave + NW*i (i < MAXB: K / S <= NW * MAXB * 256), consumed in
    // order, with only RING blocks per wave requested ahead: block i + RING is
    // requested once block i has been consumed.  Requesting the whole weight
    // stream at once made every request wait behind the full queue, so a
    // wave's blocks all arrived at the end of the stream and the matrix work
    // only started then; with a short ring the blocks arrive spread over the
    // stream and the work overlaps it.  Loads are unconditional (out-of-range
    // indices are clamped to valid addresses and the values discarded), so the
    // compiler releases block i with a partial vmcnt wait.
    constexpr int RING = MB == 1 ? 4 : 2;
    uint4 wq[RING][CPW];
    uint4 aq[RING][MB][BITS / 2];
    auto load = [&](int i, int slot) __attribute__((always_inline)) {
      const int b = min(wave + NW * i, nblk - 1);
      const int kb = kbeg + b * DKB + 64 * g;                   // this lane's 64 codes of block b
  #pragma unroll
      for (int cp = 0; cp < CPW; ++cp) {
        const int n = min(ch0 + 16 * cp + c, N - 1);
        wq[slot][cp] =
            *reinterpret_cast<const uint4*>(W + wrow_base(n, K) + (size_t)((kbeg + b * DKB) >> 8) * 1024 + 16 * g);
      }
  #pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int t = min(16 * mb + c, M - 1);
        if constexpr (BLK) {
          const uint8_t* ap = A + dblk_offset(BITS, (M + 15) >> 4, t, kb);   // run d: + 1 KiB each
  #pragma unroll
          for (int d = 0; d < BITS / 2; ++d) aq[slot][mb][d] = *reinterpret_cast<const uint4*>(ap + 1024 * d);
        } else {
          const uint4* ap = reinterpret_cast<const uint4*>(A + (size_t)t * arow + (size_t)kb * BITS / 8);
  #pragma unroll
          for (int d = 0; d < BITS / 2; ++d) aq[slot][mb][d] = ap[d];
        }
      }
    };
    auto compute = [&](int slot) __attribute__((always_inline)) {
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
  #pragma unroll
        for (int cp = 0; cp < CPW; ++cp) {
          // INT8: step j = weight word j against the 16 codes it covers (the
          // codes as loaded).  INT4 keeps the other pairing -- step j = field j
          // of all four weight words against the matching nibbles of all four
          // activation words (1 op per operand dword either way): with it the
          // 64-token decode runs 15.1 us instead of 17.1 us.
          v4i wop;
          if constexpr (BITS == 8) {
            wop = wstep(u4get(wq[slot][cp], j));
          } else {
            const uint4 p = wq[slot][cp];
            wop = v4i{(int)wfield(p.x, j), (int)wfield(p.y, j), (int)wfield(p.z, j), (int)wfield(p.w, j)};
          }
  #pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            v4i aop;
            if constexpr (BITS == 8) {
              aop = as_v4i(aq[slot][mb][j]);
            } else {
              // codes 16d + 4j + i: nibble j%2 of word 2d + j/2
              const uint4 q0 = aq[slot][mb][0], q1 = aq[slot][mb][1];
              const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
              aop = v4i{(int)a4field(w[0 + (j >> 1)], j), (int)a4field(w[2 + (j >> 1)], j),
                        (int)a4field(w[4 + (j >> 1)], j), (int)a4field(w[6 + (j >> 1)], j)};
            }
            // padding tokens (16*mb + c >= M) read token M-1's codes; their
            // sums are never stored
            acc[cp][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, aop, acc[cp][mb], 0, 0, 0);
          }
        }
      }
    };
  #pragma unroll
    for (int i = 0; i < RING; ++i) load(i, i);
  #pragma unroll
    for (int i = 0; i < MAXB; ++i) {
      if (wave + NW * i < nblk) compute(i % RING);      // wave-uniform
      if (i + RING < MAXB) {
        load(i + RING, i % RING);
        __builtin_amdgcn_sched_barrier(0);              // keep the requests where they are issued
      }
    }
  } else {
    // Blocks b = wave + NW*i, taken MAXB at a time.  Loads are unconditional
    // (out-of-range indices are clamped to valid addresses and the values
    // discarded), so the compiler can release block i with a partial vmcnt
    // wait instead of waiting for every load.
    // BITS == 6: INT4 codes in the fp6 operand layout ([K/128][M][96]) on the
    // fp6 x fp4 instruction (v_mfma_scale_f32_16x16x128_f8f6f4, unit scales):
    // lane group g takes the 32-k groups 8b + 2g and 8b + 2g + 1 of 256-k
    // block b in steps 0 and 1 -- from the packed weights words 4g, 4g + 1
    // and 4g + 2, 4g + 3 turned into e2m1 nibbles of 2w, from the codes the
    // 48 contiguous bytes of token t's 128-k block 2b + g/2 at byte 48 (g & 1).
    // Half the matrix instructions of the int8 form and no activation
    // expansion; the fp32 sums are exact integers (|acc| <= 8 K < 2^24).
    constexpr int AU = BITS == 6 ? 3 : BITS / 2;                // 16-byte activation units per token group
    typedef float v4f __attribute__((ext_vector_type(4)));
    v4f accf[CPW][MB];
    if constexpr (BITS == 6) {
#pragma unroll
      for (int cp = 0; cp < CPW; ++cp)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) accf[cp][mb] = v4f{};
    }
    for (int b0 = wave; b0 < nblk; b0 += NW * MAXB) {
      uint4 wq[MAXB][CPW];
      uint4 aq[MAXB][MB][AU];
#pragma unroll
      for (int i = 0; i < MAXB; ++i) {
        const int b = min(b0 + NW * i, nblk - 1);
        const int gb = (kbeg >> 8) + b;                           // 256-k block over K
#pragma unroll
        for (int cp = 0; cp < CPW; ++cp) {
          const int n = min(ch0 + 16 * cp + c, N - 1);
          wq[i][cp] = *reinterpret_cast<const uint4*>(W + wrow_base(n, K) + (size_t)gb * 1024 + 16 * g);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int t = min(16 * mb + c, M - 1);
          const uint4* ap =
              BITS == 6 ? reinterpret_cast<const uint4*>(A + ((size_t)(2 * gb + (g >> 1)) * M + t) * 96 + 48 * (g & 1))
                        : reinterpret_cast<const uint4*>(A + (size_t)t * arow + (size_t)(gb * DKB + 64 * g) * BITS / 8);
          if constexpr (BLK && BITS != 6) {
            const uint8_t* bp = A + dblk_offset(BITS, (M + 15) >> 4, t, gb * DKB + 64 * g);
#pragma unroll
            for (int d = 0; d < AU; ++d) aq[i][mb][d] = *reinterpret_cast<const uint4*>(bp + 1024 * d);
          } else {
#pragma unroll
            for (int d = 0; d < AU; ++d) aq[i][mb][d] = ap[d];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < MAXB; ++i) {
        if (b0 + NW * i >= nblk) continue;   // wave-uniform; keeps the loop unrolled (registers, no scratch)
        if constexpr (BITS == 6) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int cp = 0; cp < CPW; ++cp) {
              const uint32_t w0 = st ? wq[i][cp].z : wq[i][cp].x, w1 = st ? wq[i][cp].w : wq[i][cp].y;
              const v8i wop = v8i{(int)((w0 << 2) & 0xCCCCCCCCu), (int)(w0 & 0xCCCCCCCCu),
                                  (int)((w1 << 2) & 0xCCCCCCCCu), (int)(w1 & 0xCCCCCCCCu), 0, 0, 0, 0};
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                const uint4 a0 = aq[i][mb][0], a1 = aq[i][mb][1], a2 = aq[i][mb][2];
                const v8i aop = st == 0 ? v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, 0, 0}
                                        : v8i{(int)a1.z, (int)a1.w, (int)a2.x, (int)a2.y, (int)a2.z, (int)a2.w, 0, 0};
                accf[cp][mb] =
                    __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop, aop, accf[cp][mb], 4, 2, 0, 127, 0, 127);
              }
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int cp = 0; cp < CPW; ++cp) {
              // INT8: step j = weight word j against the 16 codes it covers
              // (the codes as loaded).  INT4 keeps the other pairing -- step j
              // = field j of all four weight words against the matching
              // nibbles of all four activation words (1 op per operand dword
              // either way): with it the 64-token decode ran 15.1 us instead
              // of 17.1 us.
              v4i wop;
              if constexpr (BITS == 8) {
                wop = wstep(u4get(wq[i][cp], j));
              } else {
                const uint4 p = wq[i][cp];
                wop = v4i{(int)wfield(p.x, j), (int)wfield(p.y, j), (int)wfield(p.z, j), (int)wfield(p.w, j)};
              }
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                v4i aop;
                if constexpr (BITS == 8) {
                  aop = as_v4i(aq[i][mb][j]);
                } else {
                  // codes 16d + 4j + i: nibble j%2 of word 2d + j/2
                  const uint4 q0 = aq[i][mb][0], q1 = aq[i][mb][1];
                  const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                  aop = v4i{(int)a4field(w[0 + (j >> 1)], j), (int)a4field(w[2 + (j >> 1)], j),
                            (int)a4field(w[4 + (j >> 1)], j), (int)a4field(w[6 + (j >> 1)], j)};
                }
                // padding tokens (16*mb + c >= M) read token M-1's codes;
                // their sums are never stored
                acc[cp][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, aop, acc[cp][mb], 0, 0, 0);
              }
            }
          }
        }
      }
    }
    if constexpr (BITS == 6) {
#pragma unroll
      for (int cp = 0; cp < CPW; ++cp)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[cp][mb] = v4i{(int)accf[cp][mb][0], (int)accf[cp][mb][1], (int)accf[cp][mb][2], (int)accf[cp][mb][3]};
    }
  }
  if constexpr (CPW == 1) {
    // 16x16 accumulator layout: lane l / register r hold channel 4*(l/16)+r,
    // token l%16, so a lane's four registers are token 16 mb + c, quad 4 cp + g
  #pragma unroll
    for (int cp = 0; cp < CPW; ++cp)
  #pragma unroll
      for (int mb = 0; mb < MB; ++mb) slices[wave][(16 * mb + c) * (Q + 1) + 4 * cp + g] = acc[cp][mb];
    __syncthreads();
    v4i sum[GPT];
  #pragma unroll
    for (int h = 0; h < GPT; ++h) {
      const int p = min(h * 64 * NW + tid, GROUPS - 1);
      const int slot = group_token(p) * (Q + 1) + p % Q;
      v4i v = slices[0][slot];
  #pragma unroll
      for (int w = 1; w < NW; ++w) v += slices[w][slot];
      sum[h] = v;
    }
    // a group is stored when it exists, its token is present and its channels
    // are (N % 16 == 0: four channels are all inside or all outside)
    auto live = [&](int h) {
      const int p = h * 64 * NW + tid;
      return p < GROUPS && group_token(p) < M && ch0 + group_channel(p) < N;
    };
    if (S == 1) {
  #pragma unroll
      for (int h = 0; h < GPT; ++h) {
        if (!live(h)) continue;
        const int p = h * 64 * NW + tid;
        store_out4<OUT>(Y, (size_t)group_token(p) * N + ch0 + group_channel(p), unscale4<BITS>(sum[h]), ds_pre[h] * aw);
      }
      return;
    }
    // (the plan never splits these configurations; a split given anyway is
    // summed by the separate reduction kernel)
  #pragma unroll
    for (int h = 0; h < GPT; ++h) {
      if (!live(h)) continue;
      const int p = h * 64 * NW + tid;
      *reinterpret_cast<v4i*>(partial + ((size_t)s * M + group_token(p)) * N + ch0 + group_channel(p)) = sum[h];
    }
  } else {
    __syncthreads();
    // 16x16 accumulator layout: lane l / register r hold channel 4*(l/16)+r, token l%16
    // (every lane adds when the matrix work is the fp6 x fp4 instruction: the
    // compiler would otherwise move that work into the branch of the lanes whose
    // token is present, leaving the other lanes' operands unset)
  #pragma unroll
    for (int cp = 0; cp < CPW; ++cp)
  #pragma unroll
      for (int mb = 0; mb < MB; ++mb)
  #pragma unroll
        for (int r = 0; r < 4; ++r)
          if (BITS == 6 || 16 * mb + c < M) atomicAdd(&red[(16 * mb + c) * RL + 16 * cp + 4 * r + g], acc[cp][mb][r]);
    __syncthreads();
  #pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = q * 64 * NW + tid;
      if (e >= M * CH) continue;
      const int t = e / CH, n = ch0 + e % CH;
      if (n >= N) continue;
      const int v = red[t * RL + red_col(e % CH)];
      if (S == 1) store_out<OUT>(Y, (size_t)t * N + n, unscale<BITS>(v), ds_pre[q] * aw);
      else __hip_atomic_store(&partial[((size_t)s * M + t) * N + n], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (S == 1 || tile_count == nullptr) return;
    // Hand-off to the last workgroup of the channel tile.  Every thread waits
    // until its partial stores (agent-scope atomic stores: written through the
    // XCD's L2, whose contents other XCDs do not see, to the device's point of
    // coherence) have completed, the barrier makes that true for the whole
    // workgroup, and only then does one thread count the workgroup in with an
    // agent-scope atomic, performed at that same point.  The workgroup that
    // sees the count reach S - 1 reads the partials with agent-scope atomic
    // loads, served from the point of coherence and not from a possibly stale
    // L2 line.  This gives the ordering of the memory model's release /
    // acquire pair (an L2 write-back before the atomic, an L2 invalidate after
    // it) with the write-back and invalidate replaced by accesses that bypass
    // the non-coherent L2 for exactly the data handed over: a device-scope
    // fence in every workgroup slowed the 64-token forward from 21 to 55 us
    // (its invalidate discarded the codes other workgroups of the XCD were
    // still reading).  Nothing waits on another workgroup.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      is_last = __hip_atomic_fetch_add(&tile_count[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(S - 1);
    __syncthreads();
    if (!is_last) return;
    // every partial this thread sums is requested before any is waited for
    // (clamped, always in-bounds addresses; splits past S count zero)
    int tot[NQ];
  #pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = q * 64 * NW + tid;
      const int t = min(e / CH, M - 1), n = min(ch0 + e % CH, N - 1);
      tot[q] = 0;
  #pragma unroll
      for (int s2 = 0; s2 < kDecodeMaxSplit; ++s2) {
        const int v = __hip_atomic_load(&partial[((size_t)min(s2, S - 1) * M + t) * N + n], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        tot[q] += s2 < S ? v : 0;
      }
    }
  #pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = q * 64 * NW + tid;
      if (e >= M * CH) continue;
      const int t = e / CH, n = ch0 + e % CH;
      if (n >= N) continue;
      store_out<OUT>(Y, (size_t)t * N + n, unscale<BITS>(tot[q]), ds_pre[q] * aw);
    }
    if (tid == 0) __hip_atomic_store(&tile_count[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Few tokens (M <= 4): one workgroup of NW waves per 16 channels and the whole
// K.  The tokens' activation codes are staged once per workgroup in LDS,
// already in MFMA operand form (int8; INT4 codes as 16*q), so each MFMA step
// only expands its packed weights.  The staging load is issued before the
// weight stream so waiting for it is a partial wait.  Lanes of padding tokens
// read a zeroed 64-byte LDS row.
template <int BITS, int NW, int UPT, int OUT>
__global__ __launch_bounds__(64 * NW) void gemm_decode_few_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t slab[];   // [M][K] int8 operands, then 64 zero bytes
  __shared__ int red[16 * 16];
  constexpr int MAXB = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ch0 = blockIdx.x * 16;
  const int nblk = K / DKB;
  const size_t arow = (size_t)K * BITS / 8;

  // ---- epilogue scales, fetched first so their latency is not paid at the end
  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
  const float ds_mine = OUT == OUT_ACC_I32 ? 0.f : dscale[min(tid / 16, M - 1)];
  // ---- activation staging load (issued first): UPT 16-byte units per thread,
  // UPT * 64 * NW >= M * K * BITS / 128 (chosen by the launcher).
  const int units = M * (int)(arow / 16);
  uint4 st[UPT];
#pragma unroll
  for (int q = 0; q < UPT; ++q) st[q] = reinterpret_cast<const uint4*>(A)[min(q * 64 * NW + tid, units - 1)];
  // ---- weight stream: blocks b = wave + NW*i (NW*MAXB*256 >= K for K <= 16384),
  // RING of them requested ahead (the decode kernel above explains why)
  constexpr int RING = 4;
  uint4 wq[RING];
  const int n = min(ch0 + c, N - 1);
  auto load = [&](int i) __attribute__((always_inline)) {
    const int b = min(wave + NW * i, nblk - 1);
    wq[i % RING] = *reinterpret_cast<const uint4*>(W + wrow_base(n, K) + (size_t)b * 1024 + 16 * g);
  };
#pragma unroll
  for (int i = 0; i < RING; ++i) load(i);
  // ---- operand form of the staged codes, token rows of K bytes
  const int opr = K;
  const int upr = (int)(arow / 16);                        // packed units per token row
#pragma unroll
  for (int q = 0; q < UPT; ++q) {
    const int u = q * 64 * NW + tid;
    if (u >= units) continue;
    const int t = u / upr, ub = u % upr;
    if constexpr (BITS == 8) {
      *reinterpret_cast<uint4*>(slab + t * opr + 16 * ub) = st[q];
    } else {
      // 32 INT4 codes -> 32 operand bytes 16*q in k order
      const uint32_t w[4] = {st[q].x, st[q].y, st[q].z, st[q].w};
      uint4 o0, o1;
      o0.x = (w[0] << 4) & 0xF0F0F0F0u; o0.y = w[0] & 0xF0F0F0F0u;
      o0.z = (w[1] << 4) & 0xF0F0F0F0u; o0.w = w[1] & 0xF0F0F0F0u;
      o1.x = (w[2] << 4) & 0xF0F0F0F0u; o1.y = w[2] & 0xF0F0F0F0u;
      o1.z = (w[3] << 4) & 0xF0F0F0F0u; o1.w = w[3] & 0xF0F0F0F0u;
      *reinterpret_cast<uint4*>(slab + t * opr + 32 * ub) = o0;
      *reinterpret_cast<uint4*>(slab + t * opr + 32 * ub + 16) = o1;
    }
  }
  if (tid < 4) reinterpret_cast<uint4*>(slab + M * opr)[tid] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < 256; i += 64 * NW) red[i] = 0;
  __syncthreads();

  v4i acc = v4i{};
  const uint8_t* arow_lds = c < M ? slab + c * opr + 64 * g : slab + M * opr;
  const int astep = c < M ? 1 : 0;                         // padding lanes keep reading the zero row
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = wave + NW * i;
    if (b < nblk) {                                        // wave-uniform
      const uint4* ap = reinterpret_cast<const uint4*>(arow_lds + astep * b * DKB);
      const uint4 p = wq[i % RING];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i wop = wstep(u4get(p, j));
        const v4i aop = as_v4i(ap[j]);                     // codes 16j .. 16j+15 of the lane's 64
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, aop, acc, 0, 0, 0);
      }
    }
    if (i + RING < MAXB) load(i + RING);
    __builtin_amdgcn_sched_barrier(0);                     // keep the requests where they are issued
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (c < M) atomicAdd(&red[c * 16 + 4 * g + r], acc[r]);
  __syncthreads();
  if (tid < M * 16) {   // M <= 4: one pass covers every (token, channel)
    const int t = tid / 16, nn = ch0 + tid % 16;
    if (nn < N) store_out<OUT>(Y, (size_t)t * N + nn, unscale<BITS>(red[tid]), ds_mine * aw);
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
// Short rows: K = 64 or 128 at any M, and K = 256 for 5 to 64 tokens.  The
// packed weights are then plain row-major (K/4 bytes per channel; at K = 256
// the 16-row tiles of the layout are exactly that), and one
// v_mfma_i32_16x16x64_i8 step
// covers 64 k: lane group g takes weight word 4j + g (k = 64j + 16g .. +15)
// and the same 16 codes of its token, both in natural order (wstep; INT4
// nibbles moved to the top of each byte, a4field).  Each wave computes 16
// channels x 64 tokens (four token groups), a 256-thread workgroup a 64 x 64
// output tile, channel tiles fastest so that neighbouring workgroups share
// their tokens' codes in L2.  At these K the outputs (2N bytes per token in
// bf16) outweigh the codes (K or K/2 bytes), so this is a plain streaming
// kernel: operands straight from global memory into registers, no LDS.
template <int BITS, int KS, int OUT>
__global__ __launch_bounds__(256) void gemm_smallk_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ W,
                                                          const float* __restrict__ dscale,
                                                          const float* __restrict__ walpha, void* __restrict__ Y,
                                                          int M, int N, int tiles_n) {
  static_assert(KS == 64 || KS == 128 || KS == 256, "short rows only");
  constexpr int STEPS = KS / 64;
  constexpr int AROW = KS * BITS / 8;            // code bytes per token
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int t0 = (int)(blockIdx.x / tiles_n) * 64;
  const int ch0 = (int)(blockIdx.x % tiles_n) * 64 + 16 * wave;
  if (ch0 >= N) return;                          // whole wave past the last channel (N % 16 == 0)
  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
  const uint32_t* wrow = reinterpret_cast<const uint32_t*>(W + (size_t)(ch0 + c) * (KS / 4));
  uint32_t wp[STEPS];
#pragma unroll
  for (int j = 0; j < STEPS; ++j) wp[j] = wrow[4 * j + g];
  float ds[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) ds[mb] = OUT == OUT_ACC_I32 ? 0.f : dscale[min(t0 + 16 * mb + c, M - 1)];
  v4i acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    // tokens past M read token M-1's codes; their sums are never stored
    const uint8_t* arow = A + (size_t)min(t0 + 16 * mb + c, M - 1) * AROW;
    acc[mb] = v4i{};
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      v4i aop;
      if constexpr (BITS == 8) {
        aop = as_v4i(*reinterpret_cast<const uint4*>(arow + 64 * j + 16 * g));
      } else {
        // codes k0 .. k0+15: word 0 holds k0 .. k0+7 (k0+4h+i at bits 8i+4h), word 1 the next 8
        const uint2 q = *reinterpret_cast<const uint2*>(arow + 32 * j + 8 * g);
        aop = v4i{(int)a4field(q.x, 0), (int)a4field(q.x, 1), (int)a4field(q.y, 0), (int)a4field(q.y, 1)};
      }
      acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wstep(wp[j]), aop, acc[mb], 0, 0, 0);
    }
  }
  // 16x16 accumulator layout: lane l / register r hold channel 4*(l/16)+r, token l%16
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int t = t0 + 16 * mb + c;
    if (t < M) store_out4<OUT>(Y, (size_t)t * N + ch0 + 4 * g, unscale4<BITS>(acc[mb]), ds[mb] * aw);
  }
}

// ===========================================================================
// Host side

// Split-K decode workspace: int32 partials [S][M][N], then one arrival
// counter per channel tile.
static size_t partials_bytes(const DecodePlan& p, int64_t M, int64_t N) {
  return p.S > 1 ? (((size_t)p.S * M * N * 4 + 255) & ~(size_t)255) : 0;
}
int gemm_tile_counters(int64_t M, int64_t K, int64_t N, bool blocked) {
  if (M > 64 || M <= 4) return 0;
  const DecodePlan p = decode_plan(M, K, N, blocked);
  return p.S > 1 ? (int)((N + 16 * p.cpw - 1) / (16 * p.cpw)) : 0;
}
size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, bool blocked) {
  if (M > 64 || M <= 0) return 0;
  const DecodePlan p = decode_plan(M, K, N, blocked);
  const size_t nc = (size_t)gemm_tile_counters(M, K, N, blocked);
  return partials_bytes(p, M, N) + ((nc * 4 + 255) & ~(size_t)255);
}
uint32_t* gemm_tile_counter_ptr(void* ws, int64_t M, int64_t K, int64_t N, bool blocked) {
  if (gemm_tile_counters(M, K, N, blocked) == 0 || ws == nullptr) return nullptr;
  return reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + partials_bytes(decode_plan(M, K, N, blocked), M, N));
}

template <int BITS, int MB, int CPW, int NW, int OUT, bool BLK = false>
static void launch_decode_p(const GemmArgs& a, int S) {
  constexpr int CH = 16 * CPW;
  dim3 grid((a.N + CH - 1) / CH, S);
  int32_t* part = static_cast<int32_t*>(a.ws);
  // only the four-group configuration hands its partials over in the kernel
  uint32_t* counts = CPW > 1 && S > 1 && S <= kDecodeMaxSplit ? a.tile_count : nullptr;
  bool long_rows = false;   // more than 8 blocks of 256 k per wave (K / S > 16384)
  if constexpr (CPW == 1) {
    long_rows = a.K / S > NW * 8 * DKB;
    if (long_rows)
      hipLaunchKernelGGL((gemm_decode_kernel<BITS, MB, CPW, NW, OUT, 16, BLK>), grid, dim3(64 * NW), 0, a.stream,
                         a.codes, a.wpack, a.dscale, a.walpha, a.out, a.M, a.N, a.K, S, part, counts);
  }
  if (!long_rows)
    hipLaunchKernelGGL((gemm_decode_kernel<BITS, MB, CPW, NW, OUT, 8, BLK>), grid, dim3(64 * NW), 0, a.stream, a.codes,
                       a.wpack, a.dscale, a.walpha, a.out, a.M, a.N, a.K, S, part, counts);
  if (S > 1 && counts == nullptr)
    hipLaunchKernelGGL((decode_reduce_kernel<BITS, OUT>), dim3((a.M * a.N + 255) / 256), dim3(256), 0, a.stream,
                       part, S, a.M, a.N, a.dscale, a.walpha, a.out);
}

template <int BITS, int UPT, int OUT>
static void launch_decode_few_u(const GemmArgs& a) {
  const size_t lds = (size_t)a.M * a.K + 64;
  // more than 64 KiB of dynamic LDS needs the function's limit raised, once
  // per device and instantiation (thread-safe; a failure shows as the
  // launch's error)
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64)
    std::call_once(once[dev], [] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_decode_few_kernel<BITS, 8, UPT, OUT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    });
  hipLaunchKernelGGL((gemm_decode_few_kernel<BITS, 8, UPT, OUT>), dim3((a.N + 15) / 16), dim3(512), lds,
                     a.stream, a.codes, a.wpack, a.dscale, a.walpha, a.out, a.M, a.N, a.K);
}

template <int BITS, int OUT>
static void launch_decode_few(const GemmArgs& a) {
  const long units = (long)a.M * a.K * BITS / 128;        // 16-byte units of packed codes
  if (units <= 512) launch_decode_few_u<BITS, 1, OUT>(a);
  else if (units <= 1024) launch_decode_few_u<BITS, 2, OUT>(a);
  else if (units <= 2048) launch_decode_few_u<BITS, 4, OUT>(a);
  else launch_decode_few_u<BITS, 8, OUT>(a);
}

template <int BITS, int OUT>
static void launch_decode_t(const GemmArgs& a) {
  // (the few-token kernel stages all codes in LDS and streams at most 16384 k)
  if (a.M <= 4 && a.K <= 16384) { launch_decode_few<BITS, OUT>(a); return; }
  const DecodePlan p = decode_plan(a.M, a.K, a.N, a.codes_blocked);
  if (a.codes_blocked) {
    if (p.mb == 1) launch_decode_p<BITS, 1, 1, 8, OUT, true>(a, p.S);
    else if (p.mb == 2) launch_decode_p<BITS, 2, 1, 8, OUT, true>(a, p.S);
    else if (p.cpw == 1) launch_decode_p<BITS, 4, 1, 8, OUT, true>(a, p.S);
    else launch_decode_p<BITS, 4, 4, 8, OUT, true>(a, p.S);
    return;
  }
  if (p.mb == 1) launch_decode_p<BITS, 1, 1, 8, OUT>(a, p.S);
  else if (p.mb == 2) launch_decode_p<BITS, 2, 1, 8, OUT>(a, p.S);
  else launch_decode_p<BITS, 4, 4, 8, OUT>(a, p.S);
}

// INT4 stages hold 256 k (3 x 48 KiB of LDS), INT8 stages 128 k (3 x 40 KiB).
// INT4 runs 8 waves (2 per SIMD: one wave's operand expansion overlaps the
// other's MFMAs); INT8 keeps 4 (its wider activation fragments would spill).
template <int BITS>
constexpr int prefill_waves() { return BITS == 4 ? 8 : 4; }
template <int BITS>
constexpr int prefill_bk() { return BITS == 4 ? 256 : 128; }

template <int BITS, int OUT>
static void launch_prefill_t(const GemmArgs& a) {
  const int tm = (a.M + PBM - 1) / PBM, tn = (a.N + PBN - 1) / PBN;
  hipLaunchKernelGGL((gemm_prefill_kernel<BITS, prefill_bk<BITS>(), prefill_waves<BITS>(), OUT>), dim3(tm * tn),
                     dim3(64 * prefill_waves<BITS>()), 0, a.stream, a.codes, a.wpack, a.dscale, a.walpha, a.out, a.M, a.N, a.K,
                     tm, tn);
}

template <int BITS, int OUT>
static void launch_smallk(const GemmArgs& a) {
  const int tm = (a.M + 63) / 64, tn = (a.N + 63) / 64;
  if (a.K == 64)
    hipLaunchKernelGGL((gemm_smallk_kernel<BITS, 64, OUT>), dim3(tm * tn), dim3(256), 0, a.stream, a.codes, a.wpack,
                       a.dscale, a.walpha, a.out, a.M, a.N, tn);
  else if (a.K == 256)
    hipLaunchKernelGGL((gemm_smallk_kernel<BITS, 256, OUT>), dim3(tm * tn), dim3(256), 0, a.stream, a.codes, a.wpack,
                       a.dscale, a.walpha, a.out, a.M, a.N, tn);
  else
    hipLaunchKernelGGL((gemm_smallk_kernel<BITS, 128, OUT>), dim3(tm * tn), dim3(256), 0, a.stream, a.codes, a.wpack,
                       a.dscale, a.walpha, a.out, a.M, a.N, tn);
}

template <int BITS, int OUT>
static void launch_t(const GemmArgs& a) {
  // K = 256 with 5..64 tokens: the whole row is one MFMA k-loop of four steps,
  // and the short-row kernel (no K split, no LDS) beats the decode kernels
  // (8 tokens, N = 256: forward 8.7 -> 5.5 us in graph replay; at 1 token the
  // few-token kernel stays ahead)
  if (a.K < 256 || (a.K == 256 && a.M > 4 && a.M <= 64)) launch_smallk<BITS, OUT>(a);
  else if (a.M <= 64) launch_decode_t<BITS, OUT>(a);
  else launch_prefill_t<BITS, OUT>(a);
}

// fp6 codes with at most 64 tokens: the split decode matmul (64 channels per
// workgroup; K split as the row-major plan says above 32 tokens, unsplit below, where
// only stage calls bring fp6 codes).
template <int OUT>
static void launch_decode_fp6(const GemmArgs& a) {
  const DecodePlan p = decode_plan(a.M, a.K, a.N, false);
  launch_decode_p<6, 4, 4, 8, OUT>(a, p.cpw == 4 ? p.S : 1);
}

constexpr int kFp6SmallTileBelow = 256;
constexpr int kCUs = 256;   // compute units of the part: one 256-row tile each per round

template <int OUT, int T, int TN = T>
static void launch_fp6_t(const GemmArgs& a) {
  const int tm = (a.M + T - 1) / T, tn = (a.N + TN - 1) / TN;
  if (a.K == 256)
    hipLaunchKernelGGL((gemm_fp6_kernel<OUT, 2, T, TN>), dim3(tm * tn), dim3(256), 0, a.stream, a.codes, a.wpack,
                       a.dscale, a.walpha, a.out, a.M, a.N, a.K, tm, tn);
  else
    hipLaunchKernelGGL((gemm_fp6_kernel<OUT, 4, T, TN>), dim3(tm * tn), dim3(256), 0, a.stream, a.codes, a.wpack,
                       a.dscale, a.walpha, a.out, a.M, a.N, a.K, tm, tn);
}

// Tile shape of the fp6 x fp4 matmul.  256 x 192 when it gives the busiest
// compute unit less work than 256 x 256 -- rounds of 256 resident tiles times
// the tile's work, a 256 x 192 tile counted at 0.78 of a square one (three
// quarters of the products with a little less operand reuse) -- and fills at
// least three quarters of its last round (N = 3072: 256 tiles at M = 4096,
// 512 at M = 8192, against 192 and 384 square ones).  Otherwise 256 x 256,
// or 128 x 128 when there are fewer 256 x 256 tiles than compute units.
enum F6Tile { kTile256, kTile256x192, kTile128 };
static F6Tile fp6_tile(int64_t M, int64_t N) {
  const int64_t tm = (M + 255) / 256;
  const int64_t t256 = tm * ((N + 255) / 256), t192 = tm * ((N + 191) / 192);
  const int64_t r256 = (t256 + kCUs - 1) / kCUs, r192 = (t192 + kCUs - 1) / kCUs;
  if (r192 * 78 < r256 * 100 && 4 * t192 >= 3 * kCUs * r192) return kTile256x192;
  return t256 < kFp6SmallTileBelow ? kTile128 : kTile256;
}

template <int OUT>
static void launch_fp6_o(const GemmArgs& a) {
  switch (fp6_tile(a.M, a.N)) {
    case kTile256x192: launch_fp6_t<OUT, 256, 192>(a); break;
    case kTile128: launch_fp6_t<OUT, 128>(a); break;
    default: launch_fp6_t<OUT, 256>(a); break;
  }
}

hipError_t launch_gemm_fp6(const GemmArgs& a) {
  if (a.M == 0) return hipSuccess;
  if (a.M <= 64) {
    switch (a.out_kind) {
      case OUT_ACC_I32: launch_decode_fp6<OUT_ACC_I32>(a); break;
      case OUT_F32: launch_decode_fp6<OUT_F32>(a); break;
      default: launch_decode_fp6<OUT_BF16>(a); break;
    }
    return hipGetLastError();
  }
  switch (a.out_kind) {
    case OUT_ACC_I32: launch_fp6_o<OUT_ACC_I32>(a); break;
    case OUT_F32: launch_fp6_o<OUT_F32>(a); break;
    default: launch_fp6_o<OUT_BF16>(a); break;
  }
  return hipGetLastError();
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
