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
// so that the MFMA fragment reads (8 or 16 lanes per LDS cycle: rows r..r+7 or
// r..r+15 of one unit column) and the copies hit distinct banks.
template <int U>
HBL_DEV int swz(int row) {
  if constexpr (U == 8) return (row ^ (row >> 3)) & 7;
  else if constexpr (U == 4) return ((row >> 1) ^ (row >> 3)) & 3;
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
  const int KT = K / BK;
  auto phase = [&](int kt, int buf) {
    if (kt + 1 < KT) wait_vmcnt<NL>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < KT) dma(kt + 2, buf == 0 ? 2 : buf - 1);
    compute(buf);
  };
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
    store_bf16_staged<CB>(smem + wave * (64 * (CB * 64 + 32)), static_cast<uint16_t*>(Y), dscale, aw, M, N,
                          m0 + wm * 128, n0 + wn * (32 * CB), lane,
                          [&](int rb, int cb, int r) { return (float)unscale<BITS>(acc[rb][cb][r]); });
    return;
  }
#pragma unroll
  for (int rbk = 0; rbk < 4; ++rbk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 128 + rbk * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (m >= M) continue;
      const float t = OUT == OUT_ACC_I32 ? 0.f : dscale[m] * aw;
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
// compile-time constants.
template <int OUT, int US>
__global__ __launch_bounds__(256, 1) void gemm_fp6_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[F6_LDS];
  constexpr int A_LOADS = F6_A_STAGE / 16 / 256, B_LOADS = F6_B_PAIR / 16 / 256;   // 6 and 4

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
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;
  // A is blocked by 128 k: stage kt of the tile is the contiguous run of
  // 256 x 96 bytes at (kt * M + m0) * 96.
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
    const int P = (j * 4 + wave) * 64 + lane, col = P >> 2, u = (P & 3) ^ f6_bswz(col);
    const int nr = min(n0 + col, N - 1) - n0;       // tiled: 16-row blocks of 4K bytes, 64-byte row segments
    b_off[j] = (uint32_t)(nr >> 4) * (uint32_t)K * 4u + (uint32_t)(nr & 15) * 64u + 16u * u;
  }
  // A copy j (0..5) of stage kt into A buffer buf; B copy j (0..3) of stage
  // pair p into B slot sl
  auto dmaA = [&](int j, int kt, int buf) __attribute__((always_inline)) {
    lds_copy16s(a_tile + (size_t)kt * a_stage, a_off[j], lds0 + buf * F6_A_STAGE + (j * 4 + wave_s) * 1024);
  };
  auto dmaB = [&](int j, int p, int sl) __attribute__((always_inline)) {
    lds_copy16s(b_tile + (size_t)p * 1024, b_off[j], lds0 + F6_B_BASE + sl * F6_B_PAIR + (j * 4 + wave_s) * 1024);
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  // Register fragments of one stage: per lane 48 A bytes (32-k groups 2g and
  // 2g+1 of four 32-row blocks), kept as one 12-dword vector per block so the
  // two 6-dword MFMA operands (8-dword vectors, the last two unused) are
  // sub-ranges of it, and 16 packed B bytes
  // (the same groups of four 32-column blocks).  Read r of a stage: r < 4 the
  // B block r, else A block (r-4)/3, unit (r-4)%3.
  struct Frag {
    v16i a[4];
    v4i b[4];
  };
  // read r of stage kt (A buffer kt % 4, B slot (kt / 2) % 2, half kt % 2)
  auto read1 = [&](Frag& f, int r, int kt) __attribute__((always_inline)) {
    const uint8_t* sa = smem + (kt & (F6_NBUF - 1)) * F6_A_STAGE;
    if (r < 4) {
      const int n = wn * 128 + r * 32 + l32;
      const uint8_t* sb = smem + F6_B_BASE + ((kt >> 1) & 1) * F6_B_PAIR;
      f.b[r] = *reinterpret_cast<const v4i*>(sb + n * F6_BPROW + 16 * ((2 * (kt & 1) + g) ^ f6_bswz(n)));
    } else {
      const int rb = (r - 4) / 3, t = (r - 4) % 3;
      const int row = wm * 128 + rb * 32 + l32;
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
    for (int rb = 0; rb < 4; ++rb) {
      const v8i af = aop(cur, 0, rb);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        mfma(af, bf0[cb], acc[rb][cb]);
        if (cb == 1) bf1[rb] = bexp1(cur, 1, rb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (u & 1) wait_vmcnt<2 * A_LOADS>(); else wait_vmcnt<2 * A_LOADS + B_LOADS>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
    const int akt = min(kt + F6_NBUF, KT - 1);
    const int bp = min((kt + 3) >> 1, KP - 1);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const v8i af = aop(cur, 1, rb);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int i = rb * 4 + cb;
        mfma(af, bf1[cb], acc[rb][cb]);
        read1(nxt, i, u + 1);
        if (u & 1) {
          // odd stage: B pair into the slot this pair of stages used, then A
          if (i < B_LOADS) dmaB(i, bp, ((u + 3) >> 1) & 1);
          else if (i < B_LOADS + A_LOADS) dmaA(i - B_LOADS, akt, u & (F6_NBUF - 1));
        } else {
          // even stage: the A_LOADS copies of stage kt+4 after MFMAs 1, 3, ..., 2*A_LOADS-1
          if ((i & 1) && (i >> 1) < A_LOADS) dmaA(i >> 1, akt, u & (F6_NBUF - 1));
        }
        if (i >= 8 && !(i & 1)) bf0[(i - 8) >> 1] = bexp1(nxt, 0, (i - 8) >> 1);
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
  dmaA_all(0); dmaB_all(0); dmaA_all(1); dmaA_all(2); dmaB_all(1); dmaA_all(3);
  wait_vmcnt<3 * A_LOADS + B_LOADS>();     // A0 and B0 have landed
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
#pragma unroll
  for (int r = 0; r < 16; ++r) read1(f0, r, 0);
  v8i bf0[4], bf1[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) bf0[cb] = bexp1(f0, 0, cb);
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
    store_bf16_staged<4>(smem + wave * (64 * (4 * 64 + 32)), static_cast<uint16_t*>(Y), dscale, aw, M, N,
                         m0 + wm * 128, n0 + wn * 128, lane,
                         [&](int rb, int cb, int r) { return acc[rb][cb][r]; });
  } else {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 128 + rb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m >= M) continue;
        const float t = OUT == OUT_ACC_I32 ? 0.f : dscale[m] * aw;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int n = n0 + wn * 128 + cb * 32 + l32;
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
// ranges.  The range is cut into 256-k blocks dealt round-robin to the waves.
// Each wave issues every load it will need up front -- per block, its packed
// weights (16 bytes per lane per 16 channels) and then that block's
// activation codes -- so the whole weight stream is in flight at once and,
// because loads retire in issue order, block i can start as soon as its own
// two loads have landed.  Every weight byte is read from HBM once.
// v_mfma_i32_16x16x64_i8 runs with channels on the MFMA's M side and up to 16
// tokens on its N side.  The waves' int32 partials meet in LDS through integer
// atomics (exact, order free).  With S > 1 a second small kernel sums the S
// partials in order and dequantises; integer sums are exact, so the result is
// the same for every S.
constexpr int DKB = 256;

struct DecodePlan { int cpw, S, mb, nw; };
constexpr int kDecodeMaxSplit = 4;   // split-K ways the in-kernel reduction handles
static DecodePlan decode_plan(int M, int K) {
#ifdef HBL_DECODE_PLAN
  DecodePlan p = HBL_DECODE_PLAN(M);
#else
  DecodePlan p = M <= 16 ? DecodePlan{1, 1, 1, 8} : DecodePlan{4, 4, 4, 8};
#endif
  while (p.S > 1 && K / p.S < DKB) p.S /= 2;
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
template <int BITS, int MB, int CPW, int NW, int OUT>
__global__ __launch_bounds__(64 * NW) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K, int S,
    int32_t* __restrict__ partial, uint32_t* __restrict__ tile_count) {
  // Blocks held per wave per round: their loads need MAXB * (CPW + MB*BITS/2)
  // uint4 registers, kept near 48 (192 VGPRs).
  // (two with four token groups: 8 waves of 184 registers, two per SIMD, so
  // one wave's MFMAs cover another's waits)
  constexpr int MAXB = MB == 4 ? 2 : (48 / (CPW + MB * BITS / 2)) >= 8 ? 8 : (48 / (CPW + MB * BITS / 2)) >= 4 ? 4 : 2;
  constexpr int CH = 16 * CPW;
  // Partial sums per (token, channel), rows of RL ints.  Inside each block of
  // 16 channels column 4r + q holds channel 4q + r, and RL = 4 (mod 64): the
  // 64 lanes of one accumulate (token c, channel 4g + r) then hit 64 distinct
  // banks (4c + g), where plain rows of CH ints would put 16 lanes on one.
  constexpr int RL = CH + 4;
  __shared__ int red[MB * 16 * RL];
  __shared__ int is_last;
  auto red_col = [](int nl) { return (nl & ~15) | ((nl & 3) << 2) | ((nl >> 2) & 3); };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ch0 = blockIdx.x * CH, s = blockIdx.y;
  const int Kr = K / S, kbeg = s * Kr;
  const int nblk = Kr / DKB;                                   // 256-k blocks in this range
  const size_t arow = (size_t)K * BITS / 8;

  for (int i = tid; i < MB * 16 * RL; i += 64 * NW) red[i] = 0;
  // epilogue scales fetched up front (their latency is not paid at the end)
  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
  float ds_pre[(MB * 16 * CH + 64 * NW - 1) / (64 * NW)];
#pragma unroll
  for (int q = 0; q < (MB * 16 * CH + 64 * NW - 1) / (64 * NW); ++q)
    ds_pre[q] = OUT == OUT_ACC_I32 ? 0.f : dscale[min((q * 64 * NW + tid) / CH, M - 1)];

  v4i acc[CPW][MB];
#pragma unroll
  for (int cp = 0; cp < CPW; ++cp)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[cp][mb] = v4i{};

  // Blocks b = wave + NW*i, taken MAXB at a time.
  for (int b0 = wave; b0 < nblk; b0 += NW * MAXB) {
    uint4 wq[MAXB][CPW];
    uint4 aq[MAXB][MB][BITS / 2];
    // Loads are unconditional (out-of-range indices are clamped to valid
    // addresses and the values discarded), so the compiler can release block i
    // with a partial vmcnt wait instead of waiting for every load.
#pragma unroll
    for (int i = 0; i < MAXB; ++i) {
      const int b = min(b0 + NW * i, nblk - 1);
      const int kb = kbeg + b * DKB + 64 * g;                 // this lane's 64 codes of block b
#pragma unroll
      for (int cp = 0; cp < CPW; ++cp) {
        const int n = min(ch0 + 16 * cp + c, N - 1);
        wq[i][cp] = *reinterpret_cast<const uint4*>(W + wrow_base(n, K) + (size_t)((kbeg + b * DKB) >> 8) * 1024 + 16 * g);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int t = min(16 * mb + c, M - 1);
        const uint4* ap = reinterpret_cast<const uint4*>(A + (size_t)t * arow + (size_t)kb * BITS / 8);
#pragma unroll
        for (int d = 0; d < BITS / 2; ++d) aq[i][mb][d] = ap[d];
      }
    }
#pragma unroll
    for (int i = 0; i < MAXB; ++i) {
      if (b0 + NW * i >= nblk) continue;   // wave-uniform; keeps the loop unrolled (registers, no scratch)
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
            // padding tokens (16*mb + c >= M) read token M-1's codes; their
            // sums are never stored
            acc[cp][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, aop, acc[cp][mb], 0, 0, 0);
          }
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
        if (16 * mb + c < M) atomicAdd(&red[(16 * mb + c) * RL + 16 * cp + 4 * r + g], acc[cp][mb][r]);
  __syncthreads();

#pragma unroll
  for (int q = 0; q < (MB * 16 * CH + 64 * NW - 1) / (64 * NW); ++q) {
    const int e = q * 64 * NW + tid;
    if (e >= M * CH) continue;
    const int t = e / CH, n = ch0 + e % CH;
    if (n >= N) continue;
    const int v = red[t * RL + red_col(e % CH)];
    if (S == 1) store_out<OUT>(Y, (size_t)t * N + n, unscale<BITS>(v), ds_pre[q] * aw);
    else if constexpr (MB == 1) partial[((size_t)s * M + t) * N + n] = v;
    else __hip_atomic_store(&partial[((size_t)s * M + t) * N + n], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // (the single-token-group instantiation serves M <= 16, which the plan
  // never splits; it keeps the separate reduction for any split it is given)
  if constexpr (MB == 1) return;
  if (S == 1 || tile_count == nullptr) return;
  __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(&tile_count[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (uint32_t)(S - 1);
  __syncthreads();
  if (!is_last) return;
  // every partial this thread sums is requested before any is waited for
  // (clamped, always in-bounds addresses; splits past S count zero)
  constexpr int NQ = (MB * 16 * CH + 64 * NW - 1) / (64 * NW);
  int sum[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = q * 64 * NW + tid;
    const int t = min(e / CH, M - 1), n = min(ch0 + e % CH, N - 1);
    sum[q] = 0;
#pragma unroll
    for (int s2 = 0; s2 < kDecodeMaxSplit; ++s2) {
      const int v = __hip_atomic_load(&partial[((size_t)min(s2, S - 1) * M + t) * N + n], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      sum[q] += s2 < S ? v : 0;
    }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = q * 64 * NW + tid;
    if (e >= M * CH) continue;
    const int t = e / CH, n = ch0 + e % CH;
    if (n >= N) continue;
    store_out<OUT>(Y, (size_t)t * N + n, unscale<BITS>(sum[q]), ds_pre[q] * aw);
  }
  if (tid == 0) __hip_atomic_store(&tile_count[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  // ---- weight stream: blocks b = wave + NW*i (NW*MAXB*256 >= K for K <= 16384)
  uint4 wq[MAXB];
  const int n = min(ch0 + c, N - 1);
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int b = min(wave + NW * i, nblk - 1);
    wq[i] = *reinterpret_cast<const uint4*>(W + wrow_base(n, K) + (size_t)b * 1024 + 16 * g);
  }
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
    if (b >= nblk) continue;                               // wave-uniform
    const uint4* ap = reinterpret_cast<const uint4*>(arow_lds + astep * b * DKB);
    const uint4 p = wq[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4i wop = wstep(u4get(p, j));
      const v4i aop = as_v4i(ap[j]);                       // codes 16j .. 16j+15 of the lane's 64
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, aop, acc, 0, 0, 0);
    }
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
// Host side

// Split-K decode workspace: int32 partials [S][M][N], then one arrival
// counter per channel tile.
static size_t partials_bytes(const DecodePlan& p, int64_t M, int64_t N) {
  return p.S > 1 ? (((size_t)p.S * M * N * 4 + 255) & ~(size_t)255) : 0;
}
int gemm_tile_counters(int64_t M, int64_t K, int64_t N) {
  if (M > 64 || M <= 4) return 0;
  const DecodePlan p = decode_plan((int)M, (int)K);
  return p.S > 1 ? (int)((N + 16 * p.cpw - 1) / (16 * p.cpw)) : 0;
}
size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M > 64 || M <= 0) return 0;
  const DecodePlan p = decode_plan((int)M, (int)K);
  const size_t nc = (size_t)gemm_tile_counters(M, K, N);
  return partials_bytes(p, M, N) + ((nc * 4 + 255) & ~(size_t)255);
}
uint32_t* gemm_tile_counter_ptr(void* ws, int64_t M, int64_t K, int64_t N) {
  if (gemm_tile_counters(M, K, N) == 0 || ws == nullptr) return nullptr;
  return reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + partials_bytes(decode_plan((int)M, (int)K), M, N));
}

template <int BITS, int MB, int CPW, int NW, int OUT>
static void launch_decode_p(const GemmArgs& a, int S) {
  constexpr int CH = 16 * CPW;
  dim3 grid((a.N + CH - 1) / CH, S);
  int32_t* part = static_cast<int32_t*>(a.ws);
  uint32_t* counts = MB > 1 && S > 1 && S <= kDecodeMaxSplit ? a.tile_count : nullptr;
  hipLaunchKernelGGL((gemm_decode_kernel<BITS, MB, CPW, NW, OUT>), grid, dim3(64 * NW), 0, a.stream, a.codes,
                     a.wpack, a.dscale, a.walpha, a.out, a.M, a.N, a.K, S, part, counts);
  if (S > 1 && counts == nullptr)
    hipLaunchKernelGGL((decode_reduce_kernel<BITS, OUT>), dim3((a.M * a.N + 255) / 256), dim3(256), 0, a.stream,
                       part, S, a.M, a.N, a.dscale, a.walpha, a.out);
}

template <int BITS, int UPT, int OUT>
static void launch_decode_few_u(const GemmArgs& a) {
  const size_t lds = (size_t)a.M * a.K + 64;
  // more than 64 KiB of dynamic LDS needs the function's limit raised, once
  // per device (a failure shows as the launch's error)
  static bool attr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr[dev] &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_decode_few_kernel<BITS, 8, UPT, OUT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024) == hipSuccess)
    attr[dev] = true;
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
  if (a.M <= 4) { launch_decode_few<BITS, OUT>(a); return; }
  const DecodePlan p = decode_plan(a.M, a.K);
#ifdef HBL_DECODE_VARIANTS
  HBL_DECODE_VARIANTS
#endif
  if (p.mb == 1) launch_decode_p<BITS, 1, 1, 8, OUT>(a, p.S);
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
static void launch_t(const GemmArgs& a) {
  if (a.M <= 64) launch_decode_t<BITS, OUT>(a);
  else launch_prefill_t<BITS, OUT>(a);
}

hipError_t launch_gemm_fp6(const GemmArgs& a) {
  if (a.M == 0) return hipSuccess;
  const int tm = (a.M + PBM - 1) / PBM, tn = (a.N + PBN - 1) / PBN;
#define HBL_F6(OUT)                                                                                          \
  if (a.K == 256)                                                                                                \
    hipLaunchKernelGGL((gemm_fp6_kernel<OUT, 2>), dim3(tm * tn), dim3(256), 0, a.stream, a.codes, a.wpack,         \
                       a.dscale, a.walpha, a.out, a.M, a.N, a.K, tm, tn);                                          \
  else                                                                                                           \
    hipLaunchKernelGGL((gemm_fp6_kernel<OUT, 4>), dim3(tm * tn), dim3(256), 0, a.stream, a.codes, a.wpack,         \
                       a.dscale, a.walpha, a.out, a.M, a.N, a.K, tm, tn)
  switch (a.out_kind) {
    case OUT_ACC_I32: HBL_F6(OUT_ACC_I32); break;
    case OUT_F32: HBL_F6(OUT_F32); break;
    default: HBL_F6(OUT_BF16); break;
  }
#undef HBL_F6
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
