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

// 16 ternary codes (2-bit, k0+4j+i at bits 8i+2j) -> 16 int8 in k order.
HBL_DEV v4i expand_ternary(uint32_t p) {
  v4i o;
  o[0] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, p & 0x03030303u);
  o[1] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (p >> 2) & 0x03030303u);
  o[2] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (p >> 4) & 0x03030303u);
  o[3] = (int)__builtin_amdgcn_perm(0u, 0xFF000100u, (p >> 6) & 0x03030303u);
  return o;
}

// Four 4-bit two's complement codes in the low nibbles of the bytes of x
// (already XORed with 0x08 per byte) -> four int8.
HBL_DEV int sext_nibbles(uint32_t e) { return (int)((e + 0x78787878u) ^ 0x80808080u); }

// 16 INT4 codes (two words; k0+4j+i at bits 8i+4j of each) -> 16 int8 in k order.
HBL_DEV v4i expand_int4(uint32_t w0, uint32_t w1) {
  const uint32_t a = w0 ^ 0x88888888u, b = w1 ^ 0x88888888u;
  v4i o;
  o[0] = sext_nibbles(a & 0x0F0F0F0Fu);
  o[1] = sext_nibbles((a >> 4) & 0x0F0F0F0Fu);
  o[2] = sext_nibbles(b & 0x0F0F0F0Fu);
  o[3] = sext_nibbles((b >> 4) & 0x0F0F0F0Fu);
  return o;
}

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
    uint4 bq[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int n = wn * 128 + cb * 32 + l32;
      bq[cb] = *reinterpret_cast<const uint4*>(sb + n * 32 + 16 * (g ^ swz_b(n)));
    }
    uint4 aq[4][2];
    if constexpr (BITS == 4) {
#pragma unroll
      for (int rbk = 0; rbk < 4; ++rbk) {
        const int row = wm * 128 + rbk * 32 + l32;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          aq[rbk][h] = *reinterpret_cast<const uint4*>(sa + row * 64 + 16 * ((2 * g + h) ^ swz_a<4>(row)));
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      v4i bf[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const uint32_t p = ks == 0 ? bq[cb].x : ks == 1 ? bq[cb].y : ks == 2 ? bq[cb].z : bq[cb].w;
        bf[cb] = expand_ternary(p);
      }
#pragma unroll
      for (int rbk = 0; rbk < 4; ++rbk) {
        v4i af;
        if constexpr (BITS == 8) {
          const int row = wm * 128 + rbk * 32 + l32;
          af = *reinterpret_cast<const v4i*>(sa + row * 128 + 16 * ((4 * g + ks) ^ swz_a<8>(row)));
        } else {
          const uint4 u = aq[rbk][ks >> 1];
          af = (ks & 1) ? expand_int4(u.z, u.w) : expand_int4(u.x, u.y);
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
        if (n < N) store_out<OUT>(Y, (size_t)m * N + n, acc[rbk][cb][r], t);
      }
    }
  }
}

// ===========================================================================
// Decode (M <= 64)
constexpr int DWAVES = 4;          // waves per workgroup
constexpr int DCH = 16 * DWAVES;   // output channels per workgroup
constexpr int DKB = 256;           // k per load block (16 bytes of packed weights per lane)

// Split of K into KS slabs so that about 512 workgroups stream the weights,
// while the slab's activation codes still fit in 64 KiB of LDS.
static int decode_splits(int M, int K, int N, int bits) {
  const int nblk = (N + DCH - 1) / DCH;
  int ks = 1;
  while (nblk * ks < 512 && K / (2 * ks) >= DKB) ks *= 2;
  while ((long long)M * (K / ks) * bits / 8 + (long long)M * 16 > 65536 && K / (2 * ks) >= DKB) ks *= 2;
  return ks;
}

template <int BITS>
struct DCfg {
  static constexpr int PADB = BITS == 8 ? 16 : 8;  // LDS row padding (bytes) against bank conflicts
};

template <int BITS, int MB, int OUT>
__global__ __launch_bounds__(256) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, const float* __restrict__ dscale,
    const float* __restrict__ walpha, void* __restrict__ Y, int M, int N, int K, int KS,
    int32_t* __restrict__ partial, int* __restrict__ counters) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sact[];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = blockIdx.x, ks = blockIdx.y;
  const int Kslab = K / KS, kbeg = ks * Kslab;
  const int nkb = Kslab / DKB;
  const int row_bytes = Kslab * BITS / 8;
  const int srow = row_bytes + DCfg<BITS>::PADB;
  const size_t arow = (size_t)K * BITS / 8;

  // ---- stage this slab's activation codes (M rows) in LDS, 16 bytes per thread per step
  {
    const int units = row_bytes / 16;
    for (int q = tid; q < M * units; q += 256) {
      const int t = q / units, u = q % units;
      const uint4 v = *reinterpret_cast<const uint4*>(A + (size_t)t * arow + (size_t)kbeg * BITS / 8 + 16 * u);
      uint32_t* d = reinterpret_cast<uint32_t*>(sact + t * srow + 16 * u);
      if constexpr (DCfg<BITS>::PADB == 16) {
        *reinterpret_cast<uint4*>(d) = v;
      } else {
        *reinterpret_cast<uint2*>(d) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(d + 2) = make_uint2(v.z, v.w);
      }
    }
  }

  // ---- weights: lane (channel c = lane%16, group g = lane/16) takes k in
  // [kb*256 + 64g, +64) of every 256-k block: one 16-byte load per block.
  const int c = lane & 15, g = lane >> 4;
  // N is a multiple of 16, so a wave's 16 channels are all valid or all past N.
  const bool wave_ok = nblk * DCH + wave * 16 < N;
  const int n = wave_ok ? nblk * DCH + wave * 16 + c : 0;
  const uint8_t* wp = W + (size_t)n * (K / 4) + kbeg / 4 + 16 * g;
  v4i acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = v4i{};
  __syncthreads();

  constexpr int UNR = 8;  // weight loads kept in flight per lane
  for (int kb0 = 0; kb0 < nkb; kb0 += UNR) {
    uint4 wq[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      wq[u] = (wave_ok && kb0 + u < nkb) ? *reinterpret_cast<const uint4*>(wp + (size_t)(kb0 + u) * (DKB / 4))
                                         : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (kb0 + u >= nkb) break;
      const int kb = kb0 + u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t p = j == 0 ? wq[u].x : j == 1 ? wq[u].y : j == 2 ? wq[u].z : wq[u].w;
        const v4i a = expand_ternary(p);
        const int kk = kb * DKB + 64 * g + 16 * j;  // k offset inside the slab
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int t = mb * 16 + c;
          v4i b = v4i{};
          if (t < M) {
            if constexpr (BITS == 8) {
              b = *reinterpret_cast<const v4i*>(sact + t * srow + kk);
            } else {
              const uint2 w2 = *reinterpret_cast<const uint2*>(sact + t * srow + kk / 2);
              b = expand_int4(w2.x, w2.y);
            }
          }
          acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[mb], 0, 0, 0);
        }
      }
    }
  }

  // ---- 16x16 accumulator layout: lane l / register r hold channel 4*(l/16)+r, token l%16
  const float aw = OUT == OUT_ACC_I32 ? 0.f : fmaxf(walpha[0], kEpsQ);
  const int ch0 = nblk * DCH + wave * 16 + 4 * g;
  if (KS == 1) {
    if (!wave_ok) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int t = mb * 16 + c;
      if (t >= M) continue;
      const float tt = OUT == OUT_ACC_I32 ? 0.f : dscale[t] * aw;
#pragma unroll
      for (int r = 0; r < 4; ++r) store_out<OUT>(Y, (size_t)t * N + ch0 + r, acc[mb][r], tt);
    }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = mb * 16 + c;
    if (t >= M || !wave_ok) continue;
    *reinterpret_cast<int4*>(partial + ((size_t)ks * M + t) * N + ch0) =
        make_int4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
  }
  // Last workgroup of this channel block sums the slabs in slab order.
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&counters[nblk], 1) == KS - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int e = tid; e < M * DCH; e += 256) {
    const int t = e / DCH, ch = nblk * DCH + e % DCH;
    if (ch >= N) continue;
    int s = 0;
    for (int k2 = 0; k2 < KS; ++k2) s += __builtin_nontemporal_load(partial + ((size_t)k2 * M + t) * N + ch);
    const float tt = OUT == OUT_ACC_I32 ? 0.f : dscale[t] * aw;
    store_out<OUT>(Y, (size_t)t * N + ch, s, tt);
  }
  if (tid == 0) counters[nblk] = 0;
}

// ===========================================================================
// Host side

size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M > 64 || M <= 0) return 0;
  // worst case over the two activation widths
  const int ks = decode_splits((int)M, (int)K, (int)N, 8) > decode_splits((int)M, (int)K, (int)N, 4)
                     ? decode_splits((int)M, (int)K, (int)N, 8) : decode_splits((int)M, (int)K, (int)N, 4);
  const size_t part = (size_t)ks * M * N * 4;
  const size_t cnt = (size_t)((N + DCH - 1) / DCH + 64) * 4;
  return ((part + 255) & ~(size_t)255) + ((cnt + 255) & ~(size_t)255);
}

int gemm_zero_words(int64_t M, int64_t K, int64_t N) {
  (void)K;
  return (M > 0 && M <= 64) ? (int)((N + DCH - 1) / DCH) : 0;
}

// Counters live after the partials in the workspace.
static int* decode_counters(void* ws, int64_t M, int64_t K, int64_t N) {
  const size_t part = gemm_workspace_bytes(M, K, N) - (((size_t)((N + DCH - 1) / DCH + 64) * 4 + 255) & ~(size_t)255);
  return reinterpret_cast<int*>(static_cast<uint8_t*>(ws) + part);
}
int* gemm_counters(void* ws, int64_t M, int64_t K, int64_t N) { return decode_counters(ws, M, K, N); }

__global__ void zero_i32_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
hipError_t launch_zero_i32(int* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

template <int BITS, int OUT>
static void launch_decode_t(const GemmArgs& a) {
  const int KS = decode_splits(a.M, a.K, a.N, BITS);
  const int MB = (a.M + 15) / 16;
  const size_t lds = (size_t)a.M * ((size_t)(a.K / KS) * BITS / 8 + DCfg<BITS>::PADB);
  dim3 grid((a.N + DCH - 1) / DCH, KS);
  int32_t* part = static_cast<int32_t*>(a.ws);
  int* cnt = decode_counters(a.ws, a.M, a.K, a.N);
#define HBL_DEC(MBV)                                                                                      \
  hipLaunchKernelGGL((gemm_decode_kernel<BITS, MBV, OUT>), grid, dim3(256), lds, a.stream, a.codes, a.wpack, \
                     a.dscale, a.walpha, a.out, a.M, a.N, a.K, KS, part, cnt)
  switch (MB) {
    case 1: HBL_DEC(1); break;
    case 2: HBL_DEC(2); break;
    case 3: HBL_DEC(3); break;
    default: HBL_DEC(4); break;
  }
#undef HBL_DEC
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
