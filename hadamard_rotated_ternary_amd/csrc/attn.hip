// Low-bit attention states (BitNet v2): post-RoPE Q/K/V heads quantised per
// head by absmax to unsigned b-bit integers with no calibration data, a KV
// cache held in those codes (3 bits in the headline setting), and one decode
// step of attention read straight from the packed cache.
// Sources: 新智元 article "微软再放LLM量化大招", section 实验效果 (the QKV
// states and tables 2-3); 量子位 article on BitNet v2 (the 3-bit KV cache).
//
// Codes: u = n + Z with n = round_half_even(v * Qb / G), Qb = 2^(b-1) - 1,
// Z = 2^(b-1), G = max(max|v|, 1e-5) over the head's d values; the row's fp32
// scale is G / Qb and the value a code stands for is (u - Z) * scale.
// Decisions are exact: for a bf16 value v, a = v * Qb is exact in fp32 and the
// rounding of a / G is decided by the sign of the fused a - (n0 + 1/2) * G, so
// the codes never depend on how G's reciprocal rounds.
//
// Packed layout (b in {2, 3, 4, 8}): a row of d codes is d/32 groups of 32
// consecutive codes, each group b little-endian dwords (4*b bytes).  Inside a
// group the codes are placed so that a few masks and shifts turn the b dwords
// into eight "quads", dwords whose byte i holds code 4q + i (q = 0..7):
//   b = 8: quad q is dword q.
//   b = 4: quad 2j + m = (dword j >> 4m) & 0x0F0F0F0F.
//   b = 2: quad 4j + m = (dword j >> 2m) & 0x03030303.
//   b = 3: quad 2j = dword j & 0x07070707, quad 2j + 1 = (dword j >> 3) & 0x07070707
//          (j = 0..2: codes 0..23); the top two bits of byte k hold the low two
//          bits of code 24 + k in dword 0 and of code 28 + k in dword 1; in
//          dword 2 bit 6 of byte k is bit 2 of code 24 + k and bit 7 is bit 2 of
//          code 28 + k.
// Every code then sits in its own byte, ready for v_dot4 (keys) and for the
// fp8 -> fp32 pair conversion (values: a byte below 16 read as OCP e4m3 is the
// integer times a power of two, exactly).
#include "common.h"
#include "fwht.h"
#include "launch.h"

namespace hbl {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

// round_half_even(a / G) for a = v * qb exact, given an estimate p of a / G
// that is within 1/2 of it.
HBL_DEV int round_ratio(float a, float G, float p) {
  const float n0 = floorf(p);
  const float t = __builtin_fmaf(-(n0 + 0.5f), G, a);   // exact sign of a - (n0 + 1/2) G
  const int n = (int)n0;
  return n + ((t > 0.0f) | ((t == 0.0f) & (n & 1)));
}

// b packed dwords of a 32-code group -> eight quads (byte i of quad q = code 4q + i).
template <int KB>
HBL_DEV void unpack_quads(const uint32_t (&w)[KB], uint32_t (&qd)[8]) {
  if constexpr (KB == 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q) qd[q] = w[q];
  } else if constexpr (KB == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { qd[2 * j] = w[j] & 0x0F0F0F0Fu; qd[2 * j + 1] = (w[j] >> 4) & 0x0F0F0F0Fu; }
  } else if constexpr (KB == 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < 4; ++m) qd[4 * j + m] = (w[j] >> (2 * m)) & 0x03030303u;
  } else {
    static_assert(KB == 3, "code widths 2, 3, 4, 8");
#pragma unroll
    for (int j = 0; j < 3; ++j) { qd[2 * j] = w[j] & 0x07070707u; qd[2 * j + 1] = (w[j] >> 3) & 0x07070707u; }
    qd[6] = ((w[0] >> 6) & 0x03030303u) | ((w[2] >> 4) & 0x04040404u);
    qd[7] = ((w[1] >> 6) & 0x03030303u) | ((w[2] >> 5) & 0x04040404u);
  }
}

// 32 codes (each < 2^KB) -> KB packed dwords; the inverse of unpack_quads.
template <int KB>
HBL_DEV void pack_group(const uint32_t (&u)[32], uint32_t (&w)[KB]) {
  uint32_t qd[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) qd[q] = u[4 * q] | (u[4 * q + 1] << 8) | (u[4 * q + 2] << 16) | (u[4 * q + 3] << 24);
  if constexpr (KB == 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = qd[q];
  } else if constexpr (KB == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = qd[2 * j] | (qd[2 * j + 1] << 4);
  } else if constexpr (KB == 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      w[j] = qd[4 * j] | (qd[4 * j + 1] << 2) | (qd[4 * j + 2] << 4) | (qd[4 * j + 3] << 6);
  } else {
    static_assert(KB == 3, "code widths 2, 3, 4, 8");
    w[0] = qd[0] | (qd[1] << 3) | ((qd[6] & 0x03030303u) << 6);
    w[1] = qd[2] | (qd[3] << 3) | ((qd[7] & 0x03030303u) << 6);
    w[2] = qd[4] | (qd[5] << 3) | ((qd[6] & 0x04040404u) << 4) | ((qd[7] & 0x04040404u) << 5);
  }
}

template <int N>
HBL_DEV void load_words(const uint32_t* p, uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + j);
      w[j] = v.x; w[j + 1] = v.y; w[j + 2] = v.z; w[j + 3] = v.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(p + j);
      w[j] = v.x; w[j + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) w[j] = p[j];
  }
}

// Buffer descriptor word 3 for raw dword loads on gfx9-class devices (data
// format 32 bits; a zero format would make every access out of range).
constexpr int kBufferFlags = 0x00020000;

typedef unsigned u3v __attribute__((ext_vector_type(3)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

// N dwords at byte offset off of a raw buffer (zeros past its size).
template <int N>
HBL_DEV void buffer_words(__amdgpu_buffer_rsrc_t rs, int off, uint32_t (&w)[N]) {
  if constexpr (N == 2) {
    const u2v v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (N == 3) {
    const u3v v = __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  } else {
    static_assert(N % 4 == 0, "2, 3 or a multiple of 4 dwords");
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      const u4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4 * j, 0, 0);
      w[j] = v.x; w[j + 1] = v.y; w[j + 2] = v.z; w[j + 3] = v.w;
    }
  }
}

template <int N>
HBL_DEV void store_words(uint32_t* p, const uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += 4) *reinterpret_cast<uint4*>(p + j) = make_uint4(w[j], w[j + 1], w[j + 2], w[j + 3]);
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += 2) *reinterpret_cast<uint2*>(p + j) = make_uint2(w[j], w[j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) p[j] = w[j];
  }
}

// 32 bf16 values (64 bytes) -> floats.
HBL_DEV void load_bf16x32(const uint16_t* p, float (&v)[32]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = q[i];
    v[8 * i + 0] = bf16_lo(u.x); v[8 * i + 1] = bf16_hi(u.x);
    v[8 * i + 2] = bf16_lo(u.y); v[8 * i + 3] = bf16_hi(u.y);
    v[8 * i + 4] = bf16_lo(u.z); v[8 * i + 5] = bf16_hi(u.z);
    v[8 * i + 6] = bf16_lo(u.w); v[8 * i + 7] = bf16_hi(u.w);
  }
}

// ---------------------------------------------------------------------------
// Quantise rows of D bf16 values into packed codes and fp32 scales.
// Work row o = (b * H + h) * Tn + t reads input row (b * Tn + t) * H + h and
// writes cache row (b * H + h) * Tmax + pos[b] + t, so consecutive work rows
// fill consecutive cache rows of one head.  Rows whose position falls outside
// [0, Tmax) are skipped.  blockIdx.y picks tensor 0 or 1.  A lane owns one
// 32-value group: D/32 lanes per row, 256 threads per workgroup.
template <int D, int KB>
__global__ __launch_bounds__(256) void quant_heads_kernel(QuantHeadsArgs a) {
  constexpr int LPR = D / 32, RPB = 256 / LPR;
  const uint16_t* x = static_cast<const uint16_t*>(blockIdx.y ? a.x1 : a.x0);
  uint8_t* codes = blockIdx.y ? a.codes1 : a.codes0;
  float* scale = blockIdx.y ? a.scale1 : a.scale0;
  const int c = threadIdx.x % LPR;
  const int64_t o = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int64_t rows = a.B * a.H * a.Tn;
  if (o >= rows) return;                        // whole rows: the LPR lanes of a row exit together
  const int64_t t = o % a.Tn, bh = o / a.Tn;
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t p = a.pos ? (int64_t)a.pos[b] : 0;

  float v[32];
  load_bf16x32(x + ((b * a.Tn + t) * a.H + h) * D + c * 32, v);
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) m = fmaxf(m, fabsf(v[e]));
  m = lane_reduce<LPR, true>(m);
  if (p + t < 0 || p + t >= a.Tmax) return;
  const float G = fmaxf(m, kEpsQ);
  constexpr float qb = (float)((1 << (KB - 1)) - 1);
  constexpr uint32_t Z = 1u << (KB - 1);
  const float r = qb / G;
  uint32_t u[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) u[e] = (uint32_t)(round_ratio(v[e] * qb, G, v[e] * r) + (int)Z);
  uint32_t w[KB];
  pack_group<KB>(u, w);
  const int64_t orow = bh * a.Tmax + p + t;
  store_words<KB>(reinterpret_cast<uint32_t*>(codes) + orow * (D / 32 * KB) + c * KB, w);
  if (c == 0) scale[orow] = G / qb;
}

// Codes -> values (u - Z) * scale; one thread per 32-code group.
template <int KB, bool OBF16>
__global__ __launch_bounds__(256) void dequant_heads_kernel(const uint8_t* __restrict__ codes,
                                                            const float* __restrict__ scale, int64_t R, int d,
                                                            void* __restrict__ y) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int gpr = d / 32;
  if (g >= R * gpr) return;
  const int64_t row = g / gpr;
  uint32_t w[KB], qd[8];
  load_words<KB>(reinterpret_cast<const uint32_t*>(codes) + g * KB, w);
  unpack_quads<KB>(w, qd);
  const float s = scale[row];
  constexpr int Z = 1 << (KB - 1);
  float f[32];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) f[4 * q + i] = (float)((int)((qd[q] >> (8 * i)) & 0xFFu) - Z) * s;
  const int64_t base = g * 32;
  if constexpr (OBF16) {
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + base);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 t;
      t.x = f32_to_bf16(f[8 * i + 0]) | ((uint32_t)f32_to_bf16(f[8 * i + 1]) << 16);
      t.y = f32_to_bf16(f[8 * i + 2]) | ((uint32_t)f32_to_bf16(f[8 * i + 3]) << 16);
      t.z = f32_to_bf16(f[8 * i + 4]) | ((uint32_t)f32_to_bf16(f[8 * i + 5]) << 16);
      t.w = f32_to_bf16(f[8 * i + 6]) | ((uint32_t)f32_to_bf16(f[8 * i + 7]) << 16);
      o[i] = t;
    }
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(y) + base);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
  }
}

// ---------------------------------------------------------------------------
// Decode attention.  One workgroup (4 waves) per (sequence, query head, chunk
// of CT cached tokens); when the heads alone give enough workgroups, CT covers
// the whole cache and the workgroup writes the output itself, otherwise a
// second kernel merges the chunks.
// A lane holds one 32-code group (KB dwords) of one token row: LPR = D/32
// lanes cover a row and a wave covers RPI = 64/LPR rows per step; a block is
// NI = 8 steps (BT = 8 * RPI tokens) and the waves take the chunk's blocks in
// turn, each block's loads issued while the previous block is computed.
// Per block:
//   scores: integer dot of the query codes with the key codes (v_dot4 on the
//           quads), times sq * sk / sqrt(D);
//   online softmax: the wave's running max, rescaling its sums when it grows;
//   values: sum of w * sv * u per channel and of w * sv (the (u - Z) form
//           follows at the end), codes read as fp8 bytes (exact, see above).
// The four waves' sums are rescaled to one max and added through LDS.
template <int D>
struct AttnCfg {
  static constexpr int LPR = D / 32, RPI = 64 / LPR, NI = 8, BT = NI * RPI, WB = 4 * BT;
  static constexpr int STRIDE = D + 8;           // LDS row stride (floats)
  static constexpr int PROWS = 4 * RPI;          // partial rows per workgroup
  static constexpr int SUBS = 1024 / D;          // reduction lanes per 4 channels
};
// Partial record per workgroup: D sums, then the chunk max and weight sum,
// padded to a 16-byte multiple.
template <int D> constexpr int kPartStride = D + 4;

template <int KB, int NI>
struct AttnBlock {
  uint32_t k[NI][KB], v[NI][KB];
  float ks[NI], vs[NI];
};

template <int D, int KB>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  using C = AttnCfg<D>;
  constexpr int LPR = C::LPR, RPI = C::RPI, NI = C::NI, BT = C::BT;
  __shared__ float part[C::PROWS * C::STRIDE];
  __shared__ float red[16];
  __shared__ __align__(16) int8_t qbytes[D];

  // Work item, in an XCD-aware order: the query heads that share one KV head
  // and chunk get workgroup ids 8 apart, so they run on the same XCD.
  // (32-bit arithmetic: the host bounds every count below 2^31.)
  const uint32_t g = (uint32_t)(a.Hq / a.Hkv);
  const uint32_t L = blockIdx.x;
  const uint32_t unit = (L / 8u / g) * 8u + (L % 8u);
  const uint32_t j = (L / 8u) % g;
  if (unit >= (uint32_t)a.B * (uint32_t)a.Hkv * (uint32_t)a.nchunk) return;
  const uint32_t chunk = unit % (uint32_t)a.nchunk;
  const uint32_t bh = unit / (uint32_t)a.nchunk;
  const int hk = (int)(bh % (uint32_t)a.Hkv), b = (int)(bh / (uint32_t)a.Hkv);
  const int hq = hk * (int)g + (int)j;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.Tmax ? (int)a.Tmax : len);
  const int t0 = (int)chunk * a.ct;
  const bool single = a.nchunk == 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (t0 >= len) {
    // Empty context (only possible for chunk 0 of a zero length): zeros.
    if (single && chunk == 0) {
      const int64_t ob = ((int64_t)b * a.Hq + hq) * D;
      for (int e = threadIdx.x; e < D; e += 256) {
        if (a.out_bf16) static_cast<uint16_t*>(a.out)[ob + e] = 0;
        else static_cast<float*>(a.out)[ob + e] = 0.0f;
      }
    }
    return;
  }
  const int lim = len < t0 + a.ct ? len : t0 + a.ct;   // tokens [t0, lim) of this chunk
  const int c = lane % LPR, r = lane / LPR;

  constexpr int RDW = D / 32 * KB;                    // dwords per cache row
  // Buffer views of this head's cache rows 0 .. len-1: loads past the length
  // read zeros (their scores are masked), so no address is clamped.
  const int64_t head_row = ((int64_t)b * a.Hkv + hk) * a.Tmax;
  const auto krs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.kc + head_row * RDW * 4), (short)0, len * RDW * 4,
                                                     kBufferFlags);
  const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vc + head_row * RDW * 4), (short)0, len * RDW * 4,
                                                     kBufferFlags);
  const auto kss = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ks + head_row), (short)0, len * 4, kBufferFlags);
  const auto vss = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vs + head_row), (short)0, len * 4, kBufferFlags);

  auto load_block = [&](AttnBlock<KB, NI>& blk, int tb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = tb + i * RPI + r;
      buffer_words<KB>(krs, (t * RDW + c * KB) * 4, blk.k[i]);
      blk.ks[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kss, t * 4, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = tb + i * RPI + r;
      buffer_words<KB>(vrs, (t * RDW + c * KB) * 4, blk.v[i]);
      blk.vs[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vss, t * 4, 0, 0));
    }
  };
  // Blocks of this wave: t0 + (wave + 4 * n) * BT while below lim.
  const int tb0 = t0 + wave * BT;
  AttnBlock<KB, NI> A, Bk;
  if (tb0 < lim) load_block(A, tb0);

  // Query, quantised with the whole head's absmax by wave 0 (D/64 channels
  // per lane) into signed bytes in LDS; every lane then reads the quads of
  // its 32 channels.
  if (wave == 0) {
    constexpr int CPL = D / 64;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + hq) * D + lane * CPL;
    float qv[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) qv[e] = __uint_as_float((uint32_t)qp[e] << 16);
    float qm = 0.0f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) qm = fmaxf(qm, fabsf(qv[e]));
    qm = lane_reduce<64, true>(qm);
    const float G = fmaxf(qm, kEpsQ);
    const float qb = (float)((1 << (a.qbits - 1)) - 1);
    const float rq = qb / G;
    int ns = 0;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int n = round_ratio(qv[e] * qb, G, qv[e] * rq);
      ns += n;
      qbytes[lane * CPL + e] = (int8_t)n;
    }
    const float nsum = lane_reduce<64, false>((float)ns);   // |sum| < 2^24: exact
    if (lane == 0) { red[12] = nsum; red[13] = G / qb; }
  }
  __syncthreads();
  int qd[8];
  {
    const int4 q0 = *reinterpret_cast<const int4*>(qbytes + c * 32);
    const int4 q1 = *reinterpret_cast<const int4*>(qbytes + c * 32 + 16);
    qd[0] = q0.x; qd[1] = q0.y; qd[2] = q0.z; qd[3] = q0.w;
    qd[4] = q1.x; qd[5] = q1.y; qd[6] = q1.z; qd[7] = q1.w;
  }
  const float qsum = red[12], sq = red[13];
  constexpr float kInvSqrtD = D == 64 ? 0.125f : (D == 128 ? 0.08838834764831845f : 0.0625f);
  const float coef = sq * kInvSqrtD;
  constexpr int ZK = KB == 8 ? 0 : (1 << (KB - 1));   // 8-bit key codes are flipped to signed bytes
  const float fp8_unit = __builtin_amdgcn_cvt_pk_f32_fp8(1, false)[0];
  const float vmul = KB == 8 ? 1.0f : 1.0f / fp8_unit;

  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  float m = -INFINITY, lsum = 0.0f, swv = 0.0f;

  auto process = [&](const AttnBlock<KB, NI>& blk, int tb) __attribute__((always_inline)) {
    float s[NI];
    float bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t kq[8];
      unpack_quads<KB>(blk.k[i], kq);
      int dot = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        dot = __builtin_amdgcn_sdot4((int)(KB == 8 ? kq[k] ^ 0x80808080u : kq[k]), qd[k], dot, false);
      const float f = lane_reduce<LPR, false>((float)dot) - (float)ZK * qsum;   // integers below 2^24: exact
      s[i] = tb + i * RPI + r < lim ? f * (coef * blk.ks[i]) : -INFINITY;
      bmax = fmaxf(bmax, s[i]);
    }
    bmax = lane_reduce<64, true>(bmax);
    if (bmax > m) {                                   // wave-uniform
      const float sc = __builtin_amdgcn_exp2f((m - bmax) * kLog2e);
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] *= sc;
      lsum *= sc;
      swv *= sc;
      m = bmax;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float w = __builtin_amdgcn_exp2f((s[i] - m) * kLog2e);   // 0 for masked tokens
      lsum += w;
      const float wsv = w * blk.vs[i];
      swv += wsv;
      const float wv = wsv * vmul;
      uint32_t vq[8];
      unpack_quads<KB>(blk.v[i], vq);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (KB == 8) {
          acc[4 * k + 0] = __builtin_fmaf(wv, (float)((vq[k] >> 0) & 0xFFu), acc[4 * k + 0]);
          acc[4 * k + 1] = __builtin_fmaf(wv, (float)((vq[k] >> 8) & 0xFFu), acc[4 * k + 1]);
          acc[4 * k + 2] = __builtin_fmaf(wv, (float)((vq[k] >> 16) & 0xFFu), acc[4 * k + 2]);
          acc[4 * k + 3] = __builtin_fmaf(wv, (float)((vq[k] >> 24) & 0xFFu), acc[4 * k + 3]);
        } else {
          const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)vq[k], false);
          const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)vq[k], true);
          acc[4 * k + 0] = __builtin_fmaf(wv, lo.x, acc[4 * k + 0]);
          acc[4 * k + 1] = __builtin_fmaf(wv, lo.y, acc[4 * k + 1]);
          acc[4 * k + 2] = __builtin_fmaf(wv, hi.x, acc[4 * k + 2]);
          acc[4 * k + 3] = __builtin_fmaf(wv, hi.y, acc[4 * k + 3]);
        }
      }
    }
  };

  // Ping-pong over the wave's blocks (wave-uniform control flow).
  for (int tb = tb0; tb < lim; tb += 8 * BT) {
    const int tn = tb + 4 * BT;
    if (tn < lim) load_block(Bk, tn);
    process(A, tb);
    if (tn >= lim) break;
    if (tn + 4 * BT < lim) load_block(A, tn + 4 * BT);
    process(Bk, tn);
  }

  // Rescale the four waves to the workgroup max (a wave without blocks has
  // m = -inf and zero sums) and add their partial rows through LDS.
  const float lw = lane_reduce<64, false>(c == 0 ? lsum : 0.0f);
  const float sw = lane_reduce<64, false>(c == 0 ? swv : 0.0f);
  if (lane == 0) { red[wave] = m; red[4 + wave] = lw; red[8 + wave] = sw; }
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  {
    const float sc = __builtin_amdgcn_exp2f((m - M) * kLog2e);
    float* pr = part + (wave * RPI + r) * C::STRIDE + c * 32;
#pragma unroll
    for (int e = 0; e < 32; e += 4)
      *reinterpret_cast<float4*>(pr + e) = make_float4(acc[e] * sc, acc[e + 1] * sc, acc[e + 2] * sc, acc[e + 3] * sc);
  }
  float fw[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) fw[w] = __builtin_amdgcn_exp2f((red[w] - M) * kLog2e);
  const float Lsum = fw[0] * red[4] + fw[1] * red[5] + fw[2] * red[6] + fw[3] * red[7];
  const float SW = fw[0] * red[8] + fw[1] * red[9] + fw[2] * red[10] + fw[3] * red[11];
  __syncthreads();
  constexpr int SUBS = C::SUBS, RPS = C::PROWS / SUBS;   // rows per reduction lane
  const int sub = threadIdx.x % SUBS, grp = threadIdx.x / SUBS;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < RPS; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(part + (sub + k * SUBS) * C::STRIDE + grp * 4);
    sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
  }
  sum.x = lane_reduce<SUBS, false>(sum.x);
  sum.y = lane_reduce<SUBS, false>(sum.y);
  sum.z = lane_reduce<SUBS, false>(sum.z);
  sum.w = lane_reduce<SUBS, false>(sum.w);
  const float zsw = (float)(1 << (KB - 1)) * SW;
  const float4 o = make_float4(sum.x - zsw, sum.y - zsw, sum.z - zsw, sum.w - zsw);
  if (single) {
    if (sub == 0) {
      const float inv = 1.0f / Lsum;
      const int64_t ob = ((int64_t)b * a.Hq + hq) * D + grp * 4;
      if (a.out_bf16) {
        uint2 pk;
        pk.x = f32_to_bf16(o.x * inv) | ((uint32_t)f32_to_bf16(o.y * inv) << 16);
        pk.y = f32_to_bf16(o.z * inv) | ((uint32_t)f32_to_bf16(o.w * inv) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + ob) = pk;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + ob) =
            make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      }
    }
    return;
  }
  float* out = a.part + (((int64_t)b * a.Hq + hq) * a.nchunk + chunk) * kPartStride<D>;
  if (sub == 0) *reinterpret_cast<float4*>(out + grp * 4) = o;
  if (threadIdx.x == 0) {
    out[D] = M;
    out[D + 1] = Lsum;
  }
}

// Second stage (several chunks per head): merge the chunks of one
// (sequence, query head); one wave.  Latency-bound, so every load is issued
// before any result is needed: the partial sums of up to 16 chunks per round
// (chunks past the length are read too, from the workspace, and discarded by
// select), and each lane's chunk max and weight sum.
template <int D, bool OBF16>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  constexpr int PS = kPartStride<D>, PER = D / 64, NB = 16;
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / a.Hq);
  const int lane = threadIdx.x;
  const int nch = a.nchunk;
  const float* p = a.part + bh * nch * PS;
  float pv[NB][PER];
#pragma unroll
  for (int kk = 0; kk < NB; ++kk)
#pragma unroll
    for (int i = 0; i < PER; ++i) pv[kk][i] = kk < nch ? p[kk * PS + lane + 64 * i] : 0.0f;
  const bool own = lane < nch;                      // first round of lane-parallel statistics
  const float m0 = own ? p[lane * PS + D] : -INFINITY;
  const float l0 = own ? p[lane * PS + D + 1] : 0.0f;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.Tmax ? (int)a.Tmax : len);
  const int n = (len + a.ct - 1) / a.ct;

  float M = lane < n ? m0 : -INFINITY;
  for (int k = lane + 64; k < n; k += 64) M = fmaxf(M, p[k * PS + D]);
  M = lane_reduce<64, true>(M);
  float Lsum = 0.0f;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.0f;
  for (int k0 = 0; k0 < n; k0 += NB) {
    if (k0 > 0) {
#pragma unroll
      for (int kk = 0; kk < NB; ++kk)
#pragma unroll
        for (int i = 0; i < PER; ++i) pv[kk][i] = k0 + kk < n ? p[(k0 + kk) * PS + lane + 64 * i] : 0.0f;
    }
    // factors exp(m_k - M) of chunks k0 .. k0+NB-1, held by lanes 0 .. NB-1
    const int kl = k0 + (lane % NB);
    float f = 0.0f, lk = 0.0f;
    if (kl < n) {
      const float mk = kl == lane ? m0 : p[kl * PS + D];
      lk = kl == lane ? l0 : p[kl * PS + D + 1];
      f = __builtin_amdgcn_exp2f((mk - M) * kLog2e);
    }
    if (lane < NB) Lsum = __builtin_fmaf(f, lk, Lsum);
#pragma unroll
    for (int kk = 0; kk < NB; ++kk) {
      const float fk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), kk));
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] = k0 + kk < n ? __builtin_fmaf(fk, pv[kk][i], o[i]) : o[i];
    }
  }
  Lsum = lane_reduce<64, false>(Lsum);
  const float inv = n > 0 ? 1.0f / Lsum : 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float v = o[i] * inv;
    const int64_t idx = bh * D + lane + 64 * i;
    if constexpr (OBF16) static_cast<uint16_t*>(a.out)[idx] = f32_to_bf16(v);
    else static_cast<float*>(a.out)[idx] = v;
  }
}

// ---------------------------------------------------------------------------
// Prefill (causal) attention over the quantised cache, on the matrix cores.
// One workgroup per (sequence, query head, block of new tokens): 8 waves and
// 256 tokens for head sizes up to 128, 4 waves and 128 tokens for 256 (whose
// registers allow one wave per SIMD); each wave owns 32 queries (two
// 16-query tiles).  Key blocks of 64
// cached tokens, double-buffered in LDS: the raw codes of block kb+1 are
// loaded into registers while block kb is computed, then unpacked into the
// other buffer, so one barrier per block suffices.
//   keys: signed bytes u - Z, [token][channel];
//   values: bf16 of 128 + u (bit pattern 0x4300 | u, exact for u < 128) or,
//   for 8-bit codes, of u; stored [channel][token] so the value product
//   contracts over tokens, tokens of a 32-token half permuted so that the 8
//   a lane supplies to one product are adjacent (one 16-byte read);
//   scores, transposed: S^T = K . Q^T on v_mfma_i32_16x16x64_i8 (exact), so
//   a lane holds 4 tokens of one query per 16x16 tile; the key scale with
//   1/sqrt(D) and log2(e) folded in multiplies the integer score, the query
//   scale enters through one fma inside the exponential;
//   online softmax per query with a lazily raised maximum: the accumulators
//   are rescaled only when a block's maximum exceeds the running one by more
//   than 2^8, which changes no result (every term is relative to the same
//   reference) and keeps every weight below 2^8;
//   values: O^T += V^T . P'^T on v_mfma_f32_16x16x32_bf16, with P' = P * sv
//   rounded to bf16 taken straight from the score registers, plus one
//   all-ones tile that yields sum P' per query; the value offset
//   (128 + Z, or Z for 8-bit codes) is removed with that sum at the end.
// 16x16 layouts: accumulator lane l / register r: row 4*(l/16) + r, column
// l%16; A operand: row l%16, k block l/16; B operand: column l%16, k block l/16.
constexpr float kLazyMax = 8.0f;                      // log2 of the largest weight between rescalings
typedef float v4f __attribute__((ext_vector_type(4)));

template <int D>
struct PfCfg {
  static constexpr int NW = D <= 128 ? 8 : 4;         // waves per workgroup
  static constexpr int NT = 64 * NW;                  // threads
  static constexpr int QB = 32 * NW;                  // new tokens (queries) per workgroup
  static constexpr int TB = D <= 128 ? 128 : 64;      // cached tokens per key block
  static constexpr int GPR = D / 32;                  // 32-code groups per row
  // Row pitches.  Every fragment read takes 16 bytes per lane from 16 rows
  // (lane % 16) at 4 consecutive 16-byte units (lane / 16).  Measured with
  // the LDS bank-conflict counter on gfx950, that read is conflict-free when
  // the pitch is an odd multiple of 32 bytes (160, 224, 288) and two-way
  // conflicted for the other paddings tried (144, 176, 192, 208, 240, 272,
  // ...; 128 and 256 four- and eight-way): D + 32 bytes of codes and TB + 16
  // bf16 values (keys, values and queries at D = 128 went from 38 % to 6 %
  // of the LDS cycles lost to conflicts, the kernel 4 % faster).
  static constexpr int KROW = D + 32;                 // key tile row (bytes)
  static constexpr int VROW = TB + 16;                // value tile row (bf16 per channel)
  static constexpr int QROW = D + 32;                 // query codes row (bytes)
  static_assert((KROW / 32) % 2 == 1 && (VROW * 2 / 32) % 2 == 1 && KROW % 32 == 0 && (VROW * 2) % 32 == 0,
                "row pitches: odd multiples of 32 bytes");
  static constexpr int KT = TB * KROW;                // bytes of one key tile
  static constexpr int VT = D * VROW * 2;             // bytes of one value tile
  static constexpr int BUF = KT + VT + 2 * TB * 4;    // keys, values, key and value scales
  static constexpr int NIT = TB * GPR;                // staging items per block (keys; values alike)
  // with at least twice as many threads as items, one half of the threads
  // stages the keys and the other half the values
  static constexpr bool SPLIT = NT >= 2 * NIT;
  static constexpr int IPT = SPLIT ? 1 : (NIT + NT - 1) / NT;   // items per thread
  static_assert(QB * QROW + QB * 4 <= 2 * BUF, "query codes and scales reuse the buffers");
};

// Raw codes and scales of one key block held in registers between the load
// and the unpack into LDS.  Key words in w0; value words of the two tokens in
// w1, w2, or, when halves of the workgroup stage keys and values separately,
// in w0, w1 (a thread then holds only one kind).
template <int D, int KB>
struct PfRaw {
  uint32_t w0[PfCfg<D>::IPT][KB], w1[PfCfg<D>::IPT][KB], w2[PfCfg<D>::IPT][KB];
  float ks, vs;
  HBL_DEV uint32_t (&k(int u))[KB] { return w0[u]; }
  HBL_DEV uint32_t (&v0(int u))[KB] { return PfCfg<D>::SPLIT ? w0[u] : w1[u]; }
  HBL_DEV uint32_t (&v1(int u))[KB] { return PfCfg<D>::SPLIT ? w1[u] : w2[u]; }
  HBL_DEV const uint32_t (&k(int u) const)[KB] { return w0[u]; }
  HBL_DEV const uint32_t (&v0(int u) const)[KB] { return PfCfg<D>::SPLIT ? w0[u] : w1[u]; }
  HBL_DEV const uint32_t (&v1(int u) const)[KB] { return PfCfg<D>::SPLIT ? w1[u] : w2[u]; }
};

// Value staging item -> (token pair, 32-code group, half): the 64 lanes of a
// wave take 32 consecutive token pairs twice, lanes 0..31 the even quads of
// the group and lanes 32..63 the odd ones (channels 4 apart: rows whose
// pitch is an odd multiple of 32 bytes put the two halves on opposite
// halves of the banks).
template <int D>
HBL_DEV void pf_vitem(int it, int& pr, int& grp, bool& h) {
  constexpr int PB = PfCfg<D>::TB / 64;               // sets of 32 token pairs per block
  const int w = it >> 6, lane = it & 63;
  pr = (w % PB) * 32 + (lane & 31);
  grp = w / PB;
  h = lane >= 32;
}

template <int D, int KB>
HBL_DEV void pf_load(PfRaw<D, KB>& r, int t0, int tid, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                     __amdgpu_buffer_rsrc_t kss, __amdgpu_buffer_rsrc_t vss) {
  using C = PfCfg<D>;
  constexpr int RDW = D / 32 * KB;
#pragma unroll
  for (int u = 0; u < C::IPT; ++u) {
    const int itk = C::SPLIT ? tid : tid + C::NT * u;
    const int itv = C::SPLIT ? tid - C::NIT : itk;
    if (itk < C::NIT) {
      const int row = itk / C::GPR, grp = itk % C::GPR;
      buffer_words<KB>(krs, ((t0 + row) * RDW + grp * KB) * 4, r.k(u));
    }
    if (itv >= 0 && itv < C::NIT) {
      int pr, grp2;
      bool h;
      pf_vitem<D>(itv, pr, grp2, h);
      buffer_words<KB>(vrs, ((t0 + 2 * pr) * RDW + grp2 * KB) * 4, r.v0(u));
      buffer_words<KB>(vrs, ((t0 + 2 * pr + 1) * RDW + grp2 * KB) * 4, r.v1(u));
    }
  }
  if (tid < C::TB) {
    r.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kss, (t0 + tid) * 4, 0, 0));
    r.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vss, (t0 + tid) * 4, 0, 0));
  }
}

template <int D, int KB>
HBL_DEV void pf_store(const PfRaw<D, KB>& r, char* buf, int tid) {
  using C = PfCfg<D>;
  constexpr int ZK = KB == 8 ? 128 : (1 << (KB - 1));
  constexpr float kInvSqrtD = D == 64 ? 0.125f : (D == 128 ? 0.08838834764831845f : 0.0625f);
  int8_t* kt = reinterpret_cast<int8_t*>(buf);
  uint16_t* vt = reinterpret_cast<uint16_t*>(buf + C::KT);
  float* sc = reinterpret_cast<float*>(buf + C::KT + C::VT);
#pragma unroll
  for (int u = 0; u < C::IPT; ++u) {
    const int itk = C::SPLIT ? tid : tid + C::NT * u;
    const int itv = C::SPLIT ? tid - C::NIT : itk;
    {
      // keys: token row, one 32-code group
      if (itk < C::NIT) {
        const int row = itk / C::GPR, grp = itk % C::GPR;
        uint32_t qd[8], sb[8];
        unpack_quads<KB>(r.k(u), qd);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if constexpr (KB == 8) sb[k] = qd[k] ^ 0x80808080u;
          else if constexpr (KB == 3) sb[k] = __builtin_amdgcn_perm(0x03020100u, 0xFFFEFDFCu, qd[k]);   // byte table u - 4
          else if constexpr (KB == 2) sb[k] = __builtin_amdgcn_perm(0u, 0x0100FFFEu, qd[k]);            // byte table u - 2
          else sb[k] = ((qd[k] | 0x80808080u) - (uint32_t)ZK * 0x01010101u) ^ 0x80808080u;
        }
        int8_t* kd = kt + row * C::KROW + grp * 32;
        *reinterpret_cast<uint4*>(kd) = make_uint4(sb[0], sb[1], sb[2], sb[3]);
        *reinterpret_cast<uint4*>(kd + 16) = make_uint4(sb[4], sb[5], sb[6], sb[7]);
      }
      // values: token pair pr, group it / 64, quads {0,1,4,5} or {2,3,6,7}
      // (the two halves of a wave write channels 8 apart: distinct banks)
      if (itv >= 0 && itv < C::NIT) {
        int pr, grp;
        bool h;
        pf_vitem<D>(itv, pr, grp, h);
        uint32_t d0[8], d1[8], e0[4], e1[4];
        unpack_quads<KB>(r.v0(u), d0);
        unpack_quads<KB>(r.v1(u), d1);
        // quad 2kk + h: a byte permute picks one of two registers (a plain
        // select would be folded into a runtime array index)
        const uint32_t hsel = h ? 0x07060504u : 0x03020100u;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          e0[kk] = __builtin_amdgcn_perm(d0[2 * kk + 1], d0[2 * kk], hsel);
          e1[kk] = __builtin_amdgcn_perm(d1[2 * kk + 1], d1[2 * kk], hsel);
        }
        const int t = 2 * pr;                                       // 32j + 16h' + 4g + r
        const int pos = (t & ~31) | (((t >> 2) & 3) << 3) | (((t >> 4) & 1) << 2) | (t & 3);
        uint32_t* vd = reinterpret_cast<uint32_t*>(vt + (grp * 32 + (h ? 4 : 0)) * C::VROW + pos);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t w;
            if constexpr (KB == 8) {
              const uint32_t lo = __float_as_uint((float)((e0[kk] >> (8 * i)) & 0xFFu));
              const uint32_t hi = __float_as_uint((float)((e1[kk] >> (8 * i)) & 0xFFu));
              w = __builtin_amdgcn_perm(hi, lo, 0x07060302u);      // high halves: bf16 of u, exact
            } else {
              w = __builtin_amdgcn_perm(e1[kk], e0[kk], (uint32_t)i | 0x0C00u | ((uint32_t)(4 + i) << 16) | 0x0C000000u) |
                  0x43004300u;                                      // bf16 of 128 + u
            }
            vd[(8 * kk + i) * (C::VROW / 2)] = w;
          }
        }
      }
    }
  }
  if (tid < C::TB) {
    sc[tid] = r.ks * (kInvSqrtD * kLog2e);
    sc[C::TB + tid] = r.vs;
  }
}

template <int D, int KB>
__global__ __launch_bounds__(PfCfg<D>::NT) void attn_prefill_kernel(PrefillArgs a) {
  using C = PfCfg<D>;
  __shared__ __align__(16) char lds[2 * C::BUF];

  const int BH = a.B * a.Hq;
  const int nqb = (a.Tn + C::QB - 1) / C::QB;
  const int L = blockIdx.x;
  // heaviest query blocks first; consecutive workgroups (which land on
  // different XCDs) take different heads of the same query block
  const int qblk = nqb - 1 - L / BH;
  const int bh = L % BH;
  const int hq = bh % a.Hq, b = bh / a.Hq;
  const int hk = hq / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  // device-resident start, clamped to [0, Tmax]; with Tmax + Tn < 2^31 - 512
  // (checked by the host) every position below fits in 32 bits
  int start = a.start[b];
  start = start < 0 ? 0 : (start > a.Tmax ? (int)a.Tmax : start);
  const int q0 = qblk * C::QB;
  const int qend = a.Tn < q0 + C::QB ? a.Tn : q0 + C::QB;    // new tokens q0 .. qend-1
  int len = start + qend;                                     // keys needed by the last query
  len = len > a.Tmax ? (int)a.Tmax : len;

  constexpr int RDW = D / 32 * KB;
  const int64_t head_row = ((int64_t)b * a.Hkv + hk) * a.Tmax;
  const auto krs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.kc + head_row * RDW * 4), (short)0, len * RDW * 4,
                                                     kBufferFlags);
  const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vc + head_row * RDW * 4), (short)0, len * RDW * 4,
                                                     kBufferFlags);
  const auto kss = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ks + head_row), (short)0, len * 4, kBufferFlags);
  const auto vss = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vs + head_row), (short)0, len * 4, kBufferFlags);

  PfRaw<D, KB> raw;
  pf_load<D, KB>(raw, 0, tid, krs, vrs, kss, vss);

  // ---- query codes of the block's tokens (2 threads per row, D/2 channels each) and their
  // scales, in the staging buffers (free until the first key block is stored)
  int8_t* qt = reinterpret_cast<int8_t*>(lds);
  float* qsc = reinterpret_cast<float*>(lds + C::QB * C::QROW);
  {
    const int row = tid >> 1, hh = tid & 1;
    const int i = q0 + row;
    float v[D / 2];
    if (i < a.Tn) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (((int64_t)b * a.Tn + i) * a.Hq + hq) * D + hh * (D / 2);
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        const uint4 w = reinterpret_cast<const uint4*>(qp)[u];
        v[8 * u + 0] = bf16_lo(w.x); v[8 * u + 1] = bf16_hi(w.x); v[8 * u + 2] = bf16_lo(w.y);
        v[8 * u + 3] = bf16_hi(w.y); v[8 * u + 4] = bf16_lo(w.z); v[8 * u + 5] = bf16_hi(w.z);
        v[8 * u + 6] = bf16_lo(w.w); v[8 * u + 7] = bf16_hi(w.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < D / 2; ++e) v[e] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < D / 2; ++e) m = fmaxf(m, fabsf(v[e]));
    m = lane_reduce<2, true>(m);
    const float G = fmaxf(m, kEpsQ);
    const float qb = (float)((1 << (a.qbits - 1)) - 1);
    const float rq = qb / G;
#pragma unroll
    for (int e = 0; e < D / 2; e += 4) {
      uint32_t pk = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) pk |= ((uint32_t)round_ratio(v[e + k] * qb, G, v[e + k] * rq) & 0xFFu) << (8 * k);
      *reinterpret_cast<uint32_t*>(qt + row * C::QROW + hh * (D / 2) + e) = pk;
    }
    if (hh == 0) qsc[row] = G / qb;
  }
  __syncthreads();
  // query B operands of this wave's two 16-query tiles: column = query l16,
  // k-step s covers channels 64s .. 64s+63
  v4i qB[2][D / 64];
  float sq[2];
  int qpos[2];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int row = wave * 32 + qi * 16 + l16;
#pragma unroll
    for (int s2 = 0; s2 < D / 64; ++s2) qB[qi][s2] = *reinterpret_cast<const v4i*>(qt + row * C::QROW + 64 * s2 + 16 * g4);
    sq[qi] = qsc[row];
    qpos[qi] = start + q0 + row;               // keys 0 .. qpos
  }
  __syncthreads();                             // query codes and scales read: both buffers free
  pf_store<D, KB>(raw, lds, tid);
  __syncthreads();

  constexpr int ZK = KB == 8 ? 128 : (1 << (KB - 1));
  constexpr float kOff = KB == 8 ? (float)ZK : 128.0f + (float)ZK;
  const bf8v ones = __builtin_bit_cast(bf8v, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  v4f o[2][D / 16], os[2];                            // O^T tiles [query tile][channel tile]; sum P'
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) o[qi][c] = v4f{0.f, 0.f, 0.f, 0.f};
    os[qi] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  float mq[2] = {-INFINITY, -INFINITY}, lq[2] = {0.f, 0.f};

  const int wfirst = start + q0 + wave * 32;          // the wave's first and last query positions
  const int wlast = wfirst + 31;
  constexpr int TB = C::TB, NTT = TB / 16;            // key tokens per block, 16-token tiles
  const int nkb = (len + TB - 1) / TB;
  for (int kb = 0; kb < nkb; ++kb) {
    const int t0 = kb * TB;
    if (kb + 1 < nkb) pf_load<D, KB>(raw, t0 + TB, tid, krs, vrs, kss, vss);
    const char* buf = lds + (kb & 1) * C::BUF;
    const int8_t* kt = reinterpret_cast<const int8_t*>(buf);
    const uint16_t* vt = reinterpret_cast<const uint16_t*>(buf + C::KT);
    const float* ksl = reinterpret_cast<const float*>(buf + C::KT + C::VT);
    const float* vsl = ksl + TB;
    if (t0 <= wlast) {
      const bool edge = t0 + TB - 1 > wfirst || t0 + TB > len;   // a block on the diagonal or past the end
      // K fragments and key scales of the first 32-key half; each half then
      // requests the next half's fragments and its own value operands before
      // the arithmetic that waits on its scores
      v4i ka[2][D / 64];
      float4 kf[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int s2 = 0; s2 < D / 64; ++s2)
          ka[h2][s2] = *reinterpret_cast<const v4i*>(kt + (h2 * 16 + l16) * C::KROW + 64 * s2 + 16 * g4);
        kf[h2] = *reinterpret_cast<const float4*>(ksl + h2 * 16 + 4 * g4);
      }
#pragma unroll
      for (int j = 0; j < TB / 32; ++j) {
        // ---- S^T tiles of keys 32j .. 32j+31: rows = keys 16(2j+h2) + 4*g4 + r, column = query l16;
        // x = score * log2(e) / sq
        float x[2][2][4];                                // [query tile][16-key tile][register]
        v4i acc[2][2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int qi = 0; qi < 2; ++qi) {
            acc[h2][qi] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int s2 = 0; s2 < D / 64; ++s2)
              acc[h2][qi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka[h2][s2], qB[qi][s2], acc[h2][qi], 0, 0, 0);
          }
        float kscl[2][4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          kscl[h2][0] = kf[h2].x; kscl[h2][1] = kf[h2].y; kscl[h2][2] = kf[h2].z; kscl[h2][3] = kf[h2].w;
        }
        // value operands of this half (early, except with 8-bit codes, whose
        // wider staging registers leave no room) and key fragments of the next
        constexpr bool kEarlyV = KB != 8;
        bf8v va[D / 16];
        if constexpr (kEarlyV) {
#pragma unroll
          for (int c = 0; c < D / 16; ++c)
            va[c] = *reinterpret_cast<const bf8v*>(vt + (c * 16 + l16) * C::VROW + 32 * j + 8 * g4);
        }
        if (j + 1 < TB / 32) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int nt = 2 * (j + 1) + h2;
#pragma unroll
            for (int s2 = 0; s2 < D / 64; ++s2)
              ka[h2][s2] = *reinterpret_cast<const v4i*>(kt + (nt * 16 + l16) * C::KROW + 64 * s2 + 16 * g4);
            kf[h2] = *reinterpret_cast<const float4*>(ksl + nt * 16 + 4 * g4);
          }
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int qi = 0; qi < 2; ++qi)
#pragma unroll
            for (int r = 0; r < 4; ++r) x[qi][h2][r] = (float)acc[h2][qi][r] * kscl[h2][r];
        if (edge) {
#pragma unroll
          for (int qi = 0; qi < 2; ++qi)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int t = t0 + (2 * j + h2) * 16 + 4 * g4 + r;
                if (t > qpos[qi] || t >= len) x[qi][h2][r] = -INFINITY;
              }
        }
        // ---- the running maximum is raised (and everything rescaled) only when a
        // score exceeds it by more than 2^kLazyMax; otherwise the weights are formed
        // against the current one directly
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) {
          float bm = -INFINITY;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int r = 0; r < 4; ++r) bm = fmaxf(bm, x[qi][h2][r]);
          if (__any(sq[qi] * bm > mq[qi] + kLazyMax)) {
            bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const float mn = fmaxf(mq[qi], sq[qi] * bm);
            const float fac = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(mq[qi] - mn);
            mq[qi] = mn;
            lq[qi] *= fac;
            os[qi] *= fac;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) o[qi][c] *= fac;
          }
        }
        // ---- P'^T as bf16 B operands (8 keys per lane) and O^T += V^T P'^T
        float vsr[2][4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float4 vf = *reinterpret_cast<const float4*>(vsl + (2 * j + h2) * 16 + 4 * g4);
          vsr[h2][0] = vf.x; vsr[h2][1] = vf.y; vsr[h2][2] = vf.z; vsr[h2][3] = vf.w;
        }
        bf8v pb[2];
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) {
          float ls = 0.f;
          uint32_t pk[4];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[qi], x[qi][h2][r], -mq[qi]));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[qi], x[qi][h2][r + 1], -mq[qi]));
              ls += p0;
              ls += p1;
              const f2 pv = {p0 * vsr[h2][r], p1 * vsr[h2][r + 1]};
              pk[2 * h2 + r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pv, bf2));
            }
          }
          pb[qi] = __builtin_bit_cast(bf8v, make_uint4(pk[0], pk[1], pk[2], pk[3]));
          lq[qi] += ls;
        }
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          // V^T operand: channel c*16 + l16, the 8 adjacent positions 32j + 8*g4 .. +7
          if constexpr (!kEarlyV)
            va[c] = *reinterpret_cast<const bf8v*>(vt + (c * 16 + l16) * C::VROW + 32 * j + 8 * g4);
#pragma unroll
          for (int qi = 0; qi < 2; ++qi) o[qi][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[c], pb[qi], o[qi][c], 0, 0, 0);
        }
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) os[qi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qi], os[qi], 0, 0, 0);
      }
    }
    if (kb + 1 < nkb) pf_store<D, KB>(raw, lds + ((kb + 1) & 1) * C::BUF, tid);
    __syncthreads();   // the next block is staged; this one is free for the block after
  }
  // ---- per-query sums over the 4 lanes of a column, then out = (O - off * sum P') / sum P
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    lq[qi] += __shfl_xor(lq[qi], 16, 64);
    lq[qi] += __shfl_xor(lq[qi], 32, 64);
    const int i = q0 + wave * 32 + qi * 16 + l16;
    if (i >= a.Tn) continue;
    const float inv = lq[qi] > 0.0f ? 1.0f / lq[qi] : 0.0f;
    const float zs = kOff * os[qi][0];
    const int64_t ob = (((int64_t)b * a.Tn + i) * a.Hq + hq) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const int ch = c * 16 + 4 * g4;
      const float v0 = (o[qi][c][0] - zs) * inv, v1 = (o[qi][c][1] - zs) * inv;
      const float v2 = (o[qi][c][2] - zs) * inv, v3 = (o[qi][c][3] - zs) * inv;
      if (a.out_bf16) {
        uint2 pk;
        pk.x = f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
        pk.y = f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + ob + ch) = pk;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + ob + ch) = make_float4(v0, v1, v2, v3);
      }
    }
  }
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs& a) {
  using C = PfCfg<D>;
  const int nqb = (a.Tn + C::QB - 1) / C::QB;
  const dim3 grid((unsigned)((int64_t)a.B * a.Hq * nqb)), block(C::NT);
  switch (a.kvbits) {
    case 2: attn_prefill_kernel<D, 2><<<grid, block, 0, a.stream>>>(a); break;
    case 3: attn_prefill_kernel<D, 3><<<grid, block, 0, a.stream>>>(a); break;
    case 4: attn_prefill_kernel<D, 4><<<grid, block, 0, a.stream>>>(a); break;
    case 8: attn_prefill_kernel<D, 8><<<grid, block, 0, a.stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int D>
hipError_t launch_attn_d(const AttnArgs& a) {
  const int g = a.Hq / a.Hkv;
  const int64_t units = (int64_t)a.B * a.Hkv * a.nchunk;
  const int64_t blocks = (units + 7) / 8 * 8 * g;
  switch (a.kvbits) {
#define HBL_ATTN_KB(KB) \
    case KB: attn_partial_kernel<D, KB><<<dim3((unsigned)blocks), dim3(256), 0, a.stream>>>(a); break;
    HBL_ATTN_KB(2) HBL_ATTN_KB(3) HBL_ATTN_KB(4) HBL_ATTN_KB(8)
#undef HBL_ATTN_KB
    default: return hipErrorInvalidValue;
  }
  if (hipError_t e = hipGetLastError()) return e;
  if (a.nchunk == 1) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)a.B * a.Hq));
  if (a.out_bf16) attn_combine_kernel<D, true><<<grid, dim3(64), 0, a.stream>>>(a);
  else attn_combine_kernel<D, false><<<grid, dim3(64), 0, a.stream>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_quant_d(const QuantHeadsArgs& a, dim3 grid) {
  switch (a.bits) {
    case 2: quant_heads_kernel<D, 2><<<grid, dim3(256), 0, a.stream>>>(a); break;
    case 3: quant_heads_kernel<D, 3><<<grid, dim3(256), 0, a.stream>>>(a); break;
    case 4: quant_heads_kernel<D, 4><<<grid, dim3(256), 0, a.stream>>>(a); break;
    case 8: quant_heads_kernel<D, 8><<<grid, dim3(256), 0, a.stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool heads_bits_supported(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 8; }

int attn_part_stride(int d) { return d + 4; }

void attn_plan(int64_t B, int64_t Hq, int d, int64_t Tmax, int* ct, int* nchunk) {
  const int64_t wb = attn_block_tokens(d);
  const int64_t max_chunks = (Tmax + wb - 1) / wb;
  const int64_t heads = B * Hq;
  int64_t want = heads >= 512 ? 1 : (512 + heads - 1) / heads;
  if (want > max_chunks) want = max_chunks;
  const int64_t per = (Tmax + want - 1) / want;
  const int64_t c = (per + wb - 1) / wb * wb;
  *ct = (int)c;
  *nchunk = (int)((Tmax + c - 1) / c);
}

int attn_block_tokens(int d) {
  return d == 64 ? AttnCfg<64>::WB : d == 128 ? AttnCfg<128>::WB : d == 256 ? AttnCfg<256>::WB : 0;
}

hipError_t launch_quant_heads(const QuantHeadsArgs& a) {
  const int64_t rows = a.B * a.H * a.Tn;
  if (rows == 0) return hipSuccess;
  const int rpb = 256 / (a.d / 32);
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb), a.x1 ? 2u : 1u);
  switch (a.d) {
    case 64: return launch_quant_d<64>(a, grid);
    case 128: return launch_quant_d<128>(a, grid);
    case 256: return launch_quant_d<256>(a, grid);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequant_heads(const uint8_t* codes, const float* scale, int64_t R, int d, int bits, void* y,
                                bool y_bf16, hipStream_t stream) {
  const int64_t groups = R * (d / 32);
  if (groups == 0) return hipSuccess;
  const dim3 grid((unsigned)((groups + 255) / 256));
#define HBL_DQ(KB)                                                                                          \
  case KB:                                                                                                  \
    if (y_bf16) dequant_heads_kernel<KB, true><<<grid, dim3(256), 0, stream>>>(codes, scale, R, d, y);      \
    else dequant_heads_kernel<KB, false><<<grid, dim3(256), 0, stream>>>(codes, scale, R, d, y);           \
    break;
  switch (bits) {
    HBL_DQ(2) HBL_DQ(3) HBL_DQ(4) HBL_DQ(8)
    default: return hipErrorInvalidValue;
  }
#undef HBL_DQ
  return hipGetLastError();
}

hipError_t launch_attention_prefill(const PrefillArgs& a) {
  if (a.B == 0 || a.Tn == 0) return hipSuccess;
  switch (a.d) {
    case 64: return launch_prefill_d<64>(a);
    case 128: return launch_prefill_d<128>(a);
    case 256: return launch_prefill_d<256>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_decode(const AttnArgs& a) {
  switch (a.d) {
    case 64: return launch_attn_d<64>(a);
    case 128: return launch_attn_d<128>(a);
    case 256: return launch_attn_d<256>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hbl
