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
// Decode attention, first stage: one workgroup per (sequence, query head,
// chunk of CT cached tokens).  A lane holds one 32-code group (KB dwords) of
// one token row: LPR = D/32 lanes cover a row, a wave covers RPI = 64/LPR
// rows per step and each of the four waves takes NI = 8 steps.
//   pass 1: score of every token: integer dot of the query codes with the
//           key codes (v_dot4 on the quads), times sq * sk / sqrt(D);
//   max over the chunk (LDS);
//   pass 2: weights w = exp(s - max); sum of w * sv * u per channel and of
//           w * sv, from which the (u - Z) form follows;
//   the 4 * RPI partial rows are summed through LDS.
// Output per workgroup: D unnormalised sums, the chunk max and the weight sum.
template <int D>
struct AttnCfg {
  static constexpr int LPR = D / 32, RPI = 64 / LPR, NI = 8, CT = 4 * NI * RPI;
  static constexpr int STRIDE = D + 8;           // LDS row stride (floats)
  static constexpr int PROWS = 4 * RPI;          // partial rows per workgroup
  static constexpr int SUBS = 1024 / D;          // reduction lanes per 4 channels
};
// Partial record per workgroup: D sums, then the chunk max and weight sum,
// padded to a 16-byte multiple.
template <int D> constexpr int kPartStride = D + 4;

template <int D, int KB>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  using C = AttnCfg<D>;
  constexpr int LPR = C::LPR, RPI = C::RPI, NI = C::NI;
  __shared__ float part[C::PROWS * C::STRIDE];
  __shared__ float red[16];
  __shared__ __align__(16) int8_t qbytes[D];

  // Work item, in an XCD-aware order: the query heads that share one KV head
  // and chunk get workgroup ids 8 apart, so they run on the same XCD.
  const int g = a.Hq / a.Hkv;
  const int64_t L = blockIdx.x;
  const int64_t unit = (L / 8 / g) * 8 + (L % 8);
  const int j = (int)((L / 8) % g);
  if (unit >= (int64_t)a.B * a.Hkv * a.nchunk) return;
  const int chunk = (int)(unit % a.nchunk);
  const int64_t bh = unit / a.nchunk;
  const int hk = (int)(bh % a.Hkv), b = (int)(bh / a.Hkv);
  const int hq = hk * g + j;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.Tmax ? (int)a.Tmax : len);
  const int t0 = chunk * C::CT;
  if (t0 >= len) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % LPR, r = lane / LPR;

  constexpr int RDW = D / 32 * KB;                    // dwords per cache row
  const int64_t head_row = ((int64_t)b * a.Hkv + hk) * a.Tmax;
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(a.kc);
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(a.vc);
  const int tw0 = t0 + wave * (NI * RPI) + r;

  // Issue every cache load of both passes first.
  uint32_t kx[NI][KB], vx[NI][KB];
  float ksc[NI], vsc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = tw0 + i * RPI;
    const int64_t row = head_row + (t < len ? t : len - 1);
    load_words<KB>(kw + row * RDW + c * KB, kx[i]);
    ksc[i] = a.ks[row];
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = tw0 + i * RPI;
    const int64_t row = head_row + (t < len ? t : len - 1);
    load_words<KB>(vw + row * RDW + c * KB, vx[i]);
    vsc[i] = a.vs[row];
  }

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

  // Pass 1: scores.
  float s[NI];
  float smax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    uint32_t kq[8];
    unpack_quads<KB>(kx[i], kq);
    int acc = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      acc = __builtin_amdgcn_sdot4((int)(KB == 8 ? kq[k] ^ 0x80808080u : kq[k]), qd[k], acc, false);
    float f = lane_reduce<LPR, false>((float)acc) - (float)ZK * qsum;   // integers below 2^24: exact
    const int t = tw0 + i * RPI;
    s[i] = t < len ? f * (coef * ksc[i]) : -INFINITY;
    smax = fmaxf(smax, s[i]);
  }
  smax = lane_reduce<64, true>(smax);
  if (lane == 0) red[wave] = smax;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  // Pass 2: acc_e = sum_t w_t sv_t u_{t,e} and sw = sum_t w_t sv_t.  Codes
  // below 16 are read as OCP e4m3 bytes, which gives u * unit exactly.
  const float fp8_unit = __builtin_amdgcn_cvt_pk_f32_fp8(1, false)[0];
  const float vmul = KB == 8 ? 1.0f : 1.0f / fp8_unit;
  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  float lsum = 0.0f, swv = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float w = __builtin_amdgcn_exp2f((s[i] - m) * kLog2e);   // 0 for masked tokens
    lsum += w;
    const float wsv = w * vsc[i];
    swv += wsv;
    const float wv = wsv * vmul;
    uint32_t vq[8];
    unpack_quads<KB>(vx[i], vq);
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

  // Sum the partial rows (lane (r, c) of wave w is row w * RPI + r) and the
  // two per-token sums (counted once per token: lanes with c == 0).
  {
    float* pr = part + (wave * RPI + r) * C::STRIDE + c * 32;
#pragma unroll
    for (int e = 0; e < 32; e += 4)
      *reinterpret_cast<float4*>(pr + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
  const float l = lane_reduce<64, false>(c == 0 ? lsum : 0.0f);
  const float sw = lane_reduce<64, false>(c == 0 ? swv : 0.0f);
  if (lane == 0) { red[4 + wave] = l; red[8 + wave] = sw; }
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
  const float zsw = (float)(1 << (KB - 1)) * (red[8] + red[9] + red[10] + red[11]);
  float* out = a.part + (((int64_t)b * a.Hq + hq) * a.nchunk + chunk) * kPartStride<D>;
  if (sub == 0)
    *reinterpret_cast<float4*>(out + grp * 4) = make_float4(sum.x - zsw, sum.y - zsw, sum.z - zsw, sum.w - zsw);
  if (threadIdx.x == 0) {
    out[D] = m;
    out[D + 1] = red[4] + red[5] + red[6] + red[7];
  }
}

// Second stage: merge the chunks of one (sequence, query head).
template <int D, bool OBF16>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / a.Hq);
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.Tmax ? (int)a.Tmax : len);
  const int n = (len + AttnCfg<D>::CT - 1) / AttnCfg<D>::CT;
  constexpr int PS = kPartStride<D>;
  const float* p = a.part + bh * a.nchunk * PS;
  float M = -INFINITY;
  for (int k = 0; k < n; ++k) M = fmaxf(M, p[k * PS + D]);
  float Lsum = 0.0f;
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.0f;
  for (int k = 0; k < n; ++k) {
    const float f = __builtin_amdgcn_exp2f((p[k * PS + D] - M) * kLog2e);
    Lsum = __builtin_fmaf(f, p[k * PS + D + 1], Lsum);
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = __builtin_fmaf(f, p[k * PS + threadIdx.x + 64 * i], o[i]);
  }
  const float inv = n > 0 ? 1.0f / Lsum : 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float v = o[i] * inv;
    const int64_t idx = bh * D + threadIdx.x + 64 * i;
    if constexpr (OBF16) static_cast<uint16_t*>(a.out)[idx] = f32_to_bf16(v);
    else static_cast<float*>(a.out)[idx] = v;
  }
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

int attn_chunk_tokens(int d) {
  return d == 64 ? AttnCfg<64>::CT : d == 128 ? AttnCfg<128>::CT : d == 256 ? AttnCfg<256>::CT : 0;
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

hipError_t launch_attention_decode(const AttnArgs& a) {
  switch (a.d) {
    case 64: return launch_attn_d<64>(a);
    case 128: return launch_attn_d<128>(a);
    case 256: return launch_attn_d<256>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hbl
