// Walsh-Hadamard machinery shared by the prep kernel and the fused decode
// kernel: compile-time dealing of a token's index bits over threads and
// registers, the radix-2 butterflies, the padded LDS exchange between passes,
// and token-wide reductions.
//
// QbitAI article on BitNet v2, section 引入H-BitLinear模块, and 新智元 article
// "微软再放LLM量化大招", section H-BitLinear模块: the activations go through an
// orthogonal +-1 Hadamard transform computed by the fast O(n log n) algorithm.
//
// One token of K = 2^LOGK features is spread over T = 2^(LOGK-LOGE) threads
// holding E = 2^LOGE values each.  The Walsh-Hadamard transform is a product
// of independent radix-2 butterflies, one per index bit, that may be applied
// in any order; each "pass" applies the butterflies of the index bits that a
// thread currently holds in registers, and an LDS exchange between passes
// re-deals the index bits so that the not-yet-transformed ones land in
// registers.  No shuffles are needed: every add/sub is register to register.
#pragma once
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

}  // namespace hbl
