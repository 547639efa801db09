// Shared device helpers for the H-BitLinear kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define HBL_DEV __device__ __forceinline__

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v12i __attribute__((ext_vector_type(12)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned u6 __attribute__((ext_vector_type(6)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef _Float16 h32 __attribute__((ext_vector_type(32)));

namespace hbl {

constexpr float kEpsNorm = 1e-6f;   // RMSNorm epsilon, added to the mean square
constexpr float kEpsQ = 1e-5f;      // floor of the per-token and per-tensor statistics

// Packed ternary weights: one 32-bit word per 16 consecutive k of a row, laid
// out in tiles of 16 rows x TW k, TW = min(K, 256) (16 rows x TW/16 words: 1
// KiB when K >= 256), tiles row-block major; inside a tile the TW/16 words of
// a row are contiguous (TW/4 bytes).  So a run of 16 rows' segments is one
// contiguous block, and for K <= 256 the layout is plain row-major.  Word
// index of word w (k = 16w .. 16w+15) of row n:
HBL_DEV size_t wword(int n, int w, int K) {
  const int lt = K < 256 ? __builtin_ctz((unsigned)K) - 4 : 4;   // log2 of the words per row segment
  return (((size_t)(n >> 4) * (size_t)((K >> 4) >> lt) + (size_t)(w >> lt)) << (lt + 4)) +
         ((size_t)(n & 15) << lt) + (size_t)(w & ((1 << lt) - 1));
}
// Byte offset of the tile row block holding row n (rows n & ~15 .. +15) and of
// the row's segment inside every tile of that block.
HBL_DEV size_t wrow_base(int n, int K) {
  return (size_t)(n >> 4) * (size_t)K * 4 + (size_t)(n & 15) * (size_t)((K < 256 ? K : 256) / 4);
}
// Decode-blocked activation codes: the forward's own layout for 5..64 tokens
// (the stage calls keep row-major codes).  Per 256-k block gb and 16-token
// group, BITS/2 runs of 1 KiB; run d holds, lane by lane (lane = 16 g + c),
// token c's 16 bytes at byte 16 d of its codes for k = 256 gb + 64 g ..
// + 63 -- exactly the 16 bytes lane (c, g) of the decode matmul loads as its
// d-th activation fragment, so every fragment load is one contiguous KiB.
// Byte offset of the codes starting at k0 (a multiple of 8 for INT4 and 4
// for INT8) of token t, with mbt 16-token groups:
HBL_DEV size_t dblk_offset(int bits, int mbt, int t, int k0) {
  const int nb = bits / 2, cpc = 128 / bits;          // 1 KiB runs per group, codes per 16 bytes
  const int kk = k0 & 255, ci = kk / cpc, g = ci / nb, d = ci % nb;
  return (((size_t)(k0 >> 8) * mbt + (t >> 4)) * nb + d) * 1024 + (size_t)(g * 16 + (t & 15)) * 16 +
         (size_t)(kk % cpc) * bits / 8;
}
constexpr float kQ8 = 127.0f;       // INT8 absmax: max|x| maps to code 127
constexpr float kQ4 = 2.6457513110645906f;  // INT4 absmean multiplier sqrt(7), rounded to fp32
// Adding 1.5 * 2^23 rounds a float of magnitude < 2^22 to the nearest integer
// (ties to even, by the adder) and leaves that integer in the low mantissa bits.
constexpr float kRoundMagic = 12582912.0f;

HBL_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
HBL_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 with round-half-to-even (finite inputs).
HBL_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// The same rounding (nearest, ties to even) by the hardware conversion
// (v_cvt_pk_bf16_f32): one instruction instead of four; equal to the above
// for every finite input.
HBL_DEV uint16_t f32_to_bf16_hw(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <int W>
HBL_DEV float xor_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <int W>
HBL_DEV float xor_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace hbl
