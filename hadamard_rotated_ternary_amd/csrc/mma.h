// Device helpers shared by the matmul kernels: packed-operand expansion for
// the int8 matrix instructions, exact unscaling, global-to-LDS copies with
// explicit waits, and the dequantising store.
#pragma once
#include "common.h"
#include "launch.h"

namespace hbl {

// Operand expansion without lookups.
//
// A packed weight word holds the 2-bit two's complement codes of 16
// consecutive k, the code of k0+4j+i in bits 8i+2j (field j of byte i).
// Shifting field j to the top of its byte and masking gives, byte by byte,
// exactly 64*w as a signed int8 (0x40 = +64, 0xC0 = -64).
HBL_DEV uint32_t wfield(uint32_t p, int j) {
  return (j == 3 ? p : (p << (6 - 2 * j))) & 0xC0C0C0C0u;
}
// MFMA step s (0..3) of a lane's 64-k group takes the four fields of packed
// word s: operand register r = field r, whose byte i holds code
// k0 + 16s + 4r + i.  Those are the 16 consecutive codes k0+16s .. k0+16s+15,
// so int8 activations are the other operand exactly as stored (16 bytes from
// offset 16s, no regrouping); 7 VALU ops per weight word.
HBL_DEV v4i wstep(uint32_t p) { return v4i{(int)wfield(p, 0), (int)wfield(p, 1), (int)wfield(p, 2), (int)wfield(p, 3)}; }
HBL_DEV v4i as_v4i(const uint4& u) { return v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w}; }
// The INT4 matmuls pair the other way: step j takes field j of four packed
// words (codes 16d + 4j + i, d = word, i = byte) against the same codes of
// the INT4 activations.  Those words hold codes 8 at a time, the code of
// k0+4j+i in bits 8i+4j; step j takes the low (j even) or high (j odd)
// nibbles of word 2d + j/2, moved to the top of each byte: 16*q as a signed
// int8.
HBL_DEV uint32_t a4field(uint32_t w, int j) {
  return ((j & 1) ? w : (w << 4)) & 0xF0F0F0F0u;
}
// The accumulators therefore hold 64 * acc (INT8 path) or 1024 * acc (INT4),
// exact multiples whose magnitude stays below 2^27 for K <= 16384 (|q| <= 128
// after scaling, |w| = 64): an arithmetic shift recovers acc exactly.  The
// fp6 x fp4 instruction (BITS == 6: codes q/2 against weights 2w) sums acc
// itself.
template <int BITS>
HBL_DEV int unscale(int v) { return BITS == 8 ? (v >> 6) : BITS == 4 ? (v >> 10) : v; }
HBL_DEV uint32_t u4get(const uint4& u, int j) { return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w; }

// Copy 16 bytes per lane from global memory straight into LDS: the wave's
// 64 lanes fill 1 KiB at lds_base (wave-uniform), lane L at +16L.  Issued from
// inline asm so the compiler does not track it (it cannot tell which LDS
// buffer such a copy targets and would otherwise wait for every copy before
// any LDS read); the caller orders it with wait_vmcnt() and s_barrier.  The
// instruction has no destination registers and reads its address operands at
// issue.
HBL_DEV void lds_copy16(const void* gsrc, void* lds_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(l), "v"(gsrc) : "memory", "m0");
}
// The same for 4 bytes per lane: the wave fills 256 bytes at lds_base.
HBL_DEV void lds_copy4(const void* gsrc, void* lds_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" : : "s"(l), "v"(gsrc) : "memory", "m0");
}
// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt[3:0] and [15:14], expcnt and lgkmcnt at max).
template <int N>
HBL_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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

// Four consecutive outputs (16-byte aligned for int32 / fp32, 8-byte for bf16).
template <int OUT>
HBL_DEV void store_out4(void* Y, size_t off, v4i acc, float t) {
  if constexpr (OUT == OUT_ACC_I32) {
    *reinterpret_cast<v4i*>(static_cast<int32_t*>(Y) + off) = acc;
  } else if constexpr (OUT == OUT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(Y) + off) =
        make_float4((float)acc[0] * t, (float)acc[1] * t, (float)acc[2] * t, (float)acc[3] * t);
  } else {
    const uint32_t lo = f32_to_bf16((float)acc[0] * t) | ((uint32_t)f32_to_bf16((float)acc[1] * t) << 16);
    const uint32_t hi = f32_to_bf16((float)acc[2] * t) | ((uint32_t)f32_to_bf16((float)acc[3] * t) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + off) = make_uint2(lo, hi);
  }
}
template <int BITS>
HBL_DEV v4i unscale4(v4i v) { return v4i{unscale<BITS>(v[0]), unscale<BITS>(v[1]), unscale<BITS>(v[2]), unscale<BITS>(v[3])}; }


// Row scales d of a ROWS-row output tile in LDS for the epilogue: waves 0..
// ROWS/64 - 1 each copy 64 of them with one global-to-LDS instruction (lane L: row
// 64 * wave + L, clamped to the last row, so nothing past d[M-1] is read),
// issued before the tile's first operand copies, so every later wait for
// those copies also covers it and no register holds it through the main
// loop.  Reading d from global memory in the epilogue itself put four
// dependent batches of loads, each a full memory latency with one wave per
// SIMD, into every tile (9.7 us of a 107 us tile); a register-held d
// lengthened the main loop instead.
template <int ROWS = 256>
HBL_DEV void row_scale_copy(const float* __restrict__ dscale, int m0, int M, float* srow, int wave, int lane) {
  if (wave < ROWS / 64) lds_copy4(dscale + min(m0 + 64 * wave + lane, M - 1), srow + 64 * wave);
}

// bf16 output of a wave's (64*HALVES) x (32*CB) accumulator block (CB = 2,
// 3 or 4) through
// LDS: the block is rounded into the wave's own LDS rows, 64 rows at a time, then
// written with 16-byte stores as whole row segments (instead of 2-byte
// stores scattered over 64 rows).  getv(rb, cb, r) returns the unscaled
// accumulator of 32x32 block (rb, cb), register r; lane l / register r hold
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.  srow holds the scales of the
// block's 128 rows (d, in LDS) and aw the weight scale max(alpha, 1e-5).  Staged rows are CB*64 + 32 bytes, so the
// two rows one store instruction touches start 32 banks apart.  The caller
// makes sure no other wave still uses the stage area.  N % 16 == 0, so
// 8-column chunks are either whole or outside.
template <int CB, int HALVES = 2, typename GetV>
HBL_DEV void store_bf16_staged(uint8_t* stage, uint16_t* Y, const float* srow, float aw, int M, int N, int mrow0,
                               int ncol0, int lane, GetV getv) {
  constexpr int ER = CB * 64 + 32;             // staged row bytes
  constexpr int LPR = CB * 4;                  // lanes per row on the way out (16 bytes each)
  constexpr int RPI = 64 / LPR;                // rows per store instruction (lanes past RPI * LPR idle)
  constexpr int NI = (64 + RPI - 1) / RPI;     // store instructions per 64 rows
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int hf = 0; hf < HALVES; ++hf) {
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
      const int rb = 2 * hf + rh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = rh * 32 + 8 * (r >> 2) + 4 * g + (r & 3);     // row within the half
        const float t = srow[64 * hf + rl] * aw;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          *reinterpret_cast<uint16_t*>(stage + rl * ER + (cb * 32 + l32) * 2) = f32_to_bf16_hw(getv(rb, cb, r) * t);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rl = RPI * i + lane / LPR, c16 = lane % LPR;
      if (64 % LPR != 0 && (lane >= RPI * LPR || rl >= 64)) continue;
      const int m = mrow0 + 64 * hf + rl, n = ncol0 + 8 * c16;
      const uint4 v = *reinterpret_cast<const uint4*>(stage + rl * ER + 16 * c16);
      if (m < M && n < N) *reinterpret_cast<uint4*>(Y + (size_t)m * N + n) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");       // reads done before the next half overwrites
  }
}

}  // namespace hbl
