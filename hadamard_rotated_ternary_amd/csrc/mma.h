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

// Order of the int8 operand rows the decode kernels stage in LDS: inside each
// 64-byte group byte-address bits 2-3 and 4-5 trade places.  A lane's operand
// of MFMA step j is dword j of each of its four 16-byte chunks (the pairing
// wfield() fixes); in this order those four dwords are the contiguous 16 bytes
// at 16 j, one ds_read_b128 straight into the operand registers.
HBL_DEV constexpr int opswz(int a) { return (a & ~0x3C) | ((a & 0x0C) << 2) | ((a & 0x30) >> 2); }
// Store 16-byte chunk ch (k order) of an operand row in that order.
HBL_DEV void opstore16(uint8_t* row, int ch, const uint4& v) {
  uint8_t* p = row + 64 * (ch >> 2) + 4 * (ch & 3);
  reinterpret_cast<uint32_t*>(p)[0] = v.x;
  reinterpret_cast<uint32_t*>(p + 16)[0] = v.y;
  reinterpret_cast<uint32_t*>(p + 32)[0] = v.z;
  reinterpret_cast<uint32_t*>(p + 48)[0] = v.w;
}

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

// bf16 output of a wave's 128 x (32*CB) accumulator block through LDS: the
// block is rounded into the wave's own LDS rows, 64 rows at a time, then
// written with 16-byte stores as whole row segments (instead of 2-byte
// stores scattered over 64 rows).  getv(rb, cb, r) returns the unscaled
// accumulator of 32x32 block (rb, cb), register r; lane l / register r hold
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.  Staged rows are CB*64 + 32
// bytes, so the two rows one store instruction touches start 32 banks apart.
// The caller makes sure no other wave still uses the stage area.  N % 16 == 0,
// so 8-column chunks are either whole or outside.
template <int CB, typename GetV>
HBL_DEV void store_bf16_staged(uint8_t* stage, uint16_t* Y, const float* __restrict__ dscale, float aw, int M,
                               int N, int mrow0, int ncol0, int lane, GetV getv) {
  constexpr int ER = CB * 64 + 32;             // staged row bytes
  constexpr int LPR = CB * 4;                  // lanes per row on the way out (16 bytes each)
  constexpr int RPI = 64 / LPR;                // rows per store instruction
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
      const int rb = 2 * hf + rh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = rh * 32 + 8 * (r >> 2) + 4 * g + (r & 3);     // row within the half
        const float t = dscale[min(mrow0 + 64 * hf + rl, M - 1)] * aw;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          *reinterpret_cast<uint16_t*>(stage + rl * ER + (cb * 32 + l32) * 2) = f32_to_bf16(getv(rb, cb, r) * t);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
    for (int i = 0; i < 64 / RPI; ++i) {
      const int rl = RPI * i + lane / LPR, c16 = lane % LPR;
      const int m = mrow0 + 64 * hf + rl, n = ncol0 + 8 * c16;
      const uint4 v = *reinterpret_cast<const uint4*>(stage + rl * ER + 16 * c16);
      if (m < M && n < N) *reinterpret_cast<uint4*>(Y + (size_t)m * N + n) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");       // reads done before the next half overwrites
  }
}

}  // namespace hbl
