// Copy schedules of the two prefill matmuls, as compile-time descriptions
// that the kernels use and a compile-time model checks.
//
// Both kernels fill LDS stage buffers with direct global-to-LDS copies issued
// several stages ahead of use, wait for them with a count of copy
// instructions left in flight (vmcnt), and order them against the other
// waves with one barrier per stage.  A copy that lands in a buffer still
// being read, or a wait that leaves a needed copy in flight, corrupts outputs
// silently and only now and then.  The model below replays the issue order of
// every copy instruction of one wave (every wave issues the same sequence)
// and checks, for every stage:
//   * the wait before a stage's reads leaves none of that stage's copies in
//     flight, and the latest copies into the buffers it reads carry that
//     stage (not an older one, nor a later one that overwrote it);
//   * no copy issued while a buffer is being read targets that buffer;
//   * every copy index of a stage is issued exactly once, and its 1 KiB
//     lands inside its buffer.
// Host-only constexpr code: gemm.hip static_asserts it for the shipped
// schedules, and a CPU test checks that broken schedules fail to compile.
#pragma once

namespace hbl {
namespace sched {

constexpr int cmin(int a, int b) { return a < b ? a : b; }

// One copy instruction of a wave: kind 1 = A (activation codes), 2 = B
// (packed weights); j = its index among the stage's copies (it fills LDS
// bytes [(j * waves + wave) KiB, +1 KiB) of the buffer).
struct Copy {
  int kind, j;
};

// ---------------------------------------------------------------------------
// gemm_fp6_kernel: A in a ring of 4 stage buffers, B fetched per pair of
// stages into 2 slots.  A stage kt's first MFMA step reads registers only;
// after it the wave waits (wait(kt odd)), all waves meet at a barrier, and
// the second step (16 MFMAs) reads stage kt+1's fragments from LDS while the
// copy issued after MFMA i is after(i, kt odd): on even stages the 6 A copies
// of stage kt+4 after MFMAs 1, 3, ..., 11; on odd stages first the 4 B copies
// of pair (kt+3)/2, then the 6 A copies.  Past the last stage the copies
// repeat the last stage or pair (clamped), so the counts stay constant.
struct Fp6 {
  static constexpr int NBUF = 4, SLOTS = 2, WAVES = 4;
  static constexpr int A_COPIES = 6, B_COPIES = 4;   // per wave: A stage 24 KiB, B pair 16 KiB
  static constexpr int MFMAS = 16;                   // MFMAs of a stage's second step
  static constexpr Copy after(int i, bool odd) {
    if (odd) {
      if (i < B_COPIES) return {2, i};
      if (i < B_COPIES + A_COPIES) return {1, i - B_COPIES};
      return {0, 0};
    }
    if ((i & 1) && (i >> 1) < A_COPIES) return {1, i >> 1};
    return {0, 0};
  }
  // stage / pair a copy issued during stage kt carries, and where it goes
  static constexpr int a_stage(int kt, int KT) { return cmin(kt + NBUF, KT - 1); }
  static constexpr int a_buf(int kt) { return kt % NBUF; }
  static constexpr int b_pair(int kt, int KT) { return cmin((kt + 3) >> 1, (KT >> 1) - 1); }
  static constexpr int b_slot(int kt) { return ((kt + 3) / 2) % SLOTS; }
  // buffers a stage is read from
  static constexpr int read_buf(int kt) { return kt % NBUF; }
  static constexpr int read_slot(int kt) { return (kt / 2) % SLOTS; }
  // copy instructions left in flight by the wait before stage kt+1 is read
  static constexpr int wait(bool odd) { return odd ? 2 * A_COPIES : 2 * A_COPIES + B_COPIES; }
  // prologue: A0 B0 A1 A2 B1 A3 (j = stage or pair), then a wait for A0, B0
  static constexpr int PROLOGUE = 6;
  static constexpr Copy prologue(int p) {
    return p == 0 ? Copy{1, 0} : p == 1 ? Copy{2, 0} : p == 2 ? Copy{1, 1} : p == 3 ? Copy{1, 2}
         : p == 4 ? Copy{2, 1} : Copy{1, 3};
  }
  static constexpr int wait_prologue() { return 3 * A_COPIES + B_COPIES; }
};

// gemm_fp6_kernel with 128x128 tiles (four waves of 64x64): an A stage is 3
// copies per wave and a B pair 2; the second MFMA step has 4 matrix
// instructions with two issue slots after each (8 slots): even stages take
// the A copies in slots 1, 3, 5; odd stages the B copies in slots 0-1 and the
// A copies in slots 2-4.  Buffers, slots, stage choice and prologue as Fp6.
struct Fp6Small : Fp6 {
  static constexpr int A_COPIES = 3, B_COPIES = 2;
  static constexpr int MFMAS = 8;                    // issue slots of the second step
  static constexpr Copy after(int i, bool odd) {
    if (odd) {
      if (i < B_COPIES) return {2, i};
      if (i < B_COPIES + A_COPIES) return {1, i - B_COPIES};
      return {0, 0};
    }
    if ((i & 1) && (i >> 1) < A_COPIES) return {1, i >> 1};
    return {0, 0};
  }
  static constexpr int wait(bool odd) { return odd ? 2 * A_COPIES : 2 * A_COPIES + B_COPIES; }
  static constexpr int wait_prologue() { return 3 * A_COPIES + B_COPIES; }
};

// gemm_fp6_kernel with 256x192 tiles (four waves of 128x96): an A stage is
// still 6 copies per wave, a B pair 3 (192 columns of 64 bytes), and the
// second MFMA step has 12 matrix instructions: even stages take the A copies
// after MFMAs 1, 3, ..., 11; odd stages the B copies after MFMAs 0-2 and the
// A copies after 3-8.  Buffers, slots, stage choice and prologue as Fp6.
struct Fp6Wide : Fp6 {
  static constexpr int A_COPIES = 6, B_COPIES = 3;
  static constexpr int MFMAS = 12;
  static constexpr Copy after(int i, bool odd) {
    if (odd) {
      if (i < B_COPIES) return {2, i};
      if (i < B_COPIES + A_COPIES) return {1, i - B_COPIES};
      return {0, 0};
    }
    if ((i & 1) && (i >> 1) < A_COPIES) return {1, i >> 1};
    return {0, 0};
  }
  static constexpr int wait(bool odd) { return odd ? 2 * A_COPIES : 2 * A_COPIES + B_COPIES; }
  static constexpr int wait_prologue() { return 3 * A_COPIES + B_COPIES; }
};

// Issue log of one wave's copy instructions.
struct Log {
  static constexpr int CAP = 4096;
  int kind[CAP] = {}, id[CAP] = {}, j[CAP] = {}, tgt[CAP] = {};
  int n = 0;
  constexpr bool add(int k, int stage, int jj, int target) {
    if (n >= CAP) return false;
    kind[n] = k; id[n] = stage; j[n] = jj; tgt[n] = target;
    ++n;
    return true;
  }
  // The latest copies of kind k into `target` carry `stage` for every copy
  // index below `copies`, and all of them are older than the newest `left`
  // instructions (so a wait down to `left` in flight has seen them land).
  constexpr bool ready(int k, int stage, int target, int copies, int left) const {
    for (int jj = 0; jj < copies; ++jj) {
      const int last = latest(k, target, jj);
      if (last < 0 || id[last] != stage || last >= n - left) return false;
    }
    return true;
  }
  constexpr int latest(int k, int target, int jj) const {
    for (int i = n - 1; i >= 0; --i)
      if (kind[i] == k && tgt[i] == target && j[i] == jj) return i;
    return -1;
  }
  // Instructions issued after the newest one among those `ready` looks at.
  constexpr int newer_than(int k, int target, int copies) const {
    int newest = -1;
    for (int jj = 0; jj < copies; ++jj) {
      const int i = latest(k, target, jj);
      if (i > newest) newest = i;
    }
    return n - 1 - newest;
  }
};

// Checks a schedule shaped like Fp6 over KT stages (KT even).  tight: the
// waits also leave exactly as many copies in flight as they may (none of the
// wait is wasted), as the kernel's comments state.
template <class S>
constexpr bool fp6_ok(int KT, bool tight = true) {
  if (KT < 2 || KT % 2) return false;
  Log L{};
  for (int p = 0; p < S::PROLOGUE; ++p) {
    const Copy c = S::prologue(p);
    const int copies = c.kind == 1 ? S::A_COPIES : S::B_COPIES;
    for (int jj = 0; jj < copies; ++jj)
      if (!L.add(c.kind, cmin(c.j, c.kind == 1 ? KT - 1 : KT / 2 - 1), jj,
                 c.kind == 1 ? S::read_buf(c.j) : S::read_slot(2 * c.j)))
        return false;
  }
  if (!L.ready(1, 0, S::read_buf(0), S::A_COPIES, S::wait_prologue())) return false;
  if (!L.ready(2, 0, S::read_slot(0), S::B_COPIES, S::wait_prologue())) return false;
  for (int kt = 0; kt < KT; ++kt) {
    const bool odd = kt & 1;
    const int left = S::wait(odd);
    if (kt + 1 < KT) {
      if (!L.ready(1, kt + 1, S::read_buf(kt + 1), S::A_COPIES, left)) return false;
      if (!L.ready(2, (kt + 1) / 2, S::read_slot(kt + 1), S::B_COPIES, left)) return false;
      if (tight) {
        const int a = L.newer_than(1, S::read_buf(kt + 1), S::A_COPIES);
        const int b = L.newer_than(2, S::read_slot(kt + 1), S::B_COPIES);
        if ((a < b ? a : b) != left) return false;
      }
    }
    // second step: stage kt+1 is read while the copies of this stage issue
    int na[64] = {}, nb[64] = {};
    for (int i = 0; i < S::MFMAS; ++i) {
      const Copy c = S::after(i, odd);
      if (c.kind == 1) {
        if (c.j < 0 || c.j >= S::A_COPIES) return false;
        if (S::a_buf(kt) == S::read_buf(kt + 1)) return false;
        ++na[c.j];
        if (!L.add(1, S::a_stage(kt, KT), c.j, S::a_buf(kt))) return false;
      } else if (c.kind == 2) {
        if (c.j < 0 || c.j >= S::B_COPIES) return false;
        if (S::b_slot(kt) == S::read_slot(kt + 1)) return false;
        ++nb[c.j];
        if (!L.add(2, S::b_pair(kt, KT), c.j, S::b_slot(kt))) return false;
      } else if (c.kind != 0) {
        return false;
      }
    }
    for (int jj = 0; jj < S::A_COPIES; ++jj)
      if (na[jj] != 1) return false;
    for (int jj = 0; jj < S::B_COPIES; ++jj)
      if (nb[jj] != (odd ? 1 : 0)) return false;
  }
  return true;
}

// ---------------------------------------------------------------------------
// gemm_prefill_kernel (int8 instruction): a ring of 3 stage buffers, A and B
// of a stage copied together (NL instructions per wave), AHEAD = 2 stages in
// flight.  Stage kt: wait (wait(kt, KT, NL) left), barrier, copy stage kt+2
// into write_buf(kt), then read stage kt from read_buf(kt).
struct Ring3 {
  static constexpr int NBUF = 3, AHEAD = 2;
  static constexpr int read_buf(int kt) { return kt % NBUF; }
  static constexpr int write_buf(int kt) { return (kt + AHEAD) % NBUF; }
  static constexpr int wait_steady(int NL) { return NL; }
  static constexpr int wait(int kt, int KT, int NL) { return kt + 1 < KT ? wait_steady(NL) : 0; }
};

template <class R>
constexpr bool ring_ok(int KT, int NL, bool tight = true) {
  if (KT < 1 || NL < 1) return false;
  Log L{};
  for (int s = 0; s < R::AHEAD && s < KT; ++s)
    for (int jj = 0; jj < NL; ++jj)
      if (!L.add(1, s, jj, R::read_buf(s))) return false;
  for (int kt = 0; kt < KT; ++kt) {
    const int left = R::wait(kt, KT, NL);
    if (!L.ready(1, kt, R::read_buf(kt), NL, left)) return false;
    if (tight && L.newer_than(1, R::read_buf(kt), NL) != left) return false;
    // barrier; then the copies of stage kt+AHEAD, while stage kt is read
    if (kt + R::AHEAD < KT) {
      if (R::write_buf(kt) == R::read_buf(kt)) return false;
      for (int jj = 0; jj < NL; ++jj)
        if (!L.add(1, kt + R::AHEAD, jj, R::write_buf(kt))) return false;
    }
  }
  return true;
}

}  // namespace sched
}  // namespace hbl
