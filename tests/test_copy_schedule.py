"""Compile-time model of the prefill matmuls' LDS copy schedules
(hadamard_rotated_ternary_amd/csrc/copy_schedule.h).

The kernels take their copy order, buffer choice and wait counts from that
header, and gemm.hip static_asserts the model over several stage counts.
Here the host compiler checks that the shipped schedules pass and that
schedules with a planted mistake -- more copies than a stage has (the race
of an earlier fp6 schedule: two extra copies landed in the buffer being
read), a wait that leaves a needed copy in flight, a copy into the buffer
being read, a ring too short for its lead, the 256-tile counts applied to
the 128-tile or the 256 x 192 schedule -- fail to compile.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(HERE, "..", "hadamard_rotated_ternary_amd", "csrc", "copy_schedule.h")
CXX = shutil.which("g++") or shutil.which("clang++")

pytestmark = pytest.mark.skipif(CXX is None, reason="needs a host C++ compiler")


def compiles(body: str) -> bool:
    src = f'#include "{HEADER}"\nusing namespace hbl::sched;\n{body}\n'
    r = subprocess.run([CXX, "-std=c++17", "-fsyntax-only", "-x", "c++", "-"], input=src, text=True,
                       capture_output=True)
    return r.returncode == 0


def test_shipped_schedules_pass():
    assert compiles("""
        static_assert(fp6_ok<Fp6>(2) && fp6_ok<Fp6>(4) && fp6_ok<Fp6>(16) && fp6_ok<Fp6>(128), "");
        // the 128x128 tile of the same kernel
        static_assert(fp6_ok<Fp6Small>(2) && fp6_ok<Fp6Small>(6) && fp6_ok<Fp6Small>(16)
                      && fp6_ok<Fp6Small>(128), "");
        // the 256x192 tile
        static_assert(fp6_ok<Fp6Wide>(2) && fp6_ok<Fp6Wide>(4) && fp6_ok<Fp6Wide>(16)
                      && fp6_ok<Fp6Wide>(128), "");
        // the int8 instruction kernel: 10 copies per stage (INT8), 6 (INT4)
        static_assert(ring_ok<Ring3>(1, 10) && ring_ok<Ring3>(2, 10) && ring_ok<Ring3>(64, 10), "");
        static_assert(ring_ok<Ring3>(5, 6) && ring_ok<Ring3>(64, 6), "");
    """)


def test_the_checker_itself_compiles_and_rejects():
    # sanity: a false assertion must not compile (so the cases below test the model)
    assert not compiles('static_assert(!fp6_ok<Fp6>(16), "");')


@pytest.mark.parametrize("name,body", [
    ("eight A copies on even stages", """
        struct Bad : Fp6 {
          static constexpr Copy after(int i, bool odd) {
            if (!odd) return (i & 1) ? Copy{1, i >> 1} : Copy{0, 0};
            return Fp6::after(i, odd);
          }
        };"""),
    ("one A copy missing on odd stages", """
        struct Bad : Fp6 {
          static constexpr Copy after(int i, bool odd) {
            if (odd && i == B_COPIES + A_COPIES - 1) return {0, 0};
            return Fp6::after(i, odd);
          }
        };"""),
    ("wait leaves one more copy in flight", """
        struct Bad : Fp6 { static constexpr int wait(bool odd) { return Fp6::wait(odd) + 1; } };"""),
    ("prologue wait leaves B0 in flight", """
        struct Bad : Fp6 { static constexpr int wait_prologue() { return Fp6::wait_prologue() + B_COPIES; } };"""),
    ("A copies into the buffer being read", """
        struct Bad : Fp6 { static constexpr int a_buf(int kt) { return (kt + 1) % NBUF; } };"""),
    ("B pair into the slot being read", """
        struct Bad : Fp6 { static constexpr int b_slot(int kt) { return ((kt + 1) / 2) % SLOTS; } };"""),
    ("A copies five stages ahead in a ring of four", """
        struct Bad : Fp6 { static constexpr int a_stage(int kt, int KT) { return cmin(kt + 5, KT - 1); } };"""),
])
def test_broken_fp6_schedules_fail(name, body):
    assert not compiles(body + '\nstatic_assert(fp6_ok<Bad>(16), "");'), name


@pytest.mark.parametrize("name,body", [
    ("a fourth A copy per stage (the 256-tile count leaking in)", """
        struct Bad : Fp6Small {
          static constexpr Copy after(int i, bool odd) {
            if (!odd && i == 7) return {1, 3};
            return Fp6Small::after(i, odd);
          }
        };"""),
    ("B copies missing on odd stages", """
        struct Bad : Fp6Small {
          static constexpr Copy after(int i, bool odd) {
            if (odd && i == 1) return {0, 0};
            return Fp6Small::after(i, odd);
          }
        };"""),
    ("wait counts of the 256 tile", """
        struct Bad : Fp6Small { static constexpr int wait(bool odd) { return Fp6::wait(odd); } };"""),
    ("prologue wait of the 256 tile", """
        struct Bad : Fp6Small { static constexpr int wait_prologue() { return Fp6::wait_prologue(); } };"""),
])
def test_broken_small_tile_schedules_fail(name, body):
    assert not compiles(body + '\nstatic_assert(fp6_ok<Bad>(16), "");'), name


@pytest.mark.parametrize("name,body", [
    ("a fourth B copy per pair (the 256-column count)", """
        struct Bad : Fp6Wide {
          static constexpr Copy after(int i, bool odd) {
            if (odd && i == 9) return {2, 3};
            return Fp6Wide::after(i, odd);
          }
        };"""),
    ("the 256-column B count with the 192-column slots", """
        struct Bad : Fp6Wide { static constexpr int B_COPIES = 4; };"""),
    ("wait counts of the square tile", """
        struct Bad : Fp6Wide { static constexpr int wait(bool odd) { return Fp6::wait(odd); } };"""),
    ("last A copy of even stages past the twelve MFMAs", """
        struct Bad : Fp6Wide {
          static constexpr int MFMAS = 11;
        };"""),
])
def test_broken_wide_tile_schedules_fail(name, body):
    assert not compiles(body + '\nstatic_assert(fp6_ok<Bad>(16), "");'), name


@pytest.mark.parametrize("name,body", [
    ("lead of three in a ring of three", """
        struct Bad : Ring3 { static constexpr int AHEAD = 3;
          static constexpr int write_buf(int kt) { return (kt + AHEAD) % NBUF; } };"""),
    ("steady wait leaves the stage's own copies in flight", """
        struct Bad : Ring3 {
          static constexpr int wait_steady(int NL) { return NL + 1; }
          static constexpr int wait(int kt, int KT, int NL) { return kt + 1 < KT ? wait_steady(NL) : 0; }
        };"""),
    ("copy into the buffer being read", """
        struct Bad : Ring3 { static constexpr int write_buf(int kt) { return kt % NBUF; } };"""),
])
def test_broken_ring_schedules_fail(name, body):
    assert not compiles(body + '\nstatic_assert(ring_ok<Bad>(16, 10), "");'), name
