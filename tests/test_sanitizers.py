"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the oracle (oracle/oracle.c) with a C driver that runs every exported
  function on small seeded inputs (tests/sanitize/oracle_driver.c);
* the C ABI's host side -- argument validation, workspace sizing, dispatch up
  to the device check -- with the library's sources built as the library
  builds them plus the sanitizers on the host side only (device code is
  compiled but never run: there is no GPU here) and a driver that calls
  every entry point with invalid and valid arguments
  (tests/sanitize/api_driver.cpp).

Each driver prints "ok"; any sanitizer report fails the test.  Built in a
temporary directory.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "hadamard_rotated_ternary_amd", "csrc")
sys.path.insert(0, os.path.join(ROOT, "hadamard_rotated_ternary_amd"))
import build as hbl_build  # noqa: E402  (the library's own source list)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GCC = shutil.which("gcc")


def run_driver(exe, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.stdout.strip().endswith("ok"), out[-4000:]


@pytest.mark.skipif(GCC is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run([GCC, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"],
                   check=True, capture_output=True, text=True)
    run_driver(exe, {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1",
                     "OMP_NUM_THREADS": "2"})


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_api_host_side_under_sanitizers(tmp_path):
    # the sanitizers apply to host code only (each flag behind -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g"]
    common = [f for f in hbl_build.FLAGS if f != "-shared"] + ["-I", os.path.join(ROOT, "include")]
    jobs = []
    for src in [os.path.join(CSRC, n) for n in hbl_build.SOURCES] + [os.path.join(SAN, "api_driver.cpp")]:
        name = os.path.basename(src)
        obj = str(tmp_path / (name + ".o"))
        cmd = [HIPCC, *common, *hbl_build.EXTRA.get(name, []), *san, "-c", src, "-o", obj]
        jobs.append((obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for obj, p in jobs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-4000:]
    exe = str(tmp_path / "api_san")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *san, *[o for o, _ in jobs], "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    # the HIP runtime's own allocations at exit are not this code's: no leak check
    run_driver(exe, {"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1",
                     "HIP_VISIBLE_DEVICES": ""})
