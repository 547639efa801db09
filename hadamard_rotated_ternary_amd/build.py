"""Build libhbl.so (hand-written HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhbl.so")
SOURCES = ["hbl_api.cpp", "prep.hip", "wquant.hip", "gemm.hip", "decode_fused.hip", "attn.hip", "bwd.hip",
           "noalloc.hip"]
HEADERS = ["common.h", "launch.h", "mma.h", "fwht.h", "copy_schedule.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # never emit packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source additions.  The prefill attention kernel keeps its matrix-core
# accumulators in architectural VGPRs (the default heuristic parks them in
# accumulation registers and copies all of them back on every key block).
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
OBJ = os.path.join(HERE, "_build")


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(HERE, "..", "include", "hbl.h"), os.path.join(HERE, "..", "include", "hbl_attn.h")]
    return any(os.path.getmtime(p) > t for p in deps)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libhbl.so."""
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = []
    for name in SOURCES:
        obj = os.path.join(OBJ, name + ".o")
        cmd = [HIPCC, *compile_flags, *EXTRA.get(name, []), *inc, "-c", os.path.join(CSRC, name), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((name, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for name, _, proc in jobs:
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            failed.append(name)
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *[o for _, o, _ in jobs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libhbl.so")
    os.replace(tmp, LIB)
    build_calib(verbose)
    return LIB


CALIB_LIB = os.path.join(HERE, "libhbl_calib.so")


def build_calib(verbose: bool = False) -> str:
    """libhbl_calib.so: the plain streaming read the benchmark times beside
    the decode matmul (include/hbl_calib.h); kept out of libhbl.so."""
    inc = ["-I", os.path.join(HERE, "..", "include")]
    tmp = CALIB_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *inc, os.path.join(CSRC, "calib.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on calib.hip")
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


if __name__ == "__main__":
    print(build(verbose=True))
