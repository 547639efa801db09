"""CPU oracle of the H-BitLinear forward (ctypes wrapper around ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may use it; the product library never does.  It shares no
code with the HIP path.  See ``oracle.c`` for the specification of each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_quantize_weights.argtypes = [P, I64, I64, P, P]
        L.oracle_weight_scale.argtypes = [ctypes.c_float]
        L.oracle_weight_scale.restype = ctypes.c_double
        L.oracle_rmsnorm.argtypes = [P, P, I64, P]
        L.oracle_fwht.argtypes = [P, I64]
        L.oracle_hadamard_rotate.argtypes = [P, I64, P]
        L.oracle_quant_act.argtypes = [P, I64, I, P, P, P]
        L.oracle_gemm_ternary.argtypes = [P, P, I64, I64, I64, P, I]
        L.oracle_dequant.argtypes = [P, P, ctypes.c_float, I64, I64, P]
        L.oracle_forward.argtypes = [P, P, P, ctypes.c_float, I64, I64, I64, I, P, P, P, P, P, P, I]
        L.oracle_forward_ex.argtypes = [P, P, P, ctypes.c_float, I64, I64, I64, I, I, P, P, P, P, P, P, I]
        L.oracle_quantize_weights_rotated.argtypes = [P, I64, I64, P, P, P]
        L.oracle_quant_heads.argtypes = [P, I64, I64, I, P, P, P]
        L.oracle_dequant_heads.argtypes = [P, P, I64, I64, I, P]
        L.oracle_attention_decode.argtypes = [P, I, P, P, P, P, I, P, I64, I64, I64, I64, I64, P]
        L.oracle_backward.argtypes = [P, P, P, P, P, ctypes.c_float, P, I64, I64, I64, I, P, P, P, P]
        L.oracle_attention_prefill.argtypes = [P, I, P, P, P, P, I, P, I64, I64, I64, I64, I64, I64, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _chk(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def max_threads() -> int:
    return lib().oracle_max_threads()


def quantize_weights(w: np.ndarray):
    """Ternarise latent weights [N][K] -> (w_t int8 [N][K], alpha fp32)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    wt = np.empty((N, K), dtype=np.int8)
    alpha = np.zeros(1, dtype=np.float32)
    _chk(lib().oracle_quantize_weights(_p(w), N, K, _p(wt), _p(alpha)), "quantize_weights")
    return wt, np.float32(alpha[0])


def weight_scale(alpha) -> float:
    return lib().oracle_weight_scale(float(alpha))


def rmsnorm(x: np.ndarray, g: np.ndarray | None = None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    K = x.shape[-1]
    g = None if g is None else np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.float64)
    xr, orr = x.reshape(-1, K), out.reshape(-1, K)
    for m in range(xr.shape[0]):
        _chk(lib().oracle_rmsnorm(_p(xr[m]), _p(g), K, _p(orr[m])), "rmsnorm")
    return out


def fwht(v: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform (Sylvester order) of each row."""
    v = np.array(v, dtype=np.float64, order="C", copy=True)
    n = v.shape[-1]
    vr = v.reshape(-1, n)
    for m in range(vr.shape[0]):
        _chk(lib().oracle_fwht(_p(vr[m]), n), "fwht")
    return v


def hadamard_rotate(u: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.float64)
    K = u.shape[-1]
    out = np.empty(u.shape, dtype=np.float64)
    ur, orr = u.reshape(-1, K), out.reshape(-1, K)
    for m in range(ur.shape[0]):
        _chk(lib().oracle_hadamard_rotate(_p(ur[m]), K, _p(orr[m])), "hadamard_rotate")
    return out


def quant_act(xt: np.ndarray, bits: int):
    """Per-token quantisation of rows -> (codes int8, d double [M], pre double)."""
    xt = np.ascontiguousarray(xt, dtype=np.float64)
    K = xt.shape[-1]
    xr = xt.reshape(-1, K)
    q = np.empty(xr.shape, dtype=np.int8)
    pre = np.empty(xr.shape, dtype=np.float64)
    d = np.empty(xr.shape[0], dtype=np.float64)
    for m in range(xr.shape[0]):
        dm = np.zeros(1, dtype=np.float64)
        _chk(lib().oracle_quant_act(_p(xr[m]), K, bits, _p(q[m]), _p(dm), _p(pre[m])), "quant_act")
        d[m] = dm[0]
    return q.reshape(xt.shape), d, pre.reshape(xt.shape)


def gemm_ternary(q: np.ndarray, wt: np.ndarray, nthreads: int = 0) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    wt = np.ascontiguousarray(wt, dtype=np.int8)
    M, K = q.shape
    N = wt.shape[0]
    acc = np.empty((M, N), dtype=np.int32)
    _chk(lib().oracle_gemm_ternary(_p(q), _p(wt), M, N, K, _p(acc), nthreads), "gemm_ternary")
    return acc


def dequant(acc: np.ndarray, d: np.ndarray, alpha) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    d = np.ascontiguousarray(d, dtype=np.float64)
    M, N = acc.shape
    y = np.empty((M, N), dtype=np.float64)
    _chk(lib().oracle_dequant(_p(acc), _p(d), float(alpha), M, N, _p(y)), "dequant")
    return y


def forward(x: np.ndarray, wt: np.ndarray, alpha, bits: int, g: np.ndarray | None = None,
            keep: bool = True, nthreads: int = 0, rotate: bool = True) -> dict:
    """Whole layer on fp32 activations [M][K] with ternary weights [N][K]:
    H-BitLinear (rotate=True) or BitLinear without the rotation (rotate=False).

    Returns a dict with ``y`` (double [M][N]) and, if ``keep``, the stages
    ``xt`` (the quantiser's input), ``q``, ``d``, ``pre``, ``acc``.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    wt = np.ascontiguousarray(wt, dtype=np.int8)
    M, K = x.shape
    N = wt.shape[0]
    g = None if g is None else np.ascontiguousarray(g, dtype=np.float32)
    y = np.empty((M, N), dtype=np.float64)
    out = {"y": y}
    if keep:
        out.update(xt=np.empty((M, K)), q=np.empty((M, K), dtype=np.int8), d=np.empty(M),
                   pre=np.empty((M, K)), acc=np.empty((M, N), dtype=np.int32))
    rc = lib().oracle_forward_ex(_p(x), _p(g), _p(wt), float(alpha), M, K, N, bits, int(bool(rotate)),
                                 _p(out.get("xt")), _p(out.get("q")), _p(out.get("d")),
                                 _p(out.get("pre")), _p(out.get("acc")), _p(y), nthreads)
    _chk(rc, "forward")
    return out


def quantize_weights_rotated(w: np.ndarray):
    """Weight + activation rotation variant: rows rotated by H_K / sqrt(K),
    then ternarised.  Returns (w_t int8 [N][K], alpha fp32, rotated rows double)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    wt = np.empty((N, K), dtype=np.int8)
    alpha = np.zeros(1, dtype=np.float32)
    wr = np.empty((N, K), dtype=np.float64)
    _chk(lib().oracle_quantize_weights_rotated(_p(w), N, K, _p(wt), _p(alpha), _p(wr)),
         "quantize_weights_rotated")
    return wt, np.float32(alpha[0]), wr


def quant_heads(x: np.ndarray, bits: int):
    """Per-head absmax quantisation of post-RoPE attention states to unsigned
    b-bit codes.  x [R][d] (one row per token and head) -> (codes uint8 [R][d],
    scale double [R], pre double [R][d])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, d = x.shape
    codes = np.empty((R, d), dtype=np.uint8)
    scale = np.empty(R)
    pre = np.empty((R, d))
    _chk(lib().oracle_quant_heads(_p(x), R, d, bits, _p(codes), _p(scale), _p(pre)), "quant_heads")
    return codes, scale, pre


def dequant_heads(codes: np.ndarray, scale: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float64)
    R, d = codes.shape
    y = np.empty((R, d))
    _chk(lib().oracle_dequant_heads(_p(codes), _p(scale), R, d, bits, _p(y)), "dequant_heads")
    return y


def backward(x, gain, q, d, wt, alpha, dy, rotate=True, want_dxh=False):
    """Straight-through backward of the layer.  x [M][K] fp32 (the forward
    input), gain [K] or None, q int8 [M][K] and d [M] (the forward's codes and
    scales), wt int8 [N][K], alpha fp32, dy [M][N].  Returns (dx, dw, dg, dxh)
    as float64 arrays (dg None without a gain, dxh None unless requested)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float64)
    wt = np.ascontiguousarray(wt, dtype=np.int8)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    g = None if gain is None else np.ascontiguousarray(gain, dtype=np.float32)
    M, K = x.shape
    N = wt.shape[0]
    dx = np.empty((M, K)); dw = np.empty((N, K))
    dg = np.empty(K) if g is not None else None
    dxh = np.empty((M, K)) if want_dxh else None
    _chk(lib().oracle_backward(_p(x), _p(g), _p(q), _p(d), _p(wt), float(alpha), _p(dy), M, K, N, int(rotate),
                               _p(dxh), _p(dx), _p(dw), _p(dg)), "backward")
    return dx, dw, dg, dxh


def attention_decode(q, qbits, kc, ks, vc, vs, kvbits, lens):
    """One decode step of attention over a quantised KV cache.

    q [B][Hq][d] (post-RoPE, quantised inside with ``qbits``); kc, vc
    [B][Hkv][Tmax][d] unpacked codes; ks, vs [B][Hkv][Tmax] fp32 scales;
    lens [B] context lengths.  Returns out [B][Hq][d] double."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    ks = np.ascontiguousarray(ks, dtype=np.float32)
    vs = np.ascontiguousarray(vs, dtype=np.float32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    B, Hq, d = q.shape
    _, Hkv, Tmax, d2 = kc.shape
    assert d2 == d and vc.shape == kc.shape and ks.shape == (B, Hkv, Tmax) and vs.shape == ks.shape
    out = np.empty((B, Hq, d))
    _chk(lib().oracle_attention_decode(_p(q), qbits, _p(kc), _p(ks), _p(vc), _p(vs), kvbits, _p(lens),
                                       B, Hq, Hkv, d, Tmax, _p(out)), "attention_decode")
    return out


def attention_prefill(q, qbits, kc, ks, vc, vs, kvbits, start):
    """Causal attention of Tn new tokens per sequence over the quantised cache.
    q [B][Tn][Hq][d]; cache as for attention_decode; start [B] (position of
    each sequence's first new token).  Returns out [B][Tn][Hq][d] double."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    ks = np.ascontiguousarray(ks, dtype=np.float32)
    vs = np.ascontiguousarray(vs, dtype=np.float32)
    start = np.ascontiguousarray(start, dtype=np.int32)
    B, Tn, Hq, d = q.shape
    _, Hkv, Tmax, _ = kc.shape
    out = np.empty((B, Tn, Hq, d))
    _chk(lib().oracle_attention_prefill(_p(q), qbits, _p(kc), _p(ks), _p(vc), _p(vs), kvbits, _p(start),
                                        B, Tn, Hq, Hkv, d, Tmax, _p(out)), "attention_prefill")
    return out


def to_bf16_rne(y: np.ndarray) -> np.ndarray:
    """Round double outputs to bf16 values (via fp32 round-to-nearest, then
    bf16 round-half-even), returned as fp32 — the output dtype of bf16 runs."""
    f = np.ascontiguousarray(y, dtype=np.float32).view(np.uint32)
    lsb = (f >> 16) & 1
    r = ((f + np.uint32(0x7FFF) + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)
