"""Python binding of libhbl.so, the H-BitLinear (BitNet v2) forward for MI355X.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  The binding
never falls back to another implementation: a missing library or a non-gfx950
device raises.
"""
from __future__ import annotations

import ctypes
import functools
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhbl.so")
HEADERS = [os.path.join(_HERE, "..", "include", h) for h in ("hbl.h", "hbl_attn.h")]

HBL_F32, HBL_BF16 = 0, 1
OP_QUANTIZE_WEIGHTS, OP_MATMUL, OP_QUANTIZE_WEIGHTS_ROTATED, OP_FORWARD_INT4, OP_FORWARD_INT8 = 0, 1, 2, 4, 8
OP_BACKWARD = 16
STATUS = {0: "HBL_OK", 1: "HBL_ERR_NULL", 2: "HBL_ERR_SHAPE", 3: "HBL_ERR_DTYPE", 4: "HBL_ERR_ALIGN",
          5: "HBL_ERR_WORKSPACE", 6: "HBL_ERR_LAUNCH", 7: "HBL_ERR_DEVICE", 8: "HBL_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20   # HBL_NOALLOC_SCRATCH_BYTES


class HBLError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")


_lib = None
P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "hbl_status_string": ([I], ctypes.c_char_p),
    "hbl_workspace_bytes": ([I, I64, I64, I64], SZ),
    "hbl_quantize_weights": ([P, I64, I64, P, P, P, SZ, P], I),
    "hbl_forward_int8": ([P, I, P, P, P, I64, I64, I64, P, I, P, SZ, P], I),
    "hbl_forward_int4": ([P, I, P, P, P, I64, I64, I64, P, I, P, SZ, P], I),
    "hbl_forward_noalloc": ([I, P, I, P, P, P, I64, I64, I64, P, I, P], I),
    "hbl_quantize_act": ([P, I, P, I64, I64, I, P, P, P], I),
    "hbl_quantize_rotated": ([P, I64, I64, I, P, P, P], I),
    "hbl_matmul_dequant": ([P, I, P, P, P, I64, I64, I64, P, I, P, SZ, P], I),
    "hbl_rmsnorm_fwht": ([P, I, P, I64, I64, P, P], I),
    "hbl_gemm_ternary": ([P, I, P, I64, I64, I64, P, P, SZ, P], I),
    "hbl_unpack_weights": ([P, I64, I64, P, P], I),
    "hbl_bitlinear_forward": ([P, I, P, P, P, I64, I64, I64, I, P, I, P, SZ, P], I),
    "hbl_quantize_act_unrotated": ([P, I, P, I64, I64, I, P, P, P], I),
    "hbl_quantize_weights_rotated": ([P, I64, I64, P, P, P, SZ, P], I),
    "hbl_backward_weights": ([P, I64, I64, P, P], I),
    "hbl_backward": ([P, I, P, P, I, P, P, P, P, I64, I64, I64, I, P, I, P, P, P, SZ, P], I),
    "hbl_quantize_heads": ([P, I64, I64, I, P, P, P], I),
    "hbl_dequantize_heads": ([P, P, I64, I64, I, P, I, P], I),
    "hbl_kv_cache_append": ([P, P, I64, I64, I64, I64, I, P, I64, P, P, P, P, P], I),
    "hbl_attention_workspace_bytes": ([I64, I64, I64, I64], SZ),
    "hbl_attention_decode": ([P, I, P, P, P, P, I, P, I64, I64, I64, I64, I64, P, I, P, SZ, P], I),
    "hbl_attention_prefill": ([P, I, P, P, P, P, I, P, I64, I64, I64, I64, I64, I64, P, I, P], I),
}


def declared_symbols() -> list:
    """Entry points declared in include/hbl.h and include/hbl_attn.h."""
    src = ""
    for h in HEADERS:
        with open(h) as f:
            src += f.read()
    return sorted(set(re.findall(r"^\s*(?:hbl_status|size_t|const char \*)\s*\*?\s*(hbl_\w+)\s*\(", src, re.M)))


def lib() -> ctypes.CDLL:
    """Load libhbl.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with hadamard_rotated_ternary_amd/build.py "
                               "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes, fn.restype = args, res
        _lib = L
    return _lib


CALIB_PATH = os.path.join(_HERE, "libhbl_calib.so")
CALIB_HEADER = os.path.join(_HERE, "..", "include", "hbl_calib.h")
_calib = None


def calib_lib() -> ctypes.CDLL:
    """Load libhbl_calib.so, the streaming-read measurement helper
    (include/hbl_calib.h); raises if it has not been built."""
    global _calib
    if _calib is None:
        if not os.path.exists(CALIB_PATH):
            raise RuntimeError(f"{CALIB_PATH} is missing: build it with hadamard_rotated_ternary_amd/build.py")
        L = ctypes.CDLL(CALIB_PATH)
        L.hbl_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.hbl_calib_stream_read.restype = ctypes.c_int
        L.hbl_calib_broadcast_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint, ctypes.c_void_p,
                                               ctypes.c_void_p]
        L.hbl_calib_broadcast_read.restype = ctypes.c_int
        _calib = L
    return _calib


def stream_read(src: torch.Tensor, digest: torch.Tensor = None) -> torch.Tensor:
    """Plain streaming read of src's bytes; returns the per-64-KiB XOR digests
    (uint32 viewed as int32)."""
    nbytes = src.numel() * src.element_size()
    if digest is None:
        digest = torch.empty(((nbytes + 65535) // 65536,), dtype=torch.int32, device=src.device)
    rc = calib_lib().hbl_calib_stream_read(_ptr(src), nbytes, _ptr(digest), _stream())
    if rc != 0:
        raise HBLError("hbl_calib_stream_read", rc)
    return digest


def broadcast_read(src: torch.Tensor, workgroups: int, digest: torch.Tensor = None) -> torch.Tensor:
    """Every one of `workgroups` workgroups reads all of src's bytes; returns
    one XOR digest per workgroup (uint32 viewed as int32)."""
    nbytes = src.numel() * src.element_size()
    if digest is None:
        digest = torch.empty((workgroups,), dtype=torch.int32, device=src.device)
    rc = calib_lib().hbl_calib_broadcast_read(_ptr(src), nbytes, workgroups, _ptr(digest), _stream())
    if rc != 0:
        raise HBLError("hbl_calib_broadcast_read", rc)
    return digest


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise HBLError(name, rc)


# Pointers and the stream go to ctypes as plain integers (argtypes c_void_p
# converts them); building c_void_p objects per argument cost more host time
# per call than the launches of the smallest layer.
def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(dt):
    if dt == torch.float32:
        return HBL_F32
    if dt == torch.bfloat16:
        return HBL_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _dev(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


@functools.lru_cache(maxsize=4096)
def workspace_bytes(op: int, M: int, K: int, N: int) -> int:
    # a pure function of its arguments: cached, so repeated calls of one
    # shape pay no ctypes round trip for it
    return int(lib().hbl_workspace_bytes(op, M, K, N))


def _out(t, shape, name="out"):
    """A caller-given output: a contiguous device tensor of the expected shape
    (its dtype is what the call writes)."""
    _dev(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    return t


def _workspace(nbytes, device, workspace=None):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def quantize_weights(w: torch.Tensor, rotate: bool = False):
    """Latent fp32 weights [N][K] -> (packed uint8 [N][K/4], alpha fp32 [1]).
    rotate=True ternarises the rows rotated like the activations
    (weight + activation rotation variant)."""
    _dev(w, "w")
    N, K = w.shape
    wp = torch.empty((N, K // 4), dtype=torch.uint8, device=w.device)
    alpha = torch.empty(4, dtype=torch.float32, device=w.device)[:1]
    op = OP_QUANTIZE_WEIGHTS_ROTATED if rotate else OP_QUANTIZE_WEIGHTS
    ws = _workspace(workspace_bytes(op, 0, K, N), w.device)
    fn = "hbl_quantize_weights_rotated" if rotate else "hbl_quantize_weights"
    _call(fn, _ptr(w), N, K, _ptr(wp), _ptr(alpha), _ptr(ws), ws.numel(), _stream())
    return wp, alpha


def forward(x: torch.Tensor, w_packed: torch.Tensor, w_alpha: torch.Tensor, bits: int,
            gain: torch.Tensor | None = None, out_dtype=None, workspace=None, out=None,
            rotate: bool = True) -> torch.Tensor:
    """Whole H-BitLinear forward: x [M][K] (fp32/bf16) -> y [M][N].
    rotate=False runs BitLinear without the Hadamard transform."""
    _dev(x, "x")
    M, K = x.shape
    N = w_packed.shape[0]
    if out is None:
        y = torch.empty((M, N), dtype=x.dtype if out_dtype is None else out_dtype, device=x.device)
    else:
        y = _out(out, (M, N))
        if out_dtype is not None and out_dtype != y.dtype:
            raise ValueError("out_dtype differs from out.dtype")
    out_dtype = y.dtype
    op = OP_FORWARD_INT8 if bits == 8 else OP_FORWARD_INT4
    ws = _workspace(workspace_bytes(op, M, K, N), x.device, workspace)
    if rotate:
        fn = "hbl_forward_int8" if bits == 8 else "hbl_forward_int4"
        _call(fn, _ptr(x), _dtype_code(x.dtype), _ptr(gain), _ptr(w_packed), _ptr(w_alpha), M, K, N,
              _ptr(y), _dtype_code(out_dtype), _ptr(ws), ws.numel(), _stream())
    else:
        _call("hbl_bitlinear_forward", _ptr(x), _dtype_code(x.dtype), _ptr(gain), _ptr(w_packed), _ptr(w_alpha),
              M, K, N, bits, _ptr(y), _dtype_code(out_dtype), _ptr(ws), ws.numel(), _stream())
    return y


def forward_noalloc(x: torch.Tensor, w_packed: torch.Tensor, w_alpha: torch.Tensor, bits: int,
                    gain: torch.Tensor | None = None, out_dtype=None, out=None) -> torch.Tensor:
    """The H-BitLinear forward with the library's static scratch instead of a
    workspace (no device allocation inside the call; `out` may be given so
    that the call allocates nothing at all)."""
    _dev(x, "x")
    M, K = x.shape
    N = w_packed.shape[0]
    if out is None:
        y = torch.empty((M, N), dtype=x.dtype if out_dtype is None else out_dtype, device=x.device)
    else:
        y = _out(out, (M, N))
        if out_dtype is not None and out_dtype != y.dtype:
            raise ValueError("out_dtype differs from out.dtype")
    _call("hbl_forward_noalloc", bits, _ptr(x), _dtype_code(x.dtype), _ptr(gain), _ptr(w_packed), _ptr(w_alpha),
          M, K, N, _ptr(y), _dtype_code(y.dtype), _stream())
    return y


BITS_INT4, BITS_INT4_FP6, BITS_INT8 = 4, 6, 8


def codes_row_bytes(bits: int, K: int) -> int:
    """Bytes per token of the activation codes in format `bits` (8, 4 or 6)."""
    return {8: K, 4: K // 2, 6: K // 4 * 3}[bits]


def codes_shape(bits: int, M: int, K: int) -> tuple:
    """Tensor shape of the codes: [M][K] (8), [M][K/2] (4), [K/128][M][96] (6)."""
    return (K // 128, M, 96) if bits == 6 else (M, codes_row_bytes(bits, K))


def _codes_m(codes, bits: int) -> int:
    return codes.shape[1] if bits == 6 else codes.shape[0]


def quantize_act(x: torch.Tensor, bits: int, gain: torch.Tensor | None = None, out=None, rotate: bool = True):
    """Stage 1: x [M][K] -> (codes, per-token scales fp32 [M]); rotate=False
    leaves the Hadamard transform out."""
    _dev(x, "x")
    M, K = x.shape
    if out is not None:
        codes, d = out
    else:
        codes = torch.empty(codes_shape(bits, M, K), dtype=torch.int8 if bits == 8 else torch.uint8,
                            device=x.device)
        d = torch.empty(M + 4, dtype=torch.float32, device=x.device)[:M]
    _call("hbl_quantize_act" if rotate else "hbl_quantize_act_unrotated", _ptr(x), _dtype_code(x.dtype), _ptr(gain),
          M, K, bits, _ptr(codes), _ptr(d), _stream())
    return codes, d


def quantize_rotated(xt: torch.Tensor, bits: int, out=None):
    """Stage 1 from the rotated activations xt fp32 [M][K] (as rmsnorm_fwht
    returns them): the quantiser alone -> (codes, per-token scales fp32 [M])."""
    _dev(xt, "xt")
    if xt.dtype != torch.float32:
        raise ValueError("xt must be float32")
    M, K = xt.shape
    if out is not None:
        codes, d = out
    else:
        codes = torch.empty(codes_shape(bits, M, K), dtype=torch.int8 if bits == 8 else torch.uint8,
                            device=xt.device)
        d = torch.empty(M + 4, dtype=torch.float32, device=xt.device)[:M]
    _call("hbl_quantize_rotated", _ptr(xt), M, K, bits, _ptr(codes), _ptr(d), _stream())
    return codes, d


def matmul_dequant(codes, bits, dscale, w_packed, w_alpha, K, out_dtype=torch.bfloat16, workspace=None, out=None):
    """Stage 2: codes -> y [M][N]."""
    M = _codes_m(codes, bits)
    N = w_packed.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=codes.device) if out is None else _out(out, (M, N))
    out_dtype = y.dtype
    ws = _workspace(workspace_bytes(OP_MATMUL, M, K, N), codes.device, workspace)
    _call("hbl_matmul_dequant", _ptr(codes), bits, _ptr(dscale), _ptr(w_packed), _ptr(w_alpha), M, K, N,
          _ptr(y), _dtype_code(out_dtype), _ptr(ws), ws.numel(), _stream())
    return y


def rmsnorm_fwht(x: torch.Tensor, gain: torch.Tensor | None = None) -> torch.Tensor:
    """Debug view: rotated normalised activations fp32 [M][K]."""
    _dev(x, "x")
    M, K = x.shape
    xt = torch.empty((M, K), dtype=torch.float32, device=x.device)
    _call("hbl_rmsnorm_fwht", _ptr(x), _dtype_code(x.dtype), _ptr(gain), M, K, _ptr(xt), _stream())
    return xt


def gemm_ternary(codes, bits, w_packed, K, workspace=None) -> torch.Tensor:
    """Debug view: exact int32 accumulators [M][N]."""
    M = _codes_m(codes, bits)
    N = w_packed.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=codes.device)
    ws = _workspace(workspace_bytes(OP_MATMUL, M, K, N), codes.device, workspace)
    _call("hbl_gemm_ternary", _ptr(codes), bits, _ptr(w_packed), M, K, N, _ptr(acc), _ptr(ws), ws.numel(),
          _stream())
    return acc


def unpack_weights(w_packed: torch.Tensor, K: int) -> torch.Tensor:
    N = w_packed.shape[0]
    wt = torch.empty((N, K), dtype=torch.int8, device=w_packed.device)
    _call("hbl_unpack_weights", _ptr(w_packed), N, K, _ptr(wt), _stream())
    return wt


# ----------------------------------------------------------------- backward

def backward_weights(w_packed: torch.Tensor, K: int) -> torch.Tensor:
    """Packed ternary weights [N][K/4] -> W_t^T as bf16 [K][N] (once per update)."""
    _dev(w_packed, "w_packed")
    N = w_packed.shape[0]
    wbt = torch.empty((K, N), dtype=torch.bfloat16, device=w_packed.device)
    _call("hbl_backward_weights", _ptr(w_packed), N, K, _ptr(wbt), _stream())
    return wbt


def backward(x, gain, codes, bits, d, w_bf16_t, w_alpha, dy, rotate=True, dx_dtype=None, want_dgain=None,
             workspace=None):
    """Straight-through backward: returns (dx [M][K], dw fp32 [N][K], dgain fp32 [K] or None)."""
    for t, n in ((x, "x"), (codes, "codes"), (d, "d"), (w_bf16_t, "w_bf16_t"), (w_alpha, "w_alpha"), (dy, "dy")):
        _dev(t, n)
    if dy.dtype != torch.bfloat16:
        raise TypeError("dy must be bfloat16")
    M, K = x.shape
    N = dy.shape[1]
    dx_dtype = x.dtype if dx_dtype is None else dx_dtype
    dx = torch.empty((M, K), dtype=dx_dtype, device=x.device)
    dw = torch.empty((N, K), dtype=torch.float32, device=x.device)
    want = gain is not None if want_dgain is None else want_dgain
    dg = torch.empty(K, dtype=torch.float32, device=x.device) if want else None
    ws = _workspace(workspace_bytes(OP_BACKWARD, M, K, N), x.device, workspace)
    _call("hbl_backward", _ptr(x), _dtype_code(x.dtype), _ptr(gain), _ptr(codes), bits, _ptr(d), _ptr(w_bf16_t),
          _ptr(w_alpha), _ptr(dy), M, K, N, int(bool(rotate)), _ptr(dx), _dtype_code(dx_dtype), _ptr(dw), _ptr(dg),
          _ptr(ws), ws.numel() * ws.element_size(), _stream())
    return dx, dw, dg


# ------------------------------------------------------- low-bit attention states

def heads_row_bytes(bits: int, d: int) -> int:
    """Bytes of one packed row of d codes of `bits` bits."""
    return d * bits // 8


def quantize_heads(x: torch.Tensor, bits: int):
    """Per-head absmax codes: x bf16 [..., d] -> (codes uint8 [R][d*bits/8], scale fp32 [R])."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    d = x.shape[-1]
    R = x.numel() // d
    codes = torch.empty((R, heads_row_bytes(bits, d)), dtype=torch.uint8, device=x.device)
    scale = torch.empty(R, dtype=torch.float32, device=x.device)
    _call("hbl_quantize_heads", _ptr(x), R, d, bits, _ptr(codes), _ptr(scale), _stream())
    return codes, scale


def dequantize_heads(codes: torch.Tensor, scale: torch.Tensor, bits: int, d: int, out_dtype=torch.float32):
    _dev(codes, "codes")
    _dev(scale, "scale")
    R = scale.numel()
    y = torch.empty((R, d), dtype=out_dtype, device=codes.device)
    _call("hbl_dequantize_heads", _ptr(codes), _ptr(scale), R, d, bits, _ptr(y), _dtype_code(out_dtype),
          _stream())
    return y


class KVCache:
    """Quantised KV cache: codes uint8 [B][Hkv][Tmax][d*bits/8], scales fp32 [B][Hkv][Tmax]."""

    def __init__(self, B: int, Hkv: int, Tmax: int, d: int, bits: int, device="cuda"):
        self.B, self.Hkv, self.Tmax, self.d, self.bits = B, Hkv, Tmax, d, bits
        rb = heads_row_bytes(bits, d)
        self.k_codes = torch.zeros((B, Hkv, Tmax, rb), dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros((B, Hkv, Tmax, rb), dtype=torch.uint8, device=device)
        self.k_scale = torch.zeros((B, Hkv, Tmax), dtype=torch.float32, device=device)
        self.v_scale = torch.zeros((B, Hkv, Tmax), dtype=torch.float32, device=device)

    def append(self, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor | None = None):
        """k, v bf16 [B][Tn][Hkv][d]; pos device int32 [B] (None: position 0)."""
        _dev(k, "k")
        _dev(v, "v")
        if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 or k.shape != v.shape:
            raise TypeError("k and v must be bfloat16 tensors of one shape")
        B, Tn, Hkv, d = k.shape
        if pos is not None:
            _dev(pos, "pos")
            if pos.dtype != torch.int32:
                raise TypeError("pos must be int32")
        _call("hbl_kv_cache_append", _ptr(k), _ptr(v), B, Tn, Hkv, d, self.bits, _ptr(pos), self.Tmax,
              _ptr(self.k_codes), _ptr(self.k_scale), _ptr(self.v_codes), _ptr(self.v_scale), _stream())


def attention_workspace_bytes(B: int, Hq: int, d: int, Tmax: int) -> int:
    return int(lib().hbl_attention_workspace_bytes(B, Hq, d, Tmax))


def attention_decode(q: torch.Tensor, q_bits: int, k_codes, k_scale, v_codes, v_scale, kv_bits: int,
                     lens: torch.Tensor, out_dtype=torch.float32, workspace=None, out=None) -> torch.Tensor:
    """One decode step over a quantised cache: q bf16 [B][Hq][d] -> out [B][Hq][d]."""
    for t, n in ((q, "q"), (k_codes, "k_codes"), (k_scale, "k_scale"), (v_codes, "v_codes"),
                 (v_scale, "v_scale"), (lens, "lens")):
        _dev(t, n)
    if q.dtype != torch.bfloat16 or lens.dtype != torch.int32:
        raise TypeError("q must be bfloat16 and lens int32")
    B, Hq, d = q.shape
    Hkv, Tmax = k_scale.shape[1], k_scale.shape[2]
    ws = _workspace(attention_workspace_bytes(B, Hq, d, Tmax), q.device, workspace)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    else:
        _out(out, (B, Hq, d))
    _call("hbl_attention_decode", _ptr(q), q_bits, _ptr(k_codes), _ptr(k_scale), _ptr(v_codes), _ptr(v_scale),
          kv_bits, _ptr(lens), B, Hq, Hkv, d, Tmax, _ptr(out), _dtype_code(out.dtype), _ptr(ws),
          ws.numel() * ws.element_size(), _stream())
    return out


def attention_prefill(q: torch.Tensor, q_bits: int, k_codes, k_scale, v_codes, v_scale, kv_bits: int,
                      start: torch.Tensor, out_dtype=torch.float32, out=None) -> torch.Tensor:
    """Causal prefill over a quantised cache: q bf16 [B][Tn][Hq][d] -> out [B][Tn][Hq][d]."""
    for t, n in ((q, "q"), (k_codes, "k_codes"), (k_scale, "k_scale"), (v_codes, "v_codes"),
                 (v_scale, "v_scale"), (start, "start")):
        _dev(t, n)
    if q.dtype != torch.bfloat16 or start.dtype != torch.int32:
        raise TypeError("q must be bfloat16 and start int32")
    B, Tn, Hq, d = q.shape
    Hkv, Tmax = k_scale.shape[1], k_scale.shape[2]
    if out is None:
        out = torch.empty((B, Tn, Hq, d), dtype=out_dtype, device=q.device)
    else:
        _out(out, (B, Tn, Hq, d))
    _call("hbl_attention_prefill", _ptr(q), q_bits, _ptr(k_codes), _ptr(k_scale), _ptr(v_codes), _ptr(v_scale),
          kv_bits, _ptr(start), B, Tn, Hq, Hkv, d, Tmax, _ptr(out), _dtype_code(out.dtype), _stream())
    return out
