"""Seeded synthetic workloads for the H-BitLinear forward pass.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no normalisation, transform, quantisation or matmul).  Both
the CPU oracle and the HIP path are fed from here, so the two sides always see
the same inputs.

Shapes and value distributions follow what the pages say about the inputs of
the two layers that H-BitLinear replaces (attention output projection Wo and
FFN down projection Wdown): most values sit near zero and a few channels carry
large outliers (BitNet v2 article, section "H-BitLinear module", and the
Figure 1 bottom / Figures 2-3 discussion).  The trained models' real
activations are not available, so fixed outlier channels on a Gaussian or
Laplace bulk stand in for them.  Latent weights are N(0, 0.02).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int            # tokens
    K: int            # in-features (power of two)
    N: int            # out-features
    bits: int         # activation bits on the path (8 or 4)
    x_dtype: str      # "f32" or "bf16"
    dist: str         # "normal" (N(0, scale)) or "laplace" (Laplace(0, scale))
    scale: float
    n_out: int        # number of outlier channels (same channels for every token)
    factor: float     # outlier multiplier
    seed: int
    w_std: float = 0.02

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads: a tiny INT8 case, 1.3B-shaped Wo, 3B-shaped Wdown,
# 7B-shaped prefill (Wo and Wdown, both activation widths) and 7B-shaped decode.
WORKLOADS: Dict[str, Workload] = {
    "tiny_int8": Workload("tiny_int8", 8, 256, 256, 8, "f32", "normal", 1.0, 4, 40.0, 0),
    "wo_1p3b_int4": Workload("wo_1p3b_int4", 2048, 2048, 2048, 4, "bf16", "normal", 1.0, 20, 50.0, 1),
    "wdown_3b_int4": Workload("wdown_3b_int4", 4096, 8192, 3072, 4, "bf16", "laplace", 0.05, 41, 100.0, 2),
    "wo_7b_int8": Workload("wo_7b_int8", 8192, 4096, 4096, 8, "bf16", "normal", 1.0, 41, 50.0, 3),
    "wo_7b_int4": Workload("wo_7b_int4", 8192, 4096, 4096, 4, "bf16", "normal", 1.0, 41, 50.0, 3),
    "wdown_7b_int8": Workload("wdown_7b_int8", 8192, 16384, 4096, 8, "bf16", "laplace", 0.05, 82, 100.0, 3),
    "wdown_7b_int4": Workload("wdown_7b_int4", 8192, 16384, 4096, 4, "bf16", "laplace", 0.05, 82, 100.0, 3),
    "decode_7b_m1": Workload("decode_7b_m1", 1, 16384, 4096, 4, "bf16", "laplace", 0.05, 82, 100.0, 4),
    "decode_7b_m16": Workload("decode_7b_m16", 16, 16384, 4096, 4, "bf16", "laplace", 0.05, 82, 100.0, 4),
    "decode_7b_m64": Workload("decode_7b_m64", 64, 16384, 4096, 4, "bf16", "laplace", 0.05, 82, 100.0, 4),
    # input projection of a 7B-scale FFN (up/gate, N = 11008): Gaussian-like
    # inputs without outlier channels, BitLinear without the rotation
    "up_7b_bitlinear_int4": Workload("up_7b_bitlinear_int4", 8192, 4096, 11008, 4, "bf16", "normal", 1.0, 0, 1.0, 5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round half to even) and return the raw 16-bit codes.

    Pure bit manipulation of the IEEE encodings; NaN is not expected here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 codes to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(rng: np.random.Generator, K: int, n_out: int) -> np.ndarray:
    return np.sort(rng.choice(K, n_out, replace=False))


def make_inputs(w: Workload, M: int | None = None, with_weights: bool = True
                ) -> Tuple[np.ndarray, np.ndarray | None, np.ndarray | None]:
    """Draw one workload.

    Returns ``(x_f32, x_bf16_bits, w_latent)``:
      * ``x_f32``   fp32 [M][K] — the activations exactly as the layer sees them
        (for bf16 workloads this is the exact widening of the bf16 codes);
      * ``x_bf16_bits`` uint16 [M][K] bf16 codes, or None for fp32 workloads;
      * ``w_latent`` fp32 [N][K] latent weights, or None if not requested.
    Draw order is fixed: outlier channels, activations, weights.
    """
    M = w.M if M is None else M
    rng = np.random.Generator(np.random.PCG64(w.seed))
    idx = outlier_channels(rng, w.K, w.n_out)
    if w.dist == "normal":
        x = rng.normal(0.0, w.scale, (M, w.K)).astype(np.float32)
    elif w.dist == "laplace":
        x = rng.laplace(0.0, w.scale, (M, w.K)).astype(np.float32)
    else:
        raise ValueError(w.dist)
    x[:, idx] *= np.float32(w.factor)
    wl = None
    if with_weights:
        wl = rng.normal(0.0, w.w_std, (w.N, w.K)).astype(np.float32)
    if w.x_dtype == "bf16":
        xb = f32_to_bf16_bits(x)
        return bf16_bits_to_f32(xb), xb, wl
    return x, None, wl


def make_gain(K: int, seed: int) -> np.ndarray:
    """A non-trivial RMSNorm gain vector (positive, around 1) for tests."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    return rng.uniform(0.5, 1.5, K).astype(np.float32)


def sample_rows(M: int, count: int) -> np.ndarray:
    """Deterministic token sample: evenly spaced rows plus the first and last."""
    if M <= count:
        return np.arange(M)
    rows = np.unique(np.concatenate([np.linspace(0, M - 1, count - 2).astype(np.int64), [0, M - 1]]))
    return rows


# ------------------------------------------------------- attention states
@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """One decode step of attention over a quantised KV cache."""
    name: str
    B: int            # sequences
    Hq: int           # query heads
    Hkv: int          # key/value heads
    d: int            # head size
    T: int            # cached tokens per sequence
    kv_bits: int
    q_bits: int
    n_out: int        # outlier channels of the keys (same channels for every token)
    factor: float
    seed: int


# A 7B-shaped model (32 heads of 128) decoding 16 sequences against 4096
# cached tokens with the 3-bit KV cache, a small case for tests, and the
# prefill of 4 prompts of 2048 tokens into an empty 3-bit cache (T is the
# prompt length there).
ATTN_WORKLOADS: Dict[str, AttnWorkload] = {
    "decode_attn_7b_kv3": AttnWorkload("decode_attn_7b_kv3", 16, 32, 32, 128, 4096, 3, 8, 4, 8.0, 11),
    "decode_attn_small": AttnWorkload("decode_attn_small", 4, 4, 2, 128, 1100, 3, 8, 4, 8.0, 12),
    "prefill_attn_7b_kv3": AttnWorkload("prefill_attn_7b_kv3", 4, 32, 32, 128, 2048, 3, 8, 4, 8.0, 13),
}


def make_heads(w: AttnWorkload, with_cache: bool = True):
    """Draw post-RoPE states: q [B][Hq][d] and, if requested, the new keys and
    values k, v [B][T][Hkv][d] of a prefill, all as bf16 codes (uint16).

    Queries and values are N(0, 1); keys are N(0, 1) with a few channels
    scaled by ``factor`` (key states carry channel outliers).  Draw order is
    fixed: outlier channels, q, k, v.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    idx = outlier_channels(rng, w.d, w.n_out)
    q = f32_to_bf16_bits(rng.standard_normal((w.B, w.Hq, w.d), dtype=np.float32))
    if not with_cache:
        return q, None, None
    k = rng.standard_normal((w.B, w.T, w.Hkv, w.d), dtype=np.float32)
    k[..., idx] *= np.float32(w.factor)
    k = f32_to_bf16_bits(k)
    v = f32_to_bf16_bits(rng.standard_normal((w.B, w.T, w.Hkv, w.d), dtype=np.float32))
    return q, k, v


def make_prefill(w: AttnWorkload):
    """Draw the states of a whole prompt of w.T tokens: q [B][T][Hq][d] and
    k, v [B][T][Hkv][d] as bf16 codes (uint16), distributed as in
    ``make_heads``.  Draw order: outlier channels, q, k, v."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    idx = outlier_channels(rng, w.d, w.n_out)
    q = f32_to_bf16_bits(rng.standard_normal((w.B, w.T, w.Hq, w.d), dtype=np.float32))
    k = rng.standard_normal((w.B, w.T, w.Hkv, w.d), dtype=np.float32)
    k[..., idx] *= np.float32(w.factor)
    k = f32_to_bf16_bits(k)
    v = f32_to_bf16_bits(rng.standard_normal((w.B, w.T, w.Hkv, w.d), dtype=np.float32))
    return q, k, v
