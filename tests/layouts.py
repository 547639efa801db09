"""Host-side encoders/decoders of the C ABI's packed formats (include/hbl.h).

Written from the format description in the header, independently of the HIP
kernels; the parity tests use them to feed the oracle's codes to the GPU matmul
and to read the GPU's packed outputs back.
"""
import numpy as np


def pack_ternary(wt: np.ndarray) -> np.ndarray:
    """int8 [N][K] in {-1,0,1} -> uint8 [N][K/4]; per 16 k one LE word,
    code of k0+4j+i at bits 8i+2j, 2-bit codes 00=0, 01=+1, 11=-1."""
    wt = np.asarray(wt, dtype=np.int8)
    N, K = wt.shape
    code = np.where(wt == 1, 1, np.where(wt == -1, 3, 0)).astype(np.uint32)
    g = code.reshape(N, K // 16, 4, 4)          # [.., j, i] -> k0 + 4j + i
    shifts = (8 * np.arange(4)[None, :] + 2 * np.arange(4)[:, None]).astype(np.uint32)  # [j, i]
    words = (g << shifts).sum(axis=(2, 3), dtype=np.uint64).astype(np.uint32)
    return words.view(np.uint8).reshape(N, K // 4)


def unpack_ternary(wp: np.ndarray, K: int) -> np.ndarray:
    wp = np.ascontiguousarray(wp, dtype=np.uint8)
    N = wp.shape[0]
    words = wp.view(np.uint32).reshape(N, K // 16, 1, 1)
    shifts = (8 * np.arange(4)[None, :] + 2 * np.arange(4)[:, None]).astype(np.uint32)
    code = (words >> shifts) & 3
    if np.any(code == 2):
        raise ValueError("invalid 2-bit code 0b10")
    return np.where(code == 1, 1, np.where(code == 3, -1, 0)).astype(np.int8).reshape(N, K)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int8 [M][K] in [-8,7] -> uint8 [M][K/2]; per 8 k one LE word, code of
    k0+4j+i (j in 0..1) at bits 8i+4j as a two's complement nibble."""
    q = np.asarray(q, dtype=np.int8)
    M, K = q.shape
    nib = (q.astype(np.int32) & 0xF).astype(np.uint32).reshape(M, K // 8, 2, 4)
    shifts = (8 * np.arange(4)[None, :] + 4 * np.arange(2)[:, None]).astype(np.uint32)
    words = (nib << shifts).sum(axis=(2, 3), dtype=np.uint64).astype(np.uint32)
    return words.view(np.uint8).reshape(M, K // 2)


def unpack_int4(p: np.ndarray, K: int) -> np.ndarray:
    p = np.ascontiguousarray(p, dtype=np.uint8)
    M = p.shape[0]
    words = p.view(np.uint32).reshape(M, K // 8, 1, 1)
    shifts = (8 * np.arange(4)[None, :] + 4 * np.arange(2)[:, None]).astype(np.uint32)
    nib = ((words >> shifts) & 0xF).astype(np.int32)
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8).reshape(M, K)
