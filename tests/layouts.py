"""Host-side encoders/decoders of the C ABI's packed formats (include/hbl.h).

Written from the format description in the header, independently of the HIP
kernels; the parity tests use them to feed the oracle's codes to the GPU matmul
and to read the GPU's packed outputs back.
"""
import numpy as np


def _ternary_words(wt: np.ndarray) -> np.ndarray:
    """int8 [N][K] in {-1,0,1} -> row-major words [N][K/16]: per 16 k one
    word, code of k0+4j+i at bits 8i+2j, 2-bit codes 00=0, 01=+1, 11=-1."""
    wt = np.asarray(wt, dtype=np.int8)
    N, K = wt.shape
    code = np.where(wt == 1, 1, np.where(wt == -1, 3, 0)).astype(np.uint32)
    g = code.reshape(N, K // 16, 4, 4)          # [.., j, i] -> k0 + 4j + i
    shifts = (8 * np.arange(4)[None, :] + 2 * np.arange(4)[:, None]).astype(np.uint32)  # [j, i]
    return (g << shifts).sum(axis=(2, 3), dtype=np.uint64).astype(np.uint32)


def pack_ternary(wt: np.ndarray) -> np.ndarray:
    """int8 [N][K] in {-1,0,1} -> the packed buffer, uint8 [N][K/4] in size:
    the words of _ternary_words in tiles of 16 rows x TW k, TW = min(K, 256)
    (16 x TW/16 words), tiles in row-block-major order, inside a tile row by
    row (the TW/16 words of a row contiguous).  For K <= 256 that is plain
    row-major.  N % 16 == 0, K a multiple of 16 and of TW."""
    N, K = np.shape(wt)
    tw = min(K, 256)
    if N % 16 or K % 16 or K % tw:
        raise ValueError("tiled packing needs N % 16 == 0 and K a multiple of min(K, 256)")
    words = _ternary_words(wt).reshape(N // 16, 16, K // tw, tw // 16)   # [row block, row, k block, word]
    tiled = np.ascontiguousarray(words.transpose(0, 2, 1, 3))           # [row block, k block, row, word]
    return tiled.view(np.uint8).reshape(N, K // 4)


def unpack_ternary(wp: np.ndarray, K: int) -> np.ndarray:
    wp = np.ascontiguousarray(wp, dtype=np.uint8)
    N = wp.size * 4 // K
    tw = min(K, 256)
    words = (wp.view(np.uint32).reshape(N // 16, K // tw, 16, tw // 16).transpose(0, 2, 1, 3)
             .reshape(N, K // 16, 1, 1))
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


def e2m3_value(code: int) -> float:
    """Value of a six-bit OCP fp6 e2m3 code: sign bit 5, exponent bits 4..3
    (bias 1), mantissa bits 2..0; exponent 0 is subnormal (m/8)."""
    s, e, m = (code >> 5) & 1, (code >> 3) & 3, code & 7
    v = m / 8.0 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 1)
    return -v if s else v


def _fp6_field_k() -> np.ndarray:
    """k offset (within a 32-k group) carried by field p: p = h + 2b + 8d0 + 16d1
    holds k = b + 4d0 + 8h + 16d1."""
    k = np.empty(32, np.int64)
    for p in range(32):
        h, b, d0, d1 = p & 1, (p >> 1) & 3, (p >> 3) & 1, (p >> 4) & 1
        k[p] = b + 4 * d0 + 8 * h + 16 * d1
    return k


def pack_int4_fp6(q: np.ndarray) -> np.ndarray:
    """int8 [M][K] in [-8,7] -> uint8 [K/128][M][96]: per token and 32 k a
    24-byte LE group, field p (bits 6p..6p+5) = e2m3 code of q/2 for the k of
    _fp6_field_k()[p]; the four groups of a 128-k block are token m's 96 bytes
    of block kb."""
    q = np.asarray(q, dtype=np.int8)
    M, K = q.shape
    enc = {}
    for c in range(64):
        enc.setdefault(e2m3_value(c), c)          # +0 before -0
    table = np.array([enc[v / 2.0] for v in range(-8, 8)], np.uint8)
    fields = table[q.reshape(M, K // 32, 32)[:, :, _fp6_field_k()].astype(np.int32) + 8]   # [M, G, p]
    bits = ((fields[..., None] >> np.arange(6, dtype=np.uint8)) & 1).reshape(M, K // 32, 192)
    rows = np.packbits(bits, axis=-1, bitorder="little").reshape(M, K // 128, 96)
    return np.ascontiguousarray(rows.transpose(1, 0, 2))


def unpack_int4_fp6(p: np.ndarray, K: int) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8).reshape(K // 128, -1, 96)
    M = p.shape[1]
    rows = np.ascontiguousarray(p.transpose(1, 0, 2)).reshape(M, K // 32, 24)
    bits = np.unpackbits(rows, axis=-1, bitorder="little").reshape(M, K // 32, 32, 6)
    codes = (bits.astype(np.int32) << np.arange(6)).sum(-1)
    vals = np.vectorize(e2m3_value)(np.arange(64))[codes] * 2.0
    if np.any(vals != np.round(vals)) or np.any(vals < -8) or np.any(vals > 7):
        raise ValueError("fp6 field is not an INT4 code / 2")
    q = np.empty((M, K // 32, 32), np.int8)
    q[:, :, _fp6_field_k()] = vals.astype(np.int8)
    return q.reshape(M, K)


# ------------------------------------------------------------- head codes
# Packed rows of per-head codes, written from the layout description in
# include/hbl_attn.h: 32-code groups of `bits` little-endian words; code
# c = 4q + i of a group sits in byte i of a word.

def _head_places(bits):
    """For each code c of a group: list of (word, shift, value_shift, nbits)."""
    places = []
    for c in range(32):
        q, i = divmod(c, 4)
        if bits == 8:
            places.append([(q, 8 * i, 0, 8)])
        elif bits == 4:
            places.append([(q // 2, 8 * i + 4 * (q % 2), 0, 4)])
        elif bits == 2:
            places.append([(q // 4, 8 * i + 2 * (q % 4), 0, 2)])
        elif bits == 3:
            if q < 6:
                places.append([(q // 2, 8 * i + 3 * (q % 2), 0, 3)])
            elif q == 6:
                places.append([(0, 8 * i + 6, 0, 2), (2, 8 * i + 6, 2, 1)])
            else:
                places.append([(1, 8 * i + 6, 0, 2), (2, 8 * i + 7, 2, 1)])
        else:
            raise ValueError(bits)
    return places


def pack_heads(u, bits):
    """Codes uint8 [R][d] (each < 2^bits) -> packed uint8 [R][d*bits/8]."""
    u = np.asarray(u, dtype=np.uint32)
    R, d = u.shape
    assert d % 32 == 0 and np.all(u < (1 << bits))
    g = u.reshape(R, d // 32, 32)
    words = np.zeros((R, d // 32, bits), dtype=np.uint32)
    for c, pl in enumerate(_head_places(bits)):
        for (wd, sh, vs, nb) in pl:
            words[:, :, wd] |= ((g[:, :, c] >> vs) & ((1 << nb) - 1)) << sh
    return words.reshape(R, -1).astype("<u4").view(np.uint8).reshape(R, d * bits // 8)


def unpack_heads(packed, bits, d):
    """Inverse of pack_heads."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    R = packed.shape[0]
    words = packed.reshape(R, -1).view("<u4").reshape(R, d // 32, bits).astype(np.uint32)
    u = np.zeros((R, d // 32, 32), dtype=np.uint32)
    for c, pl in enumerate(_head_places(bits)):
        for (wd, sh, vs, nb) in pl:
            u[:, :, c] |= ((words[:, :, wd] >> sh) & ((1 << nb) - 1)) << vs
    return u.reshape(R, d).astype(np.uint8)
