"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects invalid arguments before touching the device.
No kernel is launched here."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import hadamard_rotated_ternary_amd as hbl
from layouts import pack_int4, pack_int4_fp6, pack_ternary, unpack_int4, unpack_int4_fp6, unpack_ternary

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5
A = ctypes.c_void_p(0x10000)        # aligned dummy address (never dereferenced here)
A2 = ctypes.c_void_p(0x20000)
BAD = ctypes.c_void_p(0x10008)      # 8-byte aligned only
S = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hbl.LIB_PATH):
        from hadamard_rotated_ternary_amd import build
        build.build()
    return hbl.lib()


def test_header_entry_points_are_exported(L):
    declared = hbl.declared_symbols()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", hbl.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared) <= exported
    assert set(hbl.SIGNATURES) == set(declared)


def test_status_strings(L):
    for code in range(9):
        assert L.hbl_status_string(code)
    assert L.hbl_status_string(99) == b"unknown status"


def test_workspace_sizes(L):
    ws8 = L.hbl_workspace_bytes(8, 8192, 16384, 4096)
    ws4 = L.hbl_workspace_bytes(4, 8192, 16384, 4096)
    assert ws8 >= 8192 * 16384 + 8192 * 4 and ws4 >= 8192 * 16384 // 2 + 8192 * 4
    assert ws4 < ws8
    assert L.hbl_workspace_bytes(0, 0, 16384, 4096) >= 4096 * 8
    assert L.hbl_workspace_bytes(1, 64, 16384, 4096) > 0      # split-K scratch of the small-M path
    # stage matmul, 33..64 tokens: int32 partials [S][M][N] (256-aligned), then
    # one arrival counter per 64-channel tile (256-aligned); S = 4, halved
    # while K / S < 256
    assert L.hbl_workspace_bytes(1, 64, 16384, 4096) == 4 * 64 * 4096 * 4 + 256
    assert L.hbl_workspace_bytes(1, 40, 512, 96) == 2 * 40 * 96 * 4 + 256
    # the forward's 33..64 tokens read decode-blocked codes (rows padded to 16)
    # and run unsplit up to K = 16384: codes + scales only; split at K = 32768
    assert L.hbl_workspace_bytes(4, 64, 16384, 4096) == 64 * 16384 // 2 + 256
    assert L.hbl_workspace_bytes(8, 40, 8192, 4096) == 48 * 8192 + 256
    assert L.hbl_workspace_bytes(4, 40, 32768, 4096) == 48 * 32768 // 2 + 256 + 4 * 40 * 4096 * 4 + 256
    assert L.hbl_workspace_bytes(1, 16, 16384, 4096) == 0      # up to 16 tokens: no split
    assert L.hbl_workspace_bytes(1, 1, 16384, 4096) == 0      # one token: no split
    assert L.hbl_workspace_bytes(1, 8192, 16384, 4096) == 0
    assert L.hbl_workspace_bytes(3, 1, 256, 16) == 0


def fwd(L, bits=8, x=A, xd=1, gain=None, wp=A, wa=A, M=8, K=256, N=256, y=A2, yd=1, ws=A, wsb=None):
    if wsb is None:
        wsb = L.hbl_workspace_bytes(bits, M if M >= 0 else 0, K, N)
    fn = L.hbl_forward_int8 if bits == 8 else L.hbl_forward_int4
    return fn(x, xd, gain, wp, wa, M, K, N, y, yd, ws, wsb, S)


@pytest.mark.parametrize("bits", [8, 4])
def test_forward_validation(L, bits):
    assert fwd(L, bits, x=None) == NULL
    assert fwd(L, bits, wp=None) == NULL
    assert fwd(L, bits, y=None) == NULL
    assert fwd(L, bits, ws=None) == NULL
    assert fwd(L, bits, xd=5) == DTYPE
    assert fwd(L, bits, yd=-1) == DTYPE
    # K: a power of two from 64 to 32768
    for K in (32, 48, 300, 65536, 0):
        assert fwd(L, bits, K=K, wsb=1 << 40) == SHAPE
    for K in (64, 128, 256, 32768):
        assert fwd(L, bits, K=K, wsb=16) == WORKSPACE      # shape accepted, workspace checked next
    for N in (0, 8, 250):
        assert fwd(L, bits, N=N, wsb=1 << 40) == SHAPE
    assert fwd(L, bits, M=-1, wsb=1 << 40) == SHAPE
    assert fwd(L, bits, x=BAD) == ALIGN
    assert fwd(L, bits, gain=BAD) == ALIGN
    assert fwd(L, bits, wsb=16) == WORKSPACE
    # empty input: valid, nothing launched
    assert fwd(L, bits, M=0) == OK


def test_noalloc_forward_validation(L):
    """hbl_forward_noalloc checks every argument, and that the problem fits
    its static scratch, before anything touches the device (no GPU here)."""
    SCRATCH = 8
    f = L.hbl_forward_noalloc
    assert f(8, A, 1, None, A, A, 8192, 16384, 4096, A2, 1, S) == SCRATCH      # needs > 32 MiB
    assert f(4, A, 1, None, A, A, 8192, 16384, 4096, A2, 1, S) == SCRATCH
    assert L.hbl_workspace_bytes(8, 8192, 16384, 4096) > hbl.NOALLOC_SCRATCH_BYTES
    assert f(5, A, 1, None, A, A, 8, 256, 256, A2, 1, S) == DTYPE
    assert f(8, A, 1, None, A, A, 8, 300, 256, A2, 1, S) == SHAPE
    assert f(8, None, 1, None, A, A, 8, 256, 256, A2, 1, S) == NULL
    assert f(4, BAD, 1, None, A, A, 8, 256, 256, A2, 1, S) == ALIGN
    assert f(4, A, 1, None, A, A, 0, 256, 256, A2, 1, S) == OK                  # empty: nothing launched
    assert L.hbl_status_string(SCRATCH).startswith(b"problem needs more scratch")


def test_stage_validation(L):
    assert L.hbl_quantize_act(A, 1, None, 4, 256, 5, A, A2, S) == DTYPE
    assert L.hbl_quantize_act(A, 1, None, 0, 256, 6, A, A2, S) == OK           # fp6 operand layout
    assert L.hbl_quantize_act(A, 1, None, 4, 256, 6, BAD, A2, S) == ALIGN
    assert L.hbl_quantize_act(A, 1, None, 4, 200, 8, A, A2, S) == SHAPE
    assert L.hbl_quantize_act(None, 1, None, 4, 256, 8, A, A2, S) == NULL
    assert L.hbl_quantize_act(A, 1, None, 0, 256, 8, A, A2, S) == OK
    assert L.hbl_rmsnorm_fwht(A, 1, None, 4, 256, BAD, S) == ALIGN
    assert L.hbl_rmsnorm_fwht(A, 1, None, 0, 256, A, S) == OK
    assert L.hbl_gemm_ternary(A, 5, A, 4, 256, 256, A, None, 0, S) == DTYPE
    assert L.hbl_gemm_ternary(A, 8, A, 4, 256, 250, A, None, 0, S) == SHAPE
    assert L.hbl_gemm_ternary(A, 8, A, 64, 1024, 256, A, None, 0, S) == NULL     # split small-M needs scratch
    assert L.hbl_gemm_ternary(A, 8, A, 64, 1024, 256, A, A2, 16, S) == WORKSPACE
    assert L.hbl_gemm_ternary(A, 6, A, 65, 1024, 256, BAD, None, 0, S) == ALIGN   # fp6 prefill: no scratch
    assert L.hbl_gemm_ternary(A, 6, A, 64, 1024, 256, A, None, 0, S) == NULL      # fp6 split decode needs scratch
    assert L.hbl_matmul_dequant(A, 8, None, A, A, 100, 256, 256, A, 1, None, 0, S) == NULL
    # format 6 needs K >= 256 (the fp6 operand is blocked by 128 k, two blocks per step)
    assert L.hbl_quantize_act(A, 1, None, 4, 128, 6, A, A2, S) == SHAPE
    assert L.hbl_gemm_ternary(A, 6, A, 100, 128, 256, A, None, 0, S) == SHAPE
    assert L.hbl_quantize_act(A, 1, None, 4, 128, 4, BAD, A2, S) == ALIGN      # format 4 at K = 128 is fine
    assert L.hbl_gemm_ternary(A, 4, A, 100, 64, 256, BAD, None, 0, S) == ALIGN
    assert L.hbl_quantize_weights(A, 256, 255, A, A, A, 1 << 20, S) == SHAPE
    assert L.hbl_quantize_weights(A, 256, 256, A, A, A, 8, S) == WORKSPACE
    assert L.hbl_unpack_weights(A, 16, 256, None, S) == NULL
    # variants: BitLinear without the rotation, weights rotated offline
    assert L.hbl_bitlinear_forward(A, 1, None, A, A, 8, 256, 256, 5, A2, 1, A, 1 << 40, S) == DTYPE
    assert L.hbl_bitlinear_forward(A, 1, None, A, A, 8, 255, 256, 8, A2, 1, A, 1 << 40, S) == SHAPE
    assert L.hbl_bitlinear_forward(None, 1, None, A, A, 8, 256, 256, 4, A2, 1, A, 1 << 40, S) == NULL
    assert L.hbl_bitlinear_forward(A, 1, None, A, A, 0, 256, 256, 4, None, 1, None, 0, S) == OK
    assert L.hbl_quantize_act_unrotated(A, 1, None, 0, 256, 6, A, A2, S) == OK
    assert L.hbl_quantize_act_unrotated(A, 1, None, 4, 256, 7, A, A2, S) == DTYPE
    # the quantiser alone, from rotated fp32 activations
    assert L.hbl_quantize_rotated(A, 4, 256, 5, A, A2, S) == DTYPE
    assert L.hbl_quantize_rotated(A, 4, 200, 8, A, A2, S) == SHAPE
    assert L.hbl_quantize_rotated(A, 4, 65536, 8, A, A2, S) == SHAPE
    assert L.hbl_quantize_rotated(A, 4, 128, 6, A, A2, S) == SHAPE          # format 6 needs K >= 256
    assert L.hbl_quantize_rotated(None, 4, 256, 4, A, A2, S) == NULL
    assert L.hbl_quantize_rotated(A, 4, 256, 4, A, None, S) == NULL
    assert L.hbl_quantize_rotated(BAD, 4, 256, 8, A, A2, S) == ALIGN
    assert L.hbl_quantize_rotated(A, 4, 64, 4, BAD, A2, S) == ALIGN
    assert L.hbl_quantize_rotated(A, 0, 256, 6, A, A2, S) == OK              # empty: nothing launched
    need = L.hbl_workspace_bytes(2, 0, 1024, 64)
    assert need >= 64 * 1024 * 4 + 64 * 8
    assert L.hbl_quantize_weights_rotated(A, 64, 1024, A, A, A, need - 1, S) == WORKSPACE
    assert L.hbl_quantize_weights_rotated(A, 64, 1000, A, A, A, need, S) == SHAPE
    assert L.hbl_quantize_weights_rotated(BAD, 64, 1024, A, A, A, need, S) == ALIGN


def test_layout_codecs_hand_examples():
    # ternary: k0..k15 = +1, -1, 0, 0 | 0 ... ; code of k (=4j+i) at bits 8i+2j
    wt = np.zeros((16, 256), np.int8)
    wt[0, 0] = 1    # i=0 j=0 -> bits 0-1 = 01
    wt[0, 1] = -1   # i=1 j=0 -> bits 8-9 = 11
    wt[0, 4] = -1   # i=0 j=1 -> bits 2-3 = 11
    wt[0, 15] = 1   # i=3 j=3 -> bits 30-31 = 01
    p = pack_ternary(wt)
    assert p.view(np.uint32).reshape(-1)[0] == 0b01 | (0b11 << 8) | (0b11 << 2) | (0b01 << 30)
    np.testing.assert_array_equal(unpack_ternary(p, 256), wt)
    # tiles of 16 rows x 256 k: word w of row n at ((n/16)(K/256) + w/16) * 256 + (n%16) * 16 + w%16
    wt = np.zeros((32, 512), np.int8)
    wt[17, 256 + 16 * 3] = 1     # row 17 (block 1, row 1), word 19 (k block 1, word 3)
    words = pack_ternary(wt).view(np.uint32).reshape(-1)
    assert np.flatnonzero(words).tolist() == [(1 * 2 + 1) * 256 + 1 * 16 + 3] and words[(1 * 2 + 1) * 256 + 19] == 1
    with pytest.raises(ValueError):
        pack_ternary(np.zeros((8, 256), np.int8))
    # K < 256: one tile spans the row, so the layout is plain row-major
    for K in (64, 128):
        wt = np.random.default_rng(K).integers(-1, 2, (32, K)).astype(np.int8)
        words = pack_ternary(wt).view(np.uint32).reshape(32, K // 16)
        for n in (0, 5, 17, 31):
            for w in range(K // 16):
                expect = 0
                for j in range(4):
                    for i in range(4):
                        c = int(wt[n, 16 * w + 4 * j + i])
                        expect |= (1 if c == 1 else 3 if c == -1 else 0) << (8 * i + 2 * j)
                assert words[n, w] == expect
        np.testing.assert_array_equal(unpack_ternary(pack_ternary(wt), K), wt)
    # int4: code of k (=4j+i) at bits 8i+4j
    q = np.array([[1, -1, 7, -8, 2, 0, 0, 3]], np.int8)
    w = pack_int4(q).view(np.uint32)[0, 0]
    assert w == (0x1 | (0xF << 8) | (0x7 << 16) | (0x8 << 24) | (0x2 << 4) | (0x3 << 28))
    np.testing.assert_array_equal(unpack_int4(pack_int4(q), 8), q)
    rng = np.random.default_rng(0)
    q = rng.integers(-8, 8, (5, 64)).astype(np.int8)
    np.testing.assert_array_equal(unpack_int4(pack_int4(q), 64), q)
    wt = rng.integers(-1, 2, (48, 768)).astype(np.int8)
    np.testing.assert_array_equal(unpack_ternary(pack_ternary(wt), 768), wt)
    # fp6 operand layout: field p = h + 2b + 8d0 + 16d1 carries k = b + 4d0 + 8h + 16d1,
    # as the e2m3 code of q/2 (q=7 -> 3.5 = 1.75*2 -> 0b010110; q=-8 -> -4 -> 0b111000;
    # q=1 -> 0.5, subnormal 4/8 -> 0b000100; q=-3 -> -1.5 -> 0b101100)
    q = np.zeros((1, 128), np.int8)
    q[0, 8] = 7      # h=1 -> p=1, bits 6..11
    q[0, 31] = -8    # b=3 d0=1 h=1 d1=1 -> p=31, bits 186..191
    q[0, 1] = 1      # b=1 -> p=2, bits 12..17
    q[0, 20] = -3    # d0=1 d1=1 -> p=24, bits 144..149
    g = int.from_bytes(pack_int4_fp6(q)[0, 0, :24].tobytes(), "little")
    assert g == (0b010110 << 6) | (0b111000 << 186) | (0b000100 << 12) | (0b101100 << 144)
    np.testing.assert_array_equal(unpack_int4_fp6(pack_int4_fp6(q), 128), q)
    # blocked by 128 k: token m's bytes of block kb at (kb * M + m) * 96
    q = rng.integers(-8, 8, (5, 256)).astype(np.int8)
    p = pack_int4_fp6(q)
    assert p.shape == (2, 5, 96)
    np.testing.assert_array_equal(p[1, 3], pack_int4_fp6(q[3:4, 128:])[0, 0])
    np.testing.assert_array_equal(unpack_int4_fp6(p, 256), q)


def test_head_code_layout_hand_examples():
    from layouts import pack_heads, unpack_heads
    # 3-bit group, worked by hand from the layout description
    u = np.zeros((1, 32), np.uint8)
    u[0, 0] = 3        # quad 0, byte 0: word 0 bits 0..2
    u[0, 13] = 7       # quad 3 (word 1, upper field), byte 1: word 1 bits 11..13
    u[0, 25] = 5       # quad 6, byte 1: 0b01 -> word 0 bits 14..15, bit 2 -> word 2 bit 14
    u[0, 30] = 6       # quad 7, byte 2: 0b10 -> word 1 bits 22..23, bit 2 -> word 2 bit 23
    w = pack_heads(u, 3).view("<u4")[0]
    assert w.tolist() == [3 | (1 << 14), (7 << 11) | (1 << 23), (1 << 14) | (1 << 23)]
    # 2-bit: code 4q + i at word q//4, bits 8i + 2(q%4); 4-bit: word q//2, bits 8i + 4(q%2)
    u2 = np.zeros((1, 32), np.uint8); u2[0, 4 * 5 + 3] = 2        # q=5, i=3 -> word 1 bit 24+2
    assert pack_heads(u2, 2).view("<u4")[0].tolist() == [0, 2 << 26]
    u4 = np.zeros((1, 32), np.uint8); u4[0, 4 * 3 + 1] = 9        # q=3, i=1 -> word 1 bit 8+4
    assert pack_heads(u4, 4).view("<u4")[0].tolist() == [0, 9 << 12, 0, 0]
    rng = np.random.default_rng(0)
    for bits in (2, 3, 4, 8):
        for d in (64, 128, 256):
            uu = rng.integers(0, 1 << bits, size=(5, d)).astype(np.uint8)
            p = pack_heads(uu, bits)
            assert p.shape == (5, d * bits // 8)
            assert np.array_equal(unpack_heads(p, bits, d), uu)


def test_attention_entry_points_validate_without_device():
    import ctypes
    L = hbl.lib()
    # unsupported widths and head sizes are rejected before any device call
    assert L.hbl_quantize_heads(None, 4, 128, 5, None, None, None) == 3
    assert L.hbl_quantize_heads(None, 4, 96, 3, None, None, None) == 2
    assert L.hbl_quantize_heads(None, 0, 128, 3, None, None, None) == 0
    assert L.hbl_kv_cache_append(None, None, 1, 1, 2, 128, 3, None, 0, None, None, None, None, None) == 2
    assert L.hbl_attention_decode(None, 9, None, None, None, None, 3, None, 1, 4, 2, 128, 16, None, 0, None, 0,
                                  None) == 3
    assert L.hbl_attention_decode(None, 8, None, None, None, None, 3, None, 1, 3, 2, 128, 16, None, 0, None, 0,
                                  None) == 2
    assert L.hbl_attention_decode(None, 8, None, None, None, None, 3, None, 1, 4, 2, 128, 16, None, 0, None, 0,
                                  None) == 1
    # prefill: (q, q_bits, kc, ks, vc, vs, kv_bits, start, B, Tn, Hq, Hkv, d, Tmax, out, out_dtype, stream)
    pf = L.hbl_attention_prefill
    assert pf(None, 8, None, None, None, None, 5, None, 1, 4, 4, 2, 128, 16, None, 0, None) == 3   # cache width
    assert pf(None, 9, None, None, None, None, 3, None, 1, 4, 4, 2, 128, 16, None, 0, None) == 3   # query width
    assert pf(None, 8, None, None, None, None, 3, None, 1, 4, 4, 2, 96, 16, None, 0, None) == 2    # head size
    assert pf(None, 8, None, None, None, None, 3, None, 1, 4, 3, 2, 128, 16, None, 0, None) == 2   # Hq % Hkv
    assert pf(None, 8, None, None, None, None, 3, None, 1, 4, 4, 2, 128, 0, None, 0, None) == 2    # Tmax
    assert pf(None, 8, None, None, None, None, 3, None, 1, 2**31 - 600, 4, 2, 128, 100, None, 0, None) == 2
    assert pf(None, 8, None, None, None, None, 3, None, 1, 0, 4, 2, 128, 16, None, 0, None) == 0   # no new tokens
    assert pf(None, 8, None, None, None, None, 3, None, 0, 4, 4, 2, 128, 16, None, 0, None) == 0   # no sequences
    assert pf(None, 8, None, None, None, None, 3, None, 1, 4, 4, 2, 128, 16, None, 0, None) == 1   # null buffers
    # partial records: B * Hq * ceil(Tmax / 512 tokens) of (d + 4) floats, rounded up to 256 bytes
    assert L.hbl_attention_workspace_bytes(2, 8, 128, 1000) == -(-(2 * 8 * 2 * 132 * 4) // 256) * 256
    assert L.hbl_attention_workspace_bytes(1, 1, 64, 1) == 0     # one chunk: the output is written directly


def test_calib_library_exports_and_validates():
    """libhbl_calib.so (the benchmark's streaming read, include/hbl_calib.h)
    exports what its header declares and rejects bad arguments before any
    launch."""
    import re
    if not os.path.exists(hbl.CALIB_PATH):
        from hadamard_rotated_ternary_amd import build
        build.build_calib()
    with open(hbl.CALIB_HEADER) as f:
        declared = set(re.findall(r"^\s*int\s+(hbl_\w+)\s*\(", f.read(), re.M))
    assert declared == {"hbl_calib_stream_read", "hbl_calib_broadcast_read"}
    out = subprocess.run(["nm", "-D", "--defined-only", hbl.CALIB_PATH], capture_output=True, text=True).stdout
    assert declared <= {line.split()[-1] for line in out.splitlines() if " T " in line}
    C = hbl.calib_lib()
    f = C.hbl_calib_stream_read
    assert f(None, 1024, A2, S) == NULL
    assert f(A, 1024, None, S) == NULL
    assert f(A, 0, A2, S) == SHAPE
    assert f(A, 1000, A2, S) == SHAPE
    assert f(BAD, 1024, A2, S) == ALIGN
    b = C.hbl_calib_broadcast_read
    assert b(None, 1024, 256, A2, S) == NULL
    assert b(A, 1024, 256, None, S) == NULL
    assert b(A, 1000, 256, A2, S) == SHAPE
    assert b(A, 1024, 0, A2, S) == SHAPE
    assert b(A, 1024, 65537, A2, S) == SHAPE
    assert b(BAD, 1024, 256, A2, S) == ALIGN
