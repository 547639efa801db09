"""GPU parity of the low-bit attention states (through the C ABI) against the oracle.

Bars:
  * head codes: bit-exact (the HIP path decides every code exactly);
  * head scales: bit-exact against the oracle's scale rounded to fp32
    (G / Qb is correctly rounded on both sides);
  * dequantised values: bit-exact in fp32 (one rounding of an exact product)
    and in bf16 (the same fp32 value rounded to nearest even);
  * decode attention: |out - ref| <= ATTN_TOL * max|v^| per (sequence, head),
    with the oracle fed the same cache (codes and fp32 scales) and the same
    bf16 query.  ATTN_TOL: the kernel's key dot products are exact integers;
    scores carry a few fp32 roundings (relative 2^-22 each, scores below 40 in
    magnitude here), so each softmax weight is within ~1e-5 relative; the
    output is a convex combination, so its error is at most twice that times
    max|v^|, plus fp32 summation over at most a few thousand terms.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_ternary_amd as hbl
import oracle
from layouts import pack_heads, unpack_heads

pytestmark = pytest.mark.gpu

ATTN_TOL = 3e-5
BITS = (2, 3, 4, 8)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a gfx950 device"
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    hbl.lib()


def bf16_bits(x):
    """fp32 array -> (bf16 bit patterns uint16, the bf16 values as fp32), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r, (r.astype(np.uint32) << 16).view(np.float32)


def to_dev_bf16(bits16):
    return torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def head_rows(rng, R, d):
    """bf16 rows with the structure of post-RoPE states: gaussian, a few
    outlier channels, plus special rows (zero, below the floor, exact ties)."""
    x = rng.normal(size=(R, d)).astype(np.float32)
    x[:, rng.integers(0, d, size=3)] *= 8.0
    x[0] = 0.0
    x[1] = x[1] * 1e-7
    x[2] = np.arange(d, dtype=np.float32) - d / 2          # many exact ties for small widths
    x[3] = np.where(np.arange(d) % 2, 1.0, -1.0)
    return bf16_bits(x)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("d", [64, 128, 256])
def test_quantize_heads_bit_exact(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    R = 1031                                                 # ragged against every rows-per-workgroup
    xb, xf = head_rows(rng, R, d)
    codes, scale = hbl.quantize_heads(to_dev_bf16(xb), bits)
    c_or, s_or, _ = oracle.quant_heads(xf, bits)
    got = unpack_heads(host(codes), bits, d)
    assert np.array_equal(got, c_or)
    assert np.array_equal(host(scale), s_or.astype(np.float32))


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("d", [64, 256])
def test_dequantize_heads_bit_exact(bits, d):
    rng = np.random.default_rng(7 + bits)
    R = 300
    _, xf = head_rows(rng, R, d)
    c_or, s_or, _ = oracle.quant_heads(xf, bits)
    s32 = s_or.astype(np.float32)
    ref = oracle.dequant_heads(c_or, s32.astype(np.float64), bits)     # exact products in double
    packed = torch.from_numpy(pack_heads(c_or, bits)).cuda()
    sc = torch.from_numpy(s32).cuda()
    y32 = host(hbl.dequantize_heads(packed, sc, bits, d, torch.float32))
    assert np.array_equal(y32, ref.astype(np.float32))
    yb = hbl.dequantize_heads(packed, sc, bits, d, torch.bfloat16)
    yb = host(yb.view(torch.int16)).view(np.uint16)
    assert np.array_equal(yb, bf16_bits(ref.astype(np.float32))[0])


def test_kv_cache_append_positions():
    rng = np.random.default_rng(3)
    B, Tn, Hkv, d, Tmax, bits = 3, 5, 4, 128, 16, 3
    kb, kf = bf16_bits(rng.normal(size=(B, Tn, Hkv, d)))
    vb, vf = bf16_bits(rng.standard_t(4, size=(B, Tn, Hkv, d)))
    pos = np.array([0, 7, 13], np.int32)                     # the last runs past Tmax: 2 rows skipped
    cache = hbl.KVCache(B, Hkv, Tmax, d, bits)
    for t in (cache.k_codes, cache.v_codes):
        t.fill_(0xAB)
    cache.k_scale.fill_(-1.0)
    cache.v_scale.fill_(-1.0)
    cache.append(to_dev_bf16(kb), to_dev_bf16(vb), torch.from_numpy(pos).cuda())
    for codes_t, scale_t, xf in ((cache.k_codes, cache.k_scale, kf), (cache.v_codes, cache.v_scale, vf)):
        codes = host(codes_t)
        scale = host(scale_t)
        for b in range(B):
            for h in range(Hkv):
                for t in range(Tmax):
                    src = t - pos[b]
                    if 0 <= src < Tn:
                        c_or, s_or, _ = oracle.quant_heads(xf[b, src, h][None], bits)
                        assert np.array_equal(unpack_heads(codes[b, h, t][None], bits, d), c_or)
                        assert scale[b, h, t] == np.float32(s_or[0])
                    else:
                        assert np.all(codes[b, h, t] == 0xAB) and scale[b, h, t] == -1.0


def make_cache(rng, B, Hkv, Tmax, d, bits):
    """Oracle-quantised cache from bf16 keys/values: (unpacked codes, fp32
    scales, packed device codes, device scales) for K and V."""
    out = []
    for dist in ("normal", "t"):
        x = rng.normal(size=(B * Hkv * Tmax, d)) if dist == "normal" else rng.standard_t(4, size=(B * Hkv * Tmax, d))
        x[:, rng.integers(0, d, size=2)] *= 6.0
        _, xf = bf16_bits(x)
        c, s, _ = oracle.quant_heads(xf, bits)
        s32 = s.astype(np.float32)
        out.append((c.reshape(B, Hkv, Tmax, d), s32.reshape(B, Hkv, Tmax),
                    torch.from_numpy(pack_heads(c, bits).reshape(B, Hkv, Tmax, -1)).cuda(),
                    torch.from_numpy(s32.reshape(B, Hkv, Tmax)).cuda()))
    return out


def check_attention(got, ref, vc, vs, bits, Hq, Hkv, lens, tol=ATTN_TOL):
    Z = 1 << (bits - 1)
    g = Hq // Hkv
    for b in range(got.shape[0]):
        for h in range(Hq):
            L = min(max(int(lens[b]), 0), vc.shape[2])
            if L == 0:
                assert np.all(got[b, h] == 0.0)
                continue
            vh = (vc[b, h // g, :L].astype(np.float64) - Z) * vs[b, h // g, :L, None]
            bound = tol * np.max(np.abs(vh))
            err = np.max(np.abs(got[b, h] - ref[b, h]))
            assert err <= bound, (b, h, err, bound)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("d", [64, 128, 256])
def test_attention_decode_matches_oracle(bits, d):
    rng = np.random.default_rng(bits * 7 + d)
    B, Hq, Hkv = 4, 4, 2
    Tmax = {64: 2100, 128: 1100, 256: 600}[d]                # several chunks and a ragged tail
    (kc, ks, kcd, ksd), (vc, vs, vcd, vsd) = make_cache(rng, B, Hkv, Tmax, d, bits)
    qb, qf = bf16_bits(rng.normal(size=(B, Hq, d)) * 2.0)
    lens = np.array([Tmax, 1, Tmax // 2 + 5, 0], np.int32)
    for qbits in (8, 4, 3):
        ref = oracle.attention_decode(qf, qbits, kc, ks, vc, vs, bits, lens)
        got = host(hbl.attention_decode(to_dev_bf16(qb), qbits, kcd, ksd, vcd, vsd, bits,
                                        torch.from_numpy(lens).cuda()))
        check_attention(got, ref, vc, vs, bits, Hq, Hkv, lens)


def test_attention_decode_bf16_out_and_length_clamps():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, d, Tmax, bits = 3, 2, 2, 128, 700, 3
    (kc, ks, kcd, ksd), (vc, vs, vcd, vsd) = make_cache(rng, B, Hkv, Tmax, d, bits)
    qb, qf = bf16_bits(rng.normal(size=(B, Hq, d)))
    lens = np.array([10 ** 6, -5, 513], np.int32)            # clamped to Tmax and 0
    ref = oracle.attention_decode(qf, 8, kc, ks, vc, vs, bits, np.clip(lens, 0, Tmax))
    out = hbl.attention_decode(to_dev_bf16(qb), 8, kcd, ksd, vcd, vsd, bits, torch.from_numpy(lens).cuda(),
                               out_dtype=torch.bfloat16)
    got = host(out.float())
    check_attention(got, ref, vc, vs, bits, Hq, Hkv, np.clip(lens, 0, Tmax), tol=ATTN_TOL + 2.0 ** -8)


def test_attention_decode_full_size_sampled():
    """The 7B-like decode workload (16 sequences, 32 heads, 4096 cached tokens,
    head size 128, 3-bit cache) in the benchmark's launch configuration;
    sampled heads against the oracle."""
    rng = np.random.default_rng(99)
    B, H, d, T, bits = 16, 32, 128, 4096, 3
    rb = d * bits // 8
    # random valid 3-bit codes and scales (the oracle takes the same cache)
    Z = 4
    codes_k = rng.integers(Z - 3, Z + 4, size=(B, H, T, d)).astype(np.uint8)
    codes_v = rng.integers(Z - 3, Z + 4, size=(B, H, T, d)).astype(np.uint8)
    ks = rng.uniform(0.02, 0.3, size=(B, H, T)).astype(np.float32)
    vs = rng.uniform(0.02, 0.3, size=(B, H, T)).astype(np.float32)
    kcd = torch.from_numpy(pack_heads(codes_k.reshape(-1, d), bits).reshape(B, H, T, rb)).cuda()
    vcd = torch.from_numpy(pack_heads(codes_v.reshape(-1, d), bits).reshape(B, H, T, rb)).cuda()
    qb, qf = bf16_bits(rng.normal(size=(B, H, d)) * 3.0)
    lens = np.full(B, T, np.int32)
    got = host(hbl.attention_decode(to_dev_bf16(qb), 8, kcd, torch.from_numpy(ks).cuda(), vcd,
                                    torch.from_numpy(vs).cuda(), bits, torch.from_numpy(lens).cuda()))
    for (b, h) in [(0, 0), (5, 17), (15, 31), (9, 3)]:
        ref = oracle.attention_decode(qf[b:b + 1, h:h + 1], 8, codes_k[b:b + 1, h:h + 1], ks[b:b + 1, h:h + 1],
                                      codes_v[b:b + 1, h:h + 1], vs[b:b + 1, h:h + 1], bits, lens[b:b + 1])
        check_attention(got[b:b + 1, h:h + 1], ref, codes_v[b:b + 1, h:h + 1], vs[b:b + 1, h:h + 1], bits, 1, 1,
                        lens[b:b + 1])


@pytest.mark.parametrize("d,Tmax,B,Hq,Hkv", [(64, 1, 1, 1, 1), (128, 5, 2, 2, 1), (256, 3, 1, 4, 4),
                                             (128, 3000, 1, 2, 2)])
def test_attention_decode_edge_shapes(d, Tmax, B, Hq, Hkv):
    # one-token and few-token caches (one workgroup per head, short context),
    # a single head split over many chunks (merge kernel), grouped heads
    rng = np.random.default_rng(d + Tmax)
    bits = 3
    (kc, ks, kcd, ksd), (vc, vs, vcd, vsd) = make_cache(rng, B, Hkv, Tmax, d, bits)
    qb, qf = bf16_bits(rng.normal(size=(B, Hq, d)))
    lens = np.full(B, Tmax, np.int32)
    lens[-1] = max(Tmax - 1, 0)
    ref = oracle.attention_decode(qf, 8, kc, ks, vc, vs, bits, lens)
    got = host(hbl.attention_decode(to_dev_bf16(qb), 8, kcd, ksd, vcd, vsd, bits, torch.from_numpy(lens).cuda()))
    check_attention(got, ref, vc, vs, bits, Hq, Hkv, lens)


def test_attention_decode_single_workgroup_per_head_short_context():
    # 512 heads (no split, the kernel writes the output itself) with ragged
    # lengths shorter than one block, including zero
    rng = np.random.default_rng(77)
    B, Hq, Hkv, d, Tmax, bits = 16, 32, 32, 128, 40, 4
    (kc, ks, kcd, ksd), (vc, vs, vcd, vsd) = make_cache(rng, B, Hkv, Tmax, d, bits)
    qb, qf = bf16_bits(rng.normal(size=(B, Hq, d)))
    lens = rng.integers(0, Tmax + 1, size=B).astype(np.int32)
    lens[0] = 0
    lens[1] = Tmax
    ref = oracle.attention_decode(qf, 8, kc, ks, vc, vs, bits, lens)
    got = host(hbl.attention_decode(to_dev_bf16(qb), 8, kcd, ksd, vcd, vsd, bits, torch.from_numpy(lens).cuda()))
    check_attention(got, ref, vc, vs, bits, Hq, Hkv, lens)


def test_quantize_heads_empty_and_single_row():
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    codes, scale = hbl.quantize_heads(x, 3)
    assert codes.shape == (0, 48) and scale.shape == (0,)
    xb, xf = bf16_bits(np.linspace(-2, 2, 64, dtype=np.float32)[None])
    codes, scale = hbl.quantize_heads(to_dev_bf16(xb), 2)
    c_or, s_or, _ = oracle.quant_heads(xf, 2)
    assert np.array_equal(unpack_heads(host(codes), 2, 64), c_or)
    assert host(scale)[0] == np.float32(s_or[0])


# ----------------------------------------------------------------- prefill
# Bar: |out - ref| <= (2^-8 + 3e-5) * max|v^| per (token, head): the scores
# are exact integers scaled in fp32 (as in the decode step); the value
# product rounds P * sv to bf16 (relative 2^-9), so the output moves by at
# most 2^-9 of the largest value it averages.  The kernel multiplies those
# weights with 128 + u (exact in bf16) and removes 128 + Z times their sum
# at the end; that cancellation costs fp32 accumulation error only, orders
# of magnitude below the bar.
PF_TOL = 2.0 ** -8 + ATTN_TOL


def check_prefill(got, ref, vc, vs, bits, Hq, Hkv, start, tol=PF_TOL):
    Z = 1 << (bits - 1)
    g = Hq // Hkv
    B, Tn = got.shape[:2]
    for b in range(B):
        for i in range(Tn):
            L = start[b] + i + 1
            for h in range(Hq):
                vh = (vc[b, h // g, :L].astype(np.float64) - Z) * vs[b, h // g, :L, None]
                bound = tol * np.max(np.abs(vh))
                err = np.max(np.abs(got[b, i, h] - ref[b, i, h]))
                assert err <= bound, (b, i, h, err, bound)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("d", [64, 128, 256])
def test_attention_prefill_matches_oracle(bits, d):
    rng = np.random.default_rng(bits * 31 + d)
    B, Hq, Hkv = 2, 4, 2
    Tn = {64: 150, 128: 97, 256: 70}[d]          # ragged query blocks
    start = np.array([0, 37], np.int32)
    Tmax = Tn + 40
    (kc, ks, kcd, ksd), (vc, vs, vcd, vsd) = make_cache(rng, B, Hkv, Tmax, d, bits)
    qb, qf = bf16_bits(rng.normal(size=(B, Tn, Hq, d)) * 2.0)
    ref = oracle.attention_prefill(qf, 8, kc, ks, vc, vs, bits, start)
    got = host(hbl.attention_prefill(to_dev_bf16(qb), 8, kcd, ksd, vcd, vsd, bits, torch.from_numpy(start).cuda()))
    check_prefill(got, ref, vc, vs, bits, Hq, Hkv, start)


def test_attention_prefill_from_appended_cache_and_qbits():
    # keys and values appended by the library, the oracle fed the same codes
    rng = np.random.default_rng(5)
    B, Tn, Hq, Hkv, d, Tmax, bits = 2, 80, 2, 2, 128, 96, 3
    kb, kf = bf16_bits(rng.normal(size=(B, Tn, Hkv, d)))
    vb, vf = bf16_bits(rng.normal(size=(B, Tn, Hkv, d)))
    cache = hbl.KVCache(B, Hkv, Tmax, d, bits)
    start = np.array([0, 10], np.int32)
    sd = torch.from_numpy(start).cuda()
    cache.append(to_dev_bf16(kb), to_dev_bf16(vb), sd)
    kc = np.zeros((B, Hkv, Tmax, d), np.uint8); vc = np.zeros_like(kc)
    ks = np.zeros((B, Hkv, Tmax), np.float32); vs = np.zeros_like(ks)
    for b in range(B):
        for h in range(Hkv):
            c, s_, _ = oracle.quant_heads(kf[b, :, h], bits)
            kc[b, h, start[b]:start[b] + Tn] = c; ks[b, h, start[b]:start[b] + Tn] = s_
            c, s_, _ = oracle.quant_heads(vf[b, :, h], bits)
            vc[b, h, start[b]:start[b] + Tn] = c; vs[b, h, start[b]:start[b] + Tn] = s_
    # rows before start[1] of sequence 1 were never written: give both sides the same (zero) rows
    qb, qf = bf16_bits(rng.normal(size=(B, Tn, Hq, d)))
    for qbits in (8, 4):
        ref = oracle.attention_prefill(qf, qbits, kc, ks, vc, vs, bits, start)
        got = host(hbl.attention_prefill(to_dev_bf16(qb), qbits, cache.k_codes, cache.k_scale, cache.v_codes,
                                         cache.v_scale, bits, sd))
        check_prefill(got, ref, vc, vs, bits, Hq, Hkv, start)


def test_attention_prefill_full_size_sampled():
    """A 7B-shaped prefill (4 sequences x 2048 new tokens, 32 heads of 128,
    3-bit cache): sampled (token, head) pairs against the oracle's decode
    step at each token's position."""
    rng = np.random.default_rng(123)
    B, Tn, H, d, bits = 4, 2048, 32, 128, 3
    Tmax = Tn
    Z = 4
    rb = d * bits // 8
    codes_k = rng.integers(Z - 3, Z + 4, size=(B, H, Tmax, d)).astype(np.uint8)
    codes_v = rng.integers(Z - 3, Z + 4, size=(B, H, Tmax, d)).astype(np.uint8)
    ks = rng.uniform(0.02, 0.3, size=(B, H, Tmax)).astype(np.float32)
    vs = rng.uniform(0.02, 0.3, size=(B, H, Tmax)).astype(np.float32)
    kcd = torch.from_numpy(pack_heads(codes_k.reshape(-1, d), bits).reshape(B, H, Tmax, rb)).cuda()
    vcd = torch.from_numpy(pack_heads(codes_v.reshape(-1, d), bits).reshape(B, H, Tmax, rb)).cuda()
    qb, qf = bf16_bits(rng.normal(size=(B, Tn, H, d)) * 3.0)
    start = np.zeros(B, np.int32)
    got = host(hbl.attention_prefill(to_dev_bf16(qb), 8, kcd, torch.from_numpy(ks).cuda(), vcd,
                                     torch.from_numpy(vs).cuda(), bits, torch.from_numpy(start).cuda()))
    for (b, i, h) in [(0, 0, 0), (1, 63, 5), (2, 64, 17), (3, 2047, 31), (0, 1000, 9), (2, 1535, 22)]:
        ref = oracle.attention_decode(qf[b:b + 1, i], 8, codes_k[b:b + 1], ks[b:b + 1], codes_v[b:b + 1],
                                      vs[b:b + 1], bits, np.array([i + 1], np.int32))
        vh = (codes_v[b, h, :i + 1].astype(np.float64) - Z) * vs[b, h, :i + 1, None]
        err = np.max(np.abs(got[b, i, h] - ref[0, h]))
        assert err <= PF_TOL * np.max(np.abs(vh)), (b, i, h, err)


@pytest.mark.parametrize("bits", [3, 8])
def test_attention_prefill_rising_scores(bits):
    """Key scales growing by 10^3 over the prompt make each key block's
    largest score exceed the running maximum by far more than 2^8, so the
    kernel's lazily raised maximum is raised (and the accumulators rescaled)
    in the middle of the prompt, not only at its first block."""
    rng = np.random.default_rng(77 + bits)
    B, Hq, Hkv, d, Tn = 1, 2, 2, 128, 300
    Z = 1 << (bits - 1)
    qb_ = (1 << (bits - 1)) - 1
    kc = rng.integers(Z - qb_, Z + qb_ + 1, size=(B, Hkv, Tn, d)).astype(np.uint8)
    vc = rng.integers(Z - qb_, Z + qb_ + 1, size=(B, Hkv, Tn, d)).astype(np.uint8)
    ks = (0.01 * 10.0 ** (3.0 * np.arange(Tn) / Tn)).astype(np.float32)[None, None].repeat(Hkv, 1)
    vs = rng.uniform(0.05, 0.2, size=(B, Hkv, Tn)).astype(np.float32)
    qb, qf = bf16_bits(rng.normal(size=(B, Tn, Hq, d)) * 3.0)
    start = np.zeros(B, np.int32)
    # the premise: block maxima of the scores (log2 units) rise by more than 8 between blocks
    kh = (kc[0, 0].astype(np.float64) - Z) * ks[0, 0, :, None]
    sc = (qf[0, -1, 0].astype(np.float64) @ kh.T) / np.sqrt(d) * np.log2(np.e)
    bm = [sc[t:t + 64].max() for t in range(0, Tn, 64)]
    assert max(np.diff(bm)) > 8.0
    dev = lambda c: torch.from_numpy(pack_heads(c.reshape(-1, d), bits).reshape(B, Hkv, Tn, -1)).cuda()
    ref = oracle.attention_prefill(qf, 8, kc, ks, vc, vs, bits, start)
    got = host(hbl.attention_prefill(to_dev_bf16(qb), 8, dev(kc), torch.from_numpy(ks).cuda(), dev(vc),
                                     torch.from_numpy(vs).cuda(), bits, torch.from_numpy(start).cuda()))
    check_prefill(got, ref, vc, vs, bits, Hq, Hkv, start)


def test_attention_prefill_empty_and_single_token():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, Tmax, bits = 2, 4, 4, 64, 20, 4
    (kc, ks, kcd, ksd), (vc, vs, vcd, vsd) = make_cache(rng, B, Hkv, Tmax, d, bits)
    # no new tokens: nothing is launched, the output is empty
    q0 = torch.empty((B, 0, Hq, d), dtype=torch.bfloat16, device="cuda")
    st = torch.tensor([3, 7], dtype=torch.int32, device="cuda")
    got0 = hbl.attention_prefill(q0, 8, kcd, ksd, vcd, vsd, bits, st)
    assert tuple(got0.shape) == (B, 0, Hq, d)
    # one new token at positions 3 and 19 (the last cache row)
    start = np.array([3, 19], np.int32)
    qb, qf = bf16_bits(rng.normal(size=(B, 1, Hq, d)))
    ref = oracle.attention_prefill(qf, 8, kc, ks, vc, vs, bits, start)
    got = host(hbl.attention_prefill(to_dev_bf16(qb), 8, kcd, ksd, vcd, vsd, bits, torch.from_numpy(start).cuda()))
    check_prefill(got, ref, vc, vs, bits, Hq, Hkv, start)


def test_attention_prefill_positions_clamped():
    """start[b] is clamped to [0, Tmax] and a query at a position past the
    cache sees all Tmax keys: each query against the oracle's decode step at
    the clamped length (the oracle's prefill itself rejects such starts)."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, d, Tmax, Tn, bits = 3, 2, 1, 128, 100, 40, 3
    (kc, ks, kcd, ksd), (vc, vs, vcd, vsd) = make_cache(rng, B, Hkv, Tmax, d, bits)
    start = np.array([80, 150, -5], np.int32)
    qb, qf = bf16_bits(rng.normal(size=(B, Tn, Hq, d)))
    got = host(hbl.attention_prefill(to_dev_bf16(qb), 8, kcd, ksd, vcd, vsd, bits, torch.from_numpy(start).cuda()))
    Z = 1 << (bits - 1)
    for b in range(B):
        s0 = min(max(int(start[b]), 0), Tmax)
        for i in range(Tn):
            L = min(s0 + i + 1, Tmax)
            ref = oracle.attention_decode(qf[b:b + 1, i], 8, kc[b:b + 1], ks[b:b + 1], vc[b:b + 1], vs[b:b + 1],
                                          bits, np.array([L], np.int32))
            for h in range(Hq):
                vh = (vc[b, h // (Hq // Hkv), :L].astype(np.float64) - Z) * vs[b, h // (Hq // Hkv), :L, None]
                err = np.max(np.abs(got[b, i, h] - ref[0, h]))
                assert err <= PF_TOL * np.max(np.abs(vh)), (b, i, h, err)
