"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bars:
  * alpha within one fp32 ulp of the oracle's; ternary codes equal except
    where the oracle's |w|/a lies within 1e-6 of the tie 0.5;
  * rotated activations: relative L2 <= 1e-5 per token;
  * activation codes: equal except +-1 at rounding ties of the oracle's
    pre-rounding value (|pre - tie| < 1e-4), in at most 1e-4 of the codes;
    per-token scales within 1e-5 relative;
  * integer matmul: bit-exact int32 on identical codes;
  * outputs: relative L2 <= 2e-3 against the oracle rounded to the output
    dtype, pooled and per token (check_layer: a token's bar grows only by the
    effect of the code flips its oracle near-ties allow).
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_ternary_amd as hbl
import oracle
import synthetic
from layouts import pack_int4, pack_int4_fp6, pack_ternary, unpack_int4, unpack_int4_fp6, unpack_ternary

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a gfx950 device"
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    hbl.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_to_dev(x_f32, x_bits):
    if x_bits is None:
        return dev(x_f32)
    return dev(x_bits.view(np.int16)).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rel_l2(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def check_codes(q_gpu, q_or, pre_or, max_frac=1e-4, tie_tol=1e-4, ties_bound=False):
    """ties_bound: bound the mismatches by the number of the oracle's
    pre-rounding values within tie_tol of a tie (unrotated bf16 inputs land on
    exact ties often: x_k * 127 / max_k |x_k| with 8-bit mantissas)."""
    q_gpu = q_gpu.astype(np.int32); q_or = q_or.astype(np.int32)
    diff = q_gpu != q_or
    n = int(diff.sum())
    if n:
        assert np.all(np.abs(q_gpu[diff] - q_or[diff]) == 1), "code differs by more than 1"
        tie = (q_gpu[diff] + q_or[diff]) / 2.0
        assert np.all(np.abs(pre_or[diff] - tie) < tie_tol), "code differs away from a rounding tie"
    if ties_bound:
        near = int((np.abs(pre_or - np.floor(pre_or) - 0.5) < tie_tol).sum())
        assert n <= max(1, near), f"{n} code mismatches, {near} near-ties"
    else:
        assert n <= max(1, max_frac * q_or.size), f"{n} code mismatches of {q_or.size}"
    return n


def gpu_codes_unpacked(codes, bits, K):
    c = host(codes)
    if bits == 6:
        return unpack_int4_fp6(c, K)
    return c.astype(np.int8) if bits == 8 else unpack_int4(c, K)


def pack_codes(q, bits):
    """Oracle codes int8 [M][K] -> the device format `bits` (8, 4 or 6)."""
    return {8: lambda: q, 4: lambda: pack_int4(q), 6: lambda: pack_int4_fp6(q)}[bits]()


# ------------------------------------------------------------------ weights

@pytest.mark.parametrize("N,K", [(16, 64), (48, 128), (16, 256), (272, 2048), (4096, 4096), (3072, 8192), (4096, 16384),
                                 (272, 32768)])
def test_weight_ternarisation(N, K):
    """alpha within one fp32 ulp of the oracle's (the GPU sums |W| in fp64 in
    another order; both are far more precise than fp32); codes exactly the
    threshold rule |w| > a/2 evaluated on the host with the GPU's own alpha,
    and equal to the oracle's except where the oracle's |w|/a lies within
    1e-6 of the tie 0.5 (only there can a one-ulp alpha move a code)."""
    rng = np.random.default_rng(N + K)
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    wt, alpha = oracle.quantize_weights(w)
    wp, a = hbl.quantize_weights(dev(w))
    ag = host(a)[0]
    assert abs(float(ag) - float(alpha)) <= float(np.spacing(np.float32(alpha))), (ag, alpha)
    wp_h = host(wp)
    wt_gpu = unpack_ternary(wp_h, K)
    a_gpu = max(float(ag), float(np.float32(1e-5)))
    rule = np.where(np.abs(w.astype(np.float64)) > np.float32(0.5 * np.float32(a_gpu)), np.sign(w), 0).astype(np.int8)
    np.testing.assert_array_equal(wt_gpu, rule)
    check_ternary_near_ties(wt_gpu, wt, w.astype(np.float64) / oracle.weight_scale(alpha), tie_tol=1e-6)
    np.testing.assert_array_equal(wp_h, pack_ternary(wt_gpu))
    np.testing.assert_array_equal(host(hbl.unpack_weights(wp, K)), wt_gpu)


def test_weight_ternarisation_ties_and_zero():
    # alpha = 1 exactly; +-0.5 are ties that must round to 0
    w = np.tile(np.array([2.0, 0.5, -0.5, 1.0], np.float32), (16, 64))
    wt, alpha = oracle.quantize_weights(w)
    wp, a = hbl.quantize_weights(dev(w))
    assert host(a)[0] == alpha == 1.0
    np.testing.assert_array_equal(unpack_ternary(host(wp), 256), wt)
    wz = np.zeros((16, 256), np.float32)
    wp, a = hbl.quantize_weights(dev(wz))
    assert host(a)[0] == 0.0 and not host(wp).any()


# ------------------------------------------------------------------ rotation and quantisation

KS = [64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768]


def make_x(M, K, seed, dist="laplace", bf16=True):
    w = synthetic.Workload("t", M, K, 16, 4, "bf16" if bf16 else "f32", dist, 0.05 if dist == "laplace" else 1.0,
                           max(1, K // 200), 100.0, seed)
    x, xb, _ = synthetic.make_inputs(w, with_weights=False)
    return x, xb


@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("M", [1, 3, 70])
def test_rotation_matches_oracle(K, M):
    x, xb = make_x(M, K, K + M)
    for gain in (None, synthetic.make_gain(K, K)):
        xt = host(hbl.rmsnorm_fwht(x_to_dev(x, xb), None if gain is None else dev(gain)))
        ref = oracle.hadamard_rotate(oracle.rmsnorm(x, gain))
        for m in range(M):
            assert rel_l2(xt[m], ref[m]) <= 1e-5, (m, rel_l2(xt[m], ref[m]))


@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("bits", [8, 4, 6])
@pytest.mark.parametrize("M", [1, 5, 64, 129])
def test_codes_match_oracle(K, bits, M):
    if bits == 6 and K < 256:
        pytest.skip("format 6 needs K >= 256")
    x, xb = make_x(M, K, 7 * K + M, dist="normal" if K % 3 else "laplace", bf16=(M != 5))
    codes, d = hbl.quantize_act(x_to_dev(x, xb), bits)
    q = gpu_codes_unpacked(codes, bits, K)
    xt = oracle.hadamard_rotate(oracle.rmsnorm(x))
    q_or, d_or, pre = oracle.quant_act(xt, 8 if bits == 8 else 4)
    check_codes(q, q_or, pre)
    np.testing.assert_allclose(host(d), d_or, rtol=1e-5)


@pytest.mark.parametrize("K,M,bf16", [(16384, 1100, True), (16384, 1100, False), (8192, 2100, True),
                                      (4096, 3200, True), (2048, 6200, True)])
@pytest.mark.parametrize("bits", [8, 4, 6])
def test_codes_with_gain_over_persistent_iterations(K, M, bf16, bits):
    """RMSNorm gain at prefill token counts: enough tokens that every
    workgroup of the persistent grid walks two or more of them (gain loads
    and the next token's prefetch in flight together).  Evenly spaced
    sampled rows against the oracle."""
    x, xb = make_x(M, K, 11 * K + M + bits, bf16=bf16)
    g = synthetic.make_gain(K, K + 1)
    codes, d = hbl.quantize_act(x_to_dev(x, xb), bits, gain=dev(g))
    rows = synthetic.sample_rows(M, 24)
    c = host(codes)
    if bits == 6:   # [K/128][M][96]: the sampled rows of every 128-k block
        q = unpack_int4_fp6(np.ascontiguousarray(c.reshape(K // 128, M, 96)[:, rows]), K)
    else:
        q = c[rows].astype(np.int8) if bits == 8 else unpack_int4(c[rows], K)
    xt = oracle.hadamard_rotate(oracle.rmsnorm(x[rows], g))
    q_or, d_or, pre = oracle.quant_act(xt, 8 if bits == 8 else 4)
    check_codes(q, q_or, pre)
    np.testing.assert_allclose(host(d)[rows], d_or, rtol=1e-5)


@pytest.mark.parametrize("K", [64, 256, 4096, 16384, 32768])
@pytest.mark.parametrize("bits", [8, 4, 6])
@pytest.mark.parametrize("M", [1, 5, 129])
def test_quantize_rotated_matches_oracle(K, bits, M):
    """The quantiser alone, on rotated fp32 activations: the oracle's
    quantiser applied to the same fp32 values."""
    if bits == 6 and K < 256:
        pytest.skip("format 6 needs K >= 256")
    x, _ = make_x(M, K, 5 * K + M + bits, dist="laplace" if K % 3 else "normal", bf16=False)
    xt = oracle.hadamard_rotate(oracle.rmsnorm(x)).astype(np.float32)
    codes, d = hbl.quantize_rotated(dev(xt), bits)
    q = gpu_codes_unpacked(codes, bits, K)
    q_or, d_or, pre = oracle.quant_act(xt.astype(np.float64), 8 if bits == 8 else 4)
    check_codes(q, q_or, pre)
    np.testing.assert_allclose(host(d), d_or, rtol=1e-5)


@pytest.mark.parametrize("bits", [8, 4, 6])
def test_stages_rotation_then_quantiser(bits):
    """rmsnorm_fwht then quantize_rotated, at a token count where the
    persistent grid walks several tokens per workgroup: codes against the
    oracle's quantiser of the oracle's rotation (and equal to the fused
    stage's except at rounding ties), then the matmul of those codes."""
    M, K, N = 1100, 16384, 272
    x, xb = make_x(M, K, 13 + bits)
    xt = hbl.rmsnorm_fwht(x_to_dev(x, xb))
    codes, d = hbl.quantize_rotated(xt, bits)
    codes_f, d_f = hbl.quantize_act(x_to_dev(x, xb), bits)
    rows = synthetic.sample_rows(M, 24)
    c, cf = host(codes), host(codes_f)
    if bits == 6:
        pick = lambda a: unpack_int4_fp6(np.ascontiguousarray(a.reshape(K // 128, M, 96)[:, rows]), K)
    else:
        pick = lambda a: a[rows].astype(np.int8) if bits == 8 else unpack_int4(a[rows], K)
    q, qf = pick(c), pick(cf)
    xt_or = oracle.hadamard_rotate(oracle.rmsnorm(x[rows]))
    q_or, d_or, pre = oracle.quant_act(xt_or, 8 if bits == 8 else 4)
    check_codes(q, q_or, pre)
    check_codes(qf, q_or, pre)
    np.testing.assert_allclose(host(d)[rows], d_or, rtol=1e-5)
    np.testing.assert_allclose(host(d), host(d_f), rtol=1e-5)
    # the matmul takes these codes like the fused stage's
    wl = synthetic.make_inputs(gaussian_workload(1, K, N, 4, 99 + bits))[2]
    wt, alpha = oracle.quantize_weights(wl)
    wp, wa = oracle_weights_dev(wt, alpha)
    acc = host(hbl.gemm_ternary(codes, bits, wp, K))
    np.testing.assert_array_equal(acc[rows], oracle.gemm_ternary(q, wt))


def test_zero_token_and_tiny_token():
    K = 1024
    x = np.zeros((3, K), np.float32)
    x[1, 5] = 1e-30
    x[2] = 1e-3
    for bits in (8, 4):
        codes, d = hbl.quantize_act(dev(x), bits)
        q = gpu_codes_unpacked(codes, bits, K)
        q_or, d_or, pre = oracle.quant_act(oracle.hadamard_rotate(oracle.rmsnorm(x)), bits)
        np.testing.assert_array_equal(q[0], 0)
        check_codes(q, q_or, pre)
        np.testing.assert_allclose(host(d), d_or, rtol=1e-5)


# ------------------------------------------------------------------ integer matmul

@pytest.mark.parametrize("bits", [8, 4, 6])
@pytest.mark.parametrize("M,K,N", [(1, 256, 16), (5, 256, 48), (17, 256, 272), (64, 256, 4096),
                                   (2, 1024, 48), (4, 16384, 272), (3, 8192, 4096),
                                   (7, 512, 272), (16, 2048, 512), (20, 4096, 272), (32, 16384, 528), (33, 4096, 64),
                                   (64, 16384, 128), (65, 256, 256), (300, 1024, 272), (512, 2048, 512),
                                   (257, 16384, 528),
                                   # short rows (one matmul kernel for every M) and the longest rows
                                   (1, 64, 16), (5, 64, 48), (64, 64, 272), (65, 64, 80), (300, 64, 272),
                                   (3, 128, 16), (70, 128, 528), (129, 128, 64),
                                   (1, 32768, 272), (3, 32768, 64), (20, 32768, 272), (40, 32768, 528),
                                   (300, 32768, 256), (200, 2048, 144), (4096, 256, 4096)])
def test_matmul_bit_exact(bits, M, K, N):
    if bits == 6 and K < 256:
        pytest.skip("format 6 needs K >= 256")
    rng = np.random.default_rng(M * 7 + K + N + bits)
    lo, hi = (-128, 128) if bits == 8 else (-8, 8)
    q = rng.integers(lo, hi, (M, K)).astype(np.int8)
    q[0, :] = lo                      # extreme magnitudes
    wt = rng.integers(-1, 2, (N, K)).astype(np.int8)
    wt[0, :] = -1
    acc_or = oracle.gemm_ternary(q, wt)
    acc = host(hbl.gemm_ternary(dev(pack_codes(q, bits)), bits, dev(pack_ternary(wt)), K))
    np.testing.assert_array_equal(acc, acc_or)


@pytest.mark.parametrize("M,K,N", [(4059, 512, 3056), (4096, 256, 3072), (8192, 1024, 3072)])
def test_fp6_wide_tile_bit_exact(M, K, N):
    """Format 6 codes on the 256 x 192 tile of the fp6 x fp4 matmul (chosen
    for these N): int32 accumulators equal the oracle's on sampled rows --
    the first and last tile rows (ragged at M = 4059), every column (ragged
    last tile at N = 3056) -- with extreme codes in the first row."""
    rng = np.random.default_rng(M + 3 * K + N)
    q = rng.integers(-8, 8, (M, K)).astype(np.int8)
    q[0, :] = -8
    q[M - 1, :] = 7
    wt = rng.integers(-1, 2, (N, K)).astype(np.int8)
    wt[N - 1, :] = -1
    acc = host(hbl.gemm_ternary(dev(pack_codes(q, 6)), 6, dev(pack_ternary(wt)), K))
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(M - 300, M), synthetic.sample_rows(M, 32)]))
    np.testing.assert_array_equal(acc[rows], oracle.gemm_ternary(np.ascontiguousarray(q[rows]), wt))


# ------------------------------------------------------------------ whole layer

def oracle_weights_dev(wt, alpha):
    """The oracle's ternary weights, packed on the host, and its alpha, on the
    device (the GPU's own ternarisation is checked against the oracle above;
    the layer tests run on the oracle's weights so the two sides multiply by
    the same codes and scale)."""
    return dev(pack_ternary(wt)), dev(np.array([alpha, 0, 0, 0], np.float32))[:1]


def run_layer(w: synthetic.Workload, M=None, gain=None, sample=None):
    x, xb, wl = synthetic.make_inputs(w, M=M)
    wt, alpha = oracle.quantize_weights(wl)
    wp, a = oracle_weights_dev(wt, alpha)
    xd = x_to_dev(x, xb)
    gd = None if gain is None else dev(gain)
    y = hbl.forward(xd, wp, a, w.bits, gain=gd)
    rows = np.arange(x.shape[0]) if sample is None else sample
    ref = oracle.forward(x[rows], wt, alpha, w.bits, g=gain)
    yh = host(y.float())[rows]
    y_ref = ref["y"] if y.dtype == torch.float32 else oracle.to_bf16_rne(ref["y"])
    ref["alpha"] = alpha
    return yh, y_ref, ref, xd, wp, a, rows


def check_layer(yh, y_ref, ref, tol=2e-3, tie_tol=1e-4):
    """Output bar, pooled and per token.  Pooled: relative L2 <= tol.  Per
    token m: ||y_m - ref_m|| <= tol ||ref_m|| + T_m d_m a sqrt(N), where T_m
    counts the oracle's pre-rounding values of token m within tie_tol of a
    rounding tie (the only codes the code bar lets differ, by one) and
    d_m a sqrt(N) bounds the output change of one such flip (it moves each of
    the N accumulators by at most 1).  T_m and the allowance come from the
    oracle alone; a token with no near-tie gets the plain bar."""
    assert rel_l2(yh, y_ref) <= tol, rel_l2(yh, y_ref)
    pre = ref["pre"]
    near = (np.abs(pre - np.floor(pre) - 0.5) < tie_tol).sum(axis=1)
    a = oracle.weight_scale(ref["alpha"])
    N = y_ref.shape[1]
    err = np.linalg.norm(np.asarray(yh, np.float64) - np.asarray(y_ref, np.float64), axis=1)
    nrm = np.linalg.norm(np.asarray(y_ref, np.float64), axis=1)
    bar = tol * np.where(nrm > 0, nrm, 1.0) + near * ref["d"] * a * np.sqrt(N)
    bad = np.nonzero(err > bar)[0]
    assert bad.size == 0, [(int(m), float(err[m] / max(nrm[m], 1e-300)), int(near[m])) for m in bad[:8]]


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N", [(8, 256, 256), (1, 16384, 4096), (17, 4096, 272), (32, 16384, 4096), (64, 8192, 512),
                                   (300, 2048, 272), (513, 16384, 256),
                                   (8, 64, 256), (100, 64, 48), (3, 128, 272), (300, 128, 272),
                                   (1, 32768, 272), (40, 32768, 272), (300, 32768, 256)])
def test_layer_small(bits, M, K, N):
    w = synthetic.Workload("t", M, K, N, bits, "bf16", "laplace", 0.05, max(1, K // 200), 100.0, M + K + N)
    yh, y_ref, ref, xd, wp, a, rows = run_layer(w)
    check_layer(yh, y_ref, ref)
    # stage view of the same call chain
    codes, d = hbl.quantize_act(xd, bits)
    check_codes(gpu_codes_unpacked(codes, bits, K), ref["q"], ref["pre"])
    np.testing.assert_allclose(host(d), ref["d"], rtol=1e-5)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N,xdt,gain", [(1, 64, 16, "bf16", False), (8, 256, 256, "f32", True),
                                            (33, 128, 272, "bf16", True), (64, 256, 4096, "bf16", False),
                                            (17, 64, 80, "f32", False), (64, 128, 48, "f32", True)])
def test_short_rows_one_launch(bits, M, K, N, xdt, gain):
    """K = 64, 128, 256 with up to 64 tokens: the whole layer is one kernel
    (every workgroup computes all tokens' codes, then its channels' outputs).
    Against the oracle at the layer bar, with and without the transform, and
    equal bit for bit to the no-alloc entry (same kernel)."""
    w = synthetic.Workload("t", M, K, N, bits, xdt, "laplace", 0.05, max(1, K // 64), 100.0, 3 * M + K + N + bits)
    g = synthetic.make_gain(K, M) if gain else None
    yh, y_ref, ref, xd, wp, a, rows = run_layer(w, gain=g)
    check_layer(yh, y_ref, ref)
    gd = None if g is None else dev(g)
    x, xb, wl = synthetic.make_inputs(w)
    wt, alpha = oracle.quantize_weights(wl)
    yu = hbl.forward(xd, wp, a, bits, gain=gd, rotate=False, out_dtype=torch.float32)
    refu = oracle.forward(x, wt, alpha, bits, g=g, rotate=False)
    refu["alpha"] = alpha
    check_layer(host(yu), refu["y"], refu)
    y = hbl.forward(xd, wp, a, bits, gain=gd)
    yn = hbl.forward_noalloc(xd, wp, a, bits, gain=gd)
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32),
                       yn.view(torch.int16) if yn.dtype == torch.bfloat16 else yn.view(torch.int32))


def test_layer_with_gain_fp32_out():
    w = synthetic.WORKLOADS["tiny_int8"]
    g = synthetic.make_gain(w.K, 3)
    yh, y_ref, ref, *_ = run_layer(w, gain=g)
    check_layer(yh, y_ref, ref)


WORKLOAD_SAMPLES = [("tiny_int8", None), ("wo_1p3b_int4", 48), ("wdown_3b_int4", 24), ("wo_7b_int8", 24),
                    ("wo_7b_int4", 24), ("wdown_7b_int8", 16), ("wdown_7b_int4", 16), ("decode_7b_m1", None),
                    ("decode_7b_m16", None), ("decode_7b_m64", None)]


@pytest.mark.parametrize("name,count", WORKLOAD_SAMPLES)
def test_layer_full_workloads(name, count):
    """Every workload at its full size; the oracle checks a deterministic token
    sample (evenly spaced rows plus first and last) of the GPU output."""
    w = synthetic.WORKLOADS[name]
    sample = None if count is None else synthetic.sample_rows(w.M, count)
    yh, y_ref, ref, xd, wp, a, rows = run_layer(w, sample=sample)
    check_layer(yh, y_ref, ref)
    # exact integer accumulators on the sampled rows, from the oracle's own codes
    q = ref["q"]
    for bits in ((8,) if w.bits == 8 else (4, 6)):
        acc = host(hbl.gemm_ternary(dev(pack_codes(q, bits)), bits, wp, w.K))
        np.testing.assert_array_equal(acc, ref["acc"])


# ------------------------------------------------------------------ variants beside H-BitLinear

def gaussian_workload(M, K, N, bits, seed, xdt="bf16"):
    """Inputs of the attention/FFN input projections: close to Gaussian."""
    return synthetic.Workload("g", M, K, N, bits, xdt, "normal", 1.0, 1, 1.0, seed)


@pytest.mark.parametrize("K", [64, 256, 2048, 16384, 32768])
@pytest.mark.parametrize("bits", [8, 4, 6])
@pytest.mark.parametrize("M", [1, 5, 129])
def test_unrotated_codes_match_oracle(K, bits, M):
    if bits == 6 and K < 256:
        pytest.skip("format 6 needs K >= 256")
    w = gaussian_workload(M, K, 16, 4, 3 * K + M + bits)
    x, xb, _ = synthetic.make_inputs(w, with_weights=False)
    codes, d = hbl.quantize_act(x_to_dev(x, xb), bits, rotate=False)
    q = gpu_codes_unpacked(codes, bits, K)
    ref = oracle.forward(x, np.zeros((16, K), np.int8), np.float32(1), 8 if bits == 8 else 4, rotate=False)
    check_codes(q, ref["q"], ref["pre"], ties_bound=True)
    np.testing.assert_allclose(host(d), ref["d"], rtol=1e-5)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N", [(1, 16384, 4096), (3, 8192, 272), (4, 8192, 48), (3, 16384, 272),
                                   (4, 16384, 96), (16, 4096, 512), (64, 2048, 256), (300, 4096, 528),
                                   (2048, 4096, 4096), (100, 64, 272), (5, 128, 48), (2, 32768, 272)])
def test_unrotated_layer(bits, M, K, N):
    """BitLinear without the transform (one-launch decode while M * K <= 49152,
    decode, int8 and fp6 prefill matmuls) against the oracle at the layer bar."""
    w = gaussian_workload(M, K, N, bits, M + K + N)
    x, xb, wl = synthetic.make_inputs(w)
    wt, alpha = oracle.quantize_weights(wl)
    wp, a = oracle_weights_dev(wt, alpha)
    xd = x_to_dev(x, xb)
    # fp32 output: without the transform, bf16 inputs put many quantiser inputs
    # on exact rounding ties, and a bf16 output would round those one-code
    # differences up to a full bf16 step
    y = hbl.forward(xd, wp, a, bits, rotate=False, out_dtype=torch.float32)
    rows = synthetic.sample_rows(M, 24) if M > 64 else np.arange(M)
    ref = oracle.forward(x[rows], wt, alpha, bits, rotate=False)
    ref["alpha"] = alpha
    check_layer(host(y)[rows], ref["y"], ref)


def check_ternary_near_ties(wt_gpu, wt_or, ratio_or, tie_tol=1e-5, max_frac=1e-4):
    """Codes equal except where the oracle's |w|/a sits within tie_tol of 0.5."""
    diff = wt_gpu != wt_or
    n = int(diff.sum())
    if n:
        assert np.all(np.abs(wt_gpu[diff].astype(int) - wt_or[diff].astype(int)) == 1)
        assert np.all(np.abs(np.abs(ratio_or[diff]) - 0.5) < tie_tol), "code differs away from the 0.5 threshold"
    assert n <= max(1, max_frac * wt_or.size), f"{n} of {wt_or.size}"


@pytest.mark.parametrize("N,K", [(16, 64), (16, 256), (272, 2048), (4096, 4096), (3072, 8192), (512, 16384),
                                 (64, 32768)])
def test_rotated_weights_match_oracle(N, K):
    rng = np.random.default_rng(N + K)
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    w[:, rng.choice(K, 3, replace=False)] *= 30          # a few large input channels
    wt_or, alpha_or, wr = oracle.quantize_weights_rotated(w)
    wp, a = hbl.quantize_weights(dev(w), rotate=True)
    alpha = host(a)[0]
    assert abs(alpha / alpha_or - 1) <= 1e-6, (alpha, alpha_or)
    check_ternary_near_ties(unpack_ternary(host(wp), K), wt_or, wr / oracle.weight_scale(alpha_or))


@pytest.mark.parametrize("bits", [8, 4])
def test_rotated_weights_layer(bits):
    """Weights and activations both rotated: the H-BitLinear forward with the
    rotated ternary weights, against the oracle's forward on its own rotated
    weights."""
    w = synthetic.WORKLOADS["wo_1p3b_int4"].with_(bits=bits, M=256)
    x, xb, wl = synthetic.make_inputs(w)
    wt, alpha, _ = oracle.quantize_weights_rotated(wl)
    wp, a = hbl.quantize_weights(dev(wl), rotate=True)
    y = hbl.forward(x_to_dev(x, xb), wp, a, bits)
    ref = oracle.forward(x, wt, alpha, bits)
    assert rel_l2(host(y.float()), oracle.to_bf16_rne(ref["y"])) <= 2e-3


# ------------------------------------------------------------------ invariants of the GPU path

@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N,xdt,gain", [(1, 16384, 4096, "bf16", False), (1, 16384, 48, "f32", True),
                                            (1, 8192, 48, "bf16", True), (2, 8192, 4096, "f32", True),
                                            (2, 8192, 272, "bf16", False), (2, 16384, 272, "bf16", True),
                                            (3, 8192, 4096, "f32", False), (4, 16384, 16, "f32", True),
                                            (4, 8192, 528, "bf16", False)])
def test_single_launch_decode(bits, M, K, N, xdt, gain):
    """A few tokens at K = 8192 / 16384: while M * K <= 16384 the forward is
    one kernel (transform, quantiser and matmul together), beyond that prep +
    matmul.  Against the oracle at the layer bar, and against the two-kernel
    stage path on the same inputs (the one-kernel transform's summation order
    differs, so codes may differ at rounding ties only)."""
    w = synthetic.Workload("t", M, K, N, bits, xdt, "laplace", 0.05, max(1, K // 200), 100.0, 5 * M + K + N)
    g = synthetic.make_gain(K, M) if gain else None
    yh, y_ref, ref, xd, wp, a, rows = run_layer(w, gain=g)
    check_layer(yh, y_ref, ref)
    gd = None if g is None else dev(g)
    codes, d = hbl.quantize_act(xd, bits, gain=gd)
    y2 = host(hbl.matmul_dequant(codes, bits, d, wp, a, K, out_dtype=xd.dtype).float())
    assert rel_l2(yh, y2) <= 1e-3, rel_l2(yh, y2)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N", [(17, 4096, 272), (33, 16384, 4096), (64, 16384, 4096), (64, 1024, 48),
                                   (40, 512, 96), (33, 32768, 272), (64, 32768, 4096)])
def test_split_k_decode_reduction_in_kernel(bits, M, K, N):
    """33..64 tokens at K = 32768: the forward's matmul splits K and the last
    workgroup of each channel tile sums the partials; the stage calls (row-
    major codes) split at every K and sum in a separate reduction kernel.  Up
    to K = 16384 the forward runs unsplit on its decode-blocked codes, and
    17..32 tokens run unsplit everywhere: those cases check the same way.
    Same codes, exact integer sums: equal bit for bit, with a workspace that
    starts full of 0xFF (the first kernel clears the arrival counters) and
    over repeated calls on it whose inputs alternate in sign, so partial
    sums left over from the call before would show."""
    w = synthetic.Workload("t", M, K, N, bits, "bf16", "laplace", 0.05, max(1, K // 200), 100.0, 9 * M + K + N)
    x, xb, wl = synthetic.make_inputs(w)
    wp, a = hbl.quantize_weights(dev(wl))
    xds = [x_to_dev(x, xb), -x_to_dev(x, xb)]
    y_refs = []
    for xd in xds:
        codes, d = hbl.quantize_act(xd, bits)
        y_refs.append(hbl.matmul_dequant(codes, bits, d, wp, a, K, out_dtype=torch.bfloat16))
    assert not torch.equal(y_refs[0], y_refs[1])
    op = hbl.OP_FORWARD_INT8 if bits == 8 else hbl.OP_FORWARD_INT4
    ws = torch.full((hbl.workspace_bytes(op, M, K, N),), 0xFF, dtype=torch.uint8, device="cuda")
    for i in range(6):
        y = hbl.forward(xds[i % 2], wp, a, bits, out_dtype=torch.bfloat16, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_refs[i % 2].view(torch.int16)), i


@pytest.mark.parametrize("M,K", [(1, 16384), (16, 16384), (24, 16384), (40, 16384), (64, 16384), (48, 32768)])
def test_forward_graph_replays(M, K):
    """The forward captured once in a HIP graph and replayed with new inputs
    written into the captured buffers between replays (eager work and a
    synchronisation in between): every replay equals the eager forward on the
    same input.  Covers the one-kernel decode (M = 1), the unsplit decode on
    decode-blocked codes, and the split-K decode (K = 32768) whose arrival
    counters the prep kernel clears inside the graph."""
    N, bits = 4096, 4
    w = synthetic.Workload("t", M, K, N, bits, "bf16", "laplace", 0.05, max(1, K // 200), 100.0, 13 * M + 5)
    x, xb, wl = synthetic.make_inputs(w)
    wp, a = hbl.quantize_weights(dev(wl))
    inputs = [x_to_dev(x, xb), -x_to_dev(x, xb), x_to_dev(x, xb) * 0.5]
    refs = [hbl.forward(xi, wp, a, bits) for xi in inputs]
    torch.cuda.synchronize()
    xbuf = inputs[0].clone()
    ybuf = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(hbl.workspace_bytes(hbl.OP_FORWARD_INT4, M, K, N) + 16, dtype=torch.uint8, device="cuda")
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        hbl.forward(xbuf, wp, a, bits, workspace=ws, out=ybuf)   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s_)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hbl.forward(xbuf, wp, a, bits, workspace=ws, out=ybuf)
    for i in range(6):
        xbuf.copy_(inputs[i % 3])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ybuf.view(torch.int16), refs[i % 3].view(torch.int16)), i


def test_fp6_matmul_repeatable_with_fresh_buffers():
    """Regression: the fp6 x fp4 matmul once issued two extra copies per even
    stage into the LDS buffer being read, which corrupted outputs only when
    the copies happened to land first.  At the 7B Wdown shape, repeated
    stage calls with freshly allocated codes, scales and outputs must equal
    the single-call forward every time."""
    M, K, N = 8192, 16384, 4096
    w = synthetic.Workload("t", M, K, N, 4, "bf16", "laplace", 0.05, max(1, K // 200), 100.0, 7)
    x, xb, wl = synthetic.make_inputs(w)
    xd = x_to_dev(x, xb)
    wd = dev(wl)
    for _ in range(6):
        wp, a = hbl.quantize_weights(wd)
        y = hbl.forward(xd, wp, a, 4)
        c6, d6 = hbl.quantize_act(xd, 6)
        y6 = hbl.matmul_dequant(c6, 6, d6, wp, a, K)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y6.view(torch.int16))


@pytest.mark.parametrize("M,K,N", [(65, 256, 16), (257, 1024, 272), (300, 2048, 512), (513, 16384, 256),
                                   (1000, 4096, 4096), (1023, 2048, 1040), (4096, 1024, 4096), (8192, 16384, 4096),
                                   (4059, 1024, 3056), (4000, 256, 3072), (4096, 8192, 3072), (8192, 2048, 3072)])
def test_int4_prefill_fp6_path_equals_int8_instruction_path(M, K, N):
    """The fused INT4 forward for more than 64 tokens runs its matmul on the
    fp6 x fp4 instruction; the stage calls run the same codes through the
    int8 instruction (bit-exact against the oracle above).  Same codes, exact
    integer accumulators and the same dequantisation: equal bit for bit.
    Shapes with fewer than 256 tiles of 256 x 256 take 128 x 128 tiles (ragged
    edges included); 4096 x 4096 and the 7B shape take 256 x 256; N = 3072
    (and 3056, ragged in both M and N; K = 256, two stages per loop trip)
    takes 256 x 192."""
    w = synthetic.Workload("t", M, K, N, 4, "bf16", "laplace", 0.05, max(1, K // 200), 100.0, M + 3 * K + N)
    x, xb, wl = synthetic.make_inputs(w)
    wp, a = hbl.quantize_weights(dev(wl))
    xd = x_to_dev(x, xb)
    y = hbl.forward(xd, wp, a, 4)
    codes, d = hbl.quantize_act(xd, 4)
    y2 = hbl.matmul_dequant(codes, 4, d, wp, a, K)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    # saturated codes at both ends of the INT4 range occur in these inputs
    q = unpack_int4(host(codes), K)
    assert (q == -8).any() and (q == 7).any()


def test_int8_layer_is_exactly_odd_and_deterministic():
    w = synthetic.WORKLOADS["wo_1p3b_int4"].with_(bits=8, M=512)
    x, xb, wl = synthetic.make_inputs(w)
    wp, a = hbl.quantize_weights(dev(wl))
    xd = x_to_dev(x, xb)
    y1 = hbl.forward(xd, wp, a, 8)
    y2 = hbl.forward(xd, wp, a, 8)
    yn = hbl.forward(-xd, wp, a, 8)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(yn, -y1)


def test_token_permutation_equivariance():
    w = synthetic.WORKLOADS["wo_1p3b_int4"].with_(M=384)
    x, xb, wl = synthetic.make_inputs(w)
    wp, a = hbl.quantize_weights(dev(wl))
    xd = x_to_dev(x, xb)
    perm = torch.randperm(xd.shape[0], generator=torch.Generator().manual_seed(0)).cuda()
    y = hbl.forward(xd, wp, a, 4)
    yp = hbl.forward(xd[perm].contiguous(), wp, a, 4)
    torch.cuda.synchronize()
    assert torch.equal(yp, y[perm])


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N", [(5, 512, 48), (16, 2048, 272), (17, 16384, 4096), (31, 4096, 64),
                                   (33, 16384, 4096), (64, 8192, 512), (40, 32768, 272),
                                   (9, 16384, 4096), (16, 16384, 4096), (13, 1024, 80), (16, 32768, 272)])
def test_forward_decode_codes_layout_matches_stages(bits, M, K, N):
    """From 5 to 64 tokens the forward keeps its codes in the decode-blocked
    layout (each fragment load one contiguous KiB); the stage calls keep them
    row-major.  Same codes, exact integer sums, same dequant: the forward
    equals quantize_act + matmul_dequant bit for bit."""
    w = synthetic.Workload("t", M, K, N, bits, "bf16", "laplace", 0.05, max(1, K // 200), 100.0, 7 * M + K + bits)
    x, xb, wl = synthetic.make_inputs(w)
    xd = x_to_dev(x, xb)
    wp, a = hbl.quantize_weights(dev(wl))
    y = hbl.forward(xd, wp, a, bits)
    codes, d = hbl.quantize_act(xd, bits)
    ys = hbl.matmul_dequant(codes, bits, d, wp, a, K)
    assert torch.equal(y, ys)
    ynone = hbl.forward_noalloc(xd, wp, a, bits)
    assert torch.equal(ynone, ys)


def test_forward_writes_the_given_output_dtype():
    """A caller-given output of another dtype than x: the call writes that
    dtype (fp32 x into a bf16 output equals the bf16 output asked for by
    out_dtype), and outputs of the wrong shape or a conflicting out_dtype
    are refused before anything is launched."""
    M, K, N = 8, 256, 256
    x, _ = make_x(M, K, 77, bf16=False)
    wl = synthetic.make_inputs(gaussian_workload(1, K, N, 8, 78))[2]
    wp, a = hbl.quantize_weights(dev(wl))
    xd = dev(x)
    for bits in (8, 4):
        ref = hbl.forward(xd, wp, a, bits, out_dtype=torch.bfloat16)
        guard = torch.full((M + 8, N), 7.0, dtype=torch.bfloat16, device="cuda")
        y = guard[:M]
        hbl.forward(xd, wp, a, bits, out=y)
        assert torch.equal(y, ref)
        assert torch.all(guard[M:] == 7.0), "wrote past the output"
        with pytest.raises(ValueError):
            hbl.forward(xd, wp, a, bits, out=torch.empty((M, N + 16), dtype=torch.bfloat16, device="cuda"))
        with pytest.raises(ValueError):
            hbl.forward(xd, wp, a, bits, out=y, out_dtype=torch.float32)


def test_empty_batch():
    wp = torch.zeros((256, 64), dtype=torch.uint8, device="cuda")
    a = torch.ones(4, dtype=torch.float32, device="cuda")[:1]
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    y = hbl.forward(x, wp, a, 8)
    assert y.shape == (0, 256)
