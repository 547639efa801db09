"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties one oracle step to something other than the oracle itself:
hand-worked fixtures under tests/golden/, closed forms, textbook identities of
the Hadamard matrix, brute force with independent numpy code, and
invariants.  No expected value here comes from the GPU path.
"""
import math

import numpy as np
import pytest

import oracle
import synthetic
from conftest import read_golden


def popcount_sign(i, j):
    """(-1)^popcount(i & j): the Sylvester Hadamard entry, closed form."""
    return -1.0 if bin(i & j).count("1") % 2 else 1.0


def dense_sylvester(n):
    """H_n built by block recursion with numpy (independent of the oracle)."""
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


# ----------------------------------------------------------------- Hadamard

def test_h8_matches_hand_written_golden():
    g = read_golden("hadamard_8.txt")
    H8 = np.array([g[f"row{i}"] for i in range(8)])
    Hor = oracle.fwht(np.eye(8))          # row i = F(e_i) = column i of H (H symmetric)
    assert np.array_equal(Hor, H8)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
def test_fwht_equals_dense_sylvester_and_closed_form(n):
    H_block = dense_sylvester(n)
    H_closed = np.array([[popcount_sign(i, j) for j in range(n)] for i in range(n)])
    assert np.array_equal(H_block, H_closed)
    Hor = oracle.fwht(np.eye(n))
    assert np.array_equal(Hor, H_closed)
    rng = np.random.default_rng(n)
    v = rng.normal(size=(5, n))
    np.testing.assert_allclose(oracle.fwht(v), v @ H_closed.T, rtol=0, atol=1e-12 * n)


@pytest.mark.parametrize("n", [2, 16, 64, 256])
def test_hadamard_is_orthogonal_with_pm1_entries(n):
    H = oracle.fwht(np.eye(n))
    assert set(np.unique(H)) <= {-1.0, 1.0}
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("K", [64, 1024, 16384])
def test_rotation_is_orthonormal_involution(K):
    rng = np.random.default_rng(K)
    u = rng.laplace(size=(3, K))
    t = oracle.hadamard_rotate(u)
    np.testing.assert_allclose(np.linalg.norm(t, axis=1), np.linalg.norm(u, axis=1), rtol=1e-12)
    np.testing.assert_allclose(oracle.hadamard_rotate(t), u, rtol=0, atol=1e-12 * np.abs(u).max())


@pytest.mark.parametrize("K", [4, 256, 4096])
def test_rotation_special_cases(K):
    e0 = np.zeros(K); e0[0] = 1.0
    np.testing.assert_allclose(oracle.hadamard_rotate(e0), np.full(K, 1 / math.sqrt(K)), rtol=1e-14)
    np.testing.assert_allclose(oracle.hadamard_rotate(np.ones(K)), math.sqrt(K) * e0, atol=1e-12)
    # one-hot at j gives the j-th Walsh function
    j = K // 2 + 1 if K > 2 else 1
    ej = np.zeros(K); ej[j] = 1.0
    expect = np.array([popcount_sign(k, j) for k in range(K)]) / math.sqrt(K)
    np.testing.assert_allclose(oracle.hadamard_rotate(ej), expect, rtol=1e-14)


def test_fwht_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.fwht(np.ones(12))


# ----------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms():
    # x = c * ones(K): mean square c^2, so u = c / sqrt(c^2 + eps)
    for c in (3.0, 1e-2, 1e-4):
        K = 64
        u = oracle.rmsnorm(np.full((1, K), c, np.float32))
        expect = float(np.float32(c)) / math.sqrt(float(np.float32(c)) ** 2 + 1e-6)
        np.testing.assert_allclose(u, expect, rtol=1e-14)
    # x = [3, 4]: mean square 12.5
    u = oracle.rmsnorm(np.array([[3.0, 4.0]], np.float32))
    r = math.sqrt(12.5 + 1e-6)
    np.testing.assert_allclose(u[0], [3 / r, 4 / r], rtol=1e-15)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(7)
    x = rng.normal(size=(4, 512)).astype(np.float32)
    u = oracle.rmsnorm(x)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    # mean(u^2) = ms / (ms + eps)
    np.testing.assert_allclose(np.mean(u ** 2, axis=1), ms / (ms + 1e-6), rtol=1e-13)
    # odd and (nearly) scale invariant; gain multiplies channel-wise
    np.testing.assert_array_equal(oracle.rmsnorm(-x), -u)
    np.testing.assert_allclose(oracle.rmsnorm(4 * x), u, rtol=2e-6)
    g = synthetic.make_gain(512, 0)
    np.testing.assert_allclose(oracle.rmsnorm(x, g), u * g, rtol=1e-14)


# ----------------------------------------------------------------- quantisers

def test_int8_absmax_hand_golden():
    g = read_golden("quant_int8_exact.txt")
    q, d, pre = oracle.quant_act(np.array([g["xt"]]), 8)
    np.testing.assert_array_equal(pre[0], g["pre"])
    np.testing.assert_array_equal(q[0], g["codes"])
    assert d[0] == g["d"][0]


def test_int4_absmean_hand_golden():
    g = read_golden("quant_int4_hand.txt")
    for case in "abcd":
        q, d, _ = oracle.quant_act(np.array([g[f"{case}_xt"]]), 4)
        np.testing.assert_array_equal(q[0], g[f"{case}_codes"])
        if f"{case}_d" in g:
            np.testing.assert_allclose(d[0], g[f"{case}_d"][0], rtol=1e-15)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantiser_ranges_and_reconstruction(bits):
    rng = np.random.default_rng(bits)
    xt = rng.laplace(size=(16, 2048))
    xt[:, :7] *= 30
    q, d, pre = oracle.quant_act(xt, bits)
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    assert q.min() >= lo and q.max() <= hi
    unclipped = (pre >= lo - 0.5) & (pre <= hi + 0.5)
    err = np.abs(xt - q * d[:, None])
    assert np.all(err[unclipped] <= (d[:, None] / 2 * (1 + 1e-12) + 1e-300).repeat(xt.shape[1], 1)[unclipped])
    if bits == 8:
        # absmax maps the largest |x| of every token onto +-127; -128 unreachable
        assert np.all(np.abs(q).max(axis=1) == 127)
        assert q.min() >= -127
        np.testing.assert_allclose(d, np.abs(xt).max(axis=1) / 127, rtol=1e-15)
    else:
        np.testing.assert_allclose(d, np.abs(xt).mean(axis=1) / math.sqrt(7), rtol=1e-14)


def test_int4_code_edges_gaussian():
    """For exactly Gaussian x (sigma 1), beta = sqrt(2/pi) and the multiplier is
    sqrt 7 / beta, so code 7 <=> x > 6.5 beta / sqrt 7 = 1.96023 (P = 0.024984)
    and code -8 <=> x <= -7.5 beta / sqrt 7 = -2.26180 (P = 0.011856)."""
    rng = np.random.default_rng(11)
    xt = rng.normal(size=(64, 16384))
    q, d, _ = oracle.quant_act(xt, 4)
    assert abs(np.mean(q == 7) - 0.024984) < 0.0007
    assert abs(np.mean(q == -8) - 0.011856) < 0.0005


# ----------------------------------------------------------------- ternary weights

def test_ternary_hand_golden():
    g = read_golden("ternary_hand.txt")
    wt, alpha = oracle.quantize_weights(np.array(g["a_w"], np.float32).reshape(2, 4))
    assert alpha == np.float32(g["a_alpha"][0])
    np.testing.assert_array_equal(wt.ravel(), g["a_codes"])
    wt, alpha = oracle.quantize_weights(np.array(g["b_w"], np.float32).reshape(1, 4))
    assert alpha == np.float32(g["b_alpha"][0])
    np.testing.assert_array_equal(wt.ravel(), g["b_codes"])


def test_ternary_statistics_gaussian():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, (256, 1024)).astype(np.float32)
    wt, alpha = oracle.quantize_weights(w)
    assert set(np.unique(wt)) <= {-1, 0, 1}
    # E|w| = sigma sqrt(2/pi)
    assert abs(alpha / (0.02 * math.sqrt(2 / math.pi)) - 1) < 0.01
    # P(|z| <= 0.5 sqrt(2/pi)) = 2 Phi(0.39894) - 1 = 0.31006
    assert abs(np.mean(wt == 0) - 0.31006) < 0.005
    # threshold form: nonzero iff |w| > a/2, sign kept
    a = oracle.weight_scale(alpha)
    np.testing.assert_array_equal(wt != 0, np.abs(w.astype(np.float64)) > a / 2)
    np.testing.assert_array_equal(wt[wt != 0], np.sign(w[wt != 0]))


def fp32_ulp(v):
    v = np.float32(v)
    return float(np.spacing(np.abs(v)))


def test_ternary_scale_is_the_mean_abs():
    """alpha is the per-tensor mean of |W| rounded to fp32, whatever the
    summation order: (a) weights on a coarse binary grid, whose sum is exact
    in fp64 in any order, give exactly fp32(sum / NK), the sum taken as an
    exact rational; (b) Gaussian weights give fp32 of the correctly rounded
    mean (math.fsum) to within one fp32 ulp (the fp64 sum's own rounding is
    ~1e-12 relative; only a near-midpoint can move the fp32 rounding)."""
    from fractions import Fraction
    rng = np.random.default_rng(21)
    N, K = 96, 1024
    w = (rng.integers(-4096, 4097, (N, K)) / 4096.0 * 0.05).astype(np.float32)
    _, alpha = oracle.quantize_weights(w)
    exact = sum(Fraction(float(abs(v))) for v in w.ravel()) / (N * K)
    assert alpha == np.float32(float(exact))
    w = rng.normal(0, 0.02, (512, 4096)).astype(np.float32)
    _, alpha = oracle.quantize_weights(w)
    mean = math.fsum(np.abs(w.astype(np.float64)).ravel()) / w.size
    assert abs(float(alpha) - mean) <= fp32_ulp(mean)
    # reversing the tensor changes the order of the oracle's sum, not alpha
    # beyond one ulp
    _, alpha_r = oracle.quantize_weights(np.ascontiguousarray(w[::-1, ::-1]))
    assert abs(float(alpha_r) - float(alpha)) <= fp32_ulp(mean)


def test_ternary_constant_and_zero():
    wt, alpha = oracle.quantize_weights(np.full((4, 8), -0.3, np.float32))
    assert alpha == np.float32(0.3) or abs(alpha - 0.3) < 1e-7
    assert np.all(wt == -1)
    wt, alpha = oracle.quantize_weights(np.zeros((2, 8), np.float32))
    assert alpha == 0 and np.all(wt == 0)
    assert oracle.weight_scale(alpha) == float(np.float32(1e-5))


# ----------------------------------------------------------------- GEMM / dequant

def test_gemm_brute_force_and_closed_forms():
    rng = np.random.default_rng(5)
    q = rng.integers(-128, 128, (7, 96)).astype(np.int8)
    wt = rng.integers(-1, 2, (5, 96)).astype(np.int8)
    acc = oracle.gemm_ternary(q, wt)
    brute = np.array([[sum(int(q[m, k]) * int(wt[n, k]) for k in range(96)) for n in range(5)] for m in range(7)])
    np.testing.assert_array_equal(acc, brute)
    # all-ones codes give the weight row sums; extreme magnitudes stay exact in int32
    K = 32768
    ones = np.ones((1, K), np.int8)
    wt2 = np.ones((2, K), np.int8); wt2[1] = -1
    np.testing.assert_array_equal(oracle.gemm_ternary(ones * -128, wt2), [[-128 * K, 128 * K]])


def test_dequant_closed_form():
    acc = np.array([[3, -5], [0, 127]], np.int32)
    d = np.array([0.5, 2.0])
    y = oracle.dequant(acc, d, np.float32(0.25))
    np.testing.assert_array_equal(y, [[0.375, -0.625], [0.0, 63.5]])


# ----------------------------------------------------------------- whole layer

@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("K,j,c", [(256, 0, 2.5), (256, 77, 1e-3), (4096, 3001, 40.0)])
def test_one_hot_layer_closed_form(bits, K, j, c):
    """x = c e_j: every rotated entry has magnitude v = c / sqrt(c^2 + K eps),
    so codes are +-127 (INT8) or +-3 (INT4, round(sqrt 7)) with the sign of
    the Walsh function, and y_n = v a S_n (INT8) or 3 v a S_n / sqrt 7 (INT4),
    S_n = sum_k W_t[n, k] (-1)^popcount(k & j)."""
    N = 24
    rng = np.random.default_rng(K + j)
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    wt, alpha = oracle.quantize_weights(w)
    a = float(alpha)
    x = np.zeros((1, K), np.float32); x[0, j] = c
    cf = float(np.float32(c))
    v = cf / math.sqrt(cf * cf + K * 1e-6)
    walsh = np.array([popcount_sign(k, j) for k in range(K)])
    S = wt.astype(np.float64) @ walsh
    out = oracle.forward(x, wt, alpha, bits)
    np.testing.assert_allclose(np.abs(out["xt"][0]), v, rtol=1e-12)
    if bits == 8:
        np.testing.assert_array_equal(out["q"][0], 127 * walsh)
        np.testing.assert_allclose(out["y"][0], v * a * S, rtol=1e-12, atol=1e-15)
    else:
        np.testing.assert_array_equal(out["q"][0], 3 * walsh)
        np.testing.assert_allclose(out["y"][0], 3 * v * a * S / math.sqrt(7), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("bits", [8, 4])
def test_brute_force_dense_small(bits):
    """Tiny inputs against an independent dense-matrix implementation."""
    rng = np.random.default_rng(21 + bits)
    M, K, N = 4, 16, 4
    x = rng.normal(size=(M, K)).astype(np.float32)
    x[:, 3] *= 20
    g = synthetic.make_gain(K, 1)
    wl = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    wt, alpha = oracle.quantize_weights(wl)
    out = oracle.forward(x, wt, alpha, bits, g=g)
    H = dense_sylvester(K) / math.sqrt(K)
    xd = x.astype(np.float64)
    u = xd * g / np.sqrt(np.mean(xd ** 2, axis=1, keepdims=True) + 1e-6)
    xt = u @ H.T
    if bits == 8:
        G = np.maximum(np.abs(xt).max(1), 1e-5); Q = 127.0; lo, hi = -128, 127
    else:
        G = np.maximum(np.abs(xt).mean(1), 1e-5); Q = math.sqrt(7); lo, hi = -8, 7
    q = np.clip(np.round(xt * (Q / G)[:, None]), lo, hi)
    y = (q @ wt.T.astype(np.float64)) * (G / Q)[:, None] * a_of(alpha)
    np.testing.assert_allclose(out["xt"], xt, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(out["q"], q)
    np.testing.assert_allclose(out["y"], y, rtol=1e-13, atol=1e-16)


def a_of(alpha):
    return max(float(alpha), float(np.float32(1e-5)))


@pytest.mark.parametrize("bits", [8, 4])
def test_layer_invariants(bits):
    w = synthetic.WORKLOADS["tiny_int8"]
    x, _, wl = synthetic.make_inputs(w)
    wt, alpha = oracle.quantize_weights(wl)
    y = oracle.forward(x, wt, alpha, bits)["y"]
    # token independence: permuting rows permutes outputs exactly
    perm = np.random.default_rng(0).permutation(x.shape[0])
    np.testing.assert_array_equal(oracle.forward(x[perm], wt, alpha, bits)["y"], y[perm])
    if bits == 8:
        # symmetric absmax + round-half-even: the layer is exactly odd
        np.testing.assert_array_equal(oracle.forward(-x, wt, alpha, bits)["y"], -y)
    # a zero token gives a zero output
    z = oracle.forward(np.zeros((1, x.shape[1]), np.float32), wt, alpha, bits)
    assert np.all(z["y"] == 0) and np.all(z["q"] == 0)


# ----------------------------------------------------------------- the method's claim

@pytest.mark.parametrize("name", ["wo_1p3b_int4", "wdown_3b_int4", "wdown_7b_int4"])
def test_hadamard_tames_outlier_channels(name):
    """The rotation turns sharp, outlier-heavy activations into Gaussian-like
    ones (QbitAI article, section 引入H-BitLinear模块; 新智元 article, Figures
    2-3 discussion): per-token max/rms drops and INT4 error falls."""
    w = synthetic.WORKLOADS[name]
    x, _, _ = synthetic.make_inputs(w, M=32, with_weights=False)
    u = oracle.rmsnorm(x)
    xt = oracle.hadamard_rotate(u)
    def peak_ratio(v):
        return np.mean(np.abs(v).max(1) / np.sqrt(np.mean(v ** 2, 1)))
    assert peak_ratio(xt) / peak_ratio(u) < 0.3
    def rel_mse(v):
        q, d, _ = oracle.quant_act(v, 4)
        return np.mean((v - q * d[:, None]) ** 2) / np.mean(v ** 2)
    assert rel_mse(xt) / rel_mse(u) < 0.1


# ----------------------------------------------------------------- BitLinear without the rotation

@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("c", [0.7, 3e-3])
def test_unrotated_constant_token_closed_form(bits, c):
    """x = c (every feature): RMSNorm gives u_k = v = c / sqrt(c^2 + eps) for all
    k, so without the rotation every code is 127 (INT8) or round(sqrt 7) = 3
    (INT4) and y_n = v a R_n (INT8) or 3 v a R_n / sqrt 7 (INT4), R_n the row
    sum of W_t."""
    K, N = 512, 20
    rng = np.random.default_rng(5)
    wt, alpha = oracle.quantize_weights(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    x = np.full((1, K), c, np.float32)
    cf = float(np.float32(c))
    v = cf / math.sqrt(cf * cf + 1e-6)
    R = wt.astype(np.float64).sum(1)
    out = oracle.forward(x, wt, alpha, bits, rotate=False)
    np.testing.assert_allclose(out["xt"][0], v, rtol=1e-14)
    if bits == 8:
        np.testing.assert_array_equal(out["q"][0], 127)
        np.testing.assert_allclose(out["y"][0], v * a_of(alpha) * R, rtol=1e-12, atol=1e-15)
    else:
        np.testing.assert_array_equal(out["q"][0], 3)
        np.testing.assert_allclose(out["y"][0], 3 * v * a_of(alpha) * R / math.sqrt(7), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("bits", [8, 4])
def test_unrotated_brute_force_dense_small(bits):
    """Tiny inputs against an independent implementation of the layer with the
    rotation left out (quantiser input = RMSNorm output)."""
    rng = np.random.default_rng(41 + bits)
    M, K, N = 5, 32, 6
    x = rng.normal(size=(M, K)).astype(np.float32)
    g = synthetic.make_gain(K, 2)
    wt, alpha = oracle.quantize_weights(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    out = oracle.forward(x, wt, alpha, bits, g=g, rotate=False)
    xd = x.astype(np.float64)
    u = xd * g / np.sqrt(np.mean(xd ** 2, axis=1, keepdims=True) + 1e-6)
    if bits == 8:
        G = np.maximum(np.abs(u).max(1), 1e-5); Q = 127.0; lo, hi = -128, 127
    else:
        G = np.maximum(np.abs(u).mean(1), 1e-5); Q = math.sqrt(7); lo, hi = -8, 7
    q = np.clip(np.round(u * (Q / G)[:, None]), lo, hi)
    y = (q @ wt.T.astype(np.float64)) * (G / Q)[:, None] * a_of(alpha)
    np.testing.assert_allclose(out["xt"], u, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(out["q"], q)
    np.testing.assert_allclose(out["y"], y, rtol=1e-13, atol=1e-16)


# ----------------------------------------------------------------- weights rotated as well

def test_rotated_weights_definition_and_cancellation():
    """Rows rotated by H / sqrt(K) (dense Sylvester matrix, independent of the
    fast transform), then ternarised as usual; and the rotation cancels in the
    layer's inner product: (H u / sqrt K) . (H w / sqrt K) = u . w."""
    rng = np.random.default_rng(9)
    N, K = 6, 64
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    wt, alpha, wr = oracle.quantize_weights_rotated(w)
    H = dense_sylvester(K) / math.sqrt(K)
    np.testing.assert_allclose(wr, w.astype(np.float64) @ H.T, rtol=0, atol=1e-15)
    S = sum(np.abs(wr[n]).sum() for n in range(N))
    assert alpha == np.float32(S / (N * K))
    a = a_of(alpha)
    np.testing.assert_array_equal(wt, np.clip(np.round(wr / a), -1, 1))
    u = rng.normal(size=(3, K))
    np.testing.assert_allclose((u @ H.T) @ wr.T, u @ w.T.astype(np.float64), rtol=1e-12, atol=1e-14)


def test_rotated_weights_one_hot_and_involution():
    """A one-hot row e_j rotates to the Walsh function (-1)^popcount(k&j)/sqrt K
    (all magnitudes equal, so every code is +-1 with alpha = 1/sqrt K), and
    rotating the rotated rows again gives back the original rows."""
    K = 256
    for j in (0, 5, 200):
        w = np.zeros((1, K), np.float32); w[0, j] = 1.0
        wt, alpha, wr = oracle.quantize_weights_rotated(w)
        walsh = np.array([popcount_sign(k, j) for k in range(K)])
        np.testing.assert_allclose(wr[0], walsh / math.sqrt(K), rtol=1e-14)
        assert alpha == np.float32(1 / math.sqrt(K))
        np.testing.assert_array_equal(wt[0], walsh)
    rng = np.random.default_rng(3)
    w = rng.normal(size=(4, K)).astype(np.float32)
    _, _, wr = oracle.quantize_weights_rotated(w)
    back = np.stack([oracle.hadamard_rotate(r) for r in wr])
    np.testing.assert_allclose(back, w, rtol=0, atol=1e-12)


# ------------------------------------------------ low-bit attention states
# Per-head absmax quantisation of post-RoPE Q/K/V to unsigned b-bit codes and
# one decode step of attention over such a cache (新智元 article, section
# 实验效果; 量子位 article on the 3-bit KV cache).

def test_heads_3bit_hand_golden():
    g = read_golden("heads_3bit_hand.txt")
    x = np.array([g["x"]], dtype=np.float32)
    codes, scale, _ = oracle.quant_heads(x, 3)
    assert codes[0].tolist() == [int(c) for c in g["codes"]]
    assert scale[0] == g["scale"][0]


def _nearest_code_fraction(v, G, bits):
    """Brute force with exact rationals: the unsigned code whose level
    (u - Z) * G / Qb is nearest to v, ties to the even signed value."""
    from fractions import Fraction
    Qb, Z = 2 ** (bits - 1) - 1, 2 ** (bits - 1)
    best = None
    for u in range(2 ** bits):
        dist = abs(Fraction(v) - Fraction(u - Z) * Fraction(G) / Qb)
        key = (dist, (u - Z) % 2)
        if best is None or key < best[0]:
            best = (key, u)
    return best[1]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_heads_brute_force_rationals(bits):
    rng = np.random.default_rng(100 + bits)
    # bf16-valued inputs with exact ties planted: multiples of G / (2 Qb)
    Qb = 2 ** (bits - 1) - 1
    x = rng.normal(size=(6, 16)).astype(np.float32)
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    x[0, :] = np.arange(-8, 8, dtype=np.float32) * 0.25     # ties for small Qb
    x[1, 0] = 4.0
    x[1, 1:] = (np.arange(15) - 7) * (4.0 / (2 * Qb))
    x[2] = (x[2] * 1e-6).astype(np.float32)                  # below the floor
    x[2] = (x[2].view(np.uint32) & 0xFFFF0000).view(np.float32)
    codes, scale, _ = oracle.quant_heads(x, bits)
    floor = float(np.float32(1e-5))
    for r in range(x.shape[0]):
        G = max(float(np.max(np.abs(x[r].astype(np.float64)))), floor)
        assert scale[r] == G / Qb
        for e in range(x.shape[1]):
            assert codes[r, e] == _nearest_code_fraction(float(x[r, e]), G, bits), (r, e)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_heads_closed_forms_and_invariants(bits):
    Qb, Z = 2 ** (bits - 1) - 1, 2 ** (bits - 1)
    # constant-magnitude row +-c: codes Z +- Qb, scale c / Qb
    c = 0.375
    x = np.array([[c, -c, c, c, -c, -c, c, -c]], dtype=np.float32)
    codes, scale, _ = oracle.quant_heads(x, bits)
    assert codes[0].tolist() == [Z + Qb if v > 0 else Z - Qb for v in x[0]]
    assert scale[0] == c / Qb
    # zero row: the floor on the statistic keeps the scale finite, all codes Z
    codes, scale, _ = oracle.quant_heads(np.zeros((1, 8), np.float32), bits)
    assert codes[0].tolist() == [Z] * 8 and scale[0] == float(np.float32(1e-5)) / Qb
    # random rows: codes within [Z - Qb, Z + Qb] (code 0 unused for b>=2),
    # the absmax element at an end, reconstruction error at most half a step
    rng = np.random.default_rng(bits)
    x = rng.standard_t(3, size=(40, 64)).astype(np.float32)
    codes, scale, _ = oracle.quant_heads(x, bits)
    assert codes.min() >= Z - Qb and codes.max() <= Z + Qb
    am = np.argmax(np.abs(x), axis=1)
    ends = codes[np.arange(40), am].astype(int) - Z
    assert np.array_equal(np.abs(ends), np.full(40, Qb))
    y = oracle.dequant_heads(codes, scale, bits)
    assert np.all(np.abs(y - x) <= scale[:, None] / 2 * (1 + 1e-12))
    # values on the grid come back exactly
    grid = ((codes.astype(np.float64) - Z) * scale[:, None]).astype(np.float32)
    c2, s2, _ = oracle.quant_heads(grid, bits)
    assert np.array_equal(c2, codes)


def _cache(rng, B, Hkv, T, d, bits):
    Qb, Z = 2 ** (bits - 1) - 1, 2 ** (bits - 1)
    kc = rng.integers(Z - Qb, Z + Qb + 1, size=(B, Hkv, T, d)).astype(np.uint8)
    vc = rng.integers(Z - Qb, Z + Qb + 1, size=(B, Hkv, T, d)).astype(np.uint8)
    ks = rng.uniform(0.05, 0.5, size=(B, Hkv, T)).astype(np.float32)
    vs = rng.uniform(0.05, 0.5, size=(B, Hkv, T)).astype(np.float32)
    return kc, ks, vc, vs


def test_attention_single_token_and_uniform_keys():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, T, d, bits = 2, 4, 2, 5, 16, 3
    Z = 4
    kc, ks, vc, vs = _cache(rng, B, Hkv, T, d, bits)
    q = rng.normal(size=(B, Hq, d)).astype(np.float32)
    vh = (vc.astype(np.float64) - Z) * vs[..., None]
    # one cached token: the output is that token's value row
    out = oracle.attention_decode(q, 8, kc, ks, vc, vs, bits, np.array([1, 1]))
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out[b, h], vh[b, h // 2, 0], rtol=0, atol=1e-15)
    # identical keys: uniform weights, the output is the mean of the values
    kc2 = np.repeat(kc[:, :, :1], T, axis=2)
    ks2 = np.repeat(ks[:, :, :1], T, axis=2)
    out = oracle.attention_decode(q, 8, kc2, ks2, vc, vs, bits, np.array([T, 3]))
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], vh[0, h // 2].mean(axis=0), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(out[1, h], vh[1, h // 2, :3].mean(axis=0), rtol=1e-13, atol=1e-15)
    # empty context: zeros
    out = oracle.attention_decode(q, 8, kc, ks, vc, vs, bits, np.array([0, 2]))
    assert np.all(out[0] == 0.0)


def test_attention_two_token_closed_form():
    # d = 4, q = (G, 0, 0, 0): on the grid for any qbits, so q^ = q.
    # Keys: k^_0 = (2 sk0, ...), k^_1 = (-1 sk1, ...); the logits are
    # G * 2 sk0 / 2 and -G * sk1 / 2 (sqrt(4) = 2), so p_0 = sigmoid(l0 - l1).
    G, sk0, sk1 = 1.5, 0.25, 0.5
    Z = 4
    q = np.array([[[G, 0, 0, 0]]], dtype=np.float32)
    kc = np.array([[[[Z + 2, Z + 3, Z - 1, Z], [Z - 1, Z + 1, Z, Z - 3]]]], dtype=np.uint8)
    ks = np.array([[[sk0, sk1]]], dtype=np.float32)
    vc = np.array([[[[Z + 1, Z - 2, Z + 3, Z], [Z - 3, Z, Z + 1, Z + 2]]]], dtype=np.uint8)
    vs = np.array([[[0.125, 0.75]]], dtype=np.float32)
    out = oracle.attention_decode(q, 4, kc, ks, vc, vs, 3, np.array([2]))
    l0, l1 = G * 2 * sk0 / 2, -G * 1 * sk1 / 2
    p0 = 1.0 / (1.0 + math.exp(l1 - l0))
    v0 = np.array([1, -2, 3, 0]) * 0.125
    v1 = np.array([-3, 0, 1, 2]) * 0.75
    np.testing.assert_allclose(out[0, 0], p0 * v0 + (1 - p0) * v1, rtol=1e-14, atol=1e-15)


def test_attention_invariants():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, T, d, bits = 2, 6, 2, 9, 32, 3
    kc, ks, vc, vs = _cache(rng, B, Hkv, T, d, bits)
    q = rng.normal(size=(B, Hq, d)).astype(np.float32)
    q[:, 1] = q[:, 0]                     # same group, same query
    lens = np.array([9, 6])
    out = oracle.attention_decode(q, 8, kc, ks, vc, vs, bits, lens)
    assert np.array_equal(out[:, 0], out[:, 1])
    # permuting the cached tokens does not change the output
    perm = rng.permutation(T)
    out_p = oracle.attention_decode(q, 8, kc[:, :, perm], ks[:, :, perm], vc[:, :, perm], vs[:, :, perm],
                                    bits, np.array([9, 9]))
    np.testing.assert_allclose(out_p[0], out[0], rtol=1e-12, atol=1e-14)
    # tokens past the length are ignored
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[1, :, 6:] = 7
    vc2[1, :, 6:] = 1
    out2 = oracle.attention_decode(q, 8, kc2, ks, vc2, vs, bits, lens)
    assert np.array_equal(out2, out)
    # a convex combination of the values
    vh = (vc.astype(np.float64) - 4) * vs[..., None]
    for b in range(B):
        for h in range(Hq):
            seg = vh[b, h // 3, :lens[b]]
            assert np.all(out[b, h] <= seg.max(axis=0) + 1e-12)
            assert np.all(out[b, h] >= seg.min(axis=0) - 1e-12)
    # a dominant key (large logit gap) selects its value row
    kc3 = np.full_like(kc, 4)
    ks3 = np.ones_like(ks)
    qd = np.zeros_like(q)
    qd[:, :, 0] = 1.0
    kc3[:, :, 2, 0] = 7                    # k^_2 = (3, 0, ...): logit 3 * 1 / sqrt(32)
    ks3[:, :, 2] = 200.0                   # gap 600 / sqrt(32) ~ 106: exp(-106) ~ 1e-46
    out3 = oracle.attention_decode(qd, 8, kc3, ks3, vc, vs, bits, np.array([9, 9]))
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out3[b, h], vh[b, h // 3, 2], rtol=1e-12, atol=1e-15)


def test_attention_quantises_the_query():
    # a query off the grid gives the same output as its dequantised grid image
    rng = np.random.default_rng(5)
    B, Hq, Hkv, T, d, bits = 1, 2, 1, 7, 16, 3
    kc, ks, vc, vs = _cache(rng, B, Hkv, T, d, bits)
    q = rng.normal(size=(B, Hq, d)).astype(np.float32)
    for qbits in (3, 4, 8):
        c, s, _ = oracle.quant_heads(q.reshape(-1, d), qbits)
        qg = oracle.dequant_heads(c, s, qbits).astype(np.float32).reshape(q.shape)
        a = oracle.attention_decode(q, qbits, kc, ks, vc, vs, bits, np.array([T]))
        g = oracle.attention_decode(qg, qbits, kc, ks, vc, vs, bits, np.array([T]))
        np.testing.assert_allclose(a, g, rtol=1e-12, atol=1e-14)
        if qbits == 3:
            full = oracle.attention_decode(q, 8, kc, ks, vc, vs, bits, np.array([T]))
            assert not np.allclose(a, full, rtol=1e-6)


# ------------------------------------------------------------------ backward
# Straight-through backward (量子位 article, section 引入H-BitLinear模块,
# training paragraph): quantisers bypassed, gradient through the transposed
# (= the same) orthonormal Hadamard transform.  Pinned by finite differences
# of the quantiser-free surrogate built from the pinned forward steps.

def _surrogate_loss(x, g, wt, a, dy, rotate):
    """<dy, xt(x) . (W_t a)^T> with xt = H RMSNorm(x) / sqrt(K) (or RMSNorm(x))."""
    u = oracle.rmsnorm(x, g)
    xt = oracle.hadamard_rotate(u) if rotate else u
    y = xt @ (wt.astype(np.float64) * a).T
    return float(np.sum(y * dy.astype(np.float64)))


def _bwd_case(seed, M=3, K=16, N=5, with_gain=True):
    rng = np.random.default_rng(seed)
    x = (rng.integers(-64, 65, size=(M, K)) / 16.0).astype(np.float32)   # multiples of 1/16: x +- 2^-10 exact
    g = (rng.integers(8, 25, size=K) / 16.0).astype(np.float32) if with_gain else None
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    wt, alpha = oracle.quantize_weights(w)
    dy = rng.normal(size=(M, N)).astype(np.float32)
    return x, g, wt, alpha, dy


@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("with_gain", [True, False])
def test_backward_input_matches_finite_differences(rotate, with_gain):
    x, g, wt, alpha, dy = _bwd_case(1 + rotate + 2 * with_gain, with_gain=with_gain)
    a = oracle.weight_scale(alpha)
    fw = oracle.forward(x, wt, alpha, 8, g=g, rotate=rotate)
    dx, dw, dg, _ = oracle.backward(x, g, fw["q"], fw["d"], wt, alpha, dy, rotate=rotate)
    h = np.float32(2.0 ** -10)
    M, K = x.shape
    for m in range(M):
        for j in range(K):
            xp, xm = x.copy(), x.copy()
            xp[m, j] += h
            xm[m, j] -= h
            fd = (_surrogate_loss(xp, g, wt, a, dy, rotate) - _surrogate_loss(xm, g, wt, a, dy, rotate)) / (
                float(xp[m, j]) - float(xm[m, j]))
            assert abs(fd - dx[m, j]) <= 1e-5 * (1.0 + abs(dx[m, j])), (m, j, fd, dx[m, j])
    if with_gain:
        for k in range(K):
            gp, gm = g.copy(), g.copy()
            gp[k] += h
            gm[k] -= h
            fd = (_surrogate_loss(x, gp, wt, a, dy, rotate) - _surrogate_loss(x, gm, wt, a, dy, rotate)) / (
                float(gp[k]) - float(gm[k]))
            assert abs(fd - dg[k]) <= 1e-5 * (1.0 + abs(dg[k])), (k, fd, dg[k])
    else:
        assert dg is None


@pytest.mark.parametrize("bits", [8, 4])
def test_backward_one_hot_closed_forms(bits):
    x, g, wt, alpha, _ = _bwd_case(7, M=4, K=32, N=6)
    a = oracle.weight_scale(alpha)
    fw = oracle.forward(x, wt, alpha, bits, g=g)
    m0, n0 = 2, 3
    dy = np.zeros((4, 6), np.float32)
    dy[m0, n0] = 1.0
    dx, dw, dg, dxh = oracle.backward(x, g, fw["q"], fw["d"], wt, alpha, dy, want_dxh=True)
    # weight gradient: row n0 is the quantised activations of token m0, the rest zero
    ref = np.zeros_like(dw)
    ref[n0] = fw["q"][m0].astype(np.float64) * fw["d"][m0]
    assert np.array_equal(dw, ref)
    # gradient at the quantiser input: a * W_t[n0] in row m0 only
    ref = np.zeros_like(dxh)
    ref[m0] = a * wt[n0].astype(np.float64)
    assert np.array_equal(dxh, ref)
    # other tokens get no input gradient
    assert np.all(dx[[0, 1, 3]] == 0.0)
    # linearity in dy
    rng = np.random.default_rng(3)
    d1 = rng.normal(size=(4, 6)).astype(np.float32)
    d2 = rng.normal(size=(4, 6)).astype(np.float32)
    r1 = oracle.backward(x, g, fw["q"], fw["d"], wt, alpha, d1)
    r2 = oracle.backward(x, g, fw["q"], fw["d"], wt, alpha, d2)
    r12 = oracle.backward(x, g, fw["q"], fw["d"], wt, alpha, (d1.astype(np.float64) + d2).astype(np.float32))
    s12 = (d1.astype(np.float64) + d2).astype(np.float32).astype(np.float64)
    if np.array_equal(s12, d1.astype(np.float64) + d2.astype(np.float64)):
        for i in range(3):
            np.testing.assert_allclose(r12[i], r1[i] + r2[i], rtol=1e-12, atol=1e-12)


def test_backward_rmsnorm_and_rotation_invariants():
    # Without a gain: sum_j x_j dx_j = (eps / r^2) <du, u> per token (RMSNorm is
    # scale invariant up to eps), and the rotation preserves the norm of the
    # gradient it carries: |du| = |dxh|.
    rng = np.random.default_rng(9)
    M, K, N = 5, 64, 7
    x = rng.normal(size=(M, K)).astype(np.float32) * 0.01        # small rows: eps matters
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    wt, alpha = oracle.quantize_weights(w)
    dy = rng.normal(size=(M, N)).astype(np.float32)
    fw = oracle.forward(x, wt, alpha, 4)
    dx, dw, dg, dxh = oracle.backward(x, None, fw["q"], fw["d"], wt, alpha, dy, want_dxh=True)
    u = oracle.rmsnorm(x)
    du = oracle.hadamard_rotate(dxh)
    for m in range(M):
        ms = np.mean(x[m].astype(np.float64) ** 2)
        r2 = ms + 1e-6
        lhs = float(np.dot(x[m].astype(np.float64), dx[m]))
        rhs = 1e-6 / r2 * float(np.dot(du[m], u[m]))
        assert abs(lhs - rhs) <= 1e-9 * (1 + abs(rhs)) + 1e-12 * np.abs(dx[m]).sum(), (m, lhs, rhs)
        np.testing.assert_allclose(np.linalg.norm(du[m]), np.linalg.norm(dxh[m]), rtol=1e-12)


def test_attention_prefill_causal_closed_forms():
    # Prefill from position 0: query i sees keys 0..i only.
    rng = np.random.default_rng(21)
    B, Tn, Hq, Hkv, d, Tmax, bits = 2, 6, 2, 1, 16, 9, 3
    kc, ks, vc, vs = _cache(rng, B, Hkv, Tmax, d, bits)
    q = rng.normal(size=(B, Tn, Hq, d)).astype(np.float32)
    start = np.array([0, 3])
    out = oracle.attention_prefill(q, 8, kc, ks, vc, vs, bits, start)
    vh = (vc.astype(np.float64) - 4) * vs[..., None]
    # the first query of sequence 0 sees one key: its value row
    for h in range(Hq):
        np.testing.assert_allclose(out[0, 0, h], vh[0, 0, 0], rtol=0, atol=1e-15)
    # identical keys: query i of sequence b gets the mean of values 0..start+i
    kc2 = np.repeat(kc[:, :, :1], Tmax, axis=2)
    ks2 = np.repeat(ks[:, :, :1], Tmax, axis=2)
    out2 = oracle.attention_prefill(q, 8, kc2, ks2, vc, vs, bits, start)
    for b in range(B):
        for i in range(Tn):
            for h in range(Hq):
                np.testing.assert_allclose(out2[b, i, h], vh[b, 0, :start[b] + i + 1].mean(axis=0),
                                           rtol=1e-13, atol=1e-15)
    # causality: cache rows after a query's position do not change its output
    kc3, vc3 = kc.copy(), vc.copy()
    kc3[1, :, 6:] = 7
    vc3[1, :, 6:] = 1
    out3 = oracle.attention_prefill(q, 8, kc3, ks, vc3, vs, bits, start)
    assert np.array_equal(out3[0], out[0])
    assert np.array_equal(out3[1, :3], out[1, :3])          # positions 3, 4, 5 see rows 0..5 only
    assert not np.allclose(out3[1, 3:], out[1, 3:])


def test_attention_prefill_two_token_closed_form():
    # query 1 (position 1) over keys 0 and 1: p_0 = sigmoid(l0 - l1), as in the decode case
    G, sk0, sk1 = 1.5, 0.25, 0.5
    Z = 4
    q = np.zeros((1, 2, 1, 4), np.float32)
    q[0, 1, 0, 0] = G
    q[0, 0, 0, 1] = 1.0
    kc = np.array([[[[Z + 2, Z + 3, Z - 1, Z], [Z - 1, Z + 1, Z, Z - 3]]]], dtype=np.uint8)
    ks = np.array([[[sk0, sk1]]], dtype=np.float32)
    vc = np.array([[[[Z + 1, Z - 2, Z + 3, Z], [Z - 3, Z, Z + 1, Z + 2]]]], dtype=np.uint8)
    vs = np.array([[[0.125, 0.75]]], dtype=np.float32)
    out = oracle.attention_prefill(q, 4, kc, ks, vc, vs, 3, np.array([0]))
    l0, l1 = G * 2 * sk0 / 2, -G * 1 * sk1 / 2
    p0 = 1.0 / (1.0 + math.exp(l1 - l0))
    v0 = np.array([1, -2, 3, 0]) * 0.125
    v1 = np.array([-3, 0, 1, 2]) * 0.75
    np.testing.assert_allclose(out[0, 1, 0], p0 * v0 + (1 - p0) * v1, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out[0, 0, 0], v0, rtol=0, atol=1e-15)   # position 0: key 0 only
