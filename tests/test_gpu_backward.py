"""GPU parity of the straight-through backward (through the C ABI) against the oracle.

Inputs of both sides: the oracle's forward codes q and scales d (d rounded to
fp32, as the HIP path stores it, and handed to the oracle as that value),
its ternary weights, and a bf16 dy.

Bars (derived from the HIP path's arithmetic):
  * W_t^T in bf16: bit-exact (values -1, 0, +1).
  * dw: elementwise |err| <= (2^-8 + M 2^-23) * sum_m |dy[m][n]| |xh[m][k]|:
    xh = q * d is rounded to bf16 (relative 2^-9), dy is exact, products are
    exact in fp32 and the fp32 sum over M tokens adds at most M ulps.
  * dx: relative L2 per token <= 2e-5: dy and the weights are exact, so dxh
    carries only fp32 summation error over N terms; the transform adds
    log2(K) roundings and the RMSNorm backward a few more.
  * dgain: relative L2 <= 2e-5 (fp32 sums over the tokens).
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_ternary_amd as hbl
import oracle
import synthetic
from layouts import pack_int4, pack_ternary

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a gfx950 device"
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    hbl.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_dev(bits16):
    return dev(np.ascontiguousarray(bits16).view(np.int16)).view(torch.bfloat16)


def rel_l2(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def setup(w, bits, M=None, gain=True, rotate=True, dy_seed=0):
    x, xb, wl = synthetic.make_inputs(w, M=M)
    M = x.shape[0]
    g = synthetic.make_gain(w.K, w.seed) if gain else None
    wt, alpha = oracle.quantize_weights(wl)
    # the forward's codes (the oracle's steps up to the quantiser; no matmul needed)
    u = oracle.rmsnorm(x, g)
    xt = oracle.hadamard_rotate(u) if rotate else u
    del u
    q, d, _ = oracle.quant_act(xt, bits)
    del xt
    d32 = d.astype(np.float32)
    rng = np.random.default_rng(1000 + dy_seed)
    dyb = synthetic.f32_to_bf16_bits(rng.normal(size=(M, w.N)).astype(np.float32))
    dyf = synthetic.bf16_bits_to_f32(dyb)
    return dict(x=x, xb=xb, g=g, wt=wt, alpha=alpha, q=q, d32=d32, dyb=dyb, dyf=dyf, M=M, K=w.K, N=w.N)


def run_gpu(s, bits, rotate=True, dx_dtype=torch.float32, x_fp32=False):
    wpack = dev(pack_ternary(s["wt"]))
    alpha = dev(np.array([s["alpha"], 0, 0, 0], np.float32))[:1]
    wbt = hbl.backward_weights(wpack, s["K"])
    xd = dev(s["x"]) if (x_fp32 or s["xb"] is None) else bf16_dev(s["xb"])
    codes = dev(s["q"]) if bits == 8 else dev(pack_int4(s["q"]))
    gd = dev(s["g"]) if s["g"] is not None else None
    dx, dw, dg = hbl.backward(xd, gd, codes, bits, dev(s["d32"]), wbt, alpha, bf16_dev(s["dyb"]), rotate=rotate,
                              dx_dtype=dx_dtype)
    return wbt, host(dx.float()), host(dw), (host(dg) if dg is not None else None)


def check_dw(dw, rdw, q, d32, dyf):
    """dw against the oracle's dw (rdw) elementwise, within the bound the
    HIP arithmetic implies: (2^-8 + M 2^-23) sum_m |dy[m][n]| |q[m][k] d[m]|
    (q d rounded to bf16, exact products, M fp32 additions)."""
    xh = q.astype(np.float64) * d32.astype(np.float64)[:, None]
    bound = (2.0 ** -8 + q.shape[0] * 2.0 ** -23) * (np.abs(dyf).astype(np.float64).T @ np.abs(xh)) + 1e-30
    err = np.abs(dw - rdw)
    assert np.all(err <= bound), float(np.max(err / bound))


def oracle_bwd(s, rotate, rows=None):
    sl = slice(None) if rows is None else rows
    return oracle.backward(s["x"][sl], s["g"], s["q"][sl], s["d32"][sl].astype(np.float64), s["wt"], s["alpha"],
                           s["dyf"][sl], rotate=rotate)


def check_dx(dx, ref, tol=2e-5):
    for m in range(ref.shape[0]):
        assert rel_l2(dx[m], ref[m]) <= tol, (m, rel_l2(dx[m], ref[m]))


SMALL = [("tiny_int8", 8), ("wo_1p3b_int4", 4), ("wdown_3b_int4", 4)]


@pytest.mark.parametrize("name,bits", SMALL)
def test_backward_weights_bit_exact(name, bits):
    w = synthetic.WORKLOADS[name]
    if w.N % 32:
        pytest.skip("N % 32 != 0")
    _, _, wl = synthetic.make_inputs(w, M=1)
    wt, _ = oracle.quantize_weights(wl)
    wbt = hbl.backward_weights(dev(pack_ternary(wt)), w.K)
    got = host(wbt.view(torch.int16)).view(np.uint16)
    ref = synthetic.f32_to_bf16_bits(wt.T.astype(np.float32))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("name,bits,M", [("tiny_int8", 8, 8), ("wo_1p3b_int4", 4, 203), ("wdown_3b_int4", 4, 130),
                                         ("wo_1p3b_int4", 8, 77)])
def test_backward_matches_oracle(name, bits, M, rotate):
    w = synthetic.WORKLOADS[name]
    s = setup(w, bits, M=M, rotate=rotate, dy_seed=M)
    _, dx, dw, dg = run_gpu(s, bits, rotate=rotate)
    rdx, rdw, rdg, _ = oracle_bwd(s, rotate)
    check_dx(dx, rdx)
    check_dw(dw, rdw, s["q"], s["d32"], s["dyf"])
    assert rel_l2(dg, rdg) <= 2e-5


@pytest.mark.parametrize("K,N,M,bits", [(64, 64, 50, 8), (128, 96, 70, 4), (32768, 64, 5, 4)])
def test_backward_short_and_long_rows(K, N, M, bits):
    """The shortest and longest rows the library takes (K = 64, 128, 32768):
    the transposed bf16 weights bit-exact, dx, dW and dgain against the
    oracle at the bars above."""
    w = synthetic.Workload("t", M, K, N, bits, "bf16", "laplace", 0.05, max(1, K // 200), 100.0, K + N + M)
    s = setup(w, bits, dy_seed=K)
    wbt, dx, dw, dg = run_gpu(s, bits)
    got = host(wbt.view(torch.int16)).view(np.uint16)
    assert np.array_equal(got, synthetic.f32_to_bf16_bits(s["wt"].T.astype(np.float32)))
    rdx, rdw, rdg, _ = oracle_bwd(s, True)
    check_dx(dx, rdx)
    check_dw(dw, rdw, s["q"], s["d32"], s["dyf"])
    assert rel_l2(dg, rdg) <= 2e-5


def test_backward_no_gain_bf16_dx_fp32_x():
    w = synthetic.WORKLOADS["wo_1p3b_int4"]
    s = setup(w, 4, M=65, gain=False)
    _, dx32, dw, dg = run_gpu(s, 4, x_fp32=True)
    assert dg is None
    rdx, rdw, _, _ = oracle_bwd(s, True)
    check_dx(dx32, rdx)
    check_dw(dw, rdw, s["q"], s["d32"], s["dyf"])
    _, dxb, _, _ = run_gpu(s, 4, dx_dtype=torch.bfloat16)
    check_dx(dxb, rdx, tol=2e-5 + 2.0 ** -8)


@pytest.mark.parametrize("bits", [4, 8])
def test_backward_full_size_sampled(bits):
    """7B-shaped Wdown (M=8192, K=16384, N=4096) in the benchmark's launch
    configuration: dx on sampled tokens against the oracle run on those
    tokens; dw on four 64-column slices (first, last and two inside; the
    product's 256-wide tiles at both edges) against the oracle's dw for each
    slice (dw never involves the transform, so a slice of q and W_t gives
    exactly the oracle's dw columns)."""
    w = synthetic.WORKLOADS["wdown_7b_int%d" % bits]
    s = setup(w, bits, dy_seed=7)
    _, dx, dw, dg = run_gpu(s, bits)
    rows = synthetic.sample_rows(s["M"], 6)
    rdx, _, _, _ = oracle_bwd(s, True, rows=rows)
    check_dx(dx[rows], rdx)
    for k0 in (0, 4096 + 64 * 7, 9000 - 9000 % 64, s["K"] - 64):
        q = np.ascontiguousarray(s["q"][:, k0:k0 + 64])
        _, rdw, _, _ = oracle.backward(np.ascontiguousarray(s["x"][:, k0:k0 + 64]), None, q,
                                       s["d32"].astype(np.float64), np.ascontiguousarray(s["wt"][:, k0:k0 + 64]),
                                       s["alpha"], s["dyf"])
        check_dw(dw[:, k0:k0 + 64], rdw, q, s["d32"], s["dyf"])
    assert np.all(np.isfinite(dg))


@pytest.mark.parametrize("bits", [4, 8])
def test_backward_gain_over_persistent_iterations(bits):
    """K=16384 with 1100 tokens: the transform + RMSNorm backward runs on a
    grid of 512 one-token workgroups, so each walks two or three tokens and
    accumulates its gain partials across them.  dgain, dx (sampled tokens)
    and dw against the oracle on the whole batch."""
    w = synthetic.WORKLOADS["wdown_7b_int%d" % bits].with_(N=512)
    s = setup(w, bits, M=1100, dy_seed=11)
    _, dx, dw, dg = run_gpu(s, bits)
    rdx, rdw, rdg, _ = oracle_bwd(s, True)
    assert rel_l2(dg, rdg) <= 2e-5, rel_l2(dg, rdg)
    rows = synthetic.sample_rows(s["M"], 32)
    check_dx(dx[rows], rdx[rows])
    check_dw(dw, rdw, s["q"], s["d32"], s["dyf"])


@pytest.mark.parametrize("bits", [8, 4])
def test_backward_single_token(bits):
    w = synthetic.WORKLOADS["wo_1p3b_int4"]
    s = setup(w, bits, M=1, dy_seed=5)
    _, dx, dw, dg = run_gpu(s, bits)
    rdx, rdw, rdg, _ = oracle_bwd(s, True)
    check_dx(dx, rdx)
    check_dw(dw, rdw, s["q"], s["d32"], s["dyf"])
    assert rel_l2(dg, rdg) <= 2e-5
