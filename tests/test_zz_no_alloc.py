"""The forward that allocates nothing (hbl_forward_noalloc: its scratch is the
library's static device array) against the forward with a caller workspace
(hbl_forward_int8 / hbl_forward_int4): the same kernels on the same inputs,
so the outputs are equal bit for bit.  Each case makes two no-alloc calls in
a row, the second with a smaller input, so whatever the first call leaves in
the shared array (codes, scales, split-K partials and arrival counters) is
there when the second runs."""
import numpy as np
import pytest
import torch

import hadamard_rotated_ternary_amd as hbl
import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a gfx950 device"
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    hbl.lib()


def layer_inputs(M, K, N, bits, seed):
    w = synthetic.Workload("t", M, K, N, bits, "bf16", "laplace", 0.05, max(1, K // 200), 100.0, seed)
    x, xb, wl = synthetic.make_inputs(w)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    wp, a = hbl.quantize_weights(torch.from_numpy(wl).cuda())
    return xd, wp, a


# (bits, first call (M, K, N), second call, smaller): the fp6 prefill then a
# decode on decode-blocked codes; two such decodes; INT8 prefill then the
# one-kernel decode; the largest INT8 problem that fits the scratch, then a
# blocked decode; a split-K decode (K = 32768) then a smaller one (partials
# and arrival counters left by the first); the 3B down projection (256 x 192
# tiles of the fp6 matmul) then a prefill on 128 x 128 tiles.
CASES = [
    (4, (4096, 8192, 3072), (300, 1024, 272)),
    (4, (1000, 16384, 512), (40, 16384, 4096)),
    (4, (64, 16384, 4096), (33, 4096, 272)),
    (8, (300, 2048, 272), (1, 16384, 4096)),
    (8, (1900, 16384, 272), (64, 8192, 528)),
    (4, (64, 32768, 4096), (33, 32768, 272)),
    (8, (48, 32768, 528), (40, 32768, 272)),
]


@pytest.mark.parametrize("bits,first,second", CASES)
def test_noalloc_forward_equals_workspace_forward(bits, first, second):
    ins = [layer_inputs(*shape, bits, 31 * i + sum(shape)) for i, shape in enumerate((first, second))]
    for (M, K, N) in (first, second):
        need = hbl.workspace_bytes(hbl.OP_FORWARD_INT8 if bits == 8 else hbl.OP_FORWARD_INT4, M, K, N)
        assert need <= hbl.NOALLOC_SCRATCH_BYTES, (M, K, N, need)
    refs = [hbl.forward(xd, wp, a, bits) for xd, wp, a in ins]
    torch.cuda.synchronize()
    outs = [torch.full_like(r, float("nan")) for r in refs]
    for (xd, wp, a), y in zip(ins, outs):
        hbl.forward_noalloc(xd, wp, a, bits, out=y)      # back to back on one stream
    torch.cuda.synchronize()
    for i, (y, r) in enumerate(zip(outs, refs)):
        assert torch.equal(y.view(torch.int16), r.view(torch.int16)), i


def test_noalloc_rejects_problems_beyond_the_scratch():
    M, K, N = 8192, 16384, 4096
    need = hbl.workspace_bytes(hbl.OP_FORWARD_INT8, M, K, N)
    assert need > hbl.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wp = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda")
    a = torch.ones(4, dtype=torch.float32, device="cuda")[:1]
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hbl.HBLError) as e:
        hbl.forward_noalloc(x, wp, a, 8, out=y)
    assert e.value.code == 8
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
