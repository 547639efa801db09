"""GPU check of the benchmark's read helpers (include/hbl_calib.h): the XOR
digests equal numpy's on the same bytes (full and ragged last chunk; every
workgroup of the broadcast read), so the timed reads really touch every
byte."""
import numpy as np
import pytest
import torch

import hadamard_rotated_ternary_amd as hbl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 65536, 16 * 2**20, 3 * 65536 + 4096 + 48])
def test_stream_read_digest(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    dig = hbl.stream_read(src)
    torch.cuda.synchronize()
    got = dig.cpu().numpy().view(np.uint32)
    chunks = (nbytes + 65535) // 65536
    ref = np.array([np.bitwise_xor.reduce(words[c * 16384:(c + 1) * 16384]) for c in range(chunks)], np.uint32)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("nbytes,wgs", [(16, 3), (128 * 1024, 256), (512 * 1024 + 48, 300)])
def test_broadcast_read_digest(nbytes, wgs):
    rng = np.random.default_rng(nbytes + wgs)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    dig = hbl.broadcast_read(src, wgs)
    torch.cuda.synchronize()
    got = dig.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, np.full(wgs, np.bitwise_xor.reduce(words), np.uint32))
