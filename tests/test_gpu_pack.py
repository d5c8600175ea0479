"""Sign packing on the GPU is bit-exact against the oracle's packer."""
import numpy as np
import pytest

import oracle
from gpu_util import say, torch_or_skip

pytestmark = pytest.mark.gpu


def _matrix(rows, cols, seed):
    rng = np.random.default_rng(seed)
    M = rng.standard_normal((rows, cols)).astype(np.float32)
    flat = M.reshape(-1)
    flat[::17] = 0.0
    flat[::19] = -0.0
    flat[::23] = np.nan
    flat[::29] = -np.inf
    flat[::31] = np.inf
    flat[::37] = -1e-40      # negative subnormal is < 0
    return M


@pytest.mark.parametrize("rows,cols", [(1, 1), (33, 65), (64, 64), (300, 1000), (1000, 48),
                                       (8192, 304), (28672, 304)])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("pad", [0, 8])
def test_pack_bit_exact(rows, cols, axis, pad):
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    M = _matrix(rows, cols, rows * 7 + cols)
    n_other = cols if axis == 0 else rows
    ld = lb.packed_ld(n_other) + pad
    say("pack", rows, cols, axis, ld)
    words = lb.pack_signs(torch.from_numpy(M).cuda(), axis, ld)
    torch.cuda.synchronize()
    got = words.cpu().numpy().view(np.uint32)
    want = oracle.pack_signs(M, axis, ld)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_pack_hadamard_parity_pattern():
    """bit(i, j) = parity(i & j) for the 256 x 256 Sylvester-Hadamard matrix."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    n = 256
    i = np.arange(n)
    par = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    H = np.where(par == 1, -1.0, 1.0).astype(np.float32)
    say("pack hadamard")
    got = lb.pack_signs(torch.from_numpy(H).cuda(), 1).cpu().numpy().view(np.uint32)
    for w in range(n // 32):
        for r in (0, 1, 3, 77, 255):
            want = sum(par[r, 32 * w + b] << b for b in range(32))
            assert int(got[w, r]) == want
