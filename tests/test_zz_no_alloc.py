"""inv_quarter_root_batched_noalloc (the workspace in the library's own
scratch array) against inv_quarter_root_batched with a caller workspace:
same kernels, same inputs, so the roots and info records agree bit for bit.
Two calls in a row, the second on a smaller batch, so the second runs on
the scratch contents the first left behind."""

import numpy as np
import pytest

from matrix_roots_amd import binding as B
from matrix_roots_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def _batch(torch, dev, sizes, seed):
    rng = W.rng_for(93, seed)
    return [torch.from_numpy(W.spd_loguniform(d, rng, -6.0, 0.0)).to(dev) for d in sizes]


@pytest.mark.parametrize("normalize", ["trace", "none"])
def test_noalloc_matches_workspace_call(torch_dev, normalize):
    torch, dev = torch_dev
    # first call: Newton sizes over several tiles with ragged tails plus
    # Jacobi sizes; second call: fewer, smaller matrices
    for k, sizes in enumerate(([160, 300, 64, 17, 512, 129], [96, 33])):
        As = _batch(torch, dev, sizes, k)
        ref, rinfo = B.inv_quarter_root_batched(As, 1e-6, normalize=normalize)
        Xs = [torch.full((d, d), float("nan"), dtype=torch.float32, device=dev) for d in sizes]
        info = torch.zeros(B.ROOT_INFO_BYTES * len(sizes), dtype=torch.uint8, device=dev)
        B.inv_quarter_root_batched_noalloc(As, 1e-6, Xs, info, normalize=normalize)
        torch.cuda.synchronize()
        got = B.decode_info(info, len(sizes))
        assert (rinfo["flags"] == 0).all()
        assert np.array_equal(got, rinfo), (k, got, rinfo)
        for d, X, R in zip(sizes, Xs, ref):
            assert torch.equal(X, R), (k, d)


def test_noalloc_rejects_batches_beyond_the_scratch(torch_dev):
    torch, dev = torch_dev
    As = [torch.zeros(1024, 1024, dtype=torch.float32, device=dev)]
    Xs = [torch.empty(1024, 1024, dtype=torch.float32, device=dev)]
    with pytest.raises(B.MatrixRootsError) as e:
        B.inv_quarter_root_batched_noalloc(As, 1e-6, Xs, None)
    assert e.value.status == 5 and "scratch" in str(e.value)
