"""GPU parity of polar_cans_batched (the ten CANS polar steps,
tilderesearch, "Online KL Shampoo", section 2.3) against the oracle's
U phi(Sigma / sqrt(L)) V^T.

Tolerances (relative Frobenius error against the oracle), from the
arithmetic: the steps act on singular values independently, so rounding
errors only perturb the final polynomial values and singular vectors; a CPU
emulation of the fp16 iteration (operands rounded to fp16, float32
accumulation) stays below 2.8e-3 on Gaussian, low-rank, power-law and
sparse-row gradients, the split one below 5e-6.  MR_CANS_F16 is held to
1e-2, MR_CANS_SPLIT to 5e-5.  Where the spectrum is in the polynomials'
range (sigma^2 / L >= 1e-6) the output is also checked to have orthonormal
columns (rows, if wide): ||O^T O - I||_F / sqrt(min(m, n)) below 2e-2 (f16)
or 1e-4 (split).
"""

import numpy as np
import pytest

import oracle
from matrix_roots_amd import binding as B
from matrix_roots_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

TOL = {"f16": 1e-2, "split": 5e-5}
ORTH = {"f16": 2e-2, "split": 1e-4}
KINDS = {"gaussian": "toy", "lowrank32": "w1024", "powerlaw": "w2048", "sparserows": "moe"}


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def grad(kind, shape, seed=1):
    return W.gradient(KINDS[kind], 7, seed, shape=shape)


def check(torch, dev, Gs, precision, orth=True):
    Gd = [torch.from_numpy(np.ascontiguousarray(g)).to(dev) for g in Gs]
    Os, info = B.polar_cans_batched(Gd, precision=precision)
    torch.cuda.synchronize()
    worst = 0.0
    for i, G in enumerate(Gs):
        assert info["flags"][i] == 0 and info["iters"][i] == 10, info[i]
        ref, rinfo = oracle.polar_cans(G.astype(np.float64))
        assert info["scale"][i] == pytest.approx(rinfo["scale"], rel=1e-6)
        O = Os[i].cpu().numpy()
        assert np.isfinite(O).all()
        err = oracle.relative_frobenius(O, ref)
        worst = max(worst, err)
        assert err <= TOL[precision], (i, G.shape, precision, err)
        if orth:
            s = np.linalg.svd(G.astype(np.float64), compute_uv=False)
            if s.min() ** 2 / (1.01 * np.sum(s * s)) >= 1e-6:
                Od = Os[i].double()
                Q = Od.T @ Od if G.shape[0] >= G.shape[1] else Od @ Od.T
                k = min(G.shape)
                r = float(torch.linalg.norm(Q - torch.eye(k, dtype=torch.float64, device=dev))) / k ** 0.5
                assert r <= ORTH[precision], (i, G.shape, r)
    return worst


@pytest.mark.parametrize("precision", ["f16", "split"])
@pytest.mark.parametrize("shape", [(1, 1), (1, 7), (7, 1), (64, 48), (48, 64), (130, 130), (257, 129), (300, 100),
                                   (100, 300), (520, 264), (384, 1152), (320, 192), (192, 640)])
def test_shapes(torch_dev, precision, shape):
    """Gaussian gradients over tall, wide, square, ragged and degenerate
    shapes (16-byte loads when both sides are multiples of 8; fp16 products
    whose contraction is a multiple of 64 copy straight into LDS, with
    ragged last tiles at 320 x 192 and 192 x 640)."""
    torch, dev = torch_dev
    worst = check(torch, dev, [grad("gaussian", shape)], precision)
    print(f"{shape} {precision}: err {worst:.2e}")


@pytest.mark.parametrize("precision", ["f16", "split"])
@pytest.mark.parametrize("kind", ["lowrank32", "powerlaw", "sparserows"])
def test_distributions_batched(torch_dev, precision, kind):
    """Each workload's gradient structure, several shapes in one call."""
    torch, dev = torch_dev
    Gs = [grad(kind, s, seed) for seed, s in enumerate([(256, 512), (512, 256), (192, 192), (200, 72)], 1)]
    worst = check(torch, dev, Gs, precision)
    print(f"{kind} {precision}: err {worst:.2e}")


def test_flags_strides_and_repeat(torch_dev):
    torch, dev = torch_dev
    good = grad("gaussian", (136, 72))
    zero = np.zeros((40, 24), np.float32)
    nanm = grad("gaussian", (24, 40))
    nanm[3, 5] = np.inf
    Gbig = torch.zeros(136, 72 + 8, dtype=torch.float32, device=dev)
    Gbig[:, :72] = torch.from_numpy(good).to(dev)
    Obig = torch.full((136, 72 + 16), 3.0, dtype=torch.float32, device=dev)
    Gs = [Gbig[:, :72], torch.from_numpy(zero).to(dev), torch.from_numpy(nanm).to(dev)]
    Os = [Obig[:, :72], torch.empty(40, 24, device=dev), torch.empty(24, 40, device=dev)]
    ws = B.RootWorkspace()
    _, info = B.polar_cans_batched(Gs, Os=Os, workspace=ws)
    first = Obig.clone()
    assert info["flags"][0] == 0
    assert info["flags"][1] == B.MR_INFO_ZERO_TRACE and not Os[1].any()
    assert info["flags"][2] == B.MR_INFO_NONFINITE and torch.isnan(Os[2]).all()
    assert bool((Obig[:, 72:] == 3.0).all())
    ref, _ = oracle.polar_cans(good.astype(np.float64))
    assert oracle.relative_frobenius(Obig[:, :72].cpu().numpy(), ref) <= TOL["f16"]
    B.polar_cans_batched(Gs, Os=Os, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, Obig)
