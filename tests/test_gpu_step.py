"""GPU parity of the streaming step kernels against the oracle: the momentum
EMA (float64 arithmetic, one float32 rounding: within 1 ulp of the oracle
rounded to float32) and the MuonH hyperball update (float64 sums, one
float32 rounding per element: relative Frobenius error <= 1e-6, and the
norm preserved to float32 rounding), over ragged shapes, strided operands,
both load widths, the 1e-10 floors, and a whole optimizer step."""

import numpy as np
import pytest

import oracle
from matrix_roots_amd import binding as B
from matrix_roots_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (7, 3), (64, 128), (130, 257), (1024, 4096), (4096, 1024), (3, 9000)]


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def test_momentum(torch_dev):
    torch, dev = torch_dev
    Gh = [W.gradient("toy", k, 1, shape=s) for k, s in enumerate(SHAPES)]
    Mh = [W.gradient("toy", k, 2, shape=s) for k, s in enumerate(SHAPES)]
    # one strided pair (ld > n, element loads)
    Gbig = torch.zeros(130, 260, device=dev)
    Gbig[:, :257] = torch.from_numpy(Gh[3]).to(dev)
    Gs = [torch.from_numpy(g).to(dev) for g in Gh]
    Gs[3] = Gbig[:, :257]
    Ms = [torch.from_numpy(m.copy()).to(dev) for m in Mh]
    for mu in (0.9, 0.0):
        B.momentum_ema_batched(Gs, Ms, mu)
        torch.cuda.synchronize()
        for k in range(len(SHAPES)):
            ref = oracle.momentum_ema(Mh[k], Gh[k], mu).astype(np.float32)
            got = Ms[k].cpu().numpy()
            ulp = np.spacing(np.maximum(np.abs(ref), np.float32(1e-30)))
            assert np.all(np.abs(got - ref) <= ulp), (SHAPES[k], mu)
            Mh[k] = got.copy()


@pytest.mark.parametrize("lr", [0.02, 0.5])
def test_hyperball(torch_dev, lr):
    torch, dev = torch_dev
    Wh = [W.gradient("w1024", k, 3, shape=s) for k, s in enumerate(SHAPES)]
    Uh = [W.gradient("moe", k, 4, shape=s) for k, s in enumerate(SHAPES)]
    Ws = [torch.from_numpy(w.copy()).to(dev) for w in Wh]
    Us = [torch.from_numpy(u).to(dev) for u in Uh]
    norms = B.hyperball_update_batched(Ws, Us, lr, return_norms=True)
    torch.cuda.synchronize()
    norms = norms.cpu().numpy()
    for k in range(len(SHAPES)):
        ref, info = oracle.hyperball_update(Wh[k], Uh[k], lr)
        got = Ws[k].cpu().numpy()
        assert oracle.relative_frobenius(got, ref) <= 1e-6, SHAPES[k]
        np.testing.assert_allclose(norms[k], [info["w_norm"], info["u_norm"], info["new_norm"]], rtol=1e-12)
        assert abs(np.linalg.norm(got.astype(np.float64)) / info["w_norm"] - 1.0) <= 1e-6


def test_hyperball_floors_and_determinism(torch_dev):
    torch, dev = torch_dev
    Wz = torch.zeros(16, 32, device=dev)
    Wk = torch.from_numpy(W.gradient("toy", 0, 5, shape=(16, 32))).to(dev)
    keep = Wk.clone()
    B.hyperball_update_batched([Wz, Wk], [torch.ones(16, 32, device=dev), torch.zeros(16, 32, device=dev)], 0.1)
    torch.cuda.synchronize()
    assert not Wz.any()
    assert torch.equal(Wk, keep)  # zero update: W' = W, rescaled by ||W|| / ||W|| = 1
    a = torch.from_numpy(W.gradient("toy", 1, 6, shape=(1024, 4096))).to(dev)
    u = torch.from_numpy(W.gradient("toy", 2, 6, shape=(1024, 4096))).to(dev)
    b = a.clone()
    B.hyperball_update_batched([a], [u], 0.1)
    B.hyperball_update_batched([b], [u], 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_whole_optimizer_step(torch_dev):
    """Three steps of momentum -> Gram EMA -> roots -> apply to the momentum ->
    hyperball update on a small transformer-like set, against the oracle
    composed the same way (the roots dominate the error: 1e-4 per update
    direction's tolerance, so 1e-3 on the weights after three steps)."""
    torch, dev = torch_dev
    shapes = [(256, 256), (256, 1024), (1024, 256)]
    beta, mu, eps, lr = 0.95, 0.9, 1e-6, 0.05
    Wh = [W.gradient("toy", k, 9, shape=s).astype(np.float64) for k, s in enumerate(shapes)]
    Wd = [torch.from_numpy(w.astype(np.float32)).to(dev) for w in Wh]
    Md = [torch.zeros(m, n, device=dev) for m, n in shapes]
    Ld = [torch.zeros(m, m, dtype=torch.float64, device=dev) for m, n in shapes]
    Rd = [torch.zeros(n, n, dtype=torch.float64, device=dev) for m, n in shapes]
    Mh = [np.zeros(s) for s in shapes]
    Lh = [np.zeros((m, m)) for m, n in shapes]
    Rh = [np.zeros((n, n)) for m, n in shapes]
    Wo = [w.astype(np.float32).astype(np.float64) for w in Wh]
    for t in range(1, 4):
        Gh = [W.gradient("w1024", k, t, shape=s) for k, s in enumerate(shapes)]
        Gd = [torch.from_numpy(g).to(dev) for g in Gh]
        B.momentum_ema_batched(Gd, Md, mu)
        B.gram_ema_update(Gd, Ld, Rd, beta)
        Xs, info = B.inv_quarter_root_batched(Ld + Rd, eps)
        assert (info["flags"] == 0).all()
        Us = B.precondition_apply(Xs[:3], Md, Xs[3:])
        B.hyperball_update_batched(Wd, Us, lr)
        for k in range(3):
            Mh[k] = oracle.momentum_ema(Mh[k], Gh[k], mu)
            Lh[k], Rh[k] = oracle.gram_ema_update(Lh[k], Rh[k], Gh[k], beta)
            XL, _ = oracle.inv_quarter_root(Lh[k], eps)
            XR, _ = oracle.inv_quarter_root(Rh[k], eps)
            Wo[k], _ = oracle.hyperball_update(Wo[k], oracle.precondition_apply(XL, Mh[k], XR), lr)
    torch.cuda.synchronize()
    for k in range(3):
        got = Wd[k].cpu().numpy()
        assert oracle.relative_frobenius(got, Wo[k]) <= 1e-3, k
        assert abs(np.linalg.norm(got.astype(np.float64)) / np.linalg.norm(Wh[k].astype(np.float32)) - 1) <= 1e-5
