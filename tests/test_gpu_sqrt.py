"""GPU parity of inv_sqrt_root_batched (scaled CANS coupled Newton-Schulz,
tilderesearch, "Online KL Shampoo", sections 2.3-2.4 and appendix D) against
the oracle's eigendecomposition S^(-1/2).

Tolerances (relative Frobenius error against the oracle), from the
arithmetic: fp16 rounding of S alone (unit roundoff 2^-11) moves an
eigenvalue lambda by up to about 2^-11 ||S|| / sqrt(3), a relative change of
W's eigenvalue of half that over lambda / ||S||; over the matrices used here
(condition number <= 1e3) a CPU emulation of the fp16 iteration gives at most
2.6e-3 (7.3e-3 on a rank-deficient Gram with eps = 1e-3), and the GPU at
most 4.9e-3 for d >= 7.  The first step's a0 y + b0 y^2 cancels to about
1/18 of its terms near the top of the spectrum; it runs on split products in
both precisions, so no fp16 rounding is amplified there (d = 1: 8.9e-5).
MR_CANS_F16 is held to 1e-2, and to 2e-2 for d <= 3, where the smallest
eigenvalue of a condition-1e3 spectrum carries most of ||W|| and the fp16
resolution of S alone moves it by several times 1e-3 (1.3e-2 measured at
d = 3).  Split products round at 2^-22; the ten-step CANS map itself stops
at 3e-5 of the exact root for lambda/L >= 1e-6; the emulation gives at most
4.7e-5 up to condition number 1e4, so MR_CANS_SPLIT is held to 1e-4.  Every
output is checked to be exactly symmetric, finite and unflagged, with the
inverse-root residual ||W S W - I||_F / sqrt(d) computed in float64 by
torch below 5e-2 (f16) or 1e-3 (split).
"""

import numpy as np
import pytest

import oracle
from matrix_roots_amd import binding as B
from matrix_roots_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

TOL = {"f16": 1e-2, "split": 1e-4}
TOL_F16_TINY = 2e-2  # d <= 3
RES = {"f16": 5e-2, "split": 1e-3}


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def spd(d, lo_exp, seed):
    return W.spd_loguniform(d, W.rng_for(90, d, seed, 0), lo_exp, 0.0)


def check(torch, dev, As, eps, normalize, precision, dtype=np.float32, tol=None):
    Ad = [torch.from_numpy(np.ascontiguousarray(a.astype(dtype))).to(dev) for a in As]
    Ws, info = B.inv_sqrt_root_batched(Ad, eps, normalize=normalize, precision=precision)
    torch.cuda.synchronize()
    worst = 0.0
    for i, A in enumerate(As):
        assert info["flags"][i] == 0, (i, info[i])
        assert info["iters"][i] == 10
        ref, rinfo = oracle.inv_sqrt_root(A.astype(dtype).astype(np.float64), eps, normalize)
        assert rinfo["flags"] == 0
        Wg = Ws[i].cpu().numpy()
        assert np.array_equal(Wg, Wg.T) and np.isfinite(Wg).all()
        err = oracle.relative_frobenius(Wg, ref)
        worst = max(worst, err)
        bound = tol or (TOL_F16_TINY if precision == "f16" and A.shape[0] <= 3 else TOL[precision])
        assert err <= bound, (i, A.shape, precision, err)
        S = Ad[i].double()
        S = 0.5 * (S + S.T) / (torch.trace(S) if normalize == "trace" else 1.0)
        S = S + eps * torch.eye(S.shape[0], dtype=torch.float64, device=dev)
        Wt = Ws[i].double()
        r = float(torch.linalg.norm(Wt @ S @ Wt - torch.eye(S.shape[0], dtype=torch.float64, device=dev)))
        assert r / S.shape[0] ** 0.5 <= RES[precision], (i, r)
    return worst, info


@pytest.mark.parametrize("precision", ["f16", "split"])
@pytest.mark.parametrize("d", [1, 7, 64, 130, 257, 300, 320, 520, 640])
def test_sizes_ragged(torch_dev, precision, d):
    """One matrix per call, condition number 1e3, the page's S^(-1/2) (no
    rescale, eps = 0); sizes cover one tile, several tiles and ragged tails,
    16-byte (d % 8 == 0) and element loads, and the direct-to-LDS fp16 core
    (d % 64 == 0) with ragged last tiles (320, 640)."""
    torch, dev = torch_dev
    A = spd(d, -3.0, 0) if d > 1 else np.array([[0.37]], dtype=np.float32)
    worst, _ = check(torch, dev, [A], 0.0, "none", precision)
    print(f"d={d} {precision}: err {worst:.2e}")


@pytest.mark.parametrize("precision", ["f16", "split"])
def test_mixed_batch(torch_dev, precision):
    """Several size classes in one call (both load widths), float32 and
    float64 inputs, condition numbers 1e2..1e3."""
    torch, dev = torch_dev
    As = [spd(d, e, s) for s, (d, e) in enumerate([(256, -3.0), (96, -2.0), (256, -2.5), (200, -3.0), (384, -3.0),
                                                   (33, -1.0)])]
    for dtype in (np.float32, np.float64):
        worst, _ = check(torch, dev, As, 0.0, "none", precision, dtype)
        print(f"mixed {precision} {np.dtype(dtype).name}: err {worst:.2e}")


def test_split_reaches_condition_1e4(torch_dev):
    torch, dev = torch_dev
    As = [spd(384, -4.0, s) for s in range(3)]
    worst, _ = check(torch, dev, As, 0.0, "none", "split")
    print(f"split kappa 1e4: err {worst:.2e}")


@pytest.mark.parametrize("precision", ["f16", "split"])
def test_trace_normalised_grams(torch_dev, precision):
    """Trace-rescaled Grams of MoE-shaped gradients (zero rows) with eps =
    1e-3, left and right, as the OKLS preconditioner would root them."""
    torch, dev = torch_dev
    As = []
    for w in range(3):
        G = W.gradient("moe", w, 1, shape=(384, 192)).astype(np.float64)
        As += [(G @ G.T).astype(np.float32), (G.T @ G).astype(np.float32)]
    worst, info = check(torch, dev, As, 1e-3, "trace", precision)
    for i, A in enumerate(As):
        assert info["scale"][i] == pytest.approx(float(np.trace(A.astype(np.float64))), rel=1e-6)
    print(f"grams {precision}: err {worst:.2e}")


def test_flags_and_special_outputs(torch_dev):
    torch, dev = torch_dev
    d = 136
    good = spd(d, -2.0, 1)
    zero = np.zeros((d, d), np.float32)
    nanm = good.copy()
    nanm[3, 5] = np.nan
    notpd = np.diag(np.linspace(-0.5, 1.0, d)).astype(np.float32)
    Ad = [torch.from_numpy(a).to(dev) for a in (good, zero, nanm, notpd)]
    for eps in (1e-2, 0.0):
        Ws, info = B.inv_sqrt_root_batched(Ad, eps, normalize="trace" if eps else "none")
        f = info["flags"]
        assert f[0] == 0
        assert f[2] == B.MR_INFO_NONFINITE and torch.isnan(Ws[2]).all()
        assert f[3] & B.MR_INFO_NOT_CONVERGED
        if eps:
            assert f[1] == B.MR_INFO_ZERO_TRACE
            assert torch.equal(Ws[1].cpu(), torch.eye(d) * (1.0 / np.sqrt(eps)).astype(np.float32))
        else:
            # no rescale, eps = 0: the zero matrix has no positive bound
            assert f[1] == B.MR_INFO_NOT_PD and torch.isnan(Ws[1]).all()
    # the good matrix is unaffected by its neighbours
    ref, _ = oracle.inv_sqrt_root(good.astype(np.float64), 0.0, "none")
    assert oracle.relative_frobenius(Ws[0].cpu().numpy(), ref) <= TOL["f16"]


def test_strided_output_and_repeat(torch_dev):
    """ld > d for A and W; two calls on one workspace give identical results."""
    torch, dev = torch_dev
    d = 200
    A = spd(d, -3.0, 7)
    big = torch.zeros(d, d + 24, dtype=torch.float32, device=dev)
    big[:, :d] = torch.from_numpy(A).to(dev)
    out = torch.full((d, d + 40), 7.0, dtype=torch.float32, device=dev)
    ws = B.RootWorkspace()
    W1, _ = B.inv_sqrt_root_batched([big[:, :d]], 0.0, Xs=[out[:, :d]], workspace=ws)
    first = out.clone()
    B.inv_sqrt_root_batched([big[:, :d]], 0.0, Xs=[out[:, :d]], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert bool((out[:, d:] == 7.0).all())
    ref, _ = oracle.inv_sqrt_root(A.astype(np.float64), 0.0, "none")
    assert oracle.relative_frobenius(out[:, :d].cpu().numpy(), ref) <= TOL["f16"]
