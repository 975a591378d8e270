"""GPU parity at the workloads' full sizes, in the same batched launch
configuration as bench.py (every weight of a step in one call of each entry
point), checked on sampled outputs the fp64 oracle computes one by one, and
on every output through properties that hold at any size:

* relative Frobenius error <= 1e-4 per sampled root, <= 1e-3 per sampled
  update direction (the EMA-Gram page's comparison, section "Results");
* every root: exactly symmetric, finite, no flags, and the symmetric
  residual ||X^2 (A/s + eps I) X^2 - I||_F / sqrt(d) <= 1e-3, computed in
  float64 with torch's own matmul (the inverse-root equation the OKLS page,
  appendix E, calls an explicit, measurable residual).

The width-2048 workload runs on a declared subset (layers 0 and 23, all six
weights, its 3 steps): generating all 432 Haar-factor gradients on the host
and eigendecomposing 8192 x 8192 Grams in the oracle would take tens of
minutes.
"""

import numpy as np
import pytest

import oracle
from matrix_roots_amd import binding as B
from matrix_roots_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

ROOT_TOL = 1e-4
UPDATE_TOL = 1e-3
RESID_RMS_TOL = 1e-3


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def sym_residual_rms(torch, A, X, eps, normalize="trace"):
    """||X^2 (A/s + eps I) X^2 - I||_F / sqrt(d) in float64 (torch matmul)."""
    A = A.to(torch.float64)
    X = X.to(torch.float64)
    d = A.shape[0]
    s = torch.trace(A) if normalize == "trace" else torch.tensor(1.0, dtype=torch.float64, device=A.device)
    Bm = 0.5 * (A + A.T) / s + eps * torch.eye(d, dtype=torch.float64, device=A.device)
    X2 = X @ X
    R = X2 @ Bm @ X2 - torch.eye(d, dtype=torch.float64, device=A.device)
    return float(torch.linalg.norm(R) / d ** 0.5)


def run_and_check(torch, dev, workload, weights, steps, samples, last_step_samples=()):
    """Run `steps` steps of `workload` restricted to `weights` (indices into the
    workload's weight list), all of them batched per call; compare the
    `samples` (subset of weights) against the oracle at every step, the
    `last_step_samples` at the last step only (the oracle runs their Gram EMA
    alone before that step, then the whole step), and every root through the
    properties above at the last step."""
    wl = W.WORKLOADS[workload]
    shapes = [wl.shapes[w][1:] for w in weights]
    nw = len(weights)
    Ls = [torch.zeros(m, m, dtype=torch.float64, device=dev) for m, n in shapes]
    Rs = [torch.zeros(n, n, dtype=torch.float64, device=dev) for m, n in shapes]
    Us = [torch.empty(m, n, dtype=torch.float32, device=dev) for m, n in shapes]
    ws = B.RootWorkspace()
    got = {w: [] for w in samples}
    grads_host = {w: [] for w in list(samples) + list(last_step_samples)}
    last = {}
    worst = [0.0, 0.0, 0.0]
    for t in range(1, steps + 1):
        Gh = [W.gradient(workload, w, t) for w in weights]
        Gd = [torch.from_numpy(g).to(dev) for g in Gh]
        B.gram_ema_update(Gd, Ls, Rs, wl.beta)
        Xs, info = B.inv_quarter_root_batched(Ls + Rs, wl.eps, normalize=wl.normalize, workspace=ws)
        B.precondition_apply(Xs[:nw], Gd, Xs[nw:], Us=Us)
        torch.cuda.synchronize()
        assert (info["flags"] == 0).all(), (t, info[info["flags"] != 0])
        for w in samples:
            k = weights.index(w)
            got[w].append((Xs[k].cpu().numpy(), Xs[nw + k].cpu().numpy(), Us[k].cpu().numpy(),
                           Ls[k].cpu().numpy(), Rs[k].cpu().numpy()))
        for w in grads_host:
            grads_host[w].append(Gh[weights.index(w)])
        if t == steps:
            for w in last_step_samples:
                k = weights.index(w)
                last[w] = (Xs[k].cpu().numpy(), Xs[nw + k].cpu().numpy(), Us[k].cpu().numpy())
        if t == steps:
            for k, (A, X) in enumerate(zip(Ls + Rs, Xs)):
                assert torch.equal(X, X.T) and bool(torch.isfinite(X).all()), k
                r = sym_residual_rms(torch, A, X, wl.eps)
                worst[2] = max(worst[2], r)
                assert r <= RESID_RMS_TOL, (k, A.shape, r)
        del Xs
    for w in samples:
        refs = list(oracle.run_sequence(grads_host[w], wl.beta, wl.eps, wl.normalize))
        for t, (XL, XR, U, L, R) in enumerate(got[w]):
            _, rL, rR, rXL, rXR, rU, flags = refs[t]
            assert flags == 0
            assert oracle.relative_frobenius(L, rL) <= 1e-12 and oracle.relative_frobenius(R, rR) <= 1e-12
            e_root = max(oracle.relative_frobenius(XL, rXL), oracle.relative_frobenius(XR, rXR))
            e_u = oracle.relative_frobenius(U, rU)
            worst[0] = max(worst[0], e_root)
            worst[1] = max(worst[1], e_u)
            assert e_root <= ROOT_TOL and e_u <= UPDATE_TOL, (workload, w, t + 1, e_root, e_u)
    for w in last_step_samples:
        G = grads_host[w]
        m, n = G[0].shape
        rL, rR = np.zeros((m, m)), np.zeros((n, n))
        for g in G[:-1]:
            rL, rR = oracle.gram_ema_update(rL, rR, g, wl.beta)
        _, _, rXL, rXR, rU, flags = oracle.preconditioner_step(rL, rR, G[-1], wl.beta, wl.eps, wl.normalize)
        assert flags == 0
        XL, XR, U = last[w]
        e_root = max(oracle.relative_frobenius(XL, rXL), oracle.relative_frobenius(XR, rXR))
        e_u = oracle.relative_frobenius(U, rU)
        print(f"{workload} weight {w} ({m}x{n}) step {steps}: root err {e_root:.2e}, update err {e_u:.2e}",
              flush=True)
        worst[0] = max(worst[0], e_root)
        worst[1] = max(worst[1], e_u)
        assert e_root <= ROOT_TOL and e_u <= UPDATE_TOL, (workload, w, steps, e_root, e_u)
    print(f"{workload}: worst root err {worst[0]:.2e}, update err {worst[1]:.2e}, "
          f"residual rms {worst[2]:.2e}")


def test_w1024_full(torch_dev):
    """All 48 weights, 5 steps; oracle on L0.q (1024x1024) and L3.up (1024x4096)."""
    torch, dev = torch_dev
    wl = W.WORKLOADS["w1024"]
    names = [s[0] for s in wl.shapes]
    run_and_check(torch, dev, "w1024", list(range(len(wl.shapes))), wl.steps,
                  [names.index("L0.q"), names.index("L3.up")])


def test_moe_full(torch_dev):
    """All 128 expert weights (64 of 3072x1536, 64 of 1536x3072) in one batch,
    4 steps; oracle on E0.in and E63.out."""
    torch, dev = torch_dev
    wl = W.WORKLOADS["moe"]
    names = [s[0] for s in wl.shapes]
    run_and_check(torch, dev, "moe", list(range(len(wl.shapes))), wl.steps,
                  [names.index("E0.in"), names.index("E63.out")])


def test_w2048_layers_0_and_23(torch_dev):
    """Layers 0 and 23 of the width-2048 set (2048x2048, 2048x8192,
    8192x2048), 3 steps; oracle on L0.q at every step, and on L0.up (its
    8192 x 8192 right root, of rank-6144 Gram plus eps, and its 2048 x 8192
    update direction) at step 3."""
    torch, dev = torch_dev
    wl = W.WORKLOADS["w2048"]
    names = [s[0] for s in wl.shapes]
    weights = [i for i, n in enumerate(names) if n.startswith("L0.") or n.startswith("L23.")]
    run_and_check(torch, dev, "w2048", weights, wl.steps, [names.index("L0.q")],
                  last_step_samples=[names.index("L0.up")])


def test_w2048_one_8192_root_against_oracle(torch_dev):
    """One 8192 x 8192 right Gram (L0.up after step 1) against the oracle."""
    torch, dev = torch_dev
    wl = W.WORKLOADS["w2048"]
    names = [s[0] for s in wl.shapes]
    G = W.gradient("w2048", names.index("L0.up"), 1)
    Gd = torch.from_numpy(G).to(dev)
    L = torch.zeros(2048, 2048, dtype=torch.float64, device=dev)
    R = torch.zeros(8192, 8192, dtype=torch.float64, device=dev)
    B.gram_ema_update([Gd], [L], [R], wl.beta)
    Xs, info = B.inv_quarter_root_batched([R], wl.eps)
    assert info["flags"][0] == 0
    # the oracle forms its own Gram from the same float32 gradient
    _, Ro = oracle.gram_ema_update(np.zeros((2048, 2048)), np.zeros((8192, 8192)), G, wl.beta)
    assert oracle.relative_frobenius(R.cpu().numpy(), Ro) <= 1e-12
    ref, rinfo = oracle.inv_quarter_root(Ro, wl.eps)
    err = oracle.relative_frobenius(Xs[0].cpu().numpy(), ref)
    print(f"8192 root err {err:.2e}, iters {info['iters'][0]}, fp64 {info['fp64_iters'][0]}")
    assert err <= ROOT_TOL, err


@pytest.mark.parametrize("eps", W.WORKLOADS["illcond"].eps_list)
def test_illcond_full(torch_dev, eps):
    """All 256 ill-conditioned 512 x 512 matrices in one call per eps (no
    rescale), every root against the oracle."""
    torch, dev = torch_dev
    A = W.illcond_batch()
    Ad = [torch.from_numpy(a).to(dev) for a in A]
    Xs, info = B.inv_quarter_root_batched(Ad, eps, normalize="none")
    assert (info["flags"] == 0).all(), info[info["flags"] != 0]
    worst = 0.0
    for i in range(len(A)):
        ref, rinfo = oracle.inv_quarter_root(A[i].astype(np.float64), eps, "none")
        assert rinfo["flags"] == 0
        X = Xs[i].cpu().numpy()
        assert np.array_equal(X, X.T)
        err = oracle.relative_frobenius(X, ref)
        worst = max(worst, err)
        assert err <= ROOT_TOL, (i, eps, err)
    print(f"illcond eps={eps:g}: worst root err {worst:.2e}, iters {info['iters'].max()}, "
          f"fp64 {info['fp64_iters'].max()}")


def test_inv_sqrt_8192_batch4(torch_dev):
    """The inverse square root at the OKLS page's benchmark shape (4 SPD
    matrices of 8192 x 8192 in one call, as bench.py --workload cans8192
    times it; S = G G^T / 8192 + 4e-3 I, condition number about 1e3), both
    precisions: every root symmetric, finite, unflagged, with ||W S W - I||_F
    / sqrt(d) below the small-size bound; the first against the oracle
    (relative Frobenius error within the small-size tolerances: 2e-2 fp16,
    1e-4 split)."""
    torch, dev = torch_dev
    d, eps = 8192, 4e-3
    rng = W.rng_for(91, 0)
    As = []
    for _ in range(4):
        G = rng.standard_normal((d, d), dtype=np.float32)
        As.append((G @ G.T) / np.float32(d))
    Ad = [torch.from_numpy(a).to(dev) for a in As]
    ref, rinfo = oracle.inv_sqrt_root(As[0].astype(np.float64), eps, "none")
    assert rinfo["flags"] == 0
    eye = torch.eye(d, dtype=torch.float64, device=dev)
    for precision, tol, res_tol in (("f16", 2e-2, 5e-2), ("split", 1e-4, 1e-3)):
        Ws, info = B.inv_sqrt_root_batched(Ad, eps, normalize="none", precision=precision)
        torch.cuda.synchronize()
        assert (info["flags"] == 0).all(), info
        worst = 0.0
        for A, Wd in zip(Ad, Ws):
            assert torch.equal(Wd, Wd.T) and bool(torch.isfinite(Wd).all())
            S = 0.5 * (A.double() + A.double().T) + eps * eye
            Wt = Wd.double()
            r = float(torch.linalg.norm(Wt @ S @ Wt - eye)) / d ** 0.5
            worst = max(worst, r)
            assert r <= res_tol, (precision, r)
        err = oracle.relative_frobenius(Ws[0].cpu().numpy(), ref)
        print(f"8192 x4 {precision}: err {err:.2e}, residual rms {worst:.2e}")
        assert err <= tol, (precision, err)
        del Ws


def test_polar_moe_share(torch_dev):
    """All 128 expert gradients of the MoE share in one polar_cans_batched
    call (as bench.py --workload polar_moe times it), both precisions: every
    output finite and unflagged, E0.in and E63.out against the oracle within
    the small-size tolerances (1e-2 fp16, 5e-5 split)."""
    torch, dev = torch_dev
    wl = W.WORKLOADS["moe"]
    names = [s[0] for s in wl.shapes]
    Gh = [W.gradient("moe", w, 1) for w in range(len(names))]
    Gd = [torch.from_numpy(g).to(dev) for g in Gh]
    samples = [names.index("E0.in"), names.index("E63.out")]
    refs = {k: oracle.polar_cans(Gh[k].astype(np.float64))[0] for k in samples}
    for precision, tol in (("f16", 1e-2), ("split", 5e-5)):
        Os, info = B.polar_cans_batched(Gd, precision=precision)
        torch.cuda.synchronize()
        assert (info["flags"] == 0).all(), info
        assert all(bool(torch.isfinite(O).all()) for O in Os)
        for k in samples:
            err = oracle.relative_frobenius(Os[k].cpu().numpy(), refs[k])
            print(f"polar moe {precision} {names[k]}: err {err:.2e}")
            assert err <= tol, (precision, names[k], err)
        del Os
