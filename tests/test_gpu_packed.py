"""Packed symmetric state (MR_PACKED: upper triangle by rows, d(d+1)/2
elements) against full storage, bitwise: the Gram EMA writes exactly the
upper triangle the full path writes, and every root computed from a packed
input equals the one computed from the full copy of the same matrix (the
statistics sum the same values in the same order; the symmetric part of a
packed matrix is its stored value, as (v + v)/2 is for the full one).  The
packed whole step is also held to the fp64 oracle directly (tilderesearch,
"Online KL Shampoo", appendix F, counts a symmetric Kronecker factor as
d(d+1)/2 stored elements)."""

import numpy as np
import pytest

import oracle
import parity
from matrix_roots_amd import binding as B
from matrix_roots_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [(64, 128), (200, 328), (130, 7), (1, 5), (257, 129), (96, 96)]


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def run_grams(torch, dev, dtype, steps=3, beta=0.9):
    """Gram EMAs of the same gradients into full and packed states."""
    Lf = [torch.zeros(m, m, dtype=dtype, device=dev) for m, n in SHAPES]
    Rf = [torch.zeros(n, n, dtype=dtype, device=dev) for m, n in SHAPES]
    Lp = [torch.zeros(m * (m + 1) // 2, dtype=dtype, device=dev) for m, n in SHAPES]
    Rp = [torch.zeros(n * (n + 1) // 2, dtype=dtype, device=dev) for m, n in SHAPES]
    for t in range(1, steps + 1):
        Gs = [torch.from_numpy(W.gradient("w1024", k, t, shape=s)).to(dev) for k, s in enumerate(SHAPES)]
        B.gram_ema_update(Gs, Lf, Rf, beta)
        B.gram_ema_update(Gs, Lp, Rp, beta)
    torch.cuda.synchronize()
    return Lf + Rf, Lp + Rp


@pytest.mark.parametrize("dtype_name", ["float64", "float32"])
def test_gram_ema_packed_bitwise(torch_dev, dtype_name):
    torch, dev = torch_dev
    full, packed = run_grams(torch, dev, getattr(torch, dtype_name))
    for F, P in zip(full, packed):
        assert torch.equal(B.pack_upper(F), P)
        assert torch.equal(B.unpack_upper(P), F)  # the full state is exactly symmetric


@pytest.mark.parametrize("method", ["auto", "newton_f64"])
@pytest.mark.parametrize("normalize", ["trace", "none"])
def test_quarter_root_from_packed_bitwise(torch_dev, method, normalize):
    torch, dev = torch_dev
    full, packed = run_grams(torch, dev, torch.float64)
    eps = 1e-6 if normalize == "trace" else 1e-3
    Xf, info_f = B.inv_quarter_root_batched(full, eps, normalize=normalize, method=method)
    Xp, info_p = B.inv_quarter_root_batched(packed, eps, normalize=normalize, method=method)
    assert (info_f["flags"] == 0).all() and (info_p["flags"] == 0).all()
    for a, b in zip(Xf, Xp):
        assert torch.equal(a, b)
    assert np.array_equal(info_f, info_p)


@pytest.mark.parametrize("precision", ["f16", "split"])
def test_sqrt_root_from_packed_bitwise(torch_dev, precision):
    torch, dev = torch_dev
    full, packed = run_grams(torch, dev, torch.float32)
    Wf, info_f = B.inv_sqrt_root_batched(full, 1e-3, normalize="trace", precision=precision)
    Wp, info_p = B.inv_sqrt_root_batched(packed, 1e-3, normalize="trace", precision=precision)
    for a, b in zip(Wf, Wp):
        assert torch.equal(a, b)
    assert np.array_equal(info_f, info_p)


def test_packed_step_end_to_end(torch_dev):
    """Three steps of the whole preconditioner step on a small transformer-like
    set with packed float64 state give bitwise the updates of full state, and
    the packed run's states, roots and updates match the fp64 oracle run on
    the same gradients (1e-12 on states, 1e-4 on roots, 1e-3 on updates)."""
    torch, dev = torch_dev
    shapes = [(256, 256), (256, 1024), (1024, 256), (200, 136)]
    grads = [[W.gradient("w1024", k, t, shape=s) for k, s in enumerate(shapes)] for t in range(1, 4)]
    refs = [list(oracle.run_sequence([grads[t][k] for t in range(3)], 0.95, 1e-6)) for k in range(len(shapes))]
    outs = []
    for packed in (False, True):
        if packed:
            Ls = [torch.zeros(m * (m + 1) // 2, dtype=torch.float64, device=dev) for m, n in shapes]
            Rs = [torch.zeros(n * (n + 1) // 2, dtype=torch.float64, device=dev) for m, n in shapes]
        else:
            Ls = [torch.zeros(m, m, dtype=torch.float64, device=dev) for m, n in shapes]
            Rs = [torch.zeros(n, n, dtype=torch.float64, device=dev) for m, n in shapes]
        Us = []
        nw = len(shapes)
        for t in range(1, 4):
            Gs = [torch.from_numpy(grads[t - 1][k]).to(dev) for k in range(nw)]
            B.gram_ema_update(Gs, Ls, Rs, 0.95)
            Xs, info = B.inv_quarter_root_batched(Ls + Rs, 1e-6)
            assert (info["flags"] == 0).all()
            Us.append(B.precondition_apply(Xs[:nw], Gs, Xs[nw:]))
            torch.cuda.synchronize()
            if packed:
                for k in range(nw):
                    _, rL, rR, rXL, rXR, rU, flags = refs[k][t - 1]
                    ctx = f"packed step {t} weight {shapes[k]}"
                    parity.assert_state(B.unpack_upper(Ls[k]), rL, 1e-12, ctx + " L")
                    parity.assert_state(B.unpack_upper(Rs[k]), rR, 1e-12, ctx + " R")
                    parity.assert_root(Xs[k], rXL, ctx + " XL")
                    parity.assert_root(Xs[nw + k], rXR, ctx + " XR")
                    parity.assert_update(Us[-1][k], rU, ctx + " U")
        outs.append(Us)
    for Uf, Up in zip(*outs):
        for a, b in zip(Uf, Up):
            assert torch.equal(a, b)
