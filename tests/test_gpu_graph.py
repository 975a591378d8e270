"""One whole preconditioner step (Gram EMA, inverse quarter roots, apply)
captured in a HIP graph through torch.cuda.graph and replayed.  With a
caller workspace the entry points only enqueue kernels (no allocation, no
synchronisation, no memset nodes), so a graph replays the same kernels on
the same buffers: every replay, with eager work and synchronisations
between replays, must equal the eager step bit for bit."""

import pytest

from matrix_roots_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def test_step_graph_replays_match_eager(torch_dev):
    torch, dev = torch_dev
    # Jacobi (24), narrow split tiles (48, 96, 160, 256 ragged in tiles), the
    # wide split tile (1024)
    shapes = [(24, 48), (96, 160), (256, 64), (1024, 96)]
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    grads = [torch.randn(m, n, generator=g, device=dev, dtype=torch.float32) for m, n in shapes]
    Ls = [torch.zeros(m, m, dtype=torch.float64, device=dev) for m, _ in shapes]
    Rs = [torch.zeros(n, n, dtype=torch.float64, device=dev) for _, n in shapes]
    Xs = [torch.empty(S.shape[0], S.shape[0], dtype=torch.float32, device=dev) for S in Ls + Rs]
    Us = [torch.empty_like(G) for G in grads]
    info = torch.zeros(B.ROOT_INFO_BYTES * len(Xs), dtype=torch.uint8, device=dev)
    ws = B.RootWorkspace()

    def step():
        B.gram_ema_update(grads, Ls, Rs, 0.95)
        B.inv_quarter_root_batched(Ls + Rs, 1e-6, Xs=Xs, workspace=ws, return_info=False, info_out=info)
        B.precondition_apply(Xs[:len(shapes)], grads, Xs[len(shapes):], Us=Us)

    # two eager steps (the workspace reaches its size), then the reference step
    step()
    step()
    torch.cuda.synchronize()
    start = [S.clone() for S in Ls + Rs]
    step()
    torch.cuda.synchronize()
    ref_states = [S.clone() for S in Ls + Rs]
    ref_X = [X.clone() for X in Xs]
    ref_U = [U.clone() for U in Us]
    ref_info = info.clone()
    assert (B.decode_info(info, len(Xs))["flags"] == 0).all()

    for S, S0 in zip(Ls + Rs, start):
        S.copy_(S0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    other = [torch.randn(200, 200, generator=g, device=dev, dtype=torch.float64) for _ in range(2)]
    other = [A @ A.T for A in other]
    for rep in range(3):
        for S, S0 in zip(Ls + Rs, start):
            S.copy_(S0)
        for X in Xs:
            X.fill_(float("nan"))
        for U in Us:
            U.fill_(float("nan"))
        info.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (S, R) in enumerate(zip(Ls + Rs, ref_states)):
            assert torch.equal(S, R), (rep, "state", k)
        for k, (X, R) in enumerate(zip(Xs, ref_X)):
            assert torch.equal(X, R), (rep, "root", k)
        for k, (U, R) in enumerate(zip(Us, ref_U)):
            assert torch.equal(U, R), (rep, "update", k)
        assert torch.equal(info, ref_info), rep
        # eager work of the library between replays
        B.inv_quarter_root_batched(other, 1e-6)
        torch.cuda.synchronize()
