"""The seeded input generators: shapes, dtypes and the structure each
workload's recipe states (rank, zero rows, singular-value decay), for the
host draws and for the device-drawn variant (run here on the CPU device)."""

import numpy as np
import pytest
import torch

from matrix_roots_amd import workloads as W


def test_host_draws_are_pure_functions_of_their_key():
    a = W.gradient("w1024", 3, 2, shape=(64, 96))
    b = W.gradient("w1024", 3, 2, shape=(64, 96))
    c = W.gradient("w1024", 3, 3, shape=(64, 96))
    assert a.dtype == np.float32 and np.array_equal(a, b) and not np.array_equal(a, c)


@pytest.mark.parametrize("source", ["host", "device"])
def test_structure(source):
    def draw(wl, i, shape):
        if source == "host":
            return torch.from_numpy(W.gradient(wl, i, 1, shape=shape))
        return W.gradient_device(wl, i, 1, "cpu", shape=shape)

    g = draw("toy", 0, None)
    assert g.shape == (64, 128) and g.dtype == torch.float32
    # rank 32 plus 0.1-scaled noise: a sharp drop after the 32nd singular value
    s = torch.linalg.svdvals(draw("w1024", 4, (128, 256)).double())
    assert s[31] > 5 * s[32]
    # exactly floor(0.3 m) zero rows
    g = draw("moe", 0, (100, 40))
    assert int((g.abs().sum(1) == 0).sum()) == 30
    # sigma_i = i^-0.7 with orthonormal factors
    s = torch.linalg.svdvals(draw("w2048", 0, (96, 160)).double())
    expect = torch.arange(1, 97, dtype=torch.float64) ** -0.7
    assert torch.allclose(s, expect, rtol=1e-5, atol=1e-6)


def test_device_stream_is_seeded_and_distinct_from_host():
    a = W.gradient_device("moe", 5, 2, "cpu", shape=(32, 16))
    b = W.gradient_device("moe", 5, 2, "cpu", shape=(32, 16))
    assert torch.equal(a, b)
    assert not torch.equal(a, torch.from_numpy(W.gradient("moe", 5, 2, shape=(32, 16))))
