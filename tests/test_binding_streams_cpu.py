"""The binding marks the buffers it allocates as in use on the caller's
stream (CPU only: a stand-in library and stand-in tensors record the calls).

When a call is enqueued on a stream other than torch's current one, the
workspace, info buffer and any outputs the binding allocated come from the
caching allocator on the current stream; without record_stream they could be
handed out again while the library's kernels still use them.
"""

import ctypes

import pytest

from matrix_roots_amd import binding as B


class FakeTensor:
    def __init__(self, shape, dtype="torch.float32", device="cuda:0"):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = device
        self.recorded = []

    def dim(self):
        return len(self.shape)

    def stride(self, k):
        return (self.shape[1], 1)[k] if len(self.shape) == 2 else 1

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def data_ptr(self):
        return 4096 * (id(self) % 1000 + 1)

    def record_stream(self, stream):
        self.recorded.append(stream)


class FakeStream:
    cuda_stream = 1234


class FakeLib:
    """Accepts every call; workspace queries ask for 1 KiB."""

    def __getattr__(self, name):
        if name.endswith("_workspace"):
            return lambda *a: 1024
        return lambda *a: 0


class FakeWorkspace:
    def __init__(self):
        self.buf = FakeTensor((1024,), "torch.uint8")
        self.info = FakeTensor((B.ROOT_INFO_BYTES * 8,), "torch.uint8")

    def get(self, nbytes, count, device):
        return self.buf, self.info


@pytest.fixture
def fake(monkeypatch):
    monkeypatch.setattr(B, "_lib", FakeLib())
    created = []

    def workspace(nbytes, device):
        t = FakeTensor((nbytes,), "torch.uint8")
        created.append(t)
        return t

    monkeypatch.setattr(B, "_workspace", workspace)
    # the null stream stands for torch's current one (no device here)
    monkeypatch.setattr(B, "_stream", lambda stream: 0 if stream is None else int(stream.cuda_stream))
    return created


@pytest.mark.parametrize("entry", ["inv_quarter_root_batched", "inv_sqrt_root_batched"])
def test_root_buffers_recorded_on_the_call_stream(fake, entry):
    s = FakeStream()
    ws = FakeWorkspace()
    As = [FakeTensor((8, 8)), FakeTensor((8, 8))]
    Xs = [FakeTensor((8, 8)), FakeTensor((8, 8))]
    getattr(B, entry)(As, 1e-6, Xs=Xs, workspace=ws, stream=s, return_info=False)
    assert ws.buf.recorded == [s] and ws.info.recorded == [s]
    assert all(x.recorded == [] for x in Xs)  # the caller's own outputs are the caller's business


def test_root_buffers_not_recorded_on_the_current_stream(fake):
    ws = FakeWorkspace()
    As = [FakeTensor((8, 8))]
    B.inv_quarter_root_batched(As, 1e-6, Xs=[FakeTensor((8, 8))], workspace=ws, stream=None, return_info=False)
    assert ws.buf.recorded == [] and ws.info.recorded == []


def test_polar_buffers_recorded(fake):
    s = FakeStream()
    ws = FakeWorkspace()
    Gs = [FakeTensor((8, 4))]
    B.polar_cans_batched(Gs, Os=[FakeTensor((8, 4))], workspace=ws, stream=s, return_info=False)
    assert ws.buf.recorded == [s] and ws.info.recorded == [s]


def test_apply_workspace_recorded(fake):
    s = FakeStream()
    Gs = [FakeTensor((8, 4))]
    B.precondition_apply([FakeTensor((8, 8))], Gs, [FakeTensor((4, 4))], Us=[FakeTensor((8, 4))], stream=s)
    assert len(fake) == 1 and fake[0].recorded == [s]


def test_hyperball_workspace_recorded(fake):
    s = FakeStream()
    B.hyperball_update_batched([FakeTensor((8, 4))], [FakeTensor((8, 4))], 0.1, stream=s)
    assert len(fake) == 1 and fake[0].recorded == [s]


def test_fake_library_is_not_the_real_one(fake):
    assert not isinstance(B.library(), ctypes.CDLL)
