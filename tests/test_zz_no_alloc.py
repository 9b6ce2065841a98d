"""ss_scan_fwd_noalloc (the forward scan with its scratch in a static device
array, for callers that cannot allocate) through the C ABI, against
ss_scan_fwd_ex with a caller-owned workspace: the same kernels on the same
inputs, so the outputs must agree bit for bit.  Two calls in a row, the second
with a smaller input (the array keeps the first call's contents), a chunked
plan, a graph capture, and the size limit."""
import ctypes

import numpy as np
import pytest

from gpu_util import log, random_problem, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def b():
    from selective_state_space_62_amd import binding
    return binding


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _problem(dev, seed, batch, D, N, L, io):
    import torch
    rng = np.random.default_rng(seed)
    raw, par, _ = random_problem(rng, batch, D, N, L, io)
    t = {k: to_dev(v, io, dev) for k, v in raw.items()}
    p = {k: (torch.from_numpy(v).to(dev) if v is not None else None) for k, v in par.items()}
    return t, p


def _call(b, dev, t, p, io, plan=None, flags=0, noalloc=True, stream=None):
    """One forward call through the C ABI; returns (y, h_final)."""
    import torch
    batch, D, L = t["x"].shape
    N = p["A"].shape[1]
    code = b.SS_BF16 if io == "bf16" else b.SS_F32
    y = torch.full_like(t["x"], float("nan"))
    hf = torch.full((batch, D, N), float("nan"), dtype=torch.float32, device=dev)
    args = [_ptr(t["x"]), _ptr(t["dt"]), _ptr(t["z"]), _ptr(t["B"]), _ptr(t["C"]), _ptr(p["A"]), _ptr(p["Dskip"]),
            _ptr(p["dt_bias"]), _ptr(p["h0"]), _ptr(y), _ptr(hf), None]
    s = ctypes.c_void_p(stream if stream is not None else torch.cuda.current_stream().cuda_stream)
    if noalloc:
        b.ss_scan_fwd_noalloc(batch, D, N, L, code, flags, *args, plan=plan, stream=s)
    else:
        nbytes = max(b.ss_scan_fwd_workspace_bytes(batch, D, N, L, code, plan), 256)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        b.ss_scan_fwd_ex(batch, D, N, L, code, flags, *args, _ptr(ws), nbytes, plan=plan, stream=s)
        torch.cuda.synchronize()
        del ws
    torch.cuda.synchronize()
    return y, hf


def _same(a, c):
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), c.view(torch.int16))
    return torch.equal(a.view(torch.int32), c.view(torch.int32))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_two_calls_match_workspace_call(b, dev, io):
    """A large call, then a smaller one on the same array: each equals the call
    with a workspace, bit for bit (also under the zero-order-hold flag)."""
    for seed, (batch, D, N, L), flags in ((1, (4, 512, 16, 2048), 0), (2, (2, 100, 16, 515), 0),
                                          (3, (1, 70, 8, 333), b.SS_FLAG_ZOH)):
        log("no-alloc %s %s flags %d" % (io, (batch, D, N, L), flags))
        t, p = _problem(dev, seed, batch, D, N, L, io)
        y1, h1 = _call(b, dev, t, p, io, flags=flags, noalloc=True)
        y0, h0 = _call(b, dev, t, p, io, flags=flags, noalloc=False)
        assert _same(y1, y0) and _same(h1, h0), (batch, D, N, L)


def test_noalloc_chunked_plan(b, dev):
    """A chunked plan keeps its chunk aggregates in the static array too."""
    t, p = _problem(dev, 4, 1, 64, 16, 20000, "bf16")
    for plan in ((4, 2, 4096), (4, 2, 1024)):
        log("no-alloc chunked plan %s" % (plan,))
        y1, h1 = _call(b, dev, t, p, "bf16", plan=plan, noalloc=True)
        y0, h0 = _call(b, dev, t, p, "bf16", plan=plan, noalloc=False)
        assert _same(y1, y0) and _same(h1, h0), plan


def test_noalloc_rejects_oversized_calls(b, dev):
    """A shape whose scratch exceeds the array is refused before any device work."""
    import torch
    limit = b.ss_scan_fwd_noalloc_max_bytes()
    assert limit == 32 << 20
    batch, D, N, L = 1, 2048, 16, 1 << 20   # the million-token plan: 256 chunks, 69 MB of chunk aggregates
    need = b.ss_scan_fwd_workspace_bytes(batch, D, N, L, b.SS_BF16, None)
    assert need > limit
    x = torch.zeros((1, 16), dtype=torch.bfloat16, device=dev)   # never read: the size check comes first
    A = torch.zeros((D, N), dtype=torch.float32, device=dev)
    st = b.lib.ss_scan_fwd_noalloc(batch, D, N, L, b.SS_BF16, 0, _ptr(x), _ptr(x), None, _ptr(x), _ptr(x), _ptr(A),
                                   None, None, None, _ptr(x), None, None, None, None)
    assert st == b.SS_ERR_WORKSPACE
    assert "scratch" in b.last_error()


def test_noalloc_in_graph_capture(b, dev):
    """Captured once and replayed: every replay equals the eager workspace call,
    with other eager work and synchronisations between the replays."""
    import torch
    t, p = _problem(dev, 5, 2, 96, 16, 512, "bf16")
    y_ref, h_ref = _call(b, dev, t, p, "bf16", noalloc=False)
    batch, D, L = t["x"].shape
    N = p["A"].shape[1]
    y = torch.empty_like(t["x"])
    hf = torch.empty((batch, D, N), dtype=torch.float32, device=dev)
    args = [_ptr(t["x"]), _ptr(t["dt"]), _ptr(t["z"]), _ptr(t["B"]), _ptr(t["C"]), _ptr(p["A"]), _ptr(p["Dskip"]),
            _ptr(p["dt_bias"]), _ptr(p["h0"]), _ptr(y), _ptr(hf), None]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # first call on the device (address lookup) outside the capture
        b.ss_scan_fwd_noalloc(batch, D, N, L, b.SS_BF16, 0, *args, stream=ctypes.c_void_p(side.cuda_stream))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.ss_scan_fwd_noalloc(batch, D, N, L, b.SS_BF16, 0, *args,
                              stream=ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    for i in range(4):
        y.zero_()
        hf.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert _same(y, y_ref) and _same(hf, h_ref), "replay %d" % i
        _call(b, dev, t, p, "bf16", noalloc=True)   # eager use of the same array between replays
    log("no-alloc graph: 4 replays equal the eager result")
