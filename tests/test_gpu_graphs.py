"""The library's calls inside HIP graphs: captured once, replayed many times.

Serving loops capture a decode step (or a prefill scan) once and replay it.  The
library's calls only launch kernels (no allocation, no memset), so they can be
captured; every replay must give the eager result, also with other eager work
and synchronisations between the replays.
"""
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
def ss():
    import selective_state_space_62_amd as m
    return m


def test_scan_graph_replays_match_eager(ss, dev):
    import torch
    rng = np.random.default_rng(61)
    batch, D, N, L = 2, 96, 16, 512
    raw, par, _ = random_problem(rng, batch, D, N, L, "bf16")
    t = {k: to_dev(v, "bf16", dev) for k, v in raw.items()}
    p = {k: torch.from_numpy(v).to(dev) for k, v in par.items()}
    ws = torch.empty(max(ss.workspace_bytes(batch, D, N, L, torch.bfloat16), 256), dtype=torch.uint8, device=dev)
    y = torch.empty_like(t["x"])
    hf = torch.empty((batch, D, N), dtype=torch.float32, device=dev)
    kw = dict(z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"], h0=p["h0"], workspace=ws, y=y, h_final=hf)
    ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], **kw)
    torch.cuda.synchronize()
    y_ref, hf_ref = y.clone(), hf.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the capture stream
        ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], **kw)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], **kw)
    for i in range(4):
        y.zero_()
        hf.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hf, hf_ref), "replay %d" % i
        # unrelated eager work between replays
        ss.scan_fwd(t["x"], t["dt"], t["C"], t["B"], p["A"], z=t["z"])
        torch.cuda.synchronize()
    log("scan graph: 4 replays equal the eager result")


def test_decode_graph_steps_match_eager(ss, dev):
    import torch
    rng = np.random.default_rng(62)
    batch, D, N = 64, 256, 16
    raw, par, _ = random_problem(rng, batch, D, N, 1, "bf16")
    t = {k: to_dev(v[..., 0].copy(), "bf16", dev) for k, v in raw.items()}
    p = {k: torch.from_numpy(v).to(dev) for k, v in par.items()}
    kw = dict(z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"])
    # eager: 5 steps from h0
    st_e = p["h0"].clone()
    ys_e = []
    for _ in range(5):
        ys_e.append(ss.state_update(st_e, t["x"], t["dt"], t["B"], t["C"], p["A"], **kw).clone())
    torch.cuda.synchronize()
    # graph: one captured step replayed 5 times on a state buffer
    st_g = p["h0"].clone()
    y_g = torch.empty_like(t["x"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tmp = st_g.clone()
        ss.state_update(tmp, t["x"], t["dt"], t["B"], t["C"], p["A"], y=y_g, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ss.state_update(st_g, t["x"], t["dt"], t["B"], t["C"], p["A"], y=y_g, **kw)
    st_g.copy_(p["h0"])   # capture does not run the step
    for i in range(5):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, ys_e[i]), "step %d" % i
    assert torch.equal(st_g, st_e)
    log("decode graph: 5 replayed steps equal 5 eager steps")
