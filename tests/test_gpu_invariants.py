"""Invariants of the GPU path that hold at any size (and a Theorem-1 closed form).

Each compares the HIP path with itself under a transformation the pages fix
(resume from a state, decode vs scan, chunked vs unchunked) or with a closed
form computed here with numpy.
"""
import numpy as np
import pytest

import oracle
from gpu_util import log, random_problem, rel_l2, run_gpu_scan, run_oracle_scan, to_dev, to_f64

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


def _upload(raw, par, io, dev):
    import torch
    t = {k: to_dev(v, io, dev) for k, v in raw.items()}
    p = {k: (torch.from_numpy(v).to(dev) if v is not None else None) for k, v in par.items()}
    return t, p


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_chunked_equals_unchunked(ss, dev, io):
    """Chunks joined by the (decay, end state) combine reproduce the single pass."""
    import torch
    rng = np.random.default_rng(21)
    raw, par, f64 = random_problem(rng, 2, 192, 16, 4096, io)
    t, p = _upload(raw, par, io, dev)
    outs = {}
    for plan in [(4, 4096), (4, 1024), (4, 256), (2, 512), (1, 64), (4, 2, 4096), (4, 2, 512), (2, 2, 64),
                 (4, 4, 4096), (4, 4, 256)]:
        log("chunked plan %s (%s)" % (plan, io))
        y, hf = ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"], Dskip=p["Dskip"],
                            dt_bias=p["dt_bias"], h0=p["h0"], plan=plan)
        torch.cuda.synchronize()
        outs[plan] = (to_f64(y), to_f64(hf))
    y0, h0 = outs[(4, 4096)]
    yr, hr = run_oracle_scan(oracle.default(), f64, par)
    tol = 1e-5 if io == "f32" else 2e-2
    for plan, (y, hf) in outs.items():
        assert rel_l2(y, yr) <= tol and rel_l2(hf, hr) <= tol, (plan, rel_l2(y, yr), rel_l2(hf, hr))
        assert rel_l2(hf, h0) <= 1e-5, (plan, rel_l2(hf, h0))


def test_split_resume(ss, dev):
    """scan(0:L) = scan(0:L1) then scan(L1:L) from the state reached at L1."""
    import torch
    rng = np.random.default_rng(22)
    raw, par, _ = random_problem(rng, 2, 130, 16, 512, "f32")
    t, p = _upload(raw, par, "f32", dev)
    kw = dict(Dskip=p["Dskip"], dt_bias=p["dt_bias"])
    y, hf = ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"], h0=p["h0"], **kw)
    for L1 in (1, 100, 256, 511):
        s1, s2 = slice(0, L1), slice(L1, None)
        c = {k: (v[..., s1].contiguous(), v[..., s2].contiguous()) for k, v in t.items()}
        ya, ha = ss.scan_fwd(c["x"][0], c["dt"][0], c["B"][0], c["C"][0], p["A"], z=c["z"][0], h0=p["h0"], **kw)
        yb, hb = ss.scan_fwd(c["x"][1], c["dt"][1], c["B"][1], c["C"][1], p["A"], z=c["z"][1], h0=ha, **kw)
        torch.cuda.synchronize()
        assert rel_l2(to_f64(torch.cat([ya, yb], -1)), to_f64(y)) <= 1e-6
        assert rel_l2(to_f64(hb), to_f64(hf)) <= 1e-6


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_steps_equal_scan(ss, dev, io):
    """T single-token updates give the scan's outputs and final state."""
    import torch
    rng = np.random.default_rng(23)
    T = 24
    raw, par, _ = random_problem(rng, 3, 96, 16, T, io)
    t, p = _upload(raw, par, io, dev)
    kw = dict(Dskip=p["Dskip"], dt_bias=p["dt_bias"])
    y, hf = ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"], h0=p["h0"], **kw)
    st = p["h0"].clone()
    ys = []
    for k in range(T):
        ys.append(ss.state_update(st, t["x"][..., k].contiguous(), t["dt"][..., k].contiguous(),
                                  t["B"][..., k].contiguous(), t["C"][..., k].contiguous(), p["A"],
                                  z=t["z"][..., k].contiguous(), **kw))
    torch.cuda.synchronize()
    yd = torch.stack(ys, -1)
    tol = 1e-6 if io == "f32" else 1e-2
    assert rel_l2(to_f64(yd), to_f64(y)) <= tol
    assert rel_l2(to_f64(st), to_f64(hf)) <= 1e-6


@pytest.mark.parametrize("dstate", [1, 2, 4, 8, 16])
def test_decode_matches_oracle(ss, dev, dstate):
    import torch
    rng = np.random.default_rng(24 + dstate)
    raw, par, f64 = random_problem(rng, 5, 77, dstate, 1, "f32")
    t, p = _upload(raw, par, "f32", dev)
    st = p["h0"].clone()
    y = ss.state_update(st, t["x"][..., 0].contiguous(), t["dt"][..., 0].contiguous(), t["B"][..., 0].contiguous(),
                        t["C"][..., 0].contiguous(), p["A"], z=t["z"][..., 0].contiguous(), Dskip=p["Dskip"],
                        dt_bias=p["dt_bias"])
    torch.cuda.synchronize()
    yr, sr = oracle.default().state_update(par["h0"], f64["x"][..., 0], f64["dt"][..., 0], f64["B"][..., 0],
                                           f64["C"][..., 0], par["A"], z=f64["z"][..., 0], Dskip=par["Dskip"],
                                           dt_bias=par["dt_bias"])
    assert rel_l2(to_f64(y), yr) <= 1e-6 and rel_l2(to_f64(st), sr) <= 1e-6


@pytest.mark.parametrize("dstate,optional", [(16, True), (16, False), (4, False), (2, True)])
def test_decode_grid_stride_ragged(ss, dev, dstate, optional):
    """More waves than the bounded grid holds (the grid-stride loop wraps over
    rows), rows that end inside a wave (dim * lanes-per-channel not a multiple of
    64), and the optional z, Dskip and dt_bias present or absent."""
    import torch
    rng = np.random.default_rng(40 + dstate + 100 * optional)
    # waves cover (pair of batch rows, 64-item piece); the grid holds at most
    # 16384 x 4 waves, so an odd batch above 2 x 65536 / pieces makes the loop wrap
    # and ends on a pair of one row
    D = 77
    lanes = dstate // min(dstate, 4)
    pieces = (D * lanes + 63) // 64
    batch = 2 * (65536 // pieces + 50) + 1
    raw, par, f64 = random_problem(rng, batch, D, dstate, 1, "f32", with_z=optional, with_skip=optional,
                                   with_bias=optional)
    t, p = _upload(raw, par, "f32", dev)
    st = p["h0"].clone()
    col = lambda k: t[k][..., 0].contiguous() if k in t else None  # noqa: E731
    y = ss.state_update(st, col("x"), col("dt"), col("B"), col("C"), p["A"], z=col("z"), Dskip=p["Dskip"],
                        dt_bias=p["dt_bias"])
    torch.cuda.synchronize()
    fcol = lambda k: f64[k][..., 0] if k in f64 else None  # noqa: E731
    yr, sr = oracle.default().state_update(par["h0"], fcol("x"), fcol("dt"), fcol("B"), fcol("C"), par["A"],
                                           z=fcol("z"), Dskip=par["Dskip"], dt_bias=par["dt_bias"])
    assert rel_l2(to_f64(y), yr) <= 1e-6 and rel_l2(to_f64(st), sr) <= 1e-6
    # every row, including the last one, was written
    assert np.abs(to_f64(y)[-1] - yr[-1]).max() <= 1e-4 * max(1.0, np.abs(yr[-1]).max())


def test_theorem1_euler_closed_form(ss, dev):
    """N = 1, A = -1, B = C = 1, no skip or gate: h_t = (1 - sigmoid(g_t)) h_(t-1) + softplus(g_t) x_t
    (reader's notes, Theorem 1, in the Euler discretisation the kernel uses)."""
    import torch
    rng = np.random.default_rng(25)
    batch, D, L = 2, 70, 300
    g = (2.0 * rng.standard_normal((batch, D, L))).astype(np.float32)
    x = rng.standard_normal((batch, D, L)).astype(np.float32)
    h0 = rng.standard_normal((batch, D, 1)).astype(np.float32)
    ones = np.ones((batch, 1, L), np.float32)
    y, hf = ss.scan_fwd(torch.from_numpy(x).to(dev), torch.from_numpy(g).to(dev), torch.from_numpy(ones).to(dev),
                        torch.from_numpy(ones).to(dev), -torch.ones(D, 1, device=dev), h0=torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    gd = g.astype(np.float64)
    h = h0[..., 0].astype(np.float64)
    ref = np.empty((batch, D, L))
    for k in range(L):
        keep = 1.0 / (1.0 + np.exp(gd[..., k]))
        h = keep * h + np.logaddexp(0.0, gd[..., k]) * x[..., k]
        ref[..., k] = h
    assert rel_l2(to_f64(y), ref) <= 1e-5 and rel_l2(to_f64(hf)[..., 0], h) <= 1e-5


def test_state_groups_agree_and_runs_are_deterministic(ss, dev):
    import torch
    rng = np.random.default_rng(26)
    raw, par, _ = random_problem(rng, 2, 128, 16, 640, "bf16")
    t, p = _upload(raw, par, "bf16", dev)
    res = []
    for plan in [(1, 640), (2, 640), (4, 2, 640), (4, 640), (4, 640), (2, 2, 640), (1, 2, 640), (4, 4, 640),
                 (4, 4, 640)]:
        y, hf = ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"], Dskip=p["Dskip"],
                            dt_bias=p["dt_bias"], h0=p["h0"], plan=plan)
        torch.cuda.synchronize()
        res.append((y.clone(), hf.clone()))
    assert torch.equal(res[3][0], res[4][0]) and torch.equal(res[3][1], res[4][1])   # bitwise repeatable
    for y, hf in res:
        assert rel_l2(to_f64(hf), to_f64(res[3][1])) <= 1e-5
        assert rel_l2(to_f64(y), to_f64(res[3][0])) <= 1e-2


def test_timing_record(ss, dev):
    import torch
    rng = np.random.default_rng(27)
    raw, par, _ = random_problem(rng, 1, 64, 16, 256, "bf16")
    t, p = _upload(raw, par, "bf16", dev)
    ss.ss_timing_reset()
    ss.ss_timing_enable(True)
    for _ in range(3):
        ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"])
    ss.ss_timing_enable(False)
    ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"])
    ms, n = ss.ss_timing_read()
    ss.ss_timing_reset()
    assert n == 3 and ms > 0.0
