"""dt shared by a row's channels (SS_FLAG_DT_PER_ROW), on the GPU.

The selective SSM's Delta is the softplus of a parameter plus a projection of
the input broadcast over channels (reader's notes, kurisu.si, "What they did",
Selective SSM item).  With dt given per (row, token), the result must be that of
the general call with dt repeated across channels (bit for bit: the kernels read
the same values), and the oracle's with dt expanded.
"""
import zlib

import numpy as np
import pytest

import oracle
from gpu_util import log, random_problem, rel_l2, to_dev, to_f64
from workloads import inputs

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


def _row_dt(rng, batch, L, io):
    v = (0.5 * rng.standard_normal((batch, L))).astype(np.float32)
    return v if io == "f32" else inputs.f32_to_bf16_bits(v)


CASES = [("f32", False, (2, 77, 16, 130), None), ("bf16", False, (2, 96, 16, 300), None),
         ("f32", True, (1, 40, 8, 67), None), ("bf16", False, (1, 64, 16, 20000), (4, 2, 4096)),
         ("f32", False, (3, 20, 4, 9), (2, 1, 16))]


@pytest.mark.parametrize("io,zoh,shape,plan", CASES, ids=["%s-%s-%s" % (c[0], "zoh" if c[1] else "euler",
                                                                          "x".join(map(str, c[2]))) for c in CASES])
def test_scan_dt_per_row(ss, dev, io, zoh, shape, plan):
    import torch
    batch, D, N, L = shape
    rng = np.random.default_rng(zlib.crc32(repr((io, zoh, shape)).encode()))
    raw, par, f64 = random_problem(rng, batch, D, N, L, io)
    dt_row = _row_dt(rng, batch, L, io)
    dt_full = np.ascontiguousarray(np.broadcast_to(dt_row[:, None, :], (batch, D, L)))
    t = {k: to_dev(v, io, dev) for k, v in raw.items()}
    p = {k: torch.from_numpy(v).to(dev) for k, v in par.items()}
    kw = dict(z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"], h0=p["h0"], plan=plan, zoh=zoh)
    y1, h1 = ss.scan_fwd(t["x"], to_dev(dt_row, io, dev), t["B"], t["C"], p["A"], **kw)
    y2, h2 = ss.scan_fwd(t["x"], to_dev(dt_full, io, dev), t["B"], t["C"], p["A"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    yr, hr = oracle.default().scan(f64["x"], inputs.raw_to_f64(dt_full, io), f64["B"], f64["C"], par["A"],
                                   z=f64["z"], Dskip=par["Dskip"], dt_bias=par["dt_bias"], h0=par["h0"], zoh=zoh)
    ey, eh = rel_l2(to_f64(y1), yr), rel_l2(to_f64(h1), hr)
    log("dt per row %s zoh=%s %s: rel-L2 y %.3e h %.3e" % (io, zoh, shape, ey, eh))
    assert ey <= (1e-5 if io == "f32" else 2e-2) and eh <= 1e-5


@pytest.mark.parametrize("io,zoh", [("f32", False), ("bf16", True)])
def test_decode_dt_per_row(ss, dev, io, zoh):
    import torch
    rng = np.random.default_rng(51 + zoh)
    batch, D, N = 300, 77, 16
    raw, par, f64 = random_problem(rng, batch, D, N, 1, io)
    dt_row = _row_dt(rng, batch, 1, io)[:, 0].copy()
    dt_full = np.ascontiguousarray(np.broadcast_to(dt_row[:, None], (batch, D)))
    t = {k: to_dev(v[..., 0].copy(), io, dev) for k, v in raw.items()}
    p = {k: torch.from_numpy(v).to(dev) for k, v in par.items()}
    s1, s2 = p["h0"].clone(), p["h0"].clone()
    kw = dict(z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"], zoh=zoh)
    y1 = ss.state_update(s1, t["x"], to_dev(dt_row, io, dev), t["B"], t["C"], p["A"], **kw)
    y2 = ss.state_update(s2, t["x"], to_dev(dt_full, io, dev), t["B"], t["C"], p["A"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
    yr, sr = oracle.default().state_update(par["h0"], f64["x"][..., 0], inputs.raw_to_f64(dt_full, io),
                                           f64["B"][..., 0], f64["C"][..., 0], par["A"], z=f64["z"][..., 0],
                                           Dskip=par["Dskip"], dt_bias=par["dt_bias"], zoh=zoh)
    assert rel_l2(to_f64(y1), yr) <= (1e-5 if io == "f32" else 2e-2) and rel_l2(to_f64(s1), sr) <= 1e-5


BWD_CASES = [("f32", (2, 77, 16, 37), False), ("f32", (3, 33, 8, 50), False), ("f32", (2, 20, 4, 31), False),
             ("f32", (1, 130, 1, 13), False), ("f32", (2, 70, 2, 9), False), ("f32", (1, 40, 16, 1), False),
             ("bf16", (2, 96, 16, 130), False), ("bf16", (2, 512, 16, 1000), True), ("f32", (2, 64, 16, 48), True)]


@pytest.mark.parametrize("io,shape,ckpt", BWD_CASES,
                         ids=["%s-%s%s" % (c[0], "x".join(map(str, c[1])), "-ckpt" if c[2] else "") for c in BWD_CASES])
def test_bwd_dt_per_row(ss, dev, io, shape, ckpt):
    """The backward with dt shared by a row's channels: the shared dt's gradient
    is the sum over channels of the per-channel gradient (the chain rule through
    the repeat), checked against the oracle's general backward with dt repeated;
    every other gradient equals the general call's bit for bit.  With ckpt, a
    forward that stores checkpoints (per-row dt too) feeds the backward, whose
    results must not change."""
    import torch
    batch, D, N, L = shape
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-row", io, shape)).encode()))
    raw, par, f64 = random_problem(rng, batch, D, N, L, io)
    dt_row = _row_dt(rng, batch, L, io)
    dt_full = np.ascontiguousarray(np.broadcast_to(dt_row[:, None, :], (batch, D, L)))
    dy = rng.standard_normal((batch, D, L)).astype(np.float32)
    dy_raw = dy if io == "f32" else inputs.f32_to_bf16_bits(dy)
    dh_final = rng.standard_normal((batch, D, N)).astype(np.float32)
    t = {k: to_dev(v, io, dev) for k, v in raw.items()}
    p = {k: torch.from_numpy(v).to(dev) for k, v in par.items() if v is not None}
    kw = dict(z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"], h0=p["h0"], dh_final=torch.from_numpy(dh_final).to(dev))
    dyd, dtr = to_dev(dy_raw, io, dev), to_dev(dt_row, io, dev)
    log("bwd dt per row %s %s ckpt=%s" % (io, shape, ckpt))
    g1 = ss.scan_bwd(t["x"], dtr, t["B"], t["C"], p["A"], dyd, **kw)
    g2 = ss.scan_bwd(t["x"], to_dev(dt_full, io, dev), t["B"], t["C"], p["A"], dyd, **kw)
    torch.cuda.synchronize()
    for k in ("dx", "dz", "dB", "dC", "dA", "dDskip", "ddt_bias", "dh0"):
        assert torch.equal(g1[k], g2[k]), k
    assert tuple(g1["ddt"].shape) == (batch, L)
    if ckpt:
        ck = torch.full((ss.ckpt_numel(batch, D, N, L),), float("nan"), device=dev)
        ss.scan_fwd(t["x"], dtr, t["B"], t["C"], p["A"], z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"],
                    h0=p["h0"], ckpt=ck)
        g3 = ss.scan_bwd(t["x"], dtr, t["B"], t["C"], p["A"], dyd, ckpt=ck, **kw)
        torch.cuda.synchronize()
        for k, v in g1.items():
            assert torch.equal(v, g3[k]), k
    r = oracle.default().scan_bwd(f64["x"], inputs.raw_to_f64(dt_full, io), f64["B"], f64["C"], par["A"],
                                  inputs.raw_to_f64(dy_raw, io), z=f64["z"], Dskip=par["Dskip"],
                                  dt_bias=par["dt_bias"], h0=par["h0"], dh_final=dh_final)
    e = rel_l2(to_f64(g1["ddt"]), r["ddt"].sum(axis=1))
    log("  shared dt gradient rel-L2 %.3e" % e)
    assert e <= (5e-5 if io == "f32" else 2e-2)
