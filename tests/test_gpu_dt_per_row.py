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
