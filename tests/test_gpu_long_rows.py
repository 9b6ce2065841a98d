"""Rows of at least 2^19 bf16 tokens (1 MB) on the GPU against the oracle.

There the scan's owners of the per-token work take 64-byte segments of 8 rows
(a wave's loads and y stores cover whole row segments), and the backward's
reverse pass loads its operands through LDS in whole row pieces: separate
kernel instantiations, chosen by row length, that the shorter cases elsewhere
never reach.  The cases run chunked plans (aggregate pass, combine, full pass),
ragged last tiles and chunks, a second channel block with inactive channels,
batch rows past the first, N = 8 and 16, the optional inputs present and
absent, one dt per (row, token), the zero-order hold, and the training-step
pair (a forward storing checkpoints, the backward reading them).  Outputs are
held to the strict bounds of the full-size tests: the whole-tensor spec bound,
every channel's rel-L2 and every element.
"""
import zlib

import numpy as np
import pytest

import oracle
from gpu_util import (BF16_CHANNEL_REL_L2, StrictCheck, check_state, log, random_problem, rel_l2, to_dev,
                      to_f64)
from workloads import inputs

pytestmark = pytest.mark.gpu

L19 = 1 << 19


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ss():
    import selective_state_space_62_amd as m
    return m


@pytest.fixture(scope="module")
def o():
    return oracle.default()


def _problem(seed_key, batch, D, N, L, optional, dt_row, with_dy=False):
    rng = np.random.default_rng(zlib.crc32(repr(seed_key).encode()))
    raw, par, f64 = random_problem(rng, batch, D, N, L, "bf16", with_z=optional, with_skip=optional,
                                   with_bias=optional, with_h0=optional)
    row = None
    if dt_row:
        row = inputs.f32_to_bf16_bits((0.5 * rng.standard_normal((batch, L))).astype(np.float32))
        full = np.ascontiguousarray(np.broadcast_to(row[:, None, :], (batch, D, L)))
        raw["dt"], f64["dt"] = full, inputs.raw_to_f64(full, "bf16")
    if with_dy:
        dy = inputs.f32_to_bf16_bits(rng.standard_normal((batch, D, L)).astype(np.float32))
        raw["dy"], f64["dy"] = dy, inputs.raw_to_f64(dy, "bf16")
    return raw, par, f64, row


def _upload(raw, par, row, dev):
    import torch
    t = {k: to_dev(v, "bf16", dev) for k, v in raw.items()}
    if row is not None:
        t["dt"] = to_dev(row, "bf16", dev)
    p = {k: (torch.from_numpy(v).to(dev) if v is not None else None) for k, v in par.items()}
    return t, p


# (batch, D, N, L, optional inputs, one dt per row, zero-order hold)
FWD = [
    (2, 40, 16, L19 + 40, True, False, False),
    (1, 33, 8, L19 + 8, False, False, True),
    (2, 36, 16, L19 + 40, True, True, False),
]


@pytest.mark.parametrize("case", FWD, ids=["x".join(map(str, c[:4])) + ("-dtrow" if c[5] else "")
                                           + ("-zoh" if c[6] else "") for c in FWD])
def test_fwd_long_rows(ss, o, dev, case):
    import torch
    batch, D, N, L, optional, dt_row, zoh = case
    plan = ss.ss_scan_fwd_plan(batch, D, N, L, ss.SS_BF16)
    log("fwd long rows %s, plan %s" % (case, plan))
    assert plan[1] == 2 and plan[2] < L, "two lanes per channel, chunked"
    raw, par, f64, row = _problem(("fwd-long-rows", case), batch, D, N, L, optional, dt_row)
    t, p = _upload(raw, par, row, dev)
    y, hf = ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t.get("z"), Dskip=p["Dskip"],
                        dt_bias=p["dt_bias"], h0=p["h0"], zoh=zoh)
    torch.cuda.synchronize()
    y, hf = to_f64(y), to_f64(hf)
    del t
    torch.cuda.empty_cache()
    ry, rh = o.scan(f64["x"], f64["dt"], f64["B"], f64["C"], par["A"], z=f64.get("z"), Dskip=par["Dskip"],
                    dt_bias=par["dt_bias"], h0=par["h0"], zoh=zoh)
    chk = StrictCheck("y", "bf16")
    chk.add(y.reshape(batch * D, L), ry.reshape(batch * D, L))
    chk.assert_ok(2e-2, BF16_CHANNEL_REL_L2)
    check_state("h_final", hf, rh)


def test_bwd_long_rows_from_checkpoints(ss, o, dev):
    """The training-step pair at long rows: the forward stores its checkpoints
    (row-segment owners), the backward reads them (whole-piece operand loads)."""
    import torch
    batch, D, N, L = 2, 40, 16, L19 + 40
    log("bwd long rows from checkpoints %s" % ((batch, D, N, L),))
    raw, par, f64, _ = _problem(("bwd-long-rows-ckpt",), batch, D, N, L, True, False, with_dy=True)
    t, p = _upload(raw, par, None, dev)
    dh = torch.from_numpy(np.random.default_rng(7).standard_normal((batch, D, N)).astype(np.float32)).to(dev)
    ck = torch.full((ss.ckpt_numel(batch, D, N, L),), float("nan"), device=dev)
    ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"],
                h0=p["h0"], ckpt=ck)
    g = ss.scan_bwd(t["x"], t["dt"], t["B"], t["C"], p["A"], t["dy"], z=t["z"], Dskip=p["Dskip"],
                    dt_bias=p["dt_bias"], h0=p["h0"], dh_final=dh, ckpt=ck)
    torch.cuda.synchronize()
    g = {k: (to_f64(v) if v is not None else None) for k, v in g.items()}
    dhn = dh.cpu().numpy().astype(np.float64)
    del t, ck
    torch.cuda.empty_cache()
    r = o.scan_bwd(f64["x"], f64["dt"], f64["B"], f64["C"], par["A"], f64["dy"], z=f64["z"], Dskip=par["Dskip"],
                   dt_bias=par["dt_bias"], h0=par["h0"], dh_final=dhn)
    errs = {k: rel_l2(g[k], r[k]) for k in ("dx", "ddt", "dz", "dh0", "dA", "dDskip", "ddt_bias", "dB", "dC")}
    log("  %s" % ", ".join("%s %.2e" % kv for kv in errs.items()))
    for k, e in errs.items():
        assert e <= 2e-2, (k, e)
    for k in ("dx", "ddt", "dz"):
        chk = StrictCheck(k, "bf16")
        chk.add(g[k].reshape(batch * D, L), r[k].reshape(batch * D, L))
        chk.assert_ok(2e-2, BF16_CHANNEL_REL_L2)
