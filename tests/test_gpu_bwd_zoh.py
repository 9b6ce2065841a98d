"""The zero-order-hold backward (ss_scan_bwd_ex with SS_FLAG_ZOH) on the GPU
against the oracle's gradients.

With the zero-order hold the input coefficient is c = (e^(Delta A) - 1)/A, the
discretisation under which Theorem 1 of the reader's notes holds exactly
(kurisu.si, "Main results (verified)"); its derivatives dc/dDelta = e^(Delta A)
and dc/dA = Delta^2 psi(Delta A) are pinned in the oracle by finite differences
(tests/pins.py).  The GPU evaluates c by a Taylor polynomial near u = Delta A
= 0 and as (E - 1)/A elsewhere, and psi by its series near 0 and its closed
form elsewhere; the cases below span both regions.  Tolerances as for the first-order backward (tests/test_gpu_bwd.py).
"""
import zlib

import numpy as np
import pytest

import oracle
from gpu_util import log, random_problem, rel_l2, to_dev, to_f64
from workloads import inputs

pytestmark = pytest.mark.gpu

ELEMENT = ("dx", "ddt", "dz", "dh0")
SUMS = ("dA", "dDskip", "ddt_bias", "dB", "dC")


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


def _tol(io, name):
    if io == "bf16":
        return 2e-2
    return 1e-5 if name in ELEMENT else 5e-5


def _problem(rng, batch, D, N, L, io, optional=True, a_range=None, dt_shift=0.0):
    raw, par, f64 = random_problem(rng, batch, D, N, L, io, with_z=optional, with_skip=optional,
                                   with_bias=optional, with_h0=optional)
    if a_range is not None:
        par["A"] = -rng.uniform(a_range[0], a_range[1], (D, N)).astype(np.float32)
    if dt_shift:
        v = inputs.raw_to_f64(raw["dt"], io).astype(np.float32) + np.float32(dt_shift)
        raw["dt"] = v if io == "f32" else inputs.f32_to_bf16_bits(v)
        f64["dt"] = inputs.raw_to_f64(raw["dt"], io)
    dy = rng.standard_normal((batch, D, L)).astype(np.float32)
    raw["dy"] = dy if io == "f32" else inputs.f32_to_bf16_bits(dy)
    f64["dy"] = inputs.raw_to_f64(raw["dy"], io)
    par["dh_final"] = rng.standard_normal((batch, D, N)).astype(np.float32) if optional else None
    return raw, par, f64


def _run(ss, raw, par, io, dev, **kw):
    import torch
    t = {k: to_dev(v, io, dev) for k, v in raw.items()}
    p = {k: (torch.from_numpy(v).to(dev) if v is not None else None) for k, v in par.items()}
    g = ss.scan_bwd(t["x"], t["dt"], t["B"], t["C"], p["A"], t["dy"], z=t.get("z"), Dskip=p["Dskip"],
                    dt_bias=p["dt_bias"], h0=p["h0"], dh_final=p["dh_final"], zoh=True, **kw)
    torch.cuda.synchronize()
    return g, t, p


def _oracle(o, f64, par):
    return o.scan_bwd(f64["x"], f64["dt"], f64["B"], f64["C"], par["A"], f64["dy"], z=f64.get("z"),
                      Dskip=par["Dskip"], dt_bias=par["dt_bias"], h0=par["h0"], dh_final=par["dh_final"], zoh=True)


def _compare(g, r, io, what):
    errs = {k: rel_l2(to_f64(g[k]), r[k]) for k in ELEMENT + SUMS if g.get(k) is not None and r.get(k) is not None}
    log("%s: %s" % (what, ", ".join("%s %.2e" % kv for kv in errs.items())))
    for k, e in errs.items():
        assert e <= _tol(io, k), (what, k, e, errs)


CASES = [(2, 77, 16, 37), (1, 64, 16, 64), (3, 33, 8, 50), (2, 20, 4, 31), (2, 70, 2, 9), (1, 130, 1, 13),
         (2, 40, 16, 1), (2, 64, 16, 17)]


@pytest.mark.parametrize("case", CASES, ids=["x".join(map(str, c)) for c in CASES])
@pytest.mark.parametrize("optional", [True, False], ids=["all-inputs", "no-optional"])
def test_bwd_zoh_f32_matches_oracle(ss, o, dev, case, optional):
    batch, D, N, L = case
    log("bwd zoh f32 %s optional=%s" % (case, optional))
    rng = np.random.default_rng(zlib.crc32(repr(("zoh", case, optional)).encode()))
    raw, par, f64 = _problem(rng, batch, D, N, L, "f32", optional)
    g, _, _ = _run(ss, raw, par, "f32", dev)
    _compare(g, _oracle(o, f64, par), "f32", "bwd zoh %s" % (case,))


@pytest.mark.parametrize("what,a_range,dt_shift", [
    ("series region: A near zero", (1e-4, 2e-2), 0.0),
    ("closed-form region: large Delta", (0.5, 8.0), 2.5),
    ("both regions in every wave", (1e-3, 40.0), 1.0),
], ids=["small-u", "large-u", "mixed-u"])
def test_bwd_zoh_u_regions(ss, o, dev, what, a_range, dt_shift):
    """u = Delta A in the series region of phi and psi (|u| below 1/4 and 1), in
    the closed-form region, and mixed within every wave."""
    rng = np.random.default_rng(zlib.crc32(repr(("zoh-u", what)).encode()))
    raw, par, f64 = _problem(rng, 2, 96, 16, 70, "f32", True, a_range=a_range, dt_shift=dt_shift)
    g, _, _ = _run(ss, raw, par, "f32", dev)
    _compare(g, _oracle(o, f64, par), "f32", "bwd zoh %s" % what)


def test_bwd_zoh_bf16(ss, o, dev):
    rng = np.random.default_rng(zlib.crc32(b"zoh-bf16"))
    raw, par, f64 = _problem(rng, 2, 512, 16, 600, "bf16", True)
    g, _, _ = _run(ss, raw, par, "bf16", dev)
    _compare(g, _oracle(o, f64, par), "bf16", "bwd zoh bf16 2x512x16x600")


def test_bwd_zoh_checkpoints_and_determinism(ss, o, dev):
    """A ZOH forward that stores checkpoints feeds the ZOH backward; two runs give
    identical bits.  Every |A| here is at least 0.3, so the forward and the
    backward's own sweep both form the input term as (E - 1) x B / A with the
    same operations: the gradients from the stored checkpoints equal those from
    the sweep bit for bit, and both are held to the oracle."""
    import torch
    batch, D, N, L = 2, 96, 16, 130
    rng = np.random.default_rng(zlib.crc32(b"zoh-ckpt"))
    raw, par, f64 = _problem(rng, batch, D, N, L, "f32", True)
    g1, t, p = _run(ss, raw, par, "f32", dev)
    g2, _, _ = _run(ss, raw, par, "f32", dev)
    ck = torch.full((ss.ckpt_numel(batch, D, N, L),), float("nan"), device=dev)
    y0, h0f = ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"],
                          h0=p["h0"], zoh=True)
    y1, h1f = ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"],
                          h0=p["h0"], zoh=True, ckpt=ck)
    g3, _, _ = _run(ss, raw, par, "f32", dev, ckpt=ck)
    assert torch.equal(y0, y1) and torch.equal(h0f, h1f)
    assert not torch.isnan(ck).any()
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), k
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g3[k]), k
    r = _oracle(o, f64, par)
    _compare(g1, r, "f32", "bwd zoh own sweep")
    _compare(g3, r, "f32", "bwd zoh from forward checkpoints")


def test_bwd_zoh_dt_per_row(ss, o, dev):
    """ZOH with one dt per (row, token): the shared dt's gradient is the channel
    sum of the oracle's per-channel gradient with dt repeated."""
    import torch
    batch, D, N, L = 2, 77, 16, 45
    rng = np.random.default_rng(zlib.crc32(b"zoh-row"))
    raw, par, f64 = _problem(rng, batch, D, N, L, "f32", True)
    dt_row = (0.5 * rng.standard_normal((batch, L))).astype(np.float32)
    raw["dt"] = np.ascontiguousarray(np.broadcast_to(dt_row[:, None, :], (batch, D, L)))
    f64["dt"] = raw["dt"].astype(np.float64)
    g_full, t, p = _run(ss, raw, par, "f32", dev)
    g_row = ss.scan_bwd(t["x"], torch.from_numpy(dt_row).to(dev), t["B"], t["C"], p["A"], t["dy"], z=t["z"],
                        Dskip=p["Dskip"], dt_bias=p["dt_bias"], h0=p["h0"], dh_final=p["dh_final"], zoh=True)
    torch.cuda.synchronize()
    for k in ("dx", "dz", "dB", "dC", "dA", "dDskip", "ddt_bias", "dh0"):
        assert torch.equal(g_row[k], g_full[k]), k
    r = _oracle(o, f64, par)
    e = rel_l2(to_f64(g_row["ddt"]), r["ddt"].sum(axis=1))
    log("bwd zoh dt per row: shared dt gradient rel-L2 %.2e" % e)
    assert e <= 5e-5
    _compare(g_full, r, "f32", "bwd zoh (dt repeated)")


def test_bwd_zoh_a_zero(ss, o, dev):
    """Entries of A exactly zero: the ZOH coefficient's limit Delta (dc/dDelta = 1,
    dc/dA = Delta^2 / 2) comes from the series branches, as in the oracle."""
    rng = np.random.default_rng(zlib.crc32(b"zoh-a0"))
    raw, par, f64 = _problem(rng, 2, 64, 16, 40, "f32", True)
    A = par["A"].copy()
    A[rng.random(A.shape) < 0.25] = 0.0
    par["A"] = A
    g, _, _ = _run(ss, raw, par, "f32", dev)
    _compare(g, _oracle(o, f64, par), "f32", "bwd zoh with A = 0 entries")


@pytest.mark.parametrize("what,lo,hi", [
    ("every |A| >= 0.07", 0.07, 0.5),
    ("|A| from 1e-3", 1e-3, 0.5),
], ids=["a-from-0.07", "a-from-1e-3"])
def test_bwd_zoh_a_of_both_signs(ss, o, dev, what, lo, hi):
    """Entries of A of either sign (e^(Delta A) above 1 where A > 0), short
    sequences so that the growing components stay finite."""
    rng = np.random.default_rng(zlib.crc32(repr(("zoh-sign", lo)).encode()))
    raw, par, f64 = _problem(rng, 2, 96, 16, 40, "f32", True)
    mag = rng.uniform(lo, hi, par["A"].shape)
    par["A"] = (np.where(rng.random(mag.shape) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    g, _, _ = _run(ss, raw, par, "f32", dev)
    _compare(g, _oracle(o, f64, par), "f32", "bwd zoh, A of both signs (%s)" % what)


@pytest.mark.parametrize("what,lo,hi,both_signs", [
    ("every Delta A small, A < 0", 0.07, 0.5, False),
    ("every Delta A small, A of either sign", 0.07, 0.5, True),
    ("Delta about 1e-3, A in [-16, -1]", 1.0, 16.0, False),
], ids=["small-u", "small-u-signs", "small-delta"])
def test_bwd_zoh_small_delta_a(ss, o, dev, what, lo, hi, both_signs):
    """Every u = Delta A small (Delta about 1e-3), where e^u, rounded, cannot hold
    u's low bits: the gradients must still reach fp32 parity."""
    rng = np.random.default_rng(zlib.crc32(repr(("zoh-bwd-small-u", what)).encode()))
    batch, D, N, L = 2, 128, 16, 256
    raw, par, f64 = _problem(rng, batch, D, N, L, "f32", True)
    raw["dt"] = (0.1 * rng.standard_normal((batch, D, L))).astype(np.float32)
    f64["dt"] = raw["dt"].astype(np.float64)
    par["dt_bias"] = np.full(D, np.log(np.expm1(1e-3)), np.float32)
    mag = rng.uniform(lo, hi, (D, N))
    sign = np.where(rng.random((D, N)) < 0.5, 1.0, -1.0) if both_signs else -1.0
    par["A"] = (sign * mag).astype(np.float32)
    g, _, _ = _run(ss, raw, par, "f32", dev)
    _compare(g, _oracle(o, f64, par), "f32", "bwd zoh, %s" % what)


def test_bwd_zoh_130m_layer_full(ss, o, dev):
    """The 130M-shaped layer (batch 8, D 1536, N 16, L 2048, fp32) with the
    zero-order hold, every gradient in full against the oracle."""
    import torch
    from workloads import M130
    from workloads import device as wdev
    cfg = M130
    t = wdev.scan_inputs(cfg, dev)
    A, dskip, bias = wdev.params(cfg, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(62103)
    dy = torch.randn(t["x"].shape, generator=gen, device=dev, dtype=torch.float32)
    dhf = torch.randn((cfg.batch, cfg.dim, cfg.dstate), generator=gen, device=dev, dtype=torch.float32)
    g = ss.scan_bwd(t["x"], t["dt"], t["B"], t["C"], A, dy, z=t["z"], Dskip=dskip, dt_bias=bias, dh_final=dhf,
                    zoh=True)
    torch.cuda.synchronize()
    f = {k: to_f64(v) for k, v in t.items()}
    r = o.scan_bwd(f["x"], f["dt"], f["B"], f["C"], to_f64(A), to_f64(dy), z=f["z"], Dskip=to_f64(dskip),
                   dt_bias=to_f64(bias), dh_final=to_f64(dhf), zoh=True)
    _compare(g, r, "f32", "bwd zoh %s in full" % cfg.name)
