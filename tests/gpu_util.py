"""Helpers for the GPU tests: uploads, rel-L2, random problems with exact bf16 inputs."""
from __future__ import annotations

import sys

import numpy as np

from workloads import inputs


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def to_dev(raw: np.ndarray, io: str, device):
    import torch
    if io == "f32":
        return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.uint16).view(np.int16)).to(device).view(torch.bfloat16)


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def random_problem(rng, batch, D, N, L, io, with_z=True, with_skip=True, with_bias=True, with_h0=True):
    """Seeded random inputs; returns (raw dict for upload, f64 dict for the oracle)."""
    def q(a):
        a = a.astype(np.float32)
        return a if io == "f32" else inputs.f32_to_bf16_bits(a)
    raw = {
        "x": q(rng.standard_normal((batch, D, L))),
        "dt": q(0.5 * rng.standard_normal((batch, D, L))),
        "B": q(rng.standard_normal((batch, N, L))),
        "C": q(rng.standard_normal((batch, N, L))),
    }
    if with_z:
        raw["z"] = q(rng.standard_normal((batch, D, L)))
    par = {
        "A": -rng.uniform(0.3, 2.0 * N, (D, N)).astype(np.float32),
        "Dskip": rng.normal(1.0, 0.2, D).astype(np.float32) if with_skip else None,
        "dt_bias": np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), D)))).astype(np.float32)
        if with_bias else None,
        "h0": rng.standard_normal((batch, D, N)).astype(np.float32) if with_h0 else None,
    }
    f64 = {k: inputs.raw_to_f64(v, io) for k, v in raw.items()}
    return raw, par, f64


def run_gpu_scan(ss, raw, par, io, device, plan=None):
    import torch
    t = {k: to_dev(v, io, device) for k, v in raw.items()}
    p = {k: (torch.from_numpy(v).to(device) if v is not None else None) for k, v in par.items()}
    y, hf = ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], p["A"], z=t.get("z"), Dskip=p["Dskip"],
                        dt_bias=p["dt_bias"], h0=p["h0"], plan=plan)
    torch.cuda.synchronize()
    return to_f64(y), to_f64(hf)


def run_oracle_scan(o, f64, par):
    return o.scan(f64["x"], f64["dt"], f64["B"], f64["C"], par["A"], z=f64.get("z"), Dskip=par["Dskip"],
                  dt_bias=par["dt_bias"], h0=par["h0"])


# ------------------------------------------------------- strict comparisons ---
# bf16 keeps 8 significant bits: rounding an fp32 value to nearest even moves it by
# at most 2^-8 of its magnitude, so one bf16 ulp of the reference (2^-7 |y_ref|)
# bounds the rounding with a factor of 2 to spare.  The fp32 arithmetic before the
# rounding adds a few 1e-7 of the sizes of the summed terms, which the absolute part
# (1e-4 of the channel's largest |y_ref|) covers a hundred times over.  A wrong
# element, token range or channel breaks both the element bound and the channel's
# rel-L2 by orders of magnitude.
BF16_ELEM_REL = 2.0 ** -7
ELEM_ABS_OF_CHANNEL_MAX = 1e-4
BF16_CHANNEL_REL_L2 = 5e-3      # bf16 output rounding alone gives about 1.7e-3 per channel
F32_CHANNEL_REL_L2 = 1e-4       # fp32 I/O and fp32 states: rounding gives about 1e-7 .. 1e-6


def per_channel_rel_l2(a, b) -> np.ndarray:
    """rel-L2 of each row of (channels, samples) arrays (a row of zeros in b uses 1)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    num = np.sqrt(np.sum((a - b) ** 2, axis=1))
    den = np.sqrt(np.sum(b * b, axis=1))
    return num / np.where(den > 0, den, 1.0)


def elementwise_excess(a, b, rel: float, abs_of_max: float = ELEM_ABS_OF_CHANNEL_MAX):
    """Rows are channels.  Returns (number of elements over the bound
    |a - b| <= rel |b| + abs_of_max * max_row |b|, the largest ratio of error to bound)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    bound = rel * np.abs(b) + abs_of_max * np.max(np.abs(b), axis=1, keepdims=True)
    err = np.abs(a - b)
    ratio = err / np.where(bound > 0, bound, np.finfo(np.float64).tiny)
    return int(np.count_nonzero(err > bound)), float(np.max(ratio)) if ratio.size else 0.0


class StrictCheck:
    """Accumulates a whole-tensor rel-L2 and per-channel / per-element bounds over
    pieces of (channels, samples) outputs, so that large tensors are checked a
    batch row at a time."""

    def __init__(self, name: str, io: str):
        self.name, self.io = name, io
        self.num = self.den = 0.0
        self.worst_channel = 0.0
        self.over = 0
        self.worst_ratio = 0.0
        self.count = 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        self.num += float(np.sum((got - ref) ** 2))
        self.den += float(np.sum(ref * ref))
        pc = per_channel_rel_l2(got, ref)
        self.worst_channel = max(self.worst_channel, float(np.max(pc)) if pc.size else 0.0)
        rel = BF16_ELEM_REL if self.io == "bf16" else 1e-5
        n, r = elementwise_excess(got, ref, rel)
        self.over += n
        self.worst_ratio = max(self.worst_ratio, r)
        self.count += got.size

    def rel_l2(self) -> float:
        return float(np.sqrt(self.num) / (np.sqrt(self.den) if self.den > 0 else 1.0))

    def summary(self) -> str:
        return ("%s: rel-L2 %.3e, worst channel %.3e, %d of %d elements over the element bound "
                "(worst error/bound %.3f)" % (self.name, self.rel_l2(), self.worst_channel, self.over, self.count,
                                               self.worst_ratio))

    def assert_ok(self, spec_tol: float, channel_tol: float):
        log("  " + self.summary())
        assert self.rel_l2() <= spec_tol, self.summary()
        assert self.worst_channel <= channel_tol, self.summary()
        assert self.over == 0, self.summary()


def check_state(name: str, got, ref, tol: float = 1e-5, channel_tol: float = F32_CHANNEL_REL_L2):
    """An fp32 state (channels, N) against the oracle's: whole-tensor rel-L2 at the
    fp32 bound and every channel's rel-L2."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(got)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    e = rel_l2(got, ref)
    pc = per_channel_rel_l2(got, ref)
    w = float(np.max(pc)) if pc.size else 0.0
    log("  %s: rel-L2 %.3e, worst channel %.3e" % (name, e, w))
    assert e <= tol and w <= channel_tol, (name, e, w)
