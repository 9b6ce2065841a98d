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
