"""Write tests/golden/oracle_small.json: small seeded inputs and the oracle's
outputs for them (scan in both discretisations, one decode step, the backward).

The pages print no numerical worked example, so nothing here is a printed value:
these are the oracle's own results, whose correctness the pins in tests/pins.py
establish.  They fix the oracle against accidental change.  Only the oracle and
numpy are called.  Run from the repository root: python tests/golden/make_golden.py
"""
import json
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

import oracle  # noqa: E402


def inputs():
    rng = np.random.default_rng(6200)
    batch, D, N, L = 2, 3, 4, 6
    return dict(
        x=rng.standard_normal((batch, D, L)), dt=0.5 * rng.standard_normal((batch, D, L)),
        z=rng.standard_normal((batch, D, L)), B=rng.standard_normal((batch, N, L)),
        C=rng.standard_normal((batch, N, L)), A=-rng.uniform(0.2, 3.0, (D, N)), Dskip=rng.normal(1.0, 0.3, D),
        dt_bias=np.log(np.expm1(rng.uniform(1e-3, 1e-1, D))), h0=rng.standard_normal((batch, D, N)),
        dy=rng.standard_normal((batch, D, L)), dh_final=rng.standard_normal((batch, D, N)))


def outputs(o, p):
    kw = dict(z=p["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"], h0=p["h0"])
    out = {}
    for zoh in (False, True):
        y, hf = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], zoh=zoh, **kw)
        out["scan_%s" % ("zoh" if zoh else "euler")] = dict(y=y, h_final=hf)
    yd, sd = o.state_update(p["h0"], p["x"][..., 0], p["dt"][..., 0], p["B"][..., 0], p["C"][..., 0], p["A"],
                            z=p["z"][..., 0], Dskip=p["Dskip"], dt_bias=p["dt_bias"])
    out["decode"] = dict(y=yd, state=sd)
    g = o.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], p["dy"], dh_final=p["dh_final"], **kw)
    out["bwd_euler"] = g
    return out


def to_lists(d):
    return {k: (to_lists(v) if isinstance(v, dict) else np.asarray(v).tolist()) for k, v in d.items()}


if __name__ == "__main__":
    p = inputs()
    doc = {"about": "seeded inputs and the CPU oracle's outputs (float64); written by make_golden.py",
           "inputs": to_lists(p), "outputs": to_lists(outputs(oracle.default(), p))}
    (Path(__file__).parent / "oracle_small.json").write_text(json.dumps(doc, indent=0) + "\n")
