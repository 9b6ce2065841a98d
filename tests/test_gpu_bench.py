"""bench.py on the GPU: a short run prints one JSON line with the contract's
fields, the roofline and ceilings objects and the secondary legs."""
import json
import subprocess
import sys
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parent.parent


def test_bench_json_line():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--steps", "3", "--warmup", "2", "--no-cpu-baseline",
                        "--no-zoh", "--no-bwd", "--no-dt-row", "--settle-ms", "300"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "ceilings", "decode"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "2.8b-layer-bf16" and d["value"] > 0
    rf = d["roofline"]
    # the graded roofline: min(HBM, transcendentals), here the transcendental issue
    assert rf["bound"] == "alu" and rf["unit"] == "T transcendental/s" and abs(rf["peak"] - 19.661) < 1e-3
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert abs(rf["frac"] - d["ceilings"]["frac_of_min_hbm_transcendentals"]) < 2e-3
    assert d["roofline_valu_issue"]["unit"] == "T VALU-slot/s"
    assert d["ceilings"]["valu_issue_slots"] < d["ceilings"]["transcendentals_only"] < d["ceilings"]["hbm"]
    assert d["decode"]["frac_hbm_cold"] > 0
    assert d["settle_ms"] >= 200 and d["settle_calls"] > 0
    assert d["cold_cache"]["kernel_ms_median"] > 0
    v = d["valu_rates"]
    assert v["exp"] > 0 and v["fma"] > 0 and len(v["rows"]) == 45
