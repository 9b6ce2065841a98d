"""bench.py's host-side contract: it measures one GPU and says so for any other count."""
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_bench_algorithmic_counts():
    sys.path.insert(0, str(ROOT))
    import bench
    from workloads import B28
    # x, dt, z read and y written in bf16 (8 B), plus B/C, parameters and h_final amortised
    assert abs(bench.algorithmic_bytes_per_tokch(B28) - 8.048) < 1e-3
    assert bench.algorithmic_slots_per_tokch(16) == 112
    assert bench.algorithmic_slots_bwd_per_tokch(16) == 411
