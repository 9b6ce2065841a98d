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
    assert bench.algorithmic_slots_bwd_per_tokch(16) == 347
    assert bench.algorithmic_slots_bwd_per_tokch(16, sweep=False) == 267


def test_cpu_baseline_repeats_passes_until_budget():
    """The oracle baseline keeps passing over the (tiny) workload until the time
    budget is spent, and reports the fraction of the workload it covered."""
    sys.path.insert(0, str(ROOT))
    import bench
    from workloads import TINY
    r = bench.cpu_baseline(TINY, 0.3)
    assert r["kind"] == "oracle" and r["unit"] == "Gtok·ch/s" and r["value"] > 0 and r["cores"] >= 1
    passes = float(r["sample"].split(" passes")[0])
    assert passes > 1.0, r["sample"]


def test_measured_traffic_tracks_kernel_sources():
    """Traffic comes from the committed counter summaries only while their kernel
    hash matches the sources (else None); a different workload name gets None."""
    sys.path.insert(0, str(ROOT))
    import json
    import bench
    from workloads import B28, TINY
    d = json.loads(bench.COUNTERS_FILES["scan"].read_text())
    got = bench.measured_traffic(B28, "scan")
    if d["kernel_hash"] == bench.kernel_hash("scan"):
        assert got == d["hbm_bytes_per_launch"] > bench.algorithmic_bytes_per_tokch(B28) * B28.tokch * 0.9
    else:
        assert got is None
    assert bench.measured_traffic(TINY, "scan") is None


def test_ceilings_at_the_2p8b_shape():
    """HBM 8 TB/s over 8.048 B, 20 transcendentals at half rate alone, and all
    112 issue slots: 994, 983 and 351 Gtok·ch/s; the kernel's fraction of each."""
    sys.path.insert(0, str(ROOT))
    import bench
    from workloads import B28
    c = bench.ceilings(B28, 245.0)
    assert abs(c["hbm"] - 994.0) < 0.5 and abs(c["transcendentals_only"] - 983.0) < 0.5
    assert abs(c["valu_issue_slots"] - 351.1) < 0.1
    assert abs(c["frac_of_valu_issue_slots"] - 245.0 / 351.08) < 1e-3
    assert abs(c["frac_of_min_hbm_transcendentals"] - 245.0 / 983.0) < 1e-3


def test_graded_roofline_at_the_2p8b_shape():
    """The line's roofline is the fraction of min(HBM, transcendentals): at the
    2.8B shape the transcendental ceiling is the lower one (983 < 994), so the
    bound is ALU, achieved is 20 transcendentals per token-channel over the
    kernel time, and the peak is the half-rate issue, 19.66 T/s."""
    sys.path.insert(0, str(ROOT))
    import bench
    from workloads import B28, DECODE
    kern_ms = 0.32
    r = bench.graded_roofline(B28, kern_ms, None, "scan")
    assert r["bound"] == "alu" and r["unit"] == "T transcendental/s"
    assert abs(r["peak"] - 19.661) < 1e-3
    ach = 20 * B28.tokch / (kern_ms * 1e-3) / 1e12
    assert abs(r["achieved"] - ach) < 1e-3 and abs(r["frac"] - ach / r["peak"]) < 1e-3
    gtokch = B28.tokch / (kern_ms * 1e-3) / 1e9
    assert abs(r["frac"] - bench.ceilings(B28, gtokch)["frac_of_min_hbm_transcendentals"]) < 1e-3


def test_bench_cli_has_settle_and_cold_options():
    """The counted warm-up steps run after a time-based settle phase, and the
    cache-flushed timing and the rate probe can be switched off."""
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for opt in ("--settle-ms", "--no-cold", "--no-rates"):
        assert opt in r.stdout, opt
