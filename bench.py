#!/usr/bin/env python3
"""Benchmark of the selective scan on one MI355X.

A step is one ss_scan_fwd call (every step of the scan: B/C re-layout, Delta,
Abar, state recurrence, readout, skip, gate, final state) over one batch of the
2.8B-shaped layer workload: batch 8, D = 5120, N = 16, L = 2048, bf16 I/O with
an fp32 state.  Inputs are generated on the device before timing and stay
resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-decode] [--no-zoh] [--copy-calib BYTES]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "selective-scan Gtok·ch/s + achieved HBM GB/s (% roofline), 2.8B-shape L=2048"

# MI355X published peaks and the derived VALU issue rate
HBM_PEAK_GBS = 8000.0
CUS, SIMDS_PER_CU, LANES_PER_SIMD_CLK, CLOCK_GHZ = 256, 4, 16, 2.4
VALU_PEAK_TOPS = CUS * SIMDS_PER_CU * LANES_PER_SIMD_CLK * CLOCK_GHZ / 1000.0   # 39.32 T lane-slots/s
TRANS_SLOTS = 2   # transcendentals issue at half rate on gfx950 and do not co-issue with FMAs
TRANS_PEAK_TPS = VALU_PEAK_TOPS / TRANS_SLOTS   # 19.66 T transcendentals/s

_CSRC = "selective_state_space_62_amd/csrc/"
# sources of each timed kernel: committed counters apply only while these are unchanged
KERNEL_SOURCES = {
    "scan": [_CSRC + f for f in ("scan_kernel.h", "scan_bf16_euler.hip", "scan_f32_euler.hip", "device_common.h")],
    "decode": [_CSRC + f for f in ("state_update.hip", "device_common.h")],
    "bwd": [_CSRC + f for f in ("scan_bwd_kernel.h", "scan_bwd.hip", "device_common.h")],
}
COUNTERS_FILES = {
    "scan": ROOT / "profiles" / "scan_2.8b_bf16_counters.json",
    "decode": ROOT / "profiles" / "decode_256x5120_bf16_counters.json",
    "bwd": ROOT / "profiles" / "bwd_2.8b_bf16_counters.json",
}


def kernel_hash(kind: str = "scan") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update((ROOT / f).read_bytes())
    return h.hexdigest()[:16]


def algorithmic_bytes_per_tokch(cfg) -> float:
    """HBM bytes per (token, channel) that the method must move: x, dt, z read once,
    y written once; B and C read once per (batch, token); A, Dskip, dt_bias once;
    the final state once."""
    eb = 4 if cfg.io == "f32" else 2
    per = 4 * eb
    shared = (2 * cfg.batch * cfg.dstate * cfg.seqlen * eb + cfg.dim * (cfg.dstate + 2) * 4
              + cfg.batch * cfg.dim * cfg.dstate * 4)
    return per + shared / cfg.tokch


def algorithmic_bytes_bwd(cfg) -> float:
    """HBM bytes one backward call must move: x, dt, z and dy read once, dx, ddt and dz
    written once; B and C read and dB, dC written once; the parameters, h0, dh_final
    and their gradients once."""
    eb = 4 if cfg.io == "f32" else 2
    nbd, nbnl = cfg.batch * cfg.dim, cfg.batch * cfg.dstate * cfg.seqlen
    return (7 * eb * cfg.tokch + 4 * eb * nbnl + 2 * 4 * cfg.dim * (cfg.dstate + 2)
            + 3 * 4 * nbd * cfg.dstate)


def algorithmic_slots_per_tokch(N: int) -> float:
    """VALU issue slots per (token, channel): per state component a multiply for
    Delta*A, the exponential, a multiply for Delta*x*B, the state FMA and the
    readout FMA (4 ops + 1 transcendental); per (token, channel) 8 more ops and 4
    transcendentals (softplus: exp, log; silu: exp, reciprocal).  A
    transcendental costs TRANS_SLOTS slots."""
    return 4 * N + 8 + TRANS_SLOTS * (N + 4)


def algorithmic_slots_bwd_per_tokch(N: int, sweep: bool = True) -> float:
    """VALU issue slots per (token, channel) of the backward pass by recomputation:
    per state component the checkpoint sweep (3 ops + exp; absent when the forward
    stored the checkpoints), the chunk recompute with the readout (4 ops + exp,
    keeping Abar) and the adjoint step (8 ops: adjoint update, dC and dB terms, the
    adjoint decayed by the kept Abar, which also scales h for the decay's
    derivative, that derivative's dDelta and dA terms, and lam B for dx); per
    (token, channel) two softplus evaluations (5 ops + 2
    transcendentals each), sigmoid(dt + dt_bias) (2 + 2), silu(z) and its derivative
    (7 + 2) and the six output formulas (8 ops).  A transcendental costs TRANS_SLOTS
    slots."""
    per_n = 4 + 8 + TRANS_SLOTS
    if sweep:
        per_n += 3 + TRANS_SLOTS
    per_tok = 10 + 2 + 7 + 8 + TRANS_SLOTS * (4 + 2 + 2)
    return per_n * N + per_tok


def ceilings(cfg, kernel_gtokch: float) -> dict:
    """The scan's throughput ceilings in Gtok·ch/s and the kernel's fraction of
    each: HBM (algorithmic bytes at 8 TB/s); transcendentals alone (N + 4 per
    token-channel at the half-rate issue of gfx950, 19.66 T/s); and the VALU
    issue slots of all the algorithmic work (transcendentals and FMAs share the
    issue port, so this lower ceiling is what any schedule of the algorithmic
    work can reach).  The graded figure is the fraction of min(HBM,
    transcendentals)."""
    hbm = HBM_PEAK_GBS / algorithmic_bytes_per_tokch(cfg)
    exp_only = TRANS_PEAK_TPS * 1e3 / (cfg.dstate + 4)
    slots = VALU_PEAK_TOPS * 1e3 / algorithmic_slots_per_tokch(cfg.dstate)
    return {"unit": "Gtok·ch/s", "hbm": round(hbm, 1), "transcendentals_only": round(exp_only, 1),
            "valu_issue_slots": round(slots, 1), "kernel": round(kernel_gtokch, 1),
            "frac_of_min_hbm_transcendentals": round(kernel_gtokch / min(hbm, exp_only), 4),
            "frac_of_valu_issue_slots": round(kernel_gtokch / slots, 4),
            "valu_issue_slots_over_min_hbm_transcendentals": round(slots / min(hbm, exp_only), 4)}


def graded_roofline(cfg, kern_ms: float, traffic, kernel: str) -> dict:
    """The scan kernel against min(HBM, transcendentals): whichever ceiling is
    lower gives the bound, the peak and the unit.  achieved = algorithmic bytes
    (HBM) or algorithmic transcendentals, N + 4 per token-channel (ALU), per
    launch over the kernel's average launch time."""
    hbm = HBM_PEAK_GBS / algorithmic_bytes_per_tokch(cfg)
    exp_only = TRANS_PEAK_TPS * 1e3 / (cfg.dstate + 4)
    sec = kern_ms * 1e-3
    if hbm <= exp_only:
        ach = algorithmic_bytes_per_tokch(cfg) * cfg.tokch / sec / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = (cfg.dstate + 4) * cfg.tokch / sec / 1e12
        r = {"bound": "alu", "achieved": round(ach, 3), "peak": round(TRANS_PEAK_TPS, 3),
             "unit": "T transcendental/s", "frac": round(ach / TRANS_PEAK_TPS, 4),
             "transcendentals_per_tokch": cfg.dstate + 4}
    r.update({"traffic": traffic, "kernel": kernel, "kernel_ms": round(kern_ms, 5)})
    return r


PROBE_MODES = ["exp2", "fma (literal operand)", "exp2 + fma, same wave", "exp2 / fma, separate waves",
               "fma, one chain", "fma (three VGPR operands)", "mul", "DPP add", "exp2 + 4 fma",
               "scan state step (2 + 5 per component)", "exp2 + 4 fma in bursts", "rcp", "log2 + add",
               "mul+exp2 / 3 fma, separate waves", "mul+exp2 / 3 fma, same wave",
               "8 exp2 then 128 fma", "exp2 then 16 fma, 8 times",
               "one exp2, then fma only"]


def run_valu_rates(reps: int = 5, ops_per_lane: float = 131072.0) -> dict:
    """The VALU issue-rate probe (libssprobe.so) at 8 waves per SIMD for every mode,
    and at 1, 2 and 4 waves per SIMD for fma, the single fma chain and the scan
    step; rates in T lane-operations per second over all CUs."""
    import ctypes
    lib = ctypes.CDLL(str(ROOT / "selective_state_space_62_amd" / "libssprobe.so"))
    lib.ss_probe_valu_mode.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_double)] * 2
    ms, ops = ctypes.c_double(), ctypes.c_double()

    def run(mode, wps):
        wg = CUS * wps
        rc = lib.ss_probe_valu_mode(mode, wg, 1, 1, ctypes.byref(ms), ctypes.byref(ops))
        if rc != 0:
            raise RuntimeError("ss_probe_valu_mode failed with HIP error %d" % rc)
        iters = max(1, int(round(ops_per_lane / ops.value)))
        rc = lib.ss_probe_valu_mode(mode, wg, iters, reps, ctypes.byref(ms), ctypes.byref(ops))
        if rc != 0:
            raise RuntimeError("ss_probe_valu_mode failed with HIP error %d" % rc)
        rate = wg * 256 * ops.value / (ms.value * 1e-3) / 1e12
        return {"mode": PROBE_MODES[mode], "waves_per_simd": wps, "ms": round(ms.value, 4),
                "ops_per_lane": ops.value, "rate": round(rate, 3),
                "cycles_per_wave_op": round(1024 * CLOCK_GHZ * 1e9 / (rate * 1e12 / 64), 3)}
    rows = [run(m, 8) for m in range(len(PROBE_MODES))]
    rows += [run(m, w) for m in (1, 4, 9, 10, 13, 14, 15, 16, 17) for w in (1, 2, 4)]
    by = {(r["mode"], r["waves_per_simd"]): r for r in rows}
    exp_r, fma_r = by[(PROBE_MODES[0], 8)]["rate"], by[(PROBE_MODES[1], 8)]["rate"]
    mixed = by[(PROBE_MODES[2], 8)]["ms"]
    return {"unit": "T lane-op/s", "exp": exp_r, "fma": fma_r,
            "exp_over_half_rate_peak": round(exp_r / TRANS_PEAK_TPS, 4),
            "fma_over_16_lanes_per_clock": round(fma_r / VALU_PEAK_TOPS, 4),
            # the mixed mode's operations are half exp2, half fma: against the
            # time of that many of each run separately
            "mixed_time_over_sum_of_parts": round(mixed / (0.5 * (by[(PROBE_MODES[0], 8)]["ms"]
                                                                  + by[(PROBE_MODES[1], 8)]["ms"])), 4),
            "rows": rows,
            "note": "cycles_per_wave_op: SIMD cycles per 64-lane operation at %.1f GHz" % CLOCK_GHZ}


def run_l_sweep(ss, torch, dev, cfg, lengths=(512, 1024, 2048, 4096, 8192, 16384), calls=20):
    """The scan at several sequence lengths with the workload's batch and channels
    (the pages claim linear scaling in L): kernel time per call and per token."""
    import dataclasses
    from workloads import device as wdev
    A, dskip, bias = wdev.params(cfg, dev)
    rows = []
    for L in lengths:
        c = dataclasses.replace(cfg, seqlen=L, name="%s-L%d" % (cfg.name, L))
        t = wdev.scan_inputs(c, dev)
        ws = torch.empty(max(ss.workspace_bytes(c.batch, c.dim, c.dstate, L, t["x"].dtype), 256), dtype=torch.uint8,
                         device=dev)

        def call():
            ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=ws)
        # warm up for at least 100 ms at every length (as the main measurement's
        # warm-up steps do), so that short sequences are not timed while the clock ramps
        t_warm = time.perf_counter() + 0.1
        while time.perf_counter() < t_warm:
            for _ in range(10):
                call()
            torch.cuda.synchronize()
        ss.ss_timing_reset()
        ss.ss_timing_enable(True)
        for _ in range(calls):
            call()
        torch.cuda.synchronize()
        ss.ss_timing_enable(False)
        ms, n = ss.ss_timing_read()
        ss.ss_timing_reset()
        ms /= n
        plan = ss.ss_scan_fwd_plan(c.batch, c.dim, c.dstate, L, ss.SS_BF16 if c.io == "bf16" else ss.SS_F32)
        rows.append({"seq_len": L, "kernel_ms": round(ms, 5), "us_per_1k_tokens": round(ms * 1e3 * 1024 / L, 3),
                     "value": round(c.tokch / (ms * 1e-3) / 1e9, 2), "plan": list(plan)})
        del t, ws
        torch.cuda.empty_cache()
    return rows


def run_long_bwd(ss, torch, dev, calls=3):
    """The backward on the million-token workload (batch 1, D 2048, N 16, bf16),
    device-generated inputs and dy: the library's automatic split into sequence
    segments against the same backward run whole (one segment).  Kernel time from
    the library's events around each call's kernels."""
    from workloads import LONG, inputs
    from workloads import device as wdev
    cfg = LONG
    b, d, n, L = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen
    t = wdev.scan_inputs(cfg, dev)
    A, dskip, bias = wdev.params(cfg, dev)
    dy = wdev.fill(torch.empty((b, d, L), dtype=torch.bfloat16, device=dev), cfg, inputs.STREAM_DY)
    seg = ss.ss_scan_bwd_segment_len(b, d, n, L, ss.SS_BF16)
    ws = torch.empty(max(ss.bwd_workspace_bytes(b, d, n, L, torch.bfloat16, 0),
                         ss.bwd_workspace_bytes(b, d, n, L, torch.bfloat16, L)), dtype=torch.uint8, device=dev)

    def timed(segment_len):
        def call():
            return ss.scan_bwd(t["x"], t["dt"], t["B"], t["C"], A, dy, z=t["z"], Dskip=dskip, dt_bias=bias,
                               workspace=ws, segment_len=segment_len)
        call()
        torch.cuda.synchronize()
        ss.ss_timing_reset()
        ss.ss_timing_enable(True)
        for _ in range(calls):
            call()
        torch.cuda.synchronize()
        ss.ss_timing_enable(False)
        ms, k = ss.ss_timing_read()
        ss.ss_timing_reset()
        return ms / k

    split_ms = timed(0)
    whole_ms = timed(L)

    # the training-step pair: the forward (chunked plan) storing checkpoints, then
    # the split backward reading them instead of running its own aggregate pass
    ck = torch.empty(ss.ckpt_numel(b, d, n, L), dtype=torch.float32, device=dev)
    fws = torch.empty(max(ss.workspace_bytes(b, d, n, L, torch.bfloat16), 256), dtype=torch.uint8, device=dev)

    def lib_ms(fn):
        fn()
        torch.cuda.synchronize()
        ss.ss_timing_reset()
        ss.ss_timing_enable(True)
        for _ in range(calls):
            fn()
        torch.cuda.synchronize()
        ss.ss_timing_enable(False)
        ms, k = ss.ss_timing_read()
        ss.ss_timing_reset()
        return ms / k

    fwd_ms = lib_ms(lambda: ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias,
                                        workspace=fws))
    fwd_ck_ms = lib_ms(lambda: ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias,
                                           workspace=fws, ckpt=ck))
    bwd_ck_ms = lib_ms(lambda: ss.scan_bwd(t["x"], t["dt"], t["B"], t["C"], A, dy, z=t["z"], Dskip=dskip,
                                           dt_bias=bias, workspace=ws, ckpt=ck))
    del t, dy, ws, ck, fws
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "entry_point": "ss_scan_bwd (automatic split) vs ss_scan_bwd_seg (whole)",
            "segment_len": seg, "segments": (L + seg - 1) // seg, "split_ms": round(split_ms, 3),
            "whole_ms": round(whole_ms, 3), "value_split": round(cfg.tokch / (split_ms * 1e-3) / 1e9, 2),
            "value_whole": round(cfg.tokch / (whole_ms * 1e-3) / 1e9, 2), "unit": "Gtok·ch/s",
            "speedup": round(whole_ms / split_ms, 2), "calls": calls,
            "training_step": {"fwd_ms": round(fwd_ms, 3), "fwd_storing_checkpoints_ms": round(fwd_ck_ms, 3),
                              "bwd_from_checkpoints_ms": round(bwd_ck_ms, 3),
                              "step_ms": round(fwd_ms + split_ms, 3),
                              "step_with_checkpoints_ms": round(fwd_ck_ms + bwd_ck_ms, 3),
                              "checkpoint_bytes": ss.ckpt_numel(b, d, n, L) * 4}}


def cpu_single_thread(budget_s: float = 2.0):
    """The oracle on one host thread over the 130M-shaped workload (fp32 I/O),
    256 channels per call until ~budget_s of oracle time."""
    import numpy as np
    import oracle
    from workloads import M130, inputs
    o = oracle.default()
    A, dskip, bias = inputs.params(M130)
    tokch, spent = 0, 0.0
    pieces = [(b, d0) for b in range(M130.batch) for d0 in range(0, M130.dim, 256)]
    for b, d0 in pieces:
        if spent >= budget_s:
            break
        ch = [(b, d) for d in range(d0, min(M130.dim, d0 + 256))]
        sub = inputs.scan_inputs(M130, channels=ch)
        f = {k: inputs.raw_to_f64(v, M130.io) for k, v in sub.items()}
        idx = np.array([d for _, d in ch])
        t0 = time.perf_counter()
        o.scan(f["x"][None], f["dt"][None], f["B"][b:b + 1], f["C"][b:b + 1], A[idx], z=f["z"][None],
               Dskip=dskip[idx], dt_bias=bias[idx], nthreads=1)
        spent += time.perf_counter() - t0
        tokch += len(ch) * M130.seqlen
    return {"value": tokch / spent / 1e9, "unit": "Gtok·ch/s", "cores": 1, "kind": "oracle",
            "sample": "%d channels x L=%d of the %s workload, one thread (%.1f s)" % (tokch // M130.seqlen,
                                                                                   M130.seqlen, M130.name, spent)}


def cpu_baseline(cfg, budget_s: float):
    """The oracle (as it stands) on host cores over the workload, 1024 channels per
    call, passing over it again until ~budget_s of oracle time; inputs are drawn on
    the host once per piece and kept (untimed).  A workload that one pass cannot
    finish within the budget is cut at a piece boundary."""
    import numpy as np
    import oracle
    from workloads import inputs
    o = oracle.default()
    A, dskip, bias = inputs.params(cfg)
    chans_per_call = 1024
    pieces = [(b, d0) for b in range(cfg.batch) for d0 in range(0, cfg.dim, chans_per_call)]
    cache = {}
    tokch = 0
    spent = 0.0
    passes = 0
    while spent < budget_s:
        for b, d0 in pieces:
            ch = [(b, d) for d in range(d0, min(cfg.dim, d0 + chans_per_call))]
            if (b, d0) not in cache:
                sub = inputs.scan_inputs(cfg, channels=ch)
                cache[(b, d0)] = {k: inputs.raw_to_f64(v, cfg.io) for k, v in sub.items()}
            f = cache[(b, d0)]
            idx = np.array([d for _, d in ch])
            t0 = time.perf_counter()
            o.scan(f["x"][None], f["dt"][None], f["B"][b:b + 1], f["C"][b:b + 1], A[idx], z=f["z"][None],
                   Dskip=dskip[idx], dt_bias=bias[idx])
            spent += time.perf_counter() - t0
            tokch += len(ch) * cfg.seqlen
            if spent >= budget_s:
                break
        passes += 1
    whole = cfg.batch * cfg.dim * cfg.seqlen
    return {"value": tokch / spent / 1e9, "unit": "Gtok·ch/s", "cores": o.max_threads(), "kind": "oracle",
            "sample": "%.2f passes over the %s workload (%d channels x L=%d each), %.1f s of oracle time, float64"
                      % (tokch / whole, cfg.name, cfg.batch * cfg.dim, cfg.seqlen, spent)}


def measured_traffic(cfg, kind: str = "scan"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if
    the kernel sources changed since the counters were taken."""
    try:
        d = json.loads(COUNTERS_FILES[kind].read_text())
    except (OSError, ValueError):
        return None
    if d.get("kernel_hash") != kernel_hash(kind) or d.get("workload") != cfg.name:
        return None
    return d.get("hbm_bytes_per_launch")


def run_cold(ss, torch, dev, cfg, step, calls=20, flush_bytes=512 << 20):
    """Each call preceded by an untimed 512 MB write, which evicts the 256 MB
    Infinity Cache (MALL), so that the call's inputs come from HBM: the scan
    kernel's time per call from the library's events, median and minimum."""
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    times = []
    for i in range(calls + 2):
        flush.fill_(i & 0xFF)
        torch.cuda.synchronize()
        ss.ss_timing_reset()
        ss.ss_timing_enable(True)
        step()
        torch.cuda.synchronize()
        ss.ss_timing_enable(False)
        ms, n = ss.ss_timing_read()
        ss.ss_timing_reset()
        if i >= 2:
            times.append(ms / n)
    del flush
    times.sort()
    med = times[len(times) // 2]
    return {"kernel_ms_median": round(med, 5), "kernel_ms_min": round(times[0], 5), "calls": calls,
            "flush_bytes": flush_bytes, "value_median": round(cfg.tokch / (med * 1e-3) / 1e9, 2),
            "unit": "Gtok·ch/s"}


def run_decode(ss, torch, dev, steps, warmup):
    """Decode step timing (secondary).  "cold": back-to-back steps that rotate over
    6 separate states (503 MB, as the layers of a model would; more than the 256 MB
    MALL, so each step's state comes from HBM).  "warm": back-to-back steps on one
    state, which can stay in the MALL (informational only)."""
    from workloads import DECODE
    from workloads import device as wdev
    cfg = DECODE
    A, dskip, bias = wdev.params(cfg, dev)
    states = [wdev.decode_state0(cfg, dev) for _ in range(6)]
    t = wdev.decode_inputs(cfg, 0, dev)
    args = (t["x"], t["dt"], t["B"], t["C"], A)
    kw = dict(z=t["z"], Dskip=dskip, dt_bias=bias)

    def timed(rotate):
        for i in range(warmup):
            ss.state_update(states[i % 6 if rotate else 0], *args, **kw)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            ss.state_update(states[i % 6 if rotate else 0], *args, **kw)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    warm_ms = timed(False)
    cold_ms = timed(True)
    nbd = cfg.batch * cfg.dim
    bytes_step = nbd * (2 * cfg.dstate * 4 + 4 * 2) + 2 * cfg.batch * cfg.dstate * 2 + cfg.dim * (cfg.dstate + 2) * 4
    return {"workload": cfg.name, "kernel": "state_update_kernel<16,BF16,euler>", "bd_per_step": nbd,
            "ms_per_step_cold": round(cold_ms, 5),
            "ms_per_step_warm": round(warm_ms, 5), "hbm_gbs_cold": round(bytes_step / cold_ms / 1e6, 1),
            "frac_hbm_cold": round(bytes_step / cold_ms / 1e6 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": bytes_step, "traffic": measured_traffic(cfg, "decode"),
            "cold_method": "back-to-back steps rotating over 6 states (503 MB > 256 MB MALL)"}


def run_bwd(ss, torch, dev, cfg, t, A, dskip, bias, fwd_kernel_ms, calls=20):
    """Backward pass of the same workload (secondary): ss_scan_bwd with a seeded
    random dy, all gradients requested; kernels timed by the library's events."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(62200)
    dy = torch.randn(t["x"].shape, generator=gen, device=dev, dtype=torch.float32).to(t["x"].dtype)
    ws = torch.empty(max(ss.bwd_workspace_bytes(cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen, t["x"].dtype), 256),
                     dtype=torch.uint8, device=dev)

    def call():
        return ss.scan_bwd(t["x"], t["dt"], t["B"], t["C"], A, dy, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=ws)

    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    ss.ss_timing_reset()
    ss.ss_timing_enable(True)
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    ss.ss_timing_enable(False)
    ms, n = ss.ss_timing_read()
    ss.ss_timing_reset()
    kms = ms / n

    # a training step's pair: the forward stores the checkpoints, the backward reads them
    ck = torch.empty(ss.ckpt_numel(cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen), dtype=torch.float32, device=dev)
    fws = torch.empty(max(ss.workspace_bytes(cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen, t["x"].dtype), 256),
                      dtype=torch.uint8, device=dev)

    def timed_pair(with_ckpt):
        def fwd():
            ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=fws,
                        ckpt=ck if with_ckpt else None)

        def bwd():
            ss.scan_bwd(t["x"], t["dt"], t["B"], t["C"], A, dy, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=ws,
                        ckpt=ck if with_ckpt else None)
        out = []
        for fn in (fwd, bwd):
            for _ in range(calls):
                fn()
            torch.cuda.synchronize()
            ss.ss_timing_reset()
            ss.ss_timing_enable(True)
            for _ in range(calls):
                fn()
            torch.cuda.synchronize()
            ss.ss_timing_enable(False)
            m, c = ss.ss_timing_read()
            ss.ss_timing_reset()
            out.append(m / c)
        return out
    f_ck, b_ck = timed_pair(True)
    f_no, b_no = timed_pair(False)

    def timed(fn):
        for _ in range(calls):
            fn()
        torch.cuda.synchronize()
        ss.ss_timing_reset()
        ss.ss_timing_enable(True)
        for _ in range(calls):
            fn()
        torch.cuda.synchronize()
        ss.ss_timing_enable(False)
        m, c = ss.ss_timing_read()
        ss.ss_timing_reset()
        return m / c
    # the other forms of the backward on the same workload: zero-order hold, and one
    # dt per (row, token) (the first channel's dt row shared by all channels)
    zoh_ms = timed(lambda: ss.scan_bwd(t["x"], t["dt"], t["B"], t["C"], A, dy, z=t["z"], Dskip=dskip,
                                       dt_bias=bias, workspace=ws, zoh=True))
    dt_row = t["dt"][:, 0, :].contiguous()
    row_ms = timed(lambda: ss.scan_bwd(t["x"], dt_row, t["B"], t["C"], A, dy, z=t["z"], Dskip=dskip,
                                       dt_bias=bias, workspace=ws))
    spt = algorithmic_slots_bwd_per_tokch(cfg.dstate)
    ach = spt * cfg.tokch / (kms * 1e-3) / 1e12
    return {"entry_point": "ss_scan_bwd", "kernel": "scan_bwd_kernel<16,4,2,%s,euler> + reduce kernels" % cfg.io,
            "roofline": {"bound": "alu", "achieved": round(ach, 3), "peak": round(VALU_PEAK_TOPS, 3),
                         "unit": "T VALU-slot/s", "frac": round(ach / VALU_PEAK_TOPS, 4), "slots_per_tokch": spt},
            "kernel_ms": round(kms, 5),
            "value": round(cfg.tokch / (kms * 1e-3) / 1e9, 3), "unit": "Gtok·ch/s",
            "ratio_to_forward": round(kms / fwd_kernel_ms, 3),
            "hbm_gbs": round(algorithmic_bytes_bwd(cfg) / (kms * 1e-3) / 1e9, 1),
            "workspace_bytes": ws.numel(), "traffic": measured_traffic(cfg, "bwd"),
            "zoh": {"entry_point": "ss_scan_bwd_ex (SS_FLAG_ZOH)", "kernel_ms": round(zoh_ms, 5),
                    "value": round(cfg.tokch / (zoh_ms * 1e-3) / 1e9, 3)},
            "dt_per_row": {"entry_point": "ss_scan_bwd_ex (SS_FLAG_DT_PER_ROW)", "kernel_ms": round(row_ms, 5),
                           "value": round(cfg.tokch / (row_ms * 1e-3) / 1e9, 3)},
            "training_step": {"fwd_kernel_ms": round(f_no, 5), "bwd_kernel_ms": round(b_no, 5),
                              "fwd_storing_checkpoints_kernel_ms": round(f_ck, 5),
                              "bwd_from_checkpoints_kernel_ms": round(b_ck, 5),
                              "bwd_from_checkpoints_frac": round(
                                  algorithmic_slots_bwd_per_tokch(cfg.dstate, sweep=False) * cfg.tokch
                                  / (b_ck * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
                              "step_ms": round(f_no + b_no, 5), "step_with_checkpoints_ms": round(f_ck + b_ck, 5),
                              "checkpoint_bytes": ck.numel() * 4}}


def run_cp(ss, torch, cfg, t, A, dskip, bias, G, reps=10):
    """One GPU's share of a context-parallel run over G shards (secondary): the
    shard's aggregate, the combine over G shards and the shard's rescan from its
    entering state, at the real shard shape (the all-gather of the pairs between
    GPUs is not part of it)."""
    L = cfg.seqlen // G
    sh = {k: v[..., :L].contiguous() for k, v in t.items()}
    dsum, h_end = ss.shard_state(sh["x"], sh["dt"], sh["B"], A, dt_bias=bias)
    ds_all = dsum.unsqueeze(0).repeat(G, 1, 1).contiguous()
    he_all = h_end.unsqueeze(0).repeat(G, 1, 1, 1).contiguous()
    h_in, _ = ss.shard_combine(A, ds_all, he_all)
    h0 = h_in[G - 1].contiguous()
    ws = torch.empty(max(ss.workspace_bytes(cfg.batch, cfg.dim, cfg.dstate, L, t["x"].dtype), 256), dtype=torch.uint8,
                     device=t["x"].device)
    y = torch.empty_like(sh["x"])

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_state = timed(lambda: ss.shard_state(sh["x"], sh["dt"], sh["B"], A, dt_bias=bias, workspace=ws))
    ms_comb = timed(lambda: ss.shard_combine(A, ds_all, he_all))
    ms_scan = timed(lambda: ss.scan_fwd(sh["x"], sh["dt"], sh["B"], sh["C"], A, z=sh["z"], Dskip=dskip, dt_bias=bias,
                                        h0=h0, workspace=ws, y=y))
    per_gpu = ms_state + ms_comb + ms_scan
    return {"shards": G, "shard_tokens": L, "ms_shard_state": round(ms_state, 4), "ms_combine": round(ms_comb, 4),
            "ms_shard_scan": round(ms_scan, 4), "ms_per_gpu": round(per_gpu, 4),
            "projected_value": round(cfg.tokch / (per_gpu * 1e-3) / 1e9, 2), "unit": "Gtok·ch/s",
            "exchange_bytes_per_gpu": G * cfg.batch * cfg.dim * (cfg.dstate + 1) * 4,
            "note": "projection for G GPUs excludes the all-gather of the (dsum, h_end) pairs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="untimed scan calls for at least this long before the counted warm-up steps, "
                         "so that the timed steps run at the steady clock")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-flushed per-call timing")
    ap.add_argument("--no-rates", action="store_true", help="skip the VALU issue-rate probe")
    ap.add_argument("--rates-only", action="store_true", help="only run the VALU issue-rate probe")
    ap.add_argument("--workload", default="2.8b-layer-bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step timing")
    ap.add_argument("--no-zoh", action="store_true", help="skip the zero-order-hold scan timing")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--no-dt-row", action="store_true", help="skip the dt-per-row scan timing")
    ap.add_argument("--cp-shards", type=int, default=0,
                    help="also time one GPU's share of a context-parallel run over this many shards")
    ap.add_argument("--copy-calib", type=int, default=0, help="only run a plain copy of this many bytes")
    ap.add_argument("--l-sweep", action="store_true",
                    help="also time the scan at L = 512 ... 16384 with the workload's batch and channels")
    ap.add_argument("--long-bwd", action="store_true",
                    help="also time the backward on the million-token workload, split into segments and whole")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the selective scan is built and measured on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_62_amd as ss
    from workloads import BY_NAME
    from workloads import device as wdev

    dev = torch.device("cuda:0")
    if args.rates_only:
        torch.cuda.init()
        print(json.dumps({"valu_rates": run_valu_rates()}))
        return
    if args.copy_calib:
        src = torch.ones(args.copy_calib // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": args.copy_calib}))
        return

    cfg = BY_NAME[args.workload]
    assert cfg.mode == "scan"
    io = ss.SS_BF16 if cfg.io == "bf16" else ss.SS_F32
    t = wdev.scan_inputs(cfg, dev)
    A, dskip, bias = wdev.params(cfg, dev)
    plan = ss.ss_scan_fwd_plan(cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen, io)
    ws = torch.empty(ss.workspace_bytes(cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen, t["x"].dtype), dtype=torch.uint8,
                     device=dev)
    y = torch.empty_like(t["x"])
    hf = torch.empty((cfg.batch, cfg.dim, cfg.dstate), dtype=torch.float32, device=dev)

    def step():
        ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=ws, y=y,
                    h_final=hf)

    # settle: untimed calls until the clock has ramped (the first launches of a
    # process run up to 30% slower), then the counted warm-up steps
    settle_calls = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        settle_calls += 10
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ss.ss_timing_reset()
    ss.ss_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ss.ss_timing_enable(False)
    kern_ms_total, calls = ss.ss_timing_read()
    ss.ss_timing_reset()
    assert calls == args.steps
    ms_step = elapsed * 1e3 / args.steps
    kern_ms = kern_ms_total / calls
    tokch = cfg.tokch
    value = tokch / (ms_step * 1e-3) / 1e9
    bpt = algorithmic_bytes_per_tokch(cfg)
    spt = algorithmic_slots_per_tokch(cfg.dstate)
    achieved_slots = spt * tokch / (kern_ms * 1e-3) / 1e12
    achieved_gbs = bpt * tokch / (kern_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg)
    kname = "scan_kernel<%d,%d,%d,%s,euler>" % (cfg.dstate, plan[0], plan[1], cfg.io)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gtok·ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": round(settle_ms, 1),
        "settle_calls": settle_calls,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.io == "bf16" else "f32",
        "data": "synthetic (seeded Philox4x32-10 draws through an inverse-normal table, generated on the device)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "channels": cfg.dim, "dstate": cfg.dstate,
                   "seq_len": cfg.seqlen, "io": cfg.io, "state": "f32", "plan": {"state_groups": plan[0],
                   "lanes_per_channel": plan[1], "chunk_len": plan[2]}},
        "hbm_gbs": round(bpt * tokch / (ms_step * 1e-3) / 1e9, 1),
        "roofline": graded_roofline(cfg, kern_ms, traffic, kname),
        "roofline_valu_issue": {"bound": "alu", "achieved": round(achieved_slots, 3),
                                "peak": round(VALU_PEAK_TOPS, 3), "unit": "T VALU-slot/s",
                                "frac": round(achieved_slots / VALU_PEAK_TOPS, 4), "slots_per_tokch": spt},
        "roofline_hbm": {"achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "bytes_per_tokch": round(bpt, 4)},
        "ceilings": ceilings(cfg, tokch / (kern_ms * 1e-3) / 1e9),
    }
    if not args.no_cold:
        out["cold_cache"] = run_cold(ss, torch, dev, cfg, step)
    if not args.no_rates:
        out["valu_rates"] = run_valu_rates()
    if not args.no_dt_row:
        # dt shared by a row's channels (SS_FLAG_DT_PER_ROW): the same workload with
        # one dt row per batch row (secondary)
        dtr = t["dt"][:, 0, :].contiguous()
        for _ in range(100):
            ss.scan_fwd(t["x"], dtr, t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=ws, y=y,
                        h_final=hf)
        torch.cuda.synchronize()
        ss.ss_timing_reset()
        ss.ss_timing_enable(True)
        for _ in range(20):
            ss.scan_fwd(t["x"], dtr, t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=ws, y=y,
                        h_final=hf)
        torch.cuda.synchronize()
        ss.ss_timing_enable(False)
        rms, rn = ss.ss_timing_read()
        ss.ss_timing_reset()
        eb = 2 if cfg.io == "bf16" else 4
        rbytes = bpt * tokch - eb * tokch + eb * cfg.batch * cfg.seqlen
        out["dt_per_row"] = {"entry_point": "ss_scan_fwd_ex (SS_FLAG_DT_PER_ROW)", "kernel_ms": round(rms / rn, 5),
                             "value": round(tokch / (rms / rn * 1e-3) / 1e9, 3), "unit": "Gtok·ch/s",
                             "algorithmic_bytes": int(rbytes),
                             "hbm_gbs": round(rbytes / (rms / rn * 1e-3) / 1e9, 1)}
    if not args.no_zoh:
        # the same workload through the zero-order-hold entry point (secondary)
        for _ in range(20):
            ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=ws, y=y,
                        h_final=hf, zoh=True)
        torch.cuda.synchronize()
        ss.ss_timing_reset()
        ss.ss_timing_enable(True)
        for _ in range(20):
            ss.scan_fwd(t["x"], t["dt"], t["B"], t["C"], A, z=t["z"], Dskip=dskip, dt_bias=bias, workspace=ws, y=y,
                        h_final=hf, zoh=True)
        torch.cuda.synchronize()
        ss.ss_timing_enable(False)
        zms, zn = ss.ss_timing_read()
        ss.ss_timing_reset()
        out["zoh"] = {"entry_point": "ss_scan_fwd_zoh", "kernel_ms": round(zms / zn, 5),
                      "value": round(tokch / (zms / zn * 1e-3) / 1e9, 3), "unit": "Gtok·ch/s"}
    if not args.no_bwd:
        out["bwd"] = run_bwd(ss, torch, dev, cfg, t, A, dskip, bias, kern_ms)
    if args.cp_shards > 1:
        out["context_parallel"] = run_cp(ss, torch, cfg, t, A, dskip, bias, args.cp_shards)
    if args.l_sweep:
        out["l_sweep"] = run_l_sweep(ss, torch, dev, cfg)
    if args.long_bwd:
        out["long_bwd"] = run_long_bwd(ss, torch, dev)
    if not args.no_decode:
        out["decode"] = run_decode(ss, torch, dev, 60, 60)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
        out["cpu_baseline"]["host_cpus_in_affinity"] = len(os.sched_getaffinity(0))
        out["cpu_baseline"]["single_thread"] = cpu_single_thread()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
