"""Seeded synthetic inputs for the selective-scan workloads (host side).

Every per-token tensor (x, dt, z, B, C) and the decode initial state are drawn
from Philox4x32-10 streams mapped through a 65536-entry inverse-normal table:
draw ``j`` (16 bits) becomes ``Phi^-1((j + 0.5) / 65536)`` rounded to the I/O
dtype (fp32 round-to-nearest; bf16 round-to-nearest-even of that fp32 value).
``dt`` uses the same table scaled by 0.5 (exact, a power of two), giving
N(0, 0.5^2).  Because the mapping is integer hashing plus a table lookup, the
device generator (``workloads.device``) reproduces these values bit for bit,
which lets the 17 GB long-context inputs be generated on the GPU while the CPU
oracle draws only the channels it checks.

Per-channel parameters (dt_bias, Dskip) are small and drawn with numpy's PCG64:
  u ~ log-uniform[1e-3, 1e-1],  dt_bias = log(expm1(u))  (the softplus inverse),
  Dskip = 1, or ~ N(1, 0.1) for the 130M-shaped layer.
A[d, n] = -(n + 1).

Nothing in this module computes any step of the selective scan.
"""
from __future__ import annotations

import functools
from statistics import NormalDist

import numpy as np

from .philox import draw_u16
from .configs import ScanConfig

# Philox stream ids, one per tensor
STREAM_X, STREAM_DT, STREAM_Z, STREAM_B, STREAM_C, STREAM_H0 = 1, 2, 3, 4, 5, 6
STREAM_DY = 7  # the upstream gradient dy of a backward workload, N(0, 1) like x
KEY1 = 0x53533632  # second key word, fixed for all workloads


@functools.lru_cache(maxsize=None)
def _normal_f64() -> np.ndarray:
    nd = NormalDist()
    j = np.arange(65536, dtype=np.float64)
    return np.array([nd.inv_cdf(p) for p in (j + 0.5) / 65536.0], dtype=np.float64)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@functools.lru_cache(maxsize=None)
def table(io: str, scale: float = 1.0) -> np.ndarray:
    """The lookup table for one I/O dtype: float32 values, or uint16 bf16 bits."""
    t32 = (_normal_f64() * scale).astype(np.float32)
    if io == "f32":
        return t32
    if io == "bf16":
        return f32_to_bf16_bits(t32)
    raise ValueError(io)


def raw_to_f64(raw: np.ndarray, io: str) -> np.ndarray:
    """Exact widening of stored I/O values (fp32, or bf16 bits) to float64."""
    if io == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(raw).astype(np.float64)


def draw(cfg: ScanConfig, stream: int, start: int, count: int, step: int = 0,
         scale: float = 1.0) -> np.ndarray:
    """Draws ``[start, start+count)`` of one tensor stream as raw I/O values."""
    idx = draw_u16(cfg.seed, KEY1, stream, step, start, count)
    return table(cfg.io, scale)[idx]


def draw_at(cfg: ScanConfig, stream: int, index: np.ndarray, step: int = 0, scale: float = 1.0,
            io: str | None = None) -> np.ndarray:
    """Draws at arbitrary element indices of one stream (vectorised)."""
    from .philox import philox4x32_10
    index = np.asarray(index, dtype=np.uint64)
    blk = index >> np.uint64(3)
    lo = (blk & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    hi = (blk >> np.uint64(32)).astype(np.uint32)
    w = np.stack(philox4x32_10(lo, hi, np.uint32(stream), np.uint32(step), cfg.seed, KEY1), axis=-1)
    k = (index & np.uint64(7)).astype(np.int64)
    word = np.take_along_axis(w, (k >> 1)[..., None], axis=-1)[..., 0]
    j = ((word >> ((k & 1) * 16).astype(np.uint32)) & 0xFFFF).astype(np.int64)
    return table(io or cfg.io, scale)[j]


def draw_state(cfg: ScanConfig, start: int, count: int) -> np.ndarray:
    """Initial decode state (always fp32), N(0, 1)."""
    idx = draw_u16(cfg.seed, KEY1, STREAM_H0, 0, start, count)
    return table("f32", 1.0)[idx]


def params(cfg: ScanConfig):
    """Per-channel parameters: (A (D,N) f32, Dskip (D,) f32, dt_bias (D,) f32)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    u = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), cfg.dim))
    dt_bias = np.log(np.expm1(u)).astype(np.float32)
    if cfg.dskip == "normal":
        dskip = rng.normal(1.0, 0.1, cfg.dim).astype(np.float32)
    else:
        dskip = np.ones(cfg.dim, dtype=np.float32)
    A = np.tile(-(np.arange(cfg.dstate, dtype=np.float32) + 1.0), (cfg.dim, 1))
    return np.ascontiguousarray(A), dskip, dt_bias


def scan_inputs(cfg: ScanConfig, channels=None, t0: int = 0, t1: int | None = None):
    """Raw scan inputs on the host.

    ``channels`` (a list of (b, d) pairs) restricts x/dt/z to those channels, returned as
    arrays of shape (len(channels), t1-t0); B and C are always returned in full for
    every batch row: (batch, N, t1-t0).  Without ``channels`` the full (batch, D, L)
    tensors are returned.
    """
    L = cfg.seqlen
    t1 = L if t1 is None else t1
    n = t1 - t0
    out = {}
    if channels is None:
        rows = [(b, d) for b in range(cfg.batch) for d in range(cfg.dim)]
    else:
        rows = list(channels)
    for name, stream, scale in (("x", STREAM_X, 1.0), ("dt", STREAM_DT, 0.5), ("z", STREAM_Z, 1.0)):
        parts = [draw(cfg, stream, (b * cfg.dim + d) * L + t0, n, scale=scale) for (b, d) in rows]
        arr = np.stack(parts) if parts else np.zeros((0, n), dtype=table(cfg.io).dtype)
        if channels is None:
            arr = arr.reshape(cfg.batch, cfg.dim, n)
        out[name] = arr
    for name, stream in (("B", STREAM_B), ("C", STREAM_C)):
        parts = [draw(cfg, stream, (b * cfg.dstate + s) * L + t0, n)
                 for b in range(cfg.batch) for s in range(cfg.dstate)]
        out[name] = np.stack(parts).reshape(cfg.batch, cfg.dstate, n)
    return out


def scan_inputs_full(cfg: ScanConfig):
    """Full raw tensors, drawn contiguously (fast path for small configs)."""
    L, nch = cfg.seqlen, cfg.batch * cfg.dim
    out = {}
    for name, stream, scale in (("x", STREAM_X, 1.0), ("dt", STREAM_DT, 0.5), ("z", STREAM_Z, 1.0)):
        out[name] = draw(cfg, stream, 0, nch * L, scale=scale).reshape(cfg.batch, cfg.dim, L)
    for name, stream in (("B", STREAM_B), ("C", STREAM_C)):
        out[name] = draw(cfg, stream, 0, cfg.batch * cfg.dstate * L).reshape(cfg.batch, cfg.dstate, L)
    return out


def decode_inputs(cfg: ScanConfig, step: int, channels=None):
    """Raw inputs of one decode step: x, dt, z (batch, D) and B, C (batch, N).

    With ``channels`` (list of (b, d)), x/dt/z come back as (len(channels),).
    """
    nch = cfg.batch * cfg.dim
    out = {}
    for name, stream, scale in (("x", STREAM_X, 1.0), ("dt", STREAM_DT, 0.5), ("z", STREAM_Z, 1.0)):
        if channels is None:
            out[name] = draw(cfg, stream, 0, nch, step=step, scale=scale).reshape(cfg.batch, cfg.dim)
        else:
            idx = np.array([b * cfg.dim + d for (b, d) in channels], dtype=np.uint64)
            out[name] = draw_at(cfg, stream, idx, step=step, scale=scale)
    for name, stream in (("B", STREAM_B), ("C", STREAM_C)):
        out[name] = draw(cfg, stream, 0, cfg.batch * cfg.dstate, step=step).reshape(cfg.batch, cfg.dstate)
    return out


def decode_state0(cfg: ScanConfig, channels=None):
    """Initial decode state (batch, D, N) fp32, or (len(channels), N)."""
    N = cfg.dstate
    if channels is None:
        return draw_state(cfg, 0, cfg.batch * cfg.dim * N).reshape(cfg.batch, cfg.dim, N)
    idx = np.array([(b * cfg.dim + d) * N + n for (b, d) in channels for n in range(N)], dtype=np.uint64)
    return draw_at(cfg, STREAM_H0, idx, io="f32").reshape(len(channels), N)


def sample_channels(cfg: ScanConfig, count: int, seed_offset: int = 40):
    """A seeded, sorted sample of ``count`` distinct (b, d) channels."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed + seed_offset))
    total = cfg.batch * cfg.dim
    flat = np.sort(rng.choice(total, size=min(count, total), replace=False))
    return [(int(f // cfg.dim), int(f % cfg.dim)) for f in flat]


def sample_rows(cfg: ScanConfig, rows: int, per_row: int, seed_offset: int = 41):
    """A seeded sample of ``per_row`` channels in each of ``rows`` batch rows, sorted."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed + seed_offset))
    bs = np.sort(rng.choice(cfg.batch, size=min(rows, cfg.batch), replace=False))
    out = []
    for b in bs:
        ds = np.sort(rng.choice(cfg.dim, size=min(per_row, cfg.dim), replace=False))
        out.extend((int(b), int(d)) for d in ds)
    return out
