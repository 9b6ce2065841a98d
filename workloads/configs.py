"""The five selective-scan workloads: shapes, I/O dtypes and value recipes.

Shapes follow the Mamba paper's language models as summarised in the reader's
notes (kurisu.si, "What they did"): expansion E = 2 over the model width, state
size N = 16, context 2048; the long-context case uses the million-token length
of the induction-heads evaluation ("Main results (verified)").
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class ScanConfig:
    index: int            # 1-based workload number
    name: str
    batch: int
    dim: int              # D = channels = E * d_model
    dstate: int           # N
    seqlen: int           # L (1 for decode)
    io: str               # "f32" or "bf16": dtype of x, dt, z, B, C, y
    dskip: str            # "one" or "normal" (N(1, 0.1))
    mode: str = "scan"    # "scan" or "decode"
    steps: int = 1        # decode steps
    check_channels: int = 0   # >0: the oracle checks this many sampled channels

    @property
    def seed(self) -> int:
        return 62000 + self.index

    @property
    def tokch(self) -> int:
        """(batch, channel, token) elements per call."""
        return self.batch * self.dim * self.seqlen


TINY = ScanConfig(1, "tiny-f32", 1, 16, 4, 64, "f32", "one")
M130 = ScanConfig(2, "130m-layer-f32", 8, 1536, 16, 2048, "f32", "normal")
B28 = ScanConfig(3, "2.8b-layer-bf16", 8, 5120, 16, 2048, "bf16", "one")
LONG = ScanConfig(4, "long-1m-bf16", 1, 2048, 16, 1 << 20, "bf16", "one", check_channels=64)
DECODE = ScanConfig(5, "decode-bf16", 256, 5120, 16, 1, "bf16", "one", mode="decode", steps=128)

CONFIGS = (TINY, M130, B28, LONG, DECODE)
BY_NAME = {c.name: c for c in CONFIGS}


def tolerance(cfg: ScanConfig) -> float:
    """rel-L2 bound: 1e-5 for fp32 I/O, 2e-2 for bf16 I/O with an fp32 state."""
    return 1e-5 if cfg.io == "f32" else 2e-2
