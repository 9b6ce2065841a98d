"""Device-side generation of the seeded workloads (bit-identical to workloads.inputs).

Used for the inputs too large to draw on the host quickly (the 2.8B-shaped
layer, the million-token sequence, the 128 decode steps).  Built from
``workloads/csrc/wlgen.hip`` into ``workloads/libwlgen.so``.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
from pathlib import Path

import numpy as np

try:
    from .configs import ScanConfig
    from . import inputs as _in
except ImportError:  # loaded as a standalone file to build the generator library
    ScanConfig = object
    _in = None

HERE = Path(__file__).resolve().parent
SRC = HERE / "csrc" / "wlgen.hip"
LIB = HERE / "libwlgen.so"


def build() -> Path:
    hipcc = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", str(tmp), str(SRC)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("wlgen build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime, see selective_state_space_62_amd.binding)
        if not LIB.exists():
            raise ImportError("workloads/libwlgen.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(str(LIB))
        lib.wl_fill.restype = ctypes.c_int
        lib.wl_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        lib.wl_philox.restype = ctypes.c_int
        lib.wl_philox.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p]
        _lib = lib
    return _lib


_tables = {}


def _table(io: str, scale: float, device):
    import torch
    key = (io, scale, str(device))
    if key not in _tables:
        t = _in.table(io, scale)
        if io == "f32":
            _tables[key] = torch.from_numpy(t.copy()).to(device)
        else:
            _tables[key] = torch.from_numpy(t.view(np.int16).copy()).to(device)
    return _tables[key]


def fill(out, cfg: ScanConfig, stream: int, step: int = 0, start: int = 0, scale: float = 1.0, io=None):
    """Fill the contiguous tensor ``out`` with draws [start, start + out.numel())."""
    import torch
    io = io or cfg.io
    tab = _table(io, scale, out.device)
    eb = 4 if io == "f32" else 2
    assert out.is_contiguous() and out.element_size() == eb
    rc = _load().wl_fill(tab.data_ptr(), eb, cfg.seed, _in.KEY1, stream, step, start, out.numel(), out.data_ptr(),
                         torch.cuda.current_stream(out.device).cuda_stream)
    if rc != 0:
        raise RuntimeError("wl_fill failed with HIP error %d" % rc)
    return out


def _dtype(cfg):
    import torch
    return torch.float32 if cfg.io == "f32" else torch.bfloat16


def scan_inputs(cfg: ScanConfig, device):
    """Full x, dt, z (batch, D, L) and B, C (batch, N, L) on the device."""
    import torch
    dt_ = _dtype(cfg)
    L = cfg.seqlen
    out = {}
    for name, st, scale in (("x", _in.STREAM_X, 1.0), ("dt", _in.STREAM_DT, 0.5), ("z", _in.STREAM_Z, 1.0)):
        out[name] = fill(torch.empty((cfg.batch, cfg.dim, L), dtype=dt_, device=device), cfg, st, scale=scale)
    for name, st in (("B", _in.STREAM_B), ("C", _in.STREAM_C)):
        out[name] = fill(torch.empty((cfg.batch, cfg.dstate, L), dtype=dt_, device=device), cfg, st)
    return out


def decode_inputs(cfg: ScanConfig, step: int, device):
    import torch
    dt_ = _dtype(cfg)
    out = {}
    for name, st, scale in (("x", _in.STREAM_X, 1.0), ("dt", _in.STREAM_DT, 0.5), ("z", _in.STREAM_Z, 1.0)):
        out[name] = fill(torch.empty((cfg.batch, cfg.dim), dtype=dt_, device=device), cfg, st, step=step, scale=scale)
    for name, st in (("B", _in.STREAM_B), ("C", _in.STREAM_C)):
        out[name] = fill(torch.empty((cfg.batch, cfg.dstate), dtype=dt_, device=device), cfg, st, step=step)
    return out


def decode_state0(cfg: ScanConfig, device):
    import torch
    return fill(torch.empty((cfg.batch, cfg.dim, cfg.dstate), dtype=torch.float32, device=device), cfg,
                _in.STREAM_H0, io="f32")


def params(cfg: ScanConfig, device):
    import torch
    A, dskip, bias = _in.params(cfg)
    return (torch.from_numpy(A).to(device), torch.from_numpy(dskip).to(device), torch.from_numpy(bias).to(device))


def philox_raw(ctr: np.ndarray, key: np.ndarray, device):
    """Raw Philox4x32-10 blocks on the device (for known-answer checks)."""
    import torch
    n = ctr.shape[0]
    c = torch.from_numpy(ctr.astype(np.uint32).view(np.int32)).to(device)
    k = torch.from_numpy(key.astype(np.uint32).view(np.int32)).to(device)
    o = torch.empty((n, 4), dtype=torch.int32, device=device)
    rc = _load().wl_philox(c.data_ptr(), k.data_ptr(), o.data_ptr(), n, torch.cuda.current_stream(device).cuda_stream)
    if rc != 0:
        raise RuntimeError("wl_philox failed with HIP error %d" % rc)
    return o.cpu().numpy().view(np.uint32)
