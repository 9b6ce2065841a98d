"""CPU oracle for the selective state-space (S6) scan — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  The GPU library never uses it, and it shares no code
with the GPU library.  The arithmetic lives in ``ss_oracle.c`` (plain C, double
precision, one channel and one token at a time); this module only builds that
file with gcc and marshals numpy arrays to it.

Every function here is pinned in ``tests/test_oracle_pins.py`` against closed
forms and invariants that the pages fix (Theorem 1 of the reader's notes, the
small/large-Delta limits, the LTI convolution, the unrolled sum, ...).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "ss_oracle.c"
LIB = HERE / "liboracle.so"

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def compile_oracle(src: Path = SRC, out: Path = LIB) -> Path:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    tmp = out.with_suffix(".so.tmp%d" % os.getpid())
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", str(tmp), str(src), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _as_f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


class Oracle:
    """ctypes handle on one compiled copy of the oracle."""

    def __init__(self, path: Path | str = LIB):
        path = Path(path)
        if not path.exists() and path == LIB:
            compile_oracle()
        self.lib = ctypes.CDLL(str(path))
        self.lib.ss_oracle_scan.restype = ctypes.c_int
        self.lib.ss_oracle_scan.argtypes = [_i64, _i64, _i64, _i64] + [_dp] * 9 + [ctypes.c_int, _dp, _dp, ctypes.c_int]
        self.lib.ss_oracle_state_update.restype = ctypes.c_int
        self.lib.ss_oracle_state_update.argtypes = [_i64, _i64, _i64, _dp] + [_dp] * 8 + [ctypes.c_int, _dp, ctypes.c_int]
        self.lib.ss_oracle_max_threads.restype = ctypes.c_int
        self.lib.ss_oracle_scan_bwd.restype = ctypes.c_int
        self.lib.ss_oracle_scan_bwd.argtypes = ([_i64, _i64, _i64, _i64] + [_dp] * 9 + [ctypes.c_int] + [_dp] * 2
                                                + [_dp] * 9 + [ctypes.c_int])

    def max_threads(self) -> int:
        return int(self.lib.ss_oracle_max_threads())

    def scan(self, x, dt, B, C, A, z=None, Dskip=None, dt_bias=None, h0=None,
             zoh=False, nthreads=0):
        """Full-sequence scan.

        x, dt, z: (batch, D, L); B, C: (batch, N, L); A: (D, N); Dskip, dt_bias: (D,);
        h0: (batch, D, N).  Returns (y (batch, D, L), h_final (batch, D, N)) in float64.
        """
        x, dt, z, B, C, A = map(_as_f64, (x, dt, z, B, C, A))
        Dskip, dt_bias, h0 = map(_as_f64, (Dskip, dt_bias, h0))
        batch, D, L = x.shape
        N = A.shape[1]
        assert dt.shape == x.shape and B.shape == (batch, N, L) and C.shape == (batch, N, L)
        assert A.shape == (D, N)
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (batch, D, N)
        y = np.empty((batch, D, L), dtype=np.float64)
        hf = np.empty((batch, D, N), dtype=np.float64)
        rc = self.lib.ss_oracle_scan(batch, D, N, L, _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C),
                                     _ptr(A), _ptr(Dskip), _ptr(dt_bias), _ptr(h0), int(bool(zoh)),
                                     _ptr(y), _ptr(hf), int(nthreads))
        if rc != 0:
            raise ValueError("ss_oracle_scan rejected its arguments (%d)" % rc)
        return y, hf

    def scan_bwd(self, x, dt, B, C, A, dy, z=None, Dskip=None, dt_bias=None, h0=None, dh_final=None,
                 zoh=False, nthreads=0):
        """Gradients of the full-sequence scan for upstream gradients dy (batch, D, L) and
        dh_final (batch, D, N) (None = 0).

        Returns a dict of float64 arrays: dx, ddt, dz (None without z) (batch, D, L);
        dB, dC (batch, N, L); dA (D, N); dDskip, ddt_bias (D,); dh0 (batch, D, N).
        The gradients with respect to Dskip, dt_bias and h0 are returned also when those
        inputs are None (they are then taken as zeros).
        """
        x, dt, z, B, C, A, dy = map(_as_f64, (x, dt, z, B, C, A, dy))
        Dskip, dt_bias, h0, dh_final = map(_as_f64, (Dskip, dt_bias, h0, dh_final))
        batch, D, L = x.shape
        N = A.shape[1]
        assert dt.shape == x.shape and dy.shape == x.shape
        assert B.shape == (batch, N, L) and C.shape == (batch, N, L) and A.shape == (D, N)
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (batch, D, N)
        assert dh_final is None or dh_final.shape == (batch, D, N)
        out = dict(dx=np.empty((batch, D, L)), ddt=np.empty((batch, D, L)),
                   dz=np.empty((batch, D, L)) if z is not None else None,
                   dB=np.empty((batch, N, L)), dC=np.empty((batch, N, L)), dA=np.empty((D, N)),
                   dDskip=np.empty(D), ddt_bias=np.empty(D), dh0=np.empty((batch, D, N)))
        rc = self.lib.ss_oracle_scan_bwd(batch, D, N, L, _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C), _ptr(A),
                                         _ptr(Dskip), _ptr(dt_bias), _ptr(h0), int(bool(zoh)), _ptr(dy),
                                         _ptr(dh_final), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dz"]),
                                         _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dA"]), _ptr(out["dDskip"]),
                                         _ptr(out["ddt_bias"]), _ptr(out["dh0"]), int(nthreads))
        if rc != 0:
            raise ValueError("ss_oracle_scan_bwd failed (%d)" % rc)
        return out

    def state_update(self, state, x, dt, B, C, A, z=None, Dskip=None, dt_bias=None,
                     zoh=False, nthreads=0):
        """One decode step.  state: (batch, D, N); x, dt, z: (batch, D); B, C: (batch, N).

        Returns (y (batch, D), new_state (batch, D, N)); the input state is not modified.
        """
        st = np.array(state, dtype=np.float64, copy=True, order="C")
        x, dt, z, B, C, A = map(_as_f64, (x, dt, z, B, C, A))
        Dskip, dt_bias = map(_as_f64, (Dskip, dt_bias))
        batch, D = x.shape
        N = A.shape[1]
        assert st.shape == (batch, D, N) and B.shape == (batch, N) and C.shape == (batch, N)
        y = np.empty((batch, D), dtype=np.float64)
        rc = self.lib.ss_oracle_state_update(batch, D, N, _ptr(st), _ptr(x), _ptr(dt), _ptr(z),
                                             _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip), _ptr(dt_bias),
                                             int(bool(zoh)), _ptr(y), int(nthreads))
        if rc != 0:
            raise ValueError("ss_oracle_state_update rejected its arguments (%d)" % rc)
        return y, st


_default = None


def default() -> Oracle:
    """The oracle built from ``ss_oracle.c`` (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not LIB.exists():
            compile_oracle()
        _default = Oracle(LIB)
    return _default
