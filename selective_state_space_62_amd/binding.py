"""Thin ctypes binding of libssscan.so (include/ssscan.h).

Only argument marshalling lives here: every step of the scan and of the decode
update runs in the library's HIP kernels.  PyTorch supplies device memory (the
tensors) and the stream (``torch.cuda.current_stream()``).  If the library is
missing this module raises ImportError: there is no fallback.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libssscan.so"
HEADER = _PKG.parent / "include" / "ssscan.h"

SS_F32, SS_BF16 = 0, 1
SS_OK, SS_ERR_INVALID_ARG, SS_ERR_UNSUPPORTED, SS_ERR_WORKSPACE, SS_ERR_HIP = range(5)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


class ss_scan_plan(ctypes.Structure):
    _fields_ = [("state_groups", ctypes.c_int32), ("lanes_per_channel", ctypes.c_int32),
                ("chunk_len", ctypes.c_int64)]


class SsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (status_string(status), message))
        self.status = status


def _load():
    # PyTorch ships its own HIP runtime (SONAME libamdhip64.so.7).  Loading torch
    # first makes the dynamic linker bind this library's libamdhip64.so.7 to that
    # same copy, so the library launches on torch's streams with torch's device
    # memory inside one runtime.  (Loaded the other way round, the process would
    # hold two HIP runtimes.)
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - torch is part of the image
        pass
    if not LIB_PATH.exists():
        raise ImportError("libssscan.so is not built (%s); run __graft_entry__.build() or "
                          "python -m selective_state_space_62_amd._build" % LIB_PATH)
    lib = ctypes.CDLL(str(LIB_PATH))
    lib.ss_abi_version.restype = _int
    lib.ss_status_string.restype = ctypes.c_char_p
    lib.ss_status_string.argtypes = [_int]
    lib.ss_last_error.restype = ctypes.c_char_p
    lib.ss_scan_fwd_plan.restype = _int
    lib.ss_scan_fwd_plan.argtypes = [_i64, _i64, _int, _i64, _int, ctypes.POINTER(ss_scan_plan)]
    lib.ss_scan_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_scan_fwd_workspace_bytes.argtypes = [_i64, _i64, _int, _i64, _int, ctypes.POINTER(ss_scan_plan)]
    lib.ss_scan_fwd.restype = _int
    lib.ss_scan_fwd.argtypes = ([_i64, _i64, _int, _i64, _int] + [_vp] * 11 + [_vp, ctypes.c_size_t,
                                ctypes.POINTER(ss_scan_plan), _vp])
    lib.ss_state_update.restype = _int
    lib.ss_state_update.argtypes = [_i64, _i64, _int, _int] + [_vp] * 11
    lib.ss_scan_fwd_zoh.restype = _int
    lib.ss_scan_fwd_zoh.argtypes = lib.ss_scan_fwd.argtypes
    lib.ss_state_update_zoh.restype = _int
    lib.ss_state_update_zoh.argtypes = lib.ss_state_update.argtypes
    lib.ss_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_scan_bwd_workspace_bytes.argtypes = [_i64, _i64, _int, _i64, _int]
    lib.ss_scan_bwd.restype = _int
    lib.ss_scan_bwd.argtypes = [_i64, _i64, _int, _i64, _int] + [_vp] * 21 + [ctypes.c_size_t, _vp]
    lib.ss_scan_fwd_ex.restype = _int
    lib.ss_scan_fwd_ex.argtypes = ([_i64, _i64, _int, _i64, _int, ctypes.c_uint32] + [_vp] * 12
                                   + [_vp, ctypes.c_size_t, ctypes.POINTER(ss_scan_plan), _vp])
    lib.ss_scan_ckpt_bytes.restype = ctypes.c_size_t
    lib.ss_scan_ckpt_bytes.argtypes = [_i64, _i64, _int, _i64]
    lib.ss_scan_bwd_ex.restype = _int
    lib.ss_scan_bwd_ex.argtypes = [_i64, _i64, _int, _i64, _int, ctypes.c_uint32] + [_vp] * 22 + [ctypes.c_size_t, _vp]
    lib.ss_scan_bwd_segment_len.restype = _i64
    lib.ss_scan_bwd_segment_len.argtypes = [_i64, _i64, _int, _i64, _int]
    lib.ss_scan_bwd_seg_workspace_bytes.restype = ctypes.c_size_t
    lib.ss_scan_bwd_seg_workspace_bytes.argtypes = [_i64, _i64, _int, _i64, _int, _i64]
    lib.ss_scan_bwd_seg.restype = _int
    lib.ss_scan_bwd_seg.argtypes = ([_i64, _i64, _int, _i64, _int, ctypes.c_uint32, _i64] + [_vp] * 22
                                    + [ctypes.c_size_t, _vp])
    lib.ss_state_update_ex.restype = _int
    lib.ss_state_update_ex.argtypes = [_i64, _i64, _int, _int, ctypes.c_uint32] + [_vp] * 11
    lib.ss_scan_shard_state.restype = _int
    lib.ss_scan_shard_state.argtypes = [_i64, _i64, _int, _i64, _int] + [_vp] * 7 + [_vp, ctypes.c_size_t, _vp]
    lib.ss_scan_shard_state_zoh.restype = _int
    lib.ss_scan_shard_state_zoh.argtypes = lib.ss_scan_shard_state.argtypes
    lib.ss_scan_shard_combine.restype = _int
    lib.ss_scan_shard_combine.argtypes = [_i64, _i64, _int, _i64] + [_vp] * 6 + [_vp]
    lib.ss_scan_fwd_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.ss_scan_fwd_noalloc_max_bytes.argtypes = []
    lib.ss_scan_fwd_noalloc.restype = _int
    lib.ss_scan_fwd_noalloc.argtypes = ([_i64, _i64, _int, _i64, _int, ctypes.c_uint32] + [_vp] * 12
                                        + [ctypes.POINTER(ss_scan_plan), _vp])
    lib.ss_timing_enable.restype = _int
    lib.ss_timing_enable.argtypes = [_int]
    lib.ss_timing_reset.restype = _int
    lib.ss_timing_read.restype = _int
    lib.ss_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]
    if lib.ss_abi_version() != 1:
        raise ImportError("libssscan.so ABI version %d, expected 1" % lib.ss_abi_version())
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.ss_status_string(int(status)).decode()


def last_error() -> str:
    return lib.ss_last_error().decode()


def _check(status: int):
    if status != SS_OK:
        raise SsError(status, last_error())


def header_functions():
    """Names of the functions declared in include/ssscan.h."""
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ss_[a-z_]+)\s*\(", text)))


def _plan_ptr(plan):
    if plan is None:
        return None
    if isinstance(plan, ss_scan_plan):
        return ctypes.byref(plan)
    if len(plan) == 2:
        groups, chunk_len = plan
        lanes = 1
    else:
        groups, lanes, chunk_len = plan
    return ctypes.byref(ss_scan_plan(int(groups), int(lanes), int(chunk_len)))


# --- the C entry points, same names, raw pointers (ints) -----------------------

def ss_scan_fwd_plan(batch, dim, dstate, seqlen, io):
    """The automatic plan: (state_groups, lanes_per_channel, chunk_len)."""
    p = ss_scan_plan()
    _check(lib.ss_scan_fwd_plan(batch, dim, dstate, seqlen, io, ctypes.byref(p)))
    return int(p.state_groups), int(p.lanes_per_channel), int(p.chunk_len)


def ss_scan_fwd_workspace_bytes(batch, dim, dstate, seqlen, io, plan=None) -> int:
    return int(lib.ss_scan_fwd_workspace_bytes(batch, dim, dstate, seqlen, io, _plan_ptr(plan)))


def ss_scan_fwd(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                workspace, workspace_bytes, plan=None, stream=None):
    _check(lib.ss_scan_fwd(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                           workspace, workspace_bytes, _plan_ptr(plan), stream))


def ss_state_update(batch, dim, dstate, io, state, x, dt, z, B, C, A, Dskip, dt_bias, y, stream=None):
    _check(lib.ss_state_update(batch, dim, dstate, io, state, x, dt, z, B, C, A, Dskip, dt_bias, y, stream))


def ss_scan_fwd_zoh(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                    workspace, workspace_bytes, plan=None, stream=None):
    _check(lib.ss_scan_fwd_zoh(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                               workspace, workspace_bytes, _plan_ptr(plan), stream))


def ss_state_update_zoh(batch, dim, dstate, io, state, x, dt, z, B, C, A, Dskip, dt_bias, y, stream=None):
    _check(lib.ss_state_update_zoh(batch, dim, dstate, io, state, x, dt, z, B, C, A, Dskip, dt_bias, y, stream))


def ss_scan_bwd_workspace_bytes(batch, dim, dstate, seqlen, io) -> int:
    return int(lib.ss_scan_bwd_workspace_bytes(batch, dim, dstate, seqlen, io))


def ss_scan_bwd(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, dy, dh_final,
                dx, ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace, workspace_bytes, stream=None):
    _check(lib.ss_scan_bwd(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, dy, dh_final,
                           dx, ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace, workspace_bytes, stream))


SS_FLAG_ZOH = 1
SS_FLAG_DT_PER_ROW = 2


def ss_scan_fwd_ex(batch, dim, dstate, seqlen, io, flags, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                   ckpt, workspace, workspace_bytes, plan=None, stream=None):
    _check(lib.ss_scan_fwd_ex(batch, dim, dstate, seqlen, io, flags, x, dt, z, B, C, A, Dskip, dt_bias, h0, y,
                              h_final, ckpt, workspace, workspace_bytes, _plan_ptr(plan), stream))


def ss_scan_fwd_noalloc_max_bytes() -> int:
    return int(lib.ss_scan_fwd_noalloc_max_bytes())


def ss_scan_fwd_noalloc(batch, dim, dstate, seqlen, io, flags, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                        ckpt, plan=None, stream=None):
    _check(lib.ss_scan_fwd_noalloc(batch, dim, dstate, seqlen, io, flags, x, dt, z, B, C, A, Dskip, dt_bias, h0, y,
                                   h_final, ckpt, _plan_ptr(plan), stream))


def ss_scan_ckpt_bytes(batch, dim, dstate, seqlen) -> int:
    return int(lib.ss_scan_ckpt_bytes(batch, dim, dstate, seqlen))


def ss_scan_bwd_ex(batch, dim, dstate, seqlen, io, flags, x, dt, z, B, C, A, Dskip, dt_bias, h0, dy, dh_final, ckpt,
                   dx, ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace, workspace_bytes, stream=None):
    _check(lib.ss_scan_bwd_ex(batch, dim, dstate, seqlen, io, flags, x, dt, z, B, C, A, Dskip, dt_bias, h0, dy,
                              dh_final, ckpt, dx, ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace,
                              workspace_bytes, stream))


def ss_scan_bwd_segment_len(batch, dim, dstate, seqlen, io) -> int:
    return int(lib.ss_scan_bwd_segment_len(batch, dim, dstate, seqlen, io))


def ss_scan_bwd_seg_workspace_bytes(batch, dim, dstate, seqlen, io, segment_len) -> int:
    return int(lib.ss_scan_bwd_seg_workspace_bytes(batch, dim, dstate, seqlen, io, segment_len))


def ss_scan_bwd_seg(batch, dim, dstate, seqlen, io, flags, segment_len, x, dt, z, B, C, A, Dskip, dt_bias, h0, dy,
                    dh_final, ckpt, dx, ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace, workspace_bytes,
                    stream=None):
    _check(lib.ss_scan_bwd_seg(batch, dim, dstate, seqlen, io, flags, segment_len, x, dt, z, B, C, A, Dskip, dt_bias,
                               h0, dy, dh_final, ckpt, dx, ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace,
                               workspace_bytes, stream))


def ss_state_update_ex(batch, dim, dstate, io, flags, state, x, dt, z, B, C, A, Dskip, dt_bias, y, stream=None):
    _check(lib.ss_state_update_ex(batch, dim, dstate, io, flags, state, x, dt, z, B, C, A, Dskip, dt_bias, y,
                                  stream))


def ss_scan_shard_state(batch, dim, dstate, seqlen, io, x, dt, B, A, dt_bias, dsum, h_end, workspace,
                        workspace_bytes, stream=None):
    _check(lib.ss_scan_shard_state(batch, dim, dstate, seqlen, io, x, dt, B, A, dt_bias, dsum, h_end, workspace,
                                   workspace_bytes, stream))


def ss_scan_shard_state_zoh(batch, dim, dstate, seqlen, io, x, dt, B, A, dt_bias, dsum, h_end, workspace,
                            workspace_bytes, stream=None):
    _check(lib.ss_scan_shard_state_zoh(batch, dim, dstate, seqlen, io, x, dt, B, A, dt_bias, dsum, h_end, workspace,
                                       workspace_bytes, stream))


def ss_scan_shard_combine(batch, dim, dstate, nshards, A, dsum, h_end, h0, h_in, h_final, stream=None):
    _check(lib.ss_scan_shard_combine(batch, dim, dstate, nshards, A, dsum, h_end, h0, h_in, h_final, stream))


def ss_timing_enable(enable: bool):
    _check(lib.ss_timing_enable(1 if enable else 0))


def ss_timing_reset():
    _check(lib.ss_timing_reset())


def ss_timing_read():
    ms = ctypes.c_double()
    n = _i64()
    _check(lib.ss_timing_read(ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def ss_abi_version() -> int:
    return int(lib.ss_abi_version())
