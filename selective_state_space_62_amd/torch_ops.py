"""Tensor-level calls over the C ABI: marshalling only.

``scan_fwd`` and ``state_update`` check dtypes, shapes, devices and contiguity,
allocate outputs and the workspace with torch on the inputs' device, and call
the library on torch's current stream.  No arithmetic of the scan happens here.
"""
from __future__ import annotations

import torch

from . import binding as _b

_IO = {torch.float32: _b.SS_F32, torch.bfloat16: _b.SS_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, shape, device):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(batch, dim, dstate, seqlen, dtype=torch.bfloat16, plan=None) -> int:
    return _b.ss_scan_fwd_workspace_bytes(batch, dim, dstate, seqlen, _IO[dtype], plan)


def ckpt_numel(batch, dim, dstate, seqlen) -> int:
    """float32 elements of the checkpoint buffer scan_fwd(ckpt=...) fills for scan_bwd."""
    return _b.ss_scan_ckpt_bytes(batch, dim, dstate, seqlen) // 4


def scan_fwd(x, dt, B, C, A, z=None, Dskip=None, dt_bias=None, h0=None, *, plan=None, workspace=None,
             y=None, h_final=None, return_final_state=True, zoh=False, ckpt=None):
    """Selective scan over full sequences (zoh=True: zero-order-hold input term).

    ckpt: optional float32 tensor of ckpt_numel(...) elements that receives the
    states the backward pass needs (pass it on to scan_bwd).

    x, z: (batch, D, L); dt: (batch, D, L), or (batch, L) for one value per row and
    token shared by the row's channels; B, C: (batch, N, L) — all float32 or all bfloat16;
    A: (D, N) float32; Dskip, dt_bias: (D,) float32; h0: (batch, D, N) float32.
    Returns (y, h_final); h_final is None when return_final_state is False.
    """
    if x.dtype not in _IO:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    batch, dim, L = x.shape
    N = A.shape[1]
    io = _IO[x.dtype]
    dt_row = dt.dim() == 2
    _need(x, "x", x.dtype, (batch, dim, L), dev)
    _need(dt, "dt", x.dtype, (batch, L) if dt_row else (batch, dim, L), dev)
    _need(z, "z", x.dtype, (batch, dim, L), dev)
    _need(B, "B", x.dtype, (batch, N, L), dev)
    _need(C, "C", x.dtype, (batch, N, L), dev)
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(Dskip, "Dskip", torch.float32, (dim,), dev)
    _need(dt_bias, "dt_bias", torch.float32, (dim,), dev)
    _need(h0, "h0", torch.float32, (batch, dim, N), dev)
    if y is None:
        y = torch.empty((batch, dim, L), dtype=x.dtype, device=dev)
    _need(y, "y", x.dtype, (batch, dim, L), dev)
    if return_final_state and h_final is None:
        h_final = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _need(h_final, "h_final", torch.float32, (batch, dim, N), dev)
    nbytes = _b.ss_scan_fwd_workspace_bytes(batch, dim, N, L, io, plan)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    if workspace.numel() < nbytes:
        raise ValueError("workspace has %d bytes, %d needed" % (workspace.numel(), nbytes))
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.float32, (ckpt_numel(batch, dim, N, L),), dev)
    head = (_ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip), _ptr(dt_bias), _ptr(h0), _ptr(y),
            _ptr(h_final))
    tail = (_ptr(workspace), workspace.numel(), plan, _stream(dev))
    if dt_row or ckpt is not None:
        flags = (_b.SS_FLAG_DT_PER_ROW if dt_row else 0) | (_b.SS_FLAG_ZOH if zoh else 0)
        _b.ss_scan_fwd_ex(batch, dim, N, L, io, flags, *head, _ptr(ckpt), *tail)
    else:
        (_b.ss_scan_fwd_zoh if zoh else _b.ss_scan_fwd)(batch, dim, N, L, io, *head, *tail)
    return y, h_final


def state_update(state, x, dt, B, C, A, z=None, Dskip=None, dt_bias=None, *, y=None, zoh=False):
    """One decode step; ``state`` (batch, D, N) float32 is updated in place (zoh=True:
    zero-order-hold input term).

    x, z: (batch, D); dt: (batch, D), or (batch,) shared by a row's channels;
    B, C: (batch, N) in float32 or bfloat16.  Returns y (batch, D).
    """
    if x.dtype not in _IO:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    batch, dim = x.shape
    N = A.shape[1]
    _need(state, "state", torch.float32, (batch, dim, N), dev)
    dt_row = dt.dim() == 1
    _need(dt, "dt", x.dtype, (batch,) if dt_row else (batch, dim), dev)
    _need(z, "z", x.dtype, (batch, dim), dev)
    _need(B, "B", x.dtype, (batch, N), dev)
    _need(C, "C", x.dtype, (batch, N), dev)
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(Dskip, "Dskip", torch.float32, (dim,), dev)
    _need(dt_bias, "dt_bias", torch.float32, (dim,), dev)
    if y is None:
        y = torch.empty((batch, dim), dtype=x.dtype, device=dev)
    _need(y, "y", x.dtype, (batch, dim), dev)
    args = (_ptr(state), _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip), _ptr(dt_bias), _ptr(y),
            _stream(dev))
    if dt_row:
        flags = _b.SS_FLAG_DT_PER_ROW | (_b.SS_FLAG_ZOH if zoh else 0)
        _b.ss_state_update_ex(batch, dim, N, _IO[x.dtype], flags, *args)
    else:
        (_b.ss_state_update_zoh if zoh else _b.ss_state_update)(batch, dim, N, _IO[x.dtype], *args)
    return y


def bwd_workspace_bytes(batch, dim, dstate, seqlen, dtype=torch.bfloat16, segment_len=None) -> int:
    return _b.ss_scan_bwd_seg_workspace_bytes(batch, dim, dstate, seqlen, _IO[dtype], int(segment_len or 0))


def scan_bwd(x, dt, B, C, A, dy, z=None, Dskip=None, dt_bias=None, h0=None, dh_final=None, *, workspace=None,
             need_dA=True, need_dDskip=True, need_ddt_bias=True, need_dh0=True, ckpt=None, zoh=False,
             segment_len=None):
    """Gradients of ``scan_fwd`` (zoh=True: of ``scan_fwd(..., zoh=True)``) for upstream
    gradients dy (batch, D, L) and dh_final (batch, D, N) float32 (None = 0).  dt may be
    (batch, L): one value per token shared by the channels (SS_FLAG_DT_PER_ROW);
    its gradient is then (batch, L), the sum over channels.  segment_len (None or 0:
    the library's choice; else a multiple of 64) cuts the sequence into segments
    run in parallel (ss_scan_bwd_seg).

    Returns a dict: dx, ddt, dz (None without z) in the I/O dtype, shaped like x
    (ddt like dt); dB, dC shaped like B; dA (D, N), dDskip (D,), ddt_bias (D,),
    dh0 (batch, D, N) in float32 (None where not requested).
    """
    if x.dtype not in _IO:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    batch, dim, L = x.shape
    N = A.shape[1]
    io = _IO[x.dtype]
    dt_row = dt is not None and dt.dim() == 2
    for t, name, shape in ((x, "x", (batch, dim, L)), (dt, "dt", (batch, L) if dt_row else (batch, dim, L)),
                           (z, "z", (batch, dim, L)), (dy, "dy", (batch, dim, L)), (B, "B", (batch, N, L)),
                           (C, "C", (batch, N, L))):
        _need(t, name, x.dtype, shape, dev)
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(Dskip, "Dskip", torch.float32, (dim,), dev)
    _need(dt_bias, "dt_bias", torch.float32, (dim,), dev)
    _need(h0, "h0", torch.float32, (batch, dim, N), dev)
    _need(dh_final, "dh_final", torch.float32, (batch, dim, N), dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt), dz=torch.empty_like(x) if z is not None else None,
               dB=torch.empty_like(B), dC=torch.empty_like(C),
               dA=torch.empty((dim, N), dtype=torch.float32, device=dev) if need_dA else None,
               dDskip=torch.empty(dim, dtype=torch.float32, device=dev) if need_dDskip else None,
               ddt_bias=torch.empty(dim, dtype=torch.float32, device=dev) if need_ddt_bias else None,
               dh0=torch.empty((batch, dim, N), dtype=torch.float32, device=dev) if need_dh0 else None)
    seg = int(segment_len or 0)
    nbytes = _b.ss_scan_bwd_seg_workspace_bytes(batch, dim, N, L, io, seg)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    if workspace.numel() < nbytes:
        raise ValueError("workspace has %d bytes, %d needed" % (workspace.numel(), nbytes))
    ins = (_ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(Dskip), _ptr(dt_bias), _ptr(h0), _ptr(dy),
           _ptr(dh_final))
    outs = (_ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dz"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dA"]),
            _ptr(out["dDskip"]), _ptr(out["ddt_bias"]), _ptr(out["dh0"]), _ptr(workspace), workspace.numel(),
            _stream(dev))
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.float32, (ckpt_numel(batch, dim, N, L),), dev)
    flags = (_b.SS_FLAG_DT_PER_ROW if dt_row else 0) | (_b.SS_FLAG_ZOH if zoh else 0)
    if seg:
        _b.ss_scan_bwd_seg(batch, dim, N, L, io, flags, seg, *ins, _ptr(ckpt), *outs)
    elif ckpt is not None or flags:
        _b.ss_scan_bwd_ex(batch, dim, N, L, io, flags, *ins, _ptr(ckpt), *outs)
    else:
        _b.ss_scan_bwd(batch, dim, N, L, io, *ins, *outs)
    return out


def shard_state(x, dt, B, A, dt_bias=None, *, zoh=False, workspace=None):
    """One shard of a sequence from a zero state: returns (dsum (batch, D), h_end
    (batch, D, N)) in float32, the shard's sum of Delta and final state."""
    if x.dtype not in _IO:
        raise TypeError("x must be float32 or bfloat16")
    dev = x.device
    batch, dim, L = x.shape
    N = A.shape[1]
    io = _IO[x.dtype]
    _need(dt, "dt", x.dtype, (batch, dim, L), dev)
    _need(B, "B", x.dtype, (batch, N, L), dev)
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(dt_bias, "dt_bias", torch.float32, (dim,), dev)
    dsum = torch.empty((batch, dim), dtype=torch.float32, device=dev)
    h_end = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    nbytes = _b.ss_scan_fwd_workspace_bytes(batch, dim, N, L, io, None)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    if workspace.numel() < nbytes:
        raise ValueError("workspace has %d bytes, %d needed" % (workspace.numel(), nbytes))
    fn = _b.ss_scan_shard_state_zoh if zoh else _b.ss_scan_shard_state
    fn(batch, dim, N, L, io, _ptr(x), _ptr(dt), _ptr(B), _ptr(A), _ptr(dt_bias), _ptr(dsum), _ptr(h_end),
       _ptr(workspace), workspace.numel(), _stream(dev))
    return dsum, h_end


def shard_combine(A, dsum, h_end, h0=None):
    """Exclusive scan over shards: dsum (S, batch, D), h_end (S, batch, D, N) ->
    (h_in (S, batch, D, N), h_final (batch, D, N)), float32."""
    dev = A.device
    S, batch, dim, N = h_end.shape
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(dsum, "dsum", torch.float32, (S, batch, dim), dev)
    _need(h_end, "h_end", torch.float32, (S, batch, dim, N), dev)
    _need(h0, "h0", torch.float32, (batch, dim, N), dev)
    h_in = torch.empty_like(h_end)
    h_final = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _b.ss_scan_shard_combine(batch, dim, N, S, _ptr(A), _ptr(dsum), _ptr(h_end), _ptr(h0), _ptr(h_in),
                             _ptr(h_final), _stream(dev))
    return h_in, h_final
