"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects invalid arguments on the host before launching anything.

No test here launches a kernel: every call either fails validation (and the
library returns before any HIP call) or only queries sizes.
"""
import ctypes
import subprocess

import pytest

from selective_state_space_62_amd import binding as b

ALIGNED = 0x7F0000000000       # fake device addresses: only compared, never dereferenced
MB = 1 << 20


def test_abi_version():
    assert b.ss_abi_version() == 1


def test_every_declared_function_is_exported():
    names = b.header_functions()
    assert "ss_scan_fwd" in names and "ss_state_update" in names
    for n in names:
        assert hasattr(b.lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", str(b.LIB_PATH)], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing


def test_status_strings():
    assert b.status_string(b.SS_OK) == "SS_OK"
    assert b.status_string(b.SS_ERR_WORKSPACE) == "SS_ERR_WORKSPACE"
    assert b.status_string(99) == "SS_ERR_UNKNOWN"


def _scan_args(**kw):
    batch, dim, N, L = kw.pop("shape", (2, 64, 16, 256))
    io = kw.pop("io", b.SS_F32)
    eb = 2 if io == b.SS_BF16 else 4
    seq = batch * dim * L * eb
    base = ALIGNED
    ptrs = {}
    for name, size in (("x", seq), ("dt", seq), ("z", seq), ("B", batch * N * L * eb), ("C", batch * N * L * eb),
                       ("A", dim * N * 4), ("Dskip", dim * 4), ("dt_bias", dim * 4), ("h0", batch * dim * N * 4),
                       ("y", seq), ("h_final", batch * dim * N * 4)):
        ptrs[name] = base
        base += ((size + 4095) // 4096) * 4096 + 4096
    plan = kw.pop("plan", (1, L))
    ws_need = b.ss_scan_fwd_workspace_bytes(batch, dim, N, L, io, plan) if plan is not None else 1 << 30
    ptrs["workspace"] = base
    ptrs["workspace_bytes"] = ws_need
    ptrs.update(kw)
    return (batch, dim, N, L, io), ptrs, plan


def _scan_status(**kw):
    (batch, dim, N, L, io), p, plan = _scan_args(**kw)
    st = b.lib.ss_scan_fwd(batch, dim, N, L, io, p["x"], p["dt"], p["z"], p["B"], p["C"], p["A"], p["Dskip"],
                           p["dt_bias"], p["h0"], p["y"], p["h_final"], p["workspace"], p["workspace_bytes"],
                           b._plan_ptr(plan), None)
    return st, b.last_error()


@pytest.mark.parametrize("case,status", [
    (dict(shape=(2, 64, 3, 256)), b.SS_ERR_UNSUPPORTED),
    (dict(shape=(2, 64, 32, 256)), b.SS_ERR_UNSUPPORTED),
    (dict(io=7), b.SS_ERR_UNSUPPORTED),
    (dict(shape=(0, 64, 16, 256)), b.SS_ERR_INVALID_ARG),
    (dict(shape=(2, 0, 16, 256)), b.SS_ERR_INVALID_ARG),
    (dict(shape=(2, 64, 16, -1)), b.SS_ERR_INVALID_ARG),
    (dict(x=None), b.SS_ERR_INVALID_ARG),
    (dict(dt=None), b.SS_ERR_INVALID_ARG),
    (dict(B=None), b.SS_ERR_INVALID_ARG),
    (dict(C=None), b.SS_ERR_INVALID_ARG),
    (dict(A=None), b.SS_ERR_INVALID_ARG),
    (dict(y=None), b.SS_ERR_INVALID_ARG),
    (dict(x=ALIGNED + 4), b.SS_ERR_INVALID_ARG),
    (dict(h_final=ALIGNED + 8 + (1 << 36)), b.SS_ERR_INVALID_ARG),
    (dict(Dskip=ALIGNED + 2), b.SS_ERR_INVALID_ARG),
    (dict(workspace=None), b.SS_ERR_WORKSPACE),
    (dict(workspace_bytes=100, plan=(1, 64)), b.SS_ERR_WORKSPACE),   # chunked: chunk aggregates
    (dict(workspace=ALIGNED + (1 << 36) + 64), b.SS_ERR_WORKSPACE),
    (dict(y=ALIGNED + 4096), b.SS_ERR_INVALID_ARG),              # overlaps x
    (dict(plan=(3, 256)), b.SS_ERR_UNSUPPORTED),
    (dict(plan=(4, 24)), b.SS_ERR_INVALID_ARG),                  # not a multiple of the 16-token tile
    (dict(plan=(1, 0)), b.SS_ERR_INVALID_ARG),
    (dict(shape=(2, 64, 2, 256), plan=(4, 256)), b.SS_ERR_UNSUPPORTED),   # more groups than states
    (dict(shape=(2, 64, 4, 256), plan=(4, 2, 256)), b.SS_ERR_UNSUPPORTED),  # 8 state groups > 4 states
    (dict(plan=(4, 3, 256)), b.SS_ERR_UNSUPPORTED),                        # 3 lanes per channel
    (dict(plan=(2, 4, 256)), b.SS_ERR_UNSUPPORTED),                        # 4 lanes need 4 state groups
    (dict(shape=(2, 64, 8, 256), plan=(4, 4, 256)), b.SS_ERR_UNSUPPORTED),  # 16 state groups > 8 states
    (dict(shape=(1 << 41, 64, 16, 256)), b.SS_ERR_INVALID_ARG),
])
def test_scan_validation(case, status):
    st, msg = _scan_status(**case)
    assert st == status, (st, msg)
    assert msg


def test_output_overlapping_workspace_is_rejected():
    (batch, dim, N, L, io), p, plan = _scan_args(plan=(1, 64))   # chunked: the workspace holds chunk aggregates
    p["h_final"] = p["workspace"] + 256
    st = b.lib.ss_scan_fwd(batch, dim, N, L, io, p["x"], p["dt"], p["z"], p["B"], p["C"], p["A"], p["Dskip"],
                           p["dt_bias"], p["h0"], p["y"], p["h_final"], p["workspace"], p["workspace_bytes"],
                           b._plan_ptr(plan), None)
    assert st == b.SS_ERR_INVALID_ARG and "overlaps" in b.last_error()


def test_workspace_bytes():
    # one chunk: the scan reads B and C itself and needs no scratch (the minimum 256 bytes)
    assert b.ss_scan_fwd_workspace_bytes(8, 5120, 16, 2048, b.SS_BF16, (4, 2048)) == 256
    assert b.ss_scan_fwd_workspace_bytes(1, 16, 4, 64, b.SS_F32, (4, 64)) == 256
    # chunked: chunk end states, Delta sums and chunk initial states, each rounded to 256 bytes
    n = b.ss_scan_fwd_workspace_bytes(1, 2048, 16, 1 << 20, b.SS_BF16, (4, 1 << 15))
    st = 2048 * 32 * 16 * 4
    assert n == st + 2048 * 32 * 4 + st
    assert b.ss_scan_fwd_workspace_bytes(1, 16, 3, 64, b.SS_F32, None) == 0
    assert b.ss_scan_fwd_workspace_bytes(1, 16, 4, 64, b.SS_F32, (4, 8)) == 0


def test_plan_choice():
    g, k, cl = b.ss_scan_fwd_plan(8, 5120, 16, 2048, b.SS_BF16)
    assert (g, k) == (4, 2) and cl >= 2048                 # enough channels: one chunk
    g, k, cl = b.ss_scan_fwd_plan(1, 2048, 16, 1 << 20, b.SS_BF16)
    assert g == 4 and cl < (1 << 20) and cl % 32 == 0      # few channels, long sequence: chunked
    g, k, cl = b.ss_scan_fwd_plan(1, 16, 2, 64, b.SS_F32)
    assert (g, k) == (2, 1)
    g, k, cl = b.ss_scan_fwd_plan(8, 1536, 16, 2048, b.SS_F32)
    assert (g, k) == (4, 4) and cl >= 2048                 # < 2 workgroups per CU with 2 lanes: 4 lanes


@pytest.mark.parametrize("case,status", [
    (dict(state=None), b.SS_ERR_INVALID_ARG),
    (dict(x=None), b.SS_ERR_INVALID_ARG),
    (dict(y=None), b.SS_ERR_INVALID_ARG),
    (dict(dstate=5), b.SS_ERR_UNSUPPORTED),
    (dict(io=3), b.SS_ERR_UNSUPPORTED),
    (dict(batch=0), b.SS_ERR_INVALID_ARG),
    (dict(state=ALIGNED + 8), b.SS_ERR_INVALID_ARG),
    (dict(y=ALIGNED + (1 << 30)), b.SS_ERR_INVALID_ARG),           # y overlaps x
    (dict(state=ALIGNED + (1 << 30) + (1 << 28)), b.SS_ERR_INVALID_ARG),   # state overlaps dt
])
def test_state_update_validation(case, status):
    a = dict(batch=4, dim=64, dstate=16, io=b.SS_BF16, state=ALIGNED, x=ALIGNED + (1 << 30),
             dt=ALIGNED + (1 << 30) + (1 << 28), z=None, B=ALIGNED + (1 << 31), C=ALIGNED + (1 << 31) + 4096,
             A=ALIGNED + (1 << 32), Dskip=None, dt_bias=None, y=ALIGNED + (1 << 33))
    a.update(case)
    st = b.lib.ss_state_update(a["batch"], a["dim"], a["dstate"], a["io"], a["state"], a["x"], a["dt"], a["z"],
                               a["B"], a["C"], a["A"], a["Dskip"], a["dt_bias"], a["y"], None)
    assert st == status, (st, b.last_error())


_BWD_NAMES = ("x", "dt", "z", "B", "C", "A", "Dskip", "dt_bias", "h0", "dy", "dh_final", "dx", "ddt", "dz", "dB",
              "dC", "dA", "dDskip", "ddt_bias", "dh0")


def _bwd_status(**kw):
    batch, dim, N, L = kw.pop("shape", (2, 64, 16, 256))
    io = kw.pop("io", b.SS_F32)
    eb = 2 if io == b.SS_BF16 else 4
    seq, bcs, st, par = batch * dim * L * eb, batch * N * L * eb, batch * dim * N * 4, dim * 4
    sizes = dict(x=seq, dt=seq, z=seq, B=bcs, C=bcs, A=dim * N * 4, Dskip=par, dt_bias=par, h0=st, dy=seq,
                 dh_final=st, dx=seq, ddt=seq, dz=seq, dB=bcs, dC=bcs, dA=dim * N * 4, dDskip=par, ddt_bias=par, dh0=st)
    ptrs, base = {}, ALIGNED
    for name in _BWD_NAMES:
        ptrs[name] = base
        base += ((sizes[name] + 4095) // 4096) * 4096 + 4096
    ptrs["workspace"] = base
    ptrs["workspace_bytes"] = b.ss_scan_bwd_workspace_bytes(batch, dim, N, L, io) if N in (1, 2, 4, 8, 16) else 0
    ptrs.update(kw)
    stt = b.lib.ss_scan_bwd(batch, dim, N, L, io, *[ptrs[n] for n in _BWD_NAMES], ptrs["workspace"],
                            ptrs["workspace_bytes"], None)
    return stt, b.last_error()


@pytest.mark.parametrize("case,status", [
    (dict(shape=(2, 64, 5, 256)), b.SS_ERR_UNSUPPORTED),
    (dict(io=9), b.SS_ERR_UNSUPPORTED),
    (dict(shape=(0, 64, 16, 256)), b.SS_ERR_INVALID_ARG),
    (dict(x=None), b.SS_ERR_INVALID_ARG),
    (dict(dy=None), b.SS_ERR_INVALID_ARG),
    (dict(dx=None), b.SS_ERR_INVALID_ARG),
    (dict(ddt=None), b.SS_ERR_INVALID_ARG),
    (dict(dB=None), b.SS_ERR_INVALID_ARG),
    (dict(dC=None), b.SS_ERR_INVALID_ARG),
    (dict(A=None), b.SS_ERR_INVALID_ARG),
    (dict(dz=None), b.SS_ERR_INVALID_ARG),                 # z given, dz missing
    (dict(z=None), b.SS_ERR_INVALID_ARG),                  # dz given, z missing
    (dict(dB=ALIGNED + (1 << 36) + 4), b.SS_ERR_INVALID_ARG),
    (dict(dDskip=ALIGNED + (1 << 36) + 2), b.SS_ERR_INVALID_ARG),
    (dict(dx=ALIGNED), b.SS_ERR_INVALID_ARG),              # dx overlaps x
    (dict(dh0=ALIGNED + (1 << 37) + 256, workspace=ALIGNED + (1 << 37)), b.SS_ERR_INVALID_ARG),  # dh0 in the workspace
    (dict(workspace=None), b.SS_ERR_WORKSPACE),
    (dict(workspace_bytes=4096), b.SS_ERR_WORKSPACE),
    (dict(workspace=ALIGNED + (1 << 37) + 64), b.SS_ERR_WORKSPACE),
])
def test_bwd_validation(case, status):
    st, msg = _bwd_status(**case)
    assert st == status, (st, msg)
    assert msg


def test_bwd_workspace_bytes():
    # (batch, L, N, 2) B/C re-layout + (batch, D, L/16, N) checkpoints + (batch, D/32, 2N + 1, L) partials
    # (dB, dC and a per-row ddt) + (batch, D, N) + 2 (batch, D) per-row sums, each rounded to 256 bytes
    n = b.ss_scan_bwd_workspace_bytes(8, 5120, 16, 2048, b.SS_BF16)
    expect = 8 * 2048 * 32 * 4 + 8 * 5120 * 128 * 16 * 4 + 8 * 160 * 33 * 2048 * 4 + 8 * 5120 * 16 * 4 + 2 * 8 * 5120 * 4
    assert n == expect
    # a ragged length pads the partials' tokens to whole 16-token chunks
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    n = b.ss_scan_bwd_workspace_bytes(1, 64, 16, 17, b.SS_F32)
    assert n == r(17 * 32 * 4) + r(64 * 2 * 16 * 4) + r(2 * 33 * 32 * 4) + r(64 * 16 * 4) + 2 * r(64 * 4)
    assert b.ss_scan_bwd_workspace_bytes(2, 64, 16, 0, b.SS_F32) == 0
    assert b.ss_scan_bwd_workspace_bytes(2, 64, 3, 16, b.SS_F32) == 0


@pytest.mark.parametrize("case,status", [
    (dict(dstate=3), b.SS_ERR_UNSUPPORTED),
    (dict(x=None), b.SS_ERR_INVALID_ARG),
    (dict(h_end=None), b.SS_ERR_INVALID_ARG),
    (dict(dsum=None), b.SS_ERR_INVALID_ARG),
    (dict(h_end=ALIGNED + (1 << 33) + 8), b.SS_ERR_INVALID_ARG),
    (dict(dsum=ALIGNED + (1 << 30)), b.SS_ERR_INVALID_ARG),        # dsum overlaps dt
    (dict(workspace=None), b.SS_ERR_WORKSPACE),
    (dict(seqlen=16384, workspace_bytes=64), b.SS_ERR_WORKSPACE),   # chunked inside the shard
])
def test_shard_state_validation(case, status):
    a = dict(batch=2, dim=64, dstate=16, seqlen=512, io=b.SS_BF16, x=ALIGNED, dt=ALIGNED + (1 << 30),
             B=ALIGNED + (1 << 31), A=ALIGNED + (1 << 32), dt_bias=None, dsum=ALIGNED + (1 << 33) + (1 << 20),
             h_end=ALIGNED + (1 << 33), workspace=ALIGNED + (1 << 34), workspace_bytes=1 << 30)
    a.update(case)
    st = b.lib.ss_scan_shard_state(a["batch"], a["dim"], a["dstate"], a["seqlen"], a["io"], a["x"], a["dt"], a["B"],
                                   a["A"], a["dt_bias"], a["dsum"], a["h_end"], a["workspace"], a["workspace_bytes"],
                                   None)
    assert st == status, (st, b.last_error())


@pytest.mark.parametrize("case,status", [
    (dict(nshards=0), b.SS_ERR_INVALID_ARG),
    (dict(dstate=6), b.SS_ERR_UNSUPPORTED),
    (dict(A=None), b.SS_ERR_INVALID_ARG),
    (dict(h_end=None), b.SS_ERR_INVALID_ARG),
    (dict(h_in=ALIGNED + 2), b.SS_ERR_INVALID_ARG),
    (dict(h_in=ALIGNED + (1 << 31)), b.SS_ERR_INVALID_ARG),        # h_in overlaps h_end
    (dict(h_final=ALIGNED), b.SS_ERR_INVALID_ARG),                 # h_final overlaps A
])
def test_shard_combine_validation(case, status):
    a = dict(batch=2, dim=64, dstate=16, nshards=8, A=ALIGNED, dsum=ALIGNED + (1 << 30), h_end=ALIGNED + (1 << 31),
             h0=None, h_in=ALIGNED + (1 << 32), h_final=ALIGNED + (1 << 33))
    a.update(case)
    st = b.lib.ss_scan_shard_combine(a["batch"], a["dim"], a["dstate"], a["nshards"], a["A"], a["dsum"], a["h_end"],
                                     a["h0"], a["h_in"], a["h_final"], None)
    assert st == status, (st, b.last_error())


def test_flags_validation():
    (batch, dim, N, L, io), p, plan = _scan_args()
    args = [p[k] for k in ("x", "dt", "z", "B", "C", "A", "Dskip", "dt_bias", "h0", "y", "h_final")]
    st = b.lib.ss_scan_fwd_ex(batch, dim, N, L, io, 4, *args, None, p["workspace"], p["workspace_bytes"],
                              b._plan_ptr(plan), None)
    assert st == b.SS_ERR_UNSUPPORTED and "flags" in b.last_error()
    ck = ALIGNED + (1 << 38)
    # checkpoints are stored under ZOH too (the backward has that form): a ZOH call
    # with a checkpoint buffer gets as far as the overlap checks
    st = b.lib.ss_scan_fwd_ex(batch, dim, N, L, io, b.SS_FLAG_ZOH, *args, p["x"], p["workspace"],
                              p["workspace_bytes"], b._plan_ptr(plan), None)
    assert st == b.SS_ERR_INVALID_ARG and "overlaps" in b.last_error()
    st = b.lib.ss_scan_fwd_ex(batch, dim, N, L, io, 0, *args, ck + 4, p["workspace"], p["workspace_bytes"],
                              b._plan_ptr(plan), None)
    assert st == b.SS_ERR_INVALID_ARG and "ckpt" in b.last_error()
    st = b.lib.ss_scan_fwd_ex(batch, dim, N, L, io, 0, *args, p["x"], p["workspace"], p["workspace_bytes"],
                              b._plan_ptr(plan), None)
    assert st == b.SS_ERR_INVALID_ARG and "overlaps" in b.last_error()
    st = b.lib.ss_state_update_ex(4, 64, 16, b.SS_BF16, 8, ALIGNED, ALIGNED + (1 << 30), ALIGNED + (1 << 31), None,
                                  ALIGNED + (1 << 32), ALIGNED + (1 << 33), ALIGNED + (1 << 34), None, None,
                                  ALIGNED + (1 << 35), None)
    assert st == b.SS_ERR_UNSUPPORTED
    # an output inside the per-row dt (batch * L elements) is rejected
    st = b.lib.ss_scan_fwd_ex(batch, dim, N, L, io, b.SS_FLAG_DT_PER_ROW,
                              *[p[k] for k in ("x", "dt", "z", "B", "C", "A", "Dskip", "dt_bias", "h0")],
                              p["dt"] + 64, p["h_final"], None, p["workspace"], p["workspace_bytes"], b._plan_ptr(plan),
                              None)
    assert st == b.SS_ERR_INVALID_ARG and "overlaps input dt" in b.last_error()


def test_ckpt_bytes_and_bwd_ex_flags():
    # the state entering every 16-token chunk at N = 16, fp32
    assert b.ss_scan_ckpt_bytes(8, 5120, 16, 2048) == 8 * 5120 * 128 * 16 * 4
    assert b.ss_scan_ckpt_bytes(2, 64, 16, 17) == 2 * 64 * 2 * 16 * 4
    assert b.ss_scan_ckpt_bytes(2, 64, 3, 17) == 0
    names = list(_BWD_NAMES)
    (batch, dim, N, L) = (2, 64, 16, 256)
    a = {n: ALIGNED + i * (1 << 30) for i, n in enumerate(names)}
    def call(flags, **over):
        v = dict(a, **over)
        return b.lib.ss_scan_bwd_ex(batch, dim, N, L, b.SS_F32, flags, *[v[n] for n in names[:11]], None,
                                    *[v[n] for n in names[11:]], ALIGNED + (1 << 36), 1 << 30, None)
    # ZOH is accepted: such a call reaches the argument checks
    assert call(b.SS_FLAG_ZOH, dx=a["x"]) == b.SS_ERR_INVALID_ARG and "dx overlaps input x" in b.last_error()
    assert call(b.SS_FLAG_ZOH | b.SS_FLAG_DT_PER_ROW, dx=a["x"]) == b.SS_ERR_INVALID_ARG
    assert call(4) == b.SS_ERR_UNSUPPORTED and "flags" in b.last_error()
    # with one dt per (row, token), dt and ddt are batch * seqlen long: a ddt that
    # starts inside that span overlaps dt
    row_bytes = batch * L * 4
    assert call(b.SS_FLAG_DT_PER_ROW, ddt=a["dt"] + row_bytes - 16) == b.SS_ERR_INVALID_ARG
    assert "ddt overlaps input dt" in b.last_error()


def test_bwd_segment_plan_and_workspace():
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    # explicit lengths are multiples of 64; a length of at least seqlen runs the sequence whole
    assert b.ss_scan_bwd_seg_workspace_bytes(1, 64, 16, 17, b.SS_F32, 64) == b.ss_scan_bwd_workspace_bytes(
        1, 64, 16, 17, b.SS_F32)
    assert b.ss_scan_bwd_seg_workspace_bytes(1, 64, 16, 300, b.SS_F32, 100) == 0
    assert b.ss_scan_bwd_seg_workspace_bytes(1, 64, 16, 300, b.SS_F32, -64) == 0
    # five segments of 64 tokens: the per-(segment, row) sums grow fivefold, and the
    # segments' entering states, their end states from zero, the carried adjoints,
    # the adjoint aggregates and the Delta sums (shared by both) are added
    n5 = b.ss_scan_bwd_seg_workspace_bytes(1, 64, 16, 300, b.SS_F32, 64)
    n1 = b.ss_scan_bwd_seg_workspace_bytes(1, 64, 16, 300, b.SS_F32, 1 << 20)
    st, sc = 64 * 5 * 16 * 4, 64 * 5 * 4
    assert n5 - n1 == (r(5 * 64 * 16 * 4) - r(64 * 16 * 4)) + 2 * (r(5 * 64 * 4) - r(64 * 4)) + 4 * r(st) + r(sc)
    # the automatic choice: the 2.8B shape runs whole; one channel block over 8192 tokens is split
    assert b.ss_scan_bwd_segment_len(8, 5120, 16, 2048, b.SS_BF16) == 2048
    assert b.ss_scan_bwd_segment_len(1, 32, 16, 8192, b.SS_F32) == 2048
    assert b.ss_scan_bwd_segment_len(1, 32, 3, 8192, b.SS_F32) == 0
    # an invalid length is rejected before the pointers are looked at
    st_ = b.lib.ss_scan_bwd_seg(1, 64, 16, 300, b.SS_F32, 0, 100, *([None] * 22), 0, None)
    assert st_ == b.SS_ERR_INVALID_ARG and "segment_len" in b.last_error()
    assert b.lib.ss_scan_bwd_seg(1, 64, 16, 300, b.SS_F32, 8, 64, *([None] * 22), 0, None) == \
        b.SS_ERR_UNSUPPORTED


def test_timing_record_empty():
    b.ss_timing_enable(False)
    b.ss_timing_reset()
    assert b.ss_timing_read() == (0.0, 0)


def test_python_errors_carry_message():
    with pytest.raises(b.SsError) as e:
        b.ss_scan_fwd(1, 16, 3, 64, b.SS_F32, *([None] * 11), None, 0)
    assert e.value.status == b.SS_ERR_UNSUPPORTED and "dstate" in str(e.value)


def test_noalloc_scan_refuses_shapes_beyond_its_static_scratch():
    """ss_scan_fwd_noalloc checks the scratch it needs against its static array
    before any device work: a shape that needs more is refused with
    SS_ERR_WORKSPACE and a message naming both sizes."""
    assert b.ss_scan_fwd_noalloc_max_bytes() == 32 * MB
    batch, dim, N, L = 1, 2048, 16, 1 << 20   # the million-token plan: 256 chunks, 69 MB of aggregates
    need = b.ss_scan_fwd_workspace_bytes(batch, dim, N, L, b.SS_BF16)
    assert need > 32 * MB
    p = ctypes.c_void_p(ALIGNED)
    st = b.lib.ss_scan_fwd_noalloc(batch, dim, N, L, b.SS_BF16, 0, p, p, None, p, p, p, None, None, None,
                                   ctypes.c_void_p(ALIGNED + 1024 * MB), None, None, None, None)
    assert st == b.SS_ERR_WORKSPACE
    msg = b.last_error()
    assert str(need) in msg and str(32 * MB) in msg
