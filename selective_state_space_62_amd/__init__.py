"""MI355X-native selective state-space (S6) scan.

``binding`` exposes the C entry points of libssscan.so under their C names;
``torch_ops`` wraps them for PyTorch tensors (memory and streams only).
"""
from . import binding  # noqa: F401  (raises ImportError if libssscan.so is missing)
from .binding import (SS_BF16, SS_F32, SS_FLAG_DT_PER_ROW, SS_FLAG_ZOH, SsError, ss_abi_version,  # noqa: F401
                      ss_scan_bwd, ss_scan_bwd_ex, ss_scan_bwd_seg, ss_scan_bwd_seg_workspace_bytes,
                      ss_scan_bwd_segment_len, ss_scan_bwd_workspace_bytes, ss_scan_ckpt_bytes, ss_scan_fwd,
                      ss_scan_fwd_ex, ss_scan_fwd_plan, ss_scan_fwd_workspace_bytes, ss_scan_fwd_zoh,
                      ss_scan_shard_combine, ss_scan_shard_state, ss_scan_shard_state_zoh, ss_state_update,
                      ss_state_update_ex, ss_state_update_zoh, ss_timing_enable, ss_timing_read, ss_timing_reset)
from .torch_ops import (bwd_workspace_bytes, ckpt_numel, scan_bwd, scan_fwd, shard_combine, shard_state,  # noqa: F401
                        state_update, workspace_bytes)

__all__ = ["ss_scan_fwd", "ss_state_update", "ss_scan_fwd_zoh", "ss_state_update_zoh", "ss_scan_bwd",
           "ss_scan_fwd_plan", "ss_scan_fwd_workspace_bytes", "ss_scan_bwd_workspace_bytes", "ss_timing_enable",
           "ss_timing_read", "ss_timing_reset", "ss_abi_version", "scan_fwd", "scan_bwd", "state_update",
           "workspace_bytes", "bwd_workspace_bytes", "ss_scan_shard_state", "ss_scan_shard_state_zoh",
           "ss_scan_shard_combine", "shard_state", "shard_combine", "ss_scan_fwd_ex", "ss_state_update_ex",
           "SS_FLAG_ZOH", "SS_FLAG_DT_PER_ROW", "ss_scan_bwd_ex", "ss_scan_ckpt_bytes", "ckpt_numel", "SsError",
           "SS_F32", "SS_BF16", "ss_scan_bwd_seg", "ss_scan_bwd_seg_workspace_bytes", "ss_scan_bwd_segment_len"]
