"""One GPU's share of a chunk-overlapped collective GEMM on MI355X (gfx950).

The work is done by libsync_overlap.so (C ABI in include/sync_overlap.h);
``_abi`` is its ctypes binding with the same function names.  ``inputs``
draws the seeded synthetic operands.  Importing the package loads nothing;
the library is loaded on the first call and a missing build raises.
"""
from . import _abi  # noqa: F401
from ._abi import (  # noqa: F401
    SyncError, make_tune_space, sync_ag_gemm, sync_autotune, sync_gemm_rs, sync_get_device_info, sync_last_error, sync_plan, sync_plan_export,
    sync_head_attn, sync_plan_get_info, sync_read_timings, sync_ring_attn_step, sync_shutdown, sync_trace_export,
    sync_tune_workspace_size, sync_workspace_init, sync_workspace_size, sync_workspace_status)
