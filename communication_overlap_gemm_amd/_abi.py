"""ctypes binding of include/sync_overlap.h (argument marshalling only).

Every function here has the name of the C entry point it wraps and does no
computation of its own: pointer arguments accept an int address or any object
with ``data_ptr()`` (a torch tensor); stream arguments accept an int handle,
None (the null stream) or an object with ``cuda_stream`` (a torch stream).
A non-zero status raises :class:`SyncError` carrying the library's message.
The library is loaded on first use; if it is not built the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsync_overlap.so")

# ---- constants (mirror sync_overlap.h) ------------------------------------
SYNC_OK, SYNC_EINVAL, SYNC_EUNSUPPORTED, SYNC_EHIP, SYNC_ETIMEOUT, SYNC_ENOMEM, SYNC_ENODEV = 0, -1, -2, -3, -4, -5, -6
SYNC_OP_AG_GEMM, SYNC_OP_GEMM_RS, SYNC_OP_RING_ATTN, SYNC_OP_HEAD_ATTN = 1, 2, 3, 4
SYNC_PAT_RING, SYNC_PAT_EXPLICIT, SYNC_PAT_HIER_SWIZZLE, SYNC_PAT_MESH = 0, 1, 2, 3
SYNC_ORDER_ROW_MAJOR, SYNC_ORDER_CHUNK_MAJOR, SYNC_ORDER_SWIZZLED = 0, 1, 2
SYNC_B_KN, SYNC_B_NK = 0, 1
SYNC_DTYPE_F32, SYNC_DTYPE_BF16 = 0, 1
SYNC_COPY_PRESET, SYNC_COPY_SDMA, SYNC_COPY_CU, SYNC_COPY_HOST_GATED, SYNC_COPY_COLOCATED = 0, 1, 2, 3, 4
SYNC_COPY_EPILOGUE = 5
SYNC_RUN_COPY_ONLY, SYNC_RUN_COMPUTE_ONLY, SYNC_RUN_TIMED, SYNC_RUN_WITHHOLD, SYNC_RUN_TRACE = 1, 2, 4, 8, 16
SYNC_ATTN_INIT, SYNC_ATTN_FINALIZE = 1, 2

EXPORTED_SYMBOLS = (
    "sync_plan", "sync_plan_destroy", "sync_plan_get_info", "sync_plan_export", "sync_workspace_size",
    "sync_workspace_init", "sync_workspace_status", "sync_ag_gemm", "sync_ag_gemm_noalloc", "sync_gemm_rs", "sync_gemm_rs_reduce", "sync_gemm_ar",
    "sync_ring_attn_step", "sync_head_attn", "sync_attn_query_block", "sync_gemm_split",
    "sync_get_device_info", "sync_last_error", "sync_shutdown", "sync_read_timings", "sync_trace_export",
    "sync_autotune", "sync_tune_workspace_size", "sync_tune_forget",
)


class SyncError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


class sync_plan_desc(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32), ("world", ctypes.c_int32), ("rank", ctypes.c_int32), ("ring_dir", ctypes.c_int32),
        ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("pattern", ctypes.c_int32), ("split", ctypes.c_int32),
        ("explicit_order", ctypes.POINTER(ctypes.c_int32)),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_order", ctypes.c_int32),
        ("group_m", ctypes.c_int32), ("local_resident", ctypes.c_int32),
        ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32), ("b_layout", ctypes.c_int32),
        ("shard_rows", ctypes.POINTER(ctypes.c_int64)), ("hier_group", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 1),
    ]


class sync_plan_info(ctypes.Structure):
    _fields_ = [("num_chunks", ctypes.c_int32), ("num_tiles", ctypes.c_int32), ("tiles_m", ctypes.c_int32),
                ("tiles_n", ctypes.c_int32), ("num_deps", ctypes.c_int64)]


_P32 = ctypes.POINTER(ctypes.c_int32)
_P64 = ctypes.POINTER(ctypes.c_int64)


class sync_plan_tables(ctypes.Structure):
    _fields_ = [("chunk_begin", _P64), ("chunk_pos", _P32), ("arrival", _P32), ("resident", _P32),
                ("tiles_in", _P32), ("tile_order", _P32), ("tile_key", _P32), ("dep_ptr", _P64),
                ("dep_idx", _P32), ("inv_ptr", _P64), ("inv_idx", _P32)]


class sync_copy_cfg(ctypes.Structure):
    _fields_ = [("backend", ctypes.c_int32), ("copy_cus", ctypes.c_int32), ("timeout_ns", ctypes.c_uint64),
                ("host_gates", ctypes.c_void_p), ("flags", ctypes.c_int32), ("copy_streaming", ctypes.c_int32),
                ("withhold_chunk", ctypes.c_int32), ("copy_teams", ctypes.c_int32),
                ("copy_kslices", ctypes.c_int32), ("copy_link_gbps", ctypes.c_float),
                ("copy_lead_slice", ctypes.c_int32)]


class sync_trace(ctypes.Structure):
    _fields_ = [("tile_wait_begin", _P64), ("tile_wait_end", _P64), ("tile_end", _P64), ("tile_xcc", _P32),
                ("tile_slot", _P32), ("chunk_ready", _P64), ("chunk_sent", _P64)]


class sync_tune_space(ctypes.Structure):
    _fields_ = [("splits", _P32), ("n_splits", ctypes.c_int32), ("tiles", _P32), ("n_tiles", ctypes.c_int32),
                ("orders", _P32), ("n_orders", ctypes.c_int32), ("copy_cus", _P32), ("n_copy_cus", ctypes.c_int32),
                ("warmup", ctypes.c_int32), ("iters", ctypes.c_int32), ("timeout_ns", ctypes.c_uint64),
                ("force", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("agents", ctypes.c_void_p), ("n_agents", ctypes.c_int32)]


class sync_tune_buffers(ctypes.Structure):
    _fields_ = [("a_peer", ctypes.c_void_p), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("c", ctypes.c_void_p),
                ("staging", ctypes.c_void_p), ("c_dtype", ctypes.c_int32), ("ws", ctypes.c_void_p),
                ("stream", ctypes.c_void_p)]


class sync_tune_result(ctypes.Structure):
    _fields_ = [("split", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_order", ctypes.c_int32), ("copy_cus", ctypes.c_int32), ("best_ms", ctypes.c_float),
                ("candidates_run", ctypes.c_int32), ("candidates_skipped", ctypes.c_int32),
                ("backend", ctypes.c_int32), ("agent", ctypes.c_int32), ("from_cache", ctypes.c_int32),
                ("call_wall_ms", ctypes.c_float), ("search_wall_ms", ctypes.c_float)]


class sync_timing(ctypes.Structure):
    _fields_ = [("kernel_ms", ctypes.c_float), ("copy_ms", ctypes.c_float)]


class sync_device_info(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int32), ("num_cus", ctypes.c_int32), ("num_xcds", ctypes.c_int32),
                ("clock_khz", ctypes.c_int32), ("wall_clock_khz", ctypes.c_int64), ("arch", ctypes.c_char * 64)]


_LIB = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise SyncError(SYNC_ENODEV, f"{LIB_PATH} is not built; run __graft_entry__.build() "
                                         "or python communication_overlap_gemm_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "sync_plan": (i32, [ctypes.POINTER(sync_plan_desc), ctypes.POINTER(vp)]),
            "sync_plan_destroy": (None, [vp]),
            "sync_plan_get_info": (i32, [vp, ctypes.POINTER(sync_plan_info)]),
            "sync_plan_export": (i32, [vp, ctypes.POINTER(sync_plan_tables)]),
            "sync_workspace_size": (ctypes.c_size_t, [vp]),
            "sync_workspace_init": (i32, [vp, vp, vp]),
            "sync_workspace_status": (i32, [vp, vp, ctypes.POINTER(i32)]),
            "sync_ag_gemm": (i32, [vp, ctypes.POINTER(sync_copy_cfg), vp, vp, vp, vp, i32, vp, vp, vp]),
            "sync_ag_gemm_noalloc": (i32, [vp, ctypes.POINTER(sync_copy_cfg), vp, vp, vp, vp, i32, vp]),
            "sync_gemm_rs": (i32, [vp, ctypes.POINTER(sync_copy_cfg), vp, vp, vp, i32, vp, vp, vp, vp]),
            "sync_gemm_rs_reduce": (i32, [vp, ctypes.POINTER(sync_copy_cfg), vp, vp, vp, vp, vp, vp, vp, vp]),
            "sync_gemm_ar": (i32, [vp, ctypes.POINTER(sync_copy_cfg), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "sync_ring_attn_step": (i32, [vp, ctypes.POINTER(sync_copy_cfg), vp, vp, vp, vp, vp, vp, vp, vp, vp, f32,
                                          i32, vp, vp, vp]),
            "sync_head_attn": (i32, [vp, ctypes.POINTER(sync_copy_cfg), vp, vp, vp, vp, vp, vp, vp, vp, f32, vp,
                                     vp, vp]),
            "sync_attn_query_block": (i32, [i32, i32]),
            "sync_gemm_split": (i32, [vp, ctypes.POINTER(sync_copy_cfg), vp, vp, vp, vp, i32, vp, vp, vp, vp]),
            "sync_get_device_info": (i32, [ctypes.POINTER(sync_device_info)]),
            "sync_read_timings": (i32, [i32, ctypes.POINTER(sync_timing), ctypes.POINTER(i32)]),
            "sync_trace_export": (i32, [vp, vp, vp, ctypes.POINTER(sync_trace)]),
            "sync_tune_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(sync_plan_desc),
                                                           ctypes.POINTER(sync_tune_space)]),
            "sync_autotune": (i32, [ctypes.POINTER(sync_plan_desc), ctypes.POINTER(sync_tune_space),
                                    ctypes.POINTER(sync_tune_buffers), ctypes.POINTER(sync_tune_result)]),
            "sync_tune_forget": (None, []),
            "sync_last_error": (ctypes.c_char_p, []),
            "sync_shutdown": (None, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(rc: int) -> int:
    if rc != SYNC_OK:
        msg = lib().sync_last_error()
        raise SyncError(rc, msg.decode() if msg else "")
    return rc


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError(f"cannot take a device pointer from {type(x).__name__}")


def _arg(x, name: str, elem: int, count: int) -> Optional[int]:
    """Device address of x.  A tensor is also checked against what the call
    will touch: on a GPU, contiguous, `elem`-byte elements and at least `count`
    of them (these are size checks only; nothing is computed)."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "data_ptr") and hasattr(x, "is_contiguous"):
        if not getattr(x, "is_cuda", False):
            raise SyncError(SYNC_EINVAL, f"{name} must be a device tensor")
        if not x.is_contiguous():
            raise SyncError(SYNC_EINVAL, f"{name} must be contiguous")
        if x.element_size() != elem:
            raise SyncError(SYNC_EINVAL, f"{name} must have {elem}-byte elements, not {x.element_size()}")
        if x.numel() < count:
            raise SyncError(SYNC_EINVAL, f"{name} holds {x.numel()} elements; the plan needs {count}")
        return int(x.data_ptr())
    return _ptr(x)


def _ws_arg(plan, ws) -> Optional[int]:
    if ws is None or isinstance(ws, int) or not hasattr(ws, "element_size"):
        return _ptr(ws)
    need = int(lib().sync_workspace_size(plan.handle))
    return _arg(ws, "ws", ws.element_size(), (need + ws.element_size() - 1) // ws.element_size())


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"cannot take a stream handle from {type(s).__name__}")


class Plan:
    """Owns a sync_plan_t handle (released with sync_plan_destroy)."""

    def __init__(self, handle: int, desc: sync_plan_desc):
        self.handle = handle
        self.desc = desc

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.sync_plan_destroy(self.handle)
            self.handle = None


def make_desc(op: int, m: int, n: int, k: int, world: int, rank: int = 0, ring_dir: int = 1,
              pattern: int = SYNC_PAT_RING, explicit_order: Optional[Sequence[int]] = None, split: int = 1,
              tile_m: int = 256, tile_n: int = 256, tile_order: int = SYNC_ORDER_CHUNK_MAJOR, group_m: int = 0,
              local_resident: int = 1, heads_q: int = 0, heads_kv: int = 0, b_layout: int = SYNC_B_KN,
              shard_rows: Optional[Sequence[int]] = None, hier_group: int = 0):
    d = sync_plan_desc()
    d.op, d.m, d.n, d.k, d.world, d.rank, d.ring_dir = op, m, n, k, world, rank, ring_dir
    d.pattern, d.split, d.tile_m, d.tile_n, d.tile_order = pattern, split, tile_m, tile_n, tile_order
    d.group_m, d.local_resident, d.heads_q, d.heads_kv, d.b_layout = group_m, local_resident, heads_q, heads_kv, b_layout
    d.hier_group = hier_group
    if explicit_order is not None:
        arr = (ctypes.c_int32 * len(explicit_order))(*explicit_order)
        d.explicit_order = ctypes.cast(arr, _P32)
        d._keep = arr  # keep alive until sync_plan() has read it
    if shard_rows is not None:
        rows = (ctypes.c_int64 * len(shard_rows))(*shard_rows)
        d.shard_rows = ctypes.cast(rows, _P64)
        d._keep_rows = rows
    return d


def sync_plan(desc: sync_plan_desc) -> Plan:
    h = ctypes.c_void_p()
    _check(lib().sync_plan(ctypes.byref(desc), ctypes.byref(h)))
    return Plan(h.value, desc)


def sync_plan_get_info(plan: Plan) -> sync_plan_info:
    info = sync_plan_info()
    _check(lib().sync_plan_get_info(plan.handle, ctypes.byref(info)))
    return info


def sync_plan_export(plan: Plan) -> dict:
    """All plan tables as numpy arrays."""
    info = sync_plan_get_info(plan)
    C, T, D = info.num_chunks, info.num_tiles, info.num_deps
    out = {
        "chunk_begin": np.zeros(C + 1, np.int64), "chunk_pos": np.zeros(C, np.int32),
        "arrival": np.zeros(C, np.int32), "resident": np.zeros(C, np.int32), "tiles_in": np.zeros(C, np.int32),
        "tile_order": np.zeros(T, np.int32), "tile_key": np.zeros(T, np.int32), "dep_ptr": np.zeros(T + 1, np.int64),
        "dep_idx": np.zeros(D, np.int32), "inv_ptr": np.zeros(C + 1, np.int64), "inv_idx": np.zeros(D, np.int32),
    }
    t = sync_plan_tables()
    for name, arr in out.items():
        setattr(t, name, arr.ctypes.data_as(_P64 if arr.dtype == np.int64 else _P32))
    _check(lib().sync_plan_export(plan.handle, ctypes.byref(t)))
    out["num_chunks"], out["num_tiles"], out["tiles_m"], out["tiles_n"] = C, T, info.tiles_m, info.tiles_n
    return out


def make_cfg(backend: int = SYNC_COPY_SDMA, copy_cus: int = 0, timeout_ns: int = 0, host_gates=None,
             flags: int = 0, copy_streaming: int = 0, withhold_chunk: int = -1, copy_teams: int = 0,
             copy_kslices: int = 0, copy_link_gbps: float = 0.0, copy_lead_slice: int = 0) -> sync_copy_cfg:
    c = sync_copy_cfg()
    c.backend, c.copy_cus, c.timeout_ns, c.flags = backend, copy_cus, timeout_ns, flags
    c.copy_streaming, c.withhold_chunk, c.copy_teams = copy_streaming, withhold_chunk, copy_teams
    c.copy_kslices, c.copy_link_gbps, c.copy_lead_slice = copy_kslices, copy_link_gbps, copy_lead_slice
    c.host_gates = _ptr(host_gates)
    return c


def sync_workspace_size(plan: Plan) -> int:
    return int(lib().sync_workspace_size(plan.handle))


def sync_workspace_init(plan: Plan, ws, stream=None) -> None:
    _check(lib().sync_workspace_init(plan.handle, _ptr(ws), _stream(stream)))


def sync_trace_export(plan: Plan, ws, stream=None) -> dict:
    """Trace of the last SYNC_RUN_TRACE GEMM call: numpy arrays in ns (-1 = not recorded)."""
    info = sync_plan_info()
    _check(lib().sync_plan_get_info(plan.handle, ctypes.byref(info)))
    T, C = info.num_tiles, info.num_chunks
    out = {"tile_wait_begin": np.zeros(T, np.int64), "tile_wait_end": np.zeros(T, np.int64),
           "tile_end": np.zeros(T, np.int64), "tile_xcc": np.zeros(T, np.int32), "tile_slot": np.zeros(T, np.int32),
           "chunk_ready": np.zeros(C, np.int64), "chunk_sent": np.zeros(C, np.int64)}
    t = sync_trace()
    for name, arr in out.items():
        setattr(t, name, arr.ctypes.data_as(_P64 if arr.dtype == np.int64 else _P32))
    _check(lib().sync_trace_export(plan.handle, _ptr(ws), _stream(stream), ctypes.byref(t)))
    return out


def make_tune_space(splits=(1, 2, 4), tiles=((256, 256), (256, 128), (128, 128)),
                    orders=(SYNC_ORDER_CHUNK_MAJOR,), copy_cus=(16, 32), warmup: int = 0, iters: int = 0,
                    timeout_ns: int = 0, force: int = 0, agents=()):
    """A sync_tune_space plus the arrays it points into (keep the tuple alive while it is used).
    agents: sync_copy_cfg entries (make_cfg) to try instead of the copy_cus list."""
    arrs = [np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))
            for x in (splits, tiles, orders, copy_cus)]
    sp = sync_tune_space()
    sp.splits, sp.tiles, sp.orders, sp.copy_cus = (a.ctypes.data_as(_P32) for a in arrs)
    sp.n_splits, sp.n_tiles, sp.n_orders, sp.n_copy_cus = len(arrs[0]), len(arrs[1]) // 2, len(arrs[2]), len(arrs[3])
    sp.warmup, sp.iters, sp.timeout_ns, sp.force = warmup, iters, timeout_ns, force
    if agents:
        ag = (sync_copy_cfg * len(agents))(*agents)
        arrs.append(ag)
        sp.agents, sp.n_agents = ctypes.cast(ag, ctypes.c_void_p), len(agents)
    return sp, arrs


def sync_tune_workspace_size(base: sync_plan_desc, space) -> int:
    sp = space[0] if isinstance(space, tuple) else space
    return int(lib().sync_tune_workspace_size(ctypes.byref(base), ctypes.byref(sp)))


def sync_autotune(base: sync_plan_desc, space, *, a, b, c, ws, c_dtype: int = SYNC_DTYPE_F32, a_peer=None,
                  staging=None, stream=None) -> dict:
    """Runs the autotuner (AG: a is a_local, a_peer the peer region; RS: a, staging)."""
    sp = space[0] if isinstance(space, tuple) else space
    bufs = sync_tune_buffers()
    bufs.a_peer, bufs.a, bufs.b, bufs.c, bufs.staging = (_ptr(x) for x in (a_peer, a, b, c, staging))
    bufs.c_dtype, bufs.ws, bufs.stream = c_dtype, _ptr(ws), _stream(stream)
    r = sync_tune_result()
    _check(lib().sync_autotune(ctypes.byref(base), ctypes.byref(sp), ctypes.byref(bufs), ctypes.byref(r)))
    return {"split": r.split, "tile_m": r.tile_m, "tile_n": r.tile_n, "tile_order": r.tile_order,
            "copy_cus": r.copy_cus, "best_ms": r.best_ms, "candidates_run": r.candidates_run,
            "candidates_skipped": r.candidates_skipped, "backend": r.backend, "agent": r.agent,
            "from_cache": r.from_cache, "call_wall_ms": r.call_wall_ms, "search_wall_ms": r.search_wall_ms}


def sync_tune_forget() -> None:
    lib().sync_tune_forget()


def sync_workspace_status(ws, stream=None):
    """(status code, chunk id or -1).  Does not raise on SYNC_ETIMEOUT."""
    ch = ctypes.c_int32(-1)
    rc = lib().sync_workspace_status(_ptr(ws), _stream(stream), ctypes.byref(ch))
    if rc not in (SYNC_OK, SYNC_ETIMEOUT):
        _check(rc)
    return rc, ch.value


def _c_elem(c_dtype: int) -> int:
    return 4 if c_dtype == SYNC_DTYPE_F32 else 2


def sync_ag_gemm(plan: Plan, cfg: Optional[sync_copy_cfg], a_peer, a_local, b, c, c_dtype: int, ws,
                 compute=None, copy=None) -> None:
    m, n, k = plan.desc.m, plan.desc.n, plan.desc.k
    _check(lib().sync_ag_gemm(plan.handle, ctypes.byref(cfg) if cfg is not None else None,
                              _arg(a_peer, "a_peer", 2, m * k), _arg(a_local, "a_local", 2, m * k),
                              _arg(b, "b", 2, k * n), _arg(c, "c", _c_elem(c_dtype), m * n), c_dtype,
                              _ws_arg(plan, ws), _stream(compute), _stream(copy)))


def sync_ag_gemm_noalloc(plan: Plan, cfg: sync_copy_cfg, a_peer, a_local, b, c, c_dtype: int, compute=None) -> None:
    m, n, k = plan.desc.m, plan.desc.n, plan.desc.k
    _check(lib().sync_ag_gemm_noalloc(plan.handle, ctypes.byref(cfg) if cfg is not None else None,
                                      _arg(a_peer, "a_peer", 2, m * k), _arg(a_local, "a_local", 2, m * k),
                                      _arg(b, "b", 2, k * n), _arg(c, "c", _c_elem(c_dtype), m * n), c_dtype,
                                      _stream(compute)))


def sync_gemm_rs(plan: Plan, cfg: Optional[sync_copy_cfg], a, b, c, c_dtype: int, staging, ws, compute=None,
                 copy=None) -> None:
    m, n, k = plan.desc.m, plan.desc.n, plan.desc.k
    e = _c_elem(c_dtype)
    _check(lib().sync_gemm_rs(plan.handle, ctypes.byref(cfg) if cfg is not None else None, _arg(a, "a", 2, m * k),
                              _arg(b, "b", 2, k * n), _arg(c, "c", e, m * n), c_dtype,
                              _arg(staging, "staging", e, m * n), _ws_arg(plan, ws), _stream(compute),
                              _stream(copy)))


def sync_gemm_rs_reduce(plan: Plan, cfg: Optional[sync_copy_cfg], a, b, c, partials, staging, ws, compute=None,
                        copy=None) -> None:
    m, n, k = plan.desc.m, plan.desc.n, plan.desc.k
    _check(lib().sync_gemm_rs_reduce(plan.handle, ctypes.byref(cfg) if cfg is not None else None,
                                     _arg(a, "a", 2, m * k), _arg(b, "b", 2, k * n), _arg(c, "c", 4, m * n),
                                     _arg(partials, "partials", 4, m * n), _arg(staging, "staging", 4, m * n),
                                     _ws_arg(plan, ws), _stream(compute), _stream(copy)))


def sync_gemm_ar(plan: Plan, cfg: Optional[sync_copy_cfg], a, b, c, partials, reduced_peer, out, staging, ws,
                 compute=None, copy=None) -> None:
    m, n, k = plan.desc.m, plan.desc.n, plan.desc.k
    _check(lib().sync_gemm_ar(plan.handle, ctypes.byref(cfg) if cfg is not None else None, _arg(a, "a", 2, m * k),
                              _arg(b, "b", 2, k * n), _arg(c, "c", 4, m * n), _arg(partials, "partials", 4, m * n),
                              _arg(reduced_peer, "reduced_peer", 4, m * n), _arg(out, "out", 4, m * n),
                              _arg(staging, "staging", 4, m * n), _ws_arg(plan, ws), _stream(compute),
                              _stream(copy)))


def sync_ring_attn_step(plan: Plan, cfg: Optional[sync_copy_cfg], q, k_peer, v_peer, k_local, v_local, o, m_state,
                        l_state, lse, scale: float, flags: int, ws, compute=None, copy=None) -> None:
    d = plan.desc
    sq, d_head, hq, hkv = d.m, d.k, d.heads_q, d.heads_kv
    kv = d.world * d.n * hkv * d_head
    _check(lib().sync_ring_attn_step(plan.handle, ctypes.byref(cfg) if cfg is not None else None,
                                     _arg(q, "q", 2, sq * hq * d_head), _arg(k_peer, "k_peer", 2, kv),
                                     _arg(v_peer, "v_peer", 2, kv), _arg(k_local, "k_local", 2, kv),
                                     _arg(v_local, "v_local", 2, kv), _arg(o, "o", 4, sq * hq * d_head),
                                     _arg(m_state, "m_state", 4, hq * sq), _arg(l_state, "l_state", 4, hq * sq),
                                     _arg(lse, "lse", 4, hq * sq), float(scale), flags, _ws_arg(plan, ws),
                                     _stream(compute), _stream(copy)))


def sync_head_attn(plan: Plan, cfg: Optional[sync_copy_cfg], q_peer, k_peer, v_peer, q, k, v, o, lse,
                   scale: float, ws, compute=None, copy=None) -> None:
    """Head-parallel attention share: the all-to-all receive side of Q, K, V
    (token block w from peer w) fused with attention over all world*n tokens."""
    d = plan.desc
    s, d_head, hq, hkv = d.m, d.k, d.heads_q, d.heads_kv
    qn, kv = s * hq * d_head, s * hkv * d_head
    _check(lib().sync_head_attn(plan.handle, ctypes.byref(cfg) if cfg is not None else None,
                                _arg(q_peer, "q_peer", 2, qn), _arg(k_peer, "k_peer", 2, kv),
                                _arg(v_peer, "v_peer", 2, kv), _arg(q, "q", 2, qn), _arg(k, "k", 2, kv),
                                _arg(v, "v", 2, kv), _arg(o, "o", 4, qn), _arg(lse, "lse", 4, hq * s),
                                float(scale), _ws_arg(plan, ws), _stream(compute), _stream(copy)))


def sync_attn_query_block(heads_q: int, heads_kv: int) -> int:
    """Query rows of one attention work item (the tile_m of a HEAD_ATTN plan); 0 if unsupported."""
    return int(lib().sync_attn_query_block(heads_q, heads_kv))


def sync_gemm_split(plan: Plan, cfg: Optional[sync_copy_cfg], a_peer, a, b, c, c_dtype: int, staging, ws, compute,
                    copy) -> None:
    """The kernel-level overlap baseline (per-chunk copies and GEMM launches
    joined by events); `copy` is a second stream."""
    m, n, k = plan.desc.m, plan.desc.n, plan.desc.k
    e = _c_elem(c_dtype)
    _check(lib().sync_gemm_split(plan.handle, ctypes.byref(cfg) if cfg is not None else None,
                                 _arg(a_peer, "a_peer", 2, m * k), _arg(a, "a", 2, m * k), _arg(b, "b", 2, k * n),
                                 _arg(c, "c", e, m * n), c_dtype, _arg(staging, "staging", e, m * n),
                                 _ws_arg(plan, ws), _stream(compute), _stream(copy)))


def sync_get_device_info() -> dict:
    d = sync_device_info()
    _check(lib().sync_get_device_info(ctypes.byref(d)))
    return {"device": d.device, "num_cus": d.num_cus, "num_xcds": d.num_xcds, "clock_khz": d.clock_khz,
            "wall_clock_khz": d.wall_clock_khz, "arch": d.arch.decode()}


def sync_read_timings(max_records: int = 1024):
    """[(kernel_ms, copy_ms), ...] of the most recent SYNC_RUN_TIMED calls, oldest first."""
    buf = (sync_timing * max(1, max_records))()
    n = ctypes.c_int32(0)
    _check(lib().sync_read_timings(max_records, buf, ctypes.byref(n)))
    return [(buf[i].kernel_ms, buf[i].copy_ms) for i in range(n.value)]


def sync_last_error() -> str:
    m = lib().sync_last_error()
    return m.decode() if m else ""


def sync_shutdown() -> None:
    lib().sync_shutdown()
