"""ORACLE for the chunk-overlapped collective-GEMM share -- test infrastructure.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import, call or load anything here.  The HIP path shares no
code with it: no kernels, headers, helpers or table generators.  The only code
both sides use is the seeded input generator, which holds none of the method's
arithmetic.

Contents (each cites the passage it follows in its own header):
  gemm_ref.c     fp64 matrix product R = A . B (full and sampled)
  attn_ref.c     fp64 direct two-pass softmax attention (full and sampled)
  attention.py   fp64 blockwise online-softmax merge (to check the merge identity)
  head_parallel.py the head-parallel attention share: the all-to-all's head
                 group of each rank, and direct attention on it
  planner_ref.py reference chunk planner (chunk rows, ring positions, tile
                 dependencies, tile orders)
Pins: tests/test_oracle_*.py check every function here against closed forms,
exact integer arithmetic, library routines and hand-worked fixtures
(tests/golden/).  The planner's parity with the pages is unpinned beyond those
(the pages give no formula for it).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .planner_ref import (  # noqa: F401
    OP_AG_GEMM, OP_GEMM_RS, OP_HEAD_ATTN, OP_RING_ATTN, ORDER_CHUNK_MAJOR, ORDER_ROW_MAJOR, ORDER_SWIZZLED,
    PAT_EXPLICIT, PAT_HIER_SWIZZLE, PAT_MESH, PAT_RING, PlanDesc, PlanError, PlanTables, plan_ref)
from .attention import attention_online_f64  # noqa: F401
from .head_parallel import head_group, head_parallel_attention_f64  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def default_threads() -> int:
    """Threads the oracle uses: every CPU this process may run on, unless
    OMP_NUM_THREADS names a smaller share (a shared machine's CPU share for
    one job)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm_f64.argtypes = [p, p, ctypes.c_int, i64, i64, i64, p, ctypes.c_int]
        lib.oracle_gemm_f64_sampled.argtypes = [p, p, ctypes.c_int, i64, i64, i64, p, p, i64, p,
                                                ctypes.c_int]
        lib.oracle_attention_f64.argtypes = [p, p, p, i64, i64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_double, p, p, ctypes.c_int]
        lib.oracle_attention_f64_sampled.argtypes = [p, p, p, i64, i64, ctypes.c_int, ctypes.c_int,
                                                     ctypes.c_int, ctypes.c_double, p, p, i64, p, p,
                                                     ctypes.c_int]
        for f in (lib.oracle_gemm_f64, lib.oracle_gemm_f64_sampled, lib.oracle_attention_f64,
                  lib.oracle_attention_f64_sampled):
            f.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _u16(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16)")
    return x


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


_B_LAYOUT = {"kn": 0, "nk": 1}


def gemm_f64(a_bits, b_bits, m, n, k, b_layout="kn", threads=None):
    """R[m,n] = A . B in fp64 (A [m,k] bf16 bits; B [k,n] or [n,k] bf16 bits)."""
    a, b = _u16(a_bits), _u16(b_bits)
    assert a.size == m * k and b.size == k * n
    out = np.empty((m, n), dtype=np.float64)
    rc = _lib().oracle_gemm_f64(_ptr(a), _ptr(b), _B_LAYOUT[b_layout], m, n, k, _ptr(out),
                                threads or default_threads())
    if rc:
        raise ValueError("oracle_gemm_f64 rejected its arguments")
    return out


def gemm_f64_sampled(a_bits, b_bits, m, n, k, rows, cols, b_layout="kn", threads=None):
    """fp64 values of (A . B)[rows[s], cols[s]]."""
    a, b = _u16(a_bits), _u16(b_bits)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.shape == cols.shape
    out = np.empty(rows.shape, dtype=np.float64)
    rc = _lib().oracle_gemm_f64_sampled(_ptr(a), _ptr(b), _B_LAYOUT[b_layout], m, n, k,
                                        _ptr(rows), _ptr(cols), rows.size, _ptr(out),
                                        threads or default_threads())
    if rc:
        raise ValueError("oracle_gemm_f64_sampled rejected its arguments")
    return out


def attention_f64(q_bits, k_bits, v_bits, scale, threads=None):
    """Direct softmax attention in fp64.  Q [Sq,Hq,d], K/V [Skv,Hkv,d] bf16 bits.
    Returns (O [Sq,Hq,d], LSE [Hq,Sq])."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    sq, hq, d = q.shape
    skv, hkv, d2 = k.shape
    assert d == d2 and v.shape == k.shape
    o = np.empty((sq, hq, d), dtype=np.float64)
    lse = np.empty((hq, sq), dtype=np.float64)
    rc = _lib().oracle_attention_f64(_ptr(q), _ptr(k), _ptr(v), sq, skv, hq, hkv, d,
                                     float(scale), _ptr(o), _ptr(lse), threads or default_threads())
    if rc:
        raise ValueError("oracle_attention_f64 rejected its arguments")
    return o, lse


def attention_f64_sampled(q_bits, k_bits, v_bits, scale, qidx, hidx, threads=None):
    """fp64 attention rows for sampled (query, head) pairs: (O [count,d], LSE [count])."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    sq, hq, d = q.shape
    skv, hkv, _ = k.shape
    qidx = np.ascontiguousarray(qidx, dtype=np.int64)
    hidx = np.ascontiguousarray(hidx, dtype=np.int32)
    o = np.empty((qidx.size, d), dtype=np.float64)
    lse = np.empty((qidx.size,), dtype=np.float64)
    rc = _lib().oracle_attention_f64_sampled(_ptr(q), _ptr(k), _ptr(v), sq, skv, hq, hkv, d,
                                             float(scale), _ptr(qidx), _ptr(hidx), qidx.size,
                                             _ptr(o), _ptr(lse), threads or default_threads())
    if rc:
        raise ValueError("oracle_attention_f64_sampled rejected its arguments")
    return o, lse


def rs_staging_expected(r_full, plan: PlanTables):
    """What the reduce-scatter share emits: staging slot p holds the rows of the
    chunk sent p-th (arrival[p]); rows are those of the chunk in R.  Returns a
    list of (chunk id, row begin, row end) in slot order and the staged array."""
    slots = []
    parts = []
    for p in range(plan.num_chunks):
        c = plan.arrival[p]
        b, e = plan.chunk_begin[c], plan.chunk_begin[c + 1]
        slots.append((c, b, e))
        parts.append(r_full[b:e])
    return slots, np.concatenate(parts, axis=0)


def rs_reduce_staging_expected(r_full, partials, plan: PlanTables):
    """The reduce-scatter step of the share (Syncopate summary page,
    "Experiments", paper sec. 6.1: GEMM-RS; a ring reduce-scatter forwards the
    sum of the rank's own partial result and the partial sum it received):
    staging slot p holds, over the rows of chunk arrival[p], R + P in fp64,
    where P is the received partial sum.  Same slot order as
    rs_staging_expected."""
    total = np.asarray(r_full, dtype=np.float64) + np.asarray(partials, dtype=np.float64)
    return rs_staging_expected(total, plan)


def ar_share_expected(r_full, partials, reduced_peer, plan: PlanTables, world: int, rank: int):
    """The GEMM-AR share's output (Syncopate summary page, "Experiments",
    paper sec. 6.1, Fig. 11: GEMM-AR; an all-reduce is a reduce-scatter then
    an all-gather): the rows of this rank's own shard hold R + P, where P is
    the partial sum received in the reduce-scatter (the reduce-scatter ends
    there); every other row holds what the all-gather brings, reduced_peer.
    fp64."""
    out = np.array(reduced_peer, dtype=np.float64, copy=True)
    per = plan.num_chunks // world
    for c in range(rank * per, (rank + 1) * per):
        b, e = plan.chunk_begin[c], plan.chunk_begin[c + 1]
        out[b:e] = np.asarray(r_full[b:e], dtype=np.float64) + np.asarray(partials[b:e], dtype=np.float64)
    return out
