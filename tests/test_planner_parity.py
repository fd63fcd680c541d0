"""The library's C++ planner (called through the C ABI, no GPU needed) must
produce tables bit-identical to the oracle planner's, for every descriptor of
a brute-force enumeration plus the workload configurations."""
import itertools

import numpy as np
import pytest

from communication_overlap_gemm_amd import _abi as A
from oracle import planner_ref as P

KEYS = ["chunk_begin", "chunk_pos", "arrival", "resident", "tiles_in", "tile_order", "tile_key", "dep_ptr",
        "dep_idx", "inv_ptr", "inv_idx"]


def _both(**kw):
    ref = P.plan_ref(P.PlanDesc(**kw))
    kw2 = dict(kw)
    order = kw2.pop("explicit_order", None)
    lib = A.sync_plan_export(A.sync_plan(A.make_desc(explicit_order=order, **kw2)))
    return ref, lib


def _same(ref, lib):
    assert lib["num_chunks"] == ref.num_chunks and lib["num_tiles"] == ref.num_tiles
    assert lib["tiles_m"] == ref.tiles_m and lib["tiles_n"] == ref.tiles_n
    for key in KEYS:
        assert np.array_equal(lib[key], np.asarray(getattr(ref, key), dtype=lib[key].dtype)), key


def _enumerate():
    for op in (P.OP_AG_GEMM, P.OP_GEMM_RS):
        for W in (1, 2, 3, 4):
            for rows_per in (1, 2, 5):
                m = W * rows_per
                for s in range(1, min(3, rows_per) + 1):
                    for tm, order, d in itertools.product((1, 2, 4), (0, 1, 2), (1, -1)):
                        yield dict(op=op, m=m, n=5, k=3, world=W, rank=W - 1, ring_dir=d, split=s, tile_m=tm,
                                   tile_n=2, tile_order=order, group_m=2)
    for W, n, s, tm in itertools.product((1, 2, 3), (2, 3), (1, 2), (1, 3)):
        yield dict(op=P.OP_RING_ATTN, m=5, n=n, k=8, world=W, rank=0, split=s, tile_m=tm, tile_n=1,
                   heads_q=4, heads_kv=2, tile_order=1)
    for W, n, s, tm, order in itertools.product((1, 2, 3, 4), (2, 5), (1, 2), (1, 3, 4), (0, 1, 2)):
        yield dict(op=P.OP_HEAD_ATTN, m=W * n, n=n, k=8, world=W, rank=W // 2, split=s, tile_m=tm, tile_n=1,
                   heads_q=4, heads_kv=1, tile_order=order, group_m=2)


def test_enumeration_bit_exact():
    n = 0
    for kw in _enumerate():
        _same(*_both(**kw))
        n += 1
    assert n > 500


WORKLOADS = [
    # tiny AG-GEMM share: 4 shards of 256 rows, 128x128 tiles
    dict(op=1, m=1024, n=1024, k=1024, world=4, tile_m=128, tile_n=128),
    # Llama-3-8B FFN up-projection AG share, split 1..4, 256x256 tiles
    *[dict(op=1, m=8192, n=1792, k=4096, world=8, split=s, tile_m=256, tile_n=256, tile_order=o)
      for s in (1, 2, 3, 4) for o in (0, 1, 2)],
    # Llama-3-8B FFN down-projection RS share
    dict(op=2, m=8192, n=4096, k=1792, world=8, tile_m=256, tile_n=256),
    # 70B-like AG share, chunk-size sweep
    *[dict(op=1, m=16384, n=3584, k=8192, world=8, split=s, tile_m=256, tile_n=256, tile_order=o)
      for s in (1, 4, 16, 64) for o in (0, 1, 2)],
    # ring-attention step: 4096 queries, 8 KV blocks of 4096 tokens, 32/8 heads
    dict(op=3, m=4096, n=4096, k=128, world=8, tile_m=128, tile_n=1, heads_q=32, heads_kv=8),
    # head-parallel attention share: 8 peers x 4096 tokens, one rank's 4/1 heads, 64-row query blocks
    *[dict(op=4, m=32768, n=4096, k=128, world=8, rank=3, split=s, tile_m=64, tile_n=1, heads_q=4, heads_kv=1,
           tile_order=o) for s in (1, 4) for o in (0, 1, 2)],
]


@pytest.mark.parametrize("kw", WORKLOADS)
def test_workload_plans_bit_exact(kw):
    _same(*_both(**kw))


def test_hier_swizzle_and_mesh_bit_exact():
    """The hierarchical-swizzle and mesh patterns: both planners agree bit
    for bit over worlds, group sizes, ranks, directions, splits and orders."""
    n = 0
    for op in (P.OP_AG_GEMM, P.OP_GEMM_RS, P.OP_RING_ATTN, P.OP_HEAD_ATTN):
        for W in (1, 2, 4, 6, 8):
            for r in sorted({0, W // 2, W - 1}):
                for s, order in itertools.product((1, 3), (0, 1, 2)):
                    attn = op in (P.OP_RING_ATTN, P.OP_HEAD_ATTN)
                    m = W * 6 if op == P.OP_HEAD_ATTN else (7 if attn else W * 6)
                    base = dict(op=op, m=m, n=6 if attn else 5, k=8 if attn else 3,
                                world=W, rank=r, split=s, tile_m=4, tile_n=1 if attn else 2, tile_order=order,
                                group_m=2, **(dict(heads_q=4, heads_kv=2) if attn else {}))
                    for g in [x for x in range(1, W + 1) if W % x == 0]:
                        _same(*_both(pattern=P.PAT_HIER_SWIZZLE, hier_group=g, **base))
                        n += 1
                    for d in (1, -1):
                        _same(*_both(pattern=P.PAT_MESH, ring_dir=d, **base))
                        n += 1
    assert n > 300
    for bad in (dict(pattern=P.PAT_HIER_SWIZZLE, hier_group=3), dict(pattern=P.PAT_RING, hier_group=2)):
        with pytest.raises(A.SyncError):
            A.sync_plan(A.make_desc(P.OP_AG_GEMM, 8, 4, 4, 4, tile_m=2, tile_n=2, **bad))


def test_explicit_order_bit_exact():
    for perm in itertools.permutations(range(4)):
        _same(*_both(op=1, m=12, n=4, k=64, world=4, rank=1, pattern=1, explicit_order=list(perm), split=3,
                      tile_m=2, tile_n=2, tile_order=2, group_m=3))


def _uneven():
    rng = np.random.default_rng(11)
    for op in (P.OP_AG_GEMM, P.OP_GEMM_RS):
        for W in (1, 2, 3, 5):
            for _ in range(6):
                rows = [int(x) for x in rng.integers(1, 9, size=W)]
                for s in range(1, min(3, min(rows)) + 1):
                    for tm, order, d in itertools.product((1, 3), (0, 1, 2), (1, -1)):
                        yield dict(op=op, m=sum(rows), n=5, k=3, world=W, rank=int(rng.integers(0, W)), ring_dir=d,
                                   split=s, tile_m=tm, tile_n=2, tile_order=order, group_m=2, shard_rows=rows)


def test_uneven_shards_bit_exact():
    """Uneven shards (an all-to-all's receive side): both planners agree bit
    for bit on random per-shard row counts."""
    n = 0
    for kw in _uneven():
        _same(*_both(**kw))
        n += 1
    assert n > 300


def test_uneven_shards_rejected_alike():
    for bad in (dict(shard_rows=[3, 0, 5]), dict(shard_rows=[3, 3, 3]), dict(shard_rows=[2, 2, 4], split=3),
                dict(m=0, shard_rows=None), dict(k=0), dict(n=0), dict(world=0, shard_rows=None)):
        kw = dict(op=P.OP_AG_GEMM, m=8, n=4, k=4, world=3, tile_m=2, tile_n=2)
        kw.update(bad)
        with pytest.raises(P.PlanError):
            P.plan_ref(P.PlanDesc(**kw))
        with pytest.raises(A.SyncError):
            A.sync_plan(A.make_desc(**kw))
    with pytest.raises(A.SyncError):
        A.sync_plan(A.make_desc(P.OP_RING_ATTN, 4, 4, 128, 2, tile_m=4, tile_n=1, heads_q=2, heads_kv=1,
                                shard_rows=[2, 2]))
