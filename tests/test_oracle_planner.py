"""Pins for the reference planner (oracle/planner_ref.py).

The pages fix no formula for chunk positions or tile orders (Syncopate summary
page, "Core method", paper sec. 5.1-5.2, Fig. 6), so this planner is pinned
by (1) hand-worked fixtures in tests/golden/plan_fixtures.json, (2) a direct
simulation of ring all-gather and ring reduce-scatter message passing,
(3) invariants checked over a brute-force enumeration of small descriptors,
with the dependency sets recomputed row by row.
"""
import itertools
import json
import os

import pytest

from oracle import planner_ref as P

GOLD = os.path.join(os.path.dirname(__file__), "golden", "plan_fixtures.json")


def _desc(d):
    kw = dict(d)
    return P.PlanDesc(**{("explicit_order" if k == "explicit_order" else k): v for k, v in kw.items()})


@pytest.mark.parametrize("case", json.load(open(GOLD))["cases"], ids=lambda c: c["name"])
def test_hand_worked_fixture(case):
    t = P.plan_ref(_desc(case["desc"]))
    for key, want in case["expect"].items():
        assert list(getattr(t, key)) == want, key


def _simulate_ring_allgather(W, r, d):
    """Each rank forwards what it last received to rank+d; returns the shards rank
    r holds, in the order it gets them (its own first)."""
    last = list(range(W))
    got = [[w] for w in range(W)]
    for _ in range(W - 1):
        incoming = [last[(w - d) % W] for w in range(W)]
        for w in range(W):
            got[w].append(incoming[w])
        last = incoming
    return got[r]


def _simulate_ring_reduce_scatter(W, r, d):
    """Ring reduce-scatter that forwards to rank+d and ends with every rank holding
    its own shard fully reduced.  Returns the order in which rank r's own partial
    results are consumed (added into the travelling sums)."""
    # at step 0 rank w starts the sum for the shard that must end at w + d*(W-1)
    carry = {w: ((w + d * (W - 1)) % W, {w}) for w in range(W)}
    used = {w: [carry[w][0]] for w in range(W)}
    for _ in range(W - 1):
        nxt = {}
        for w in range(W):
            shard, who = carry[(w - d) % W]
            nxt[w] = (shard, who | {w})
            used[w].append(shard)
        carry = nxt
    for w in range(W):
        assert carry[w][0] == w and carry[w][1] == set(range(W))
    return used[r]


@pytest.mark.parametrize("W,r,d", [(W, r, d) for W in (1, 2, 3, 4, 8) for r in range(W) for d in (1, -1)])
def test_ring_positions_follow_message_passing(W, r, d):
    ag = P.plan_ref(P.PlanDesc(op=P.OP_AG_GEMM, m=W, n=1, k=1, world=W, rank=r, ring_dir=d,
                               tile_m=1, tile_n=1))
    assert ag.arrival == _simulate_ring_allgather(W, r, d)
    rs = P.plan_ref(P.PlanDesc(op=P.OP_GEMM_RS, m=W, n=1, k=1, world=W, rank=r, ring_dir=d,
                               tile_m=1, tile_n=1))
    assert rs.arrival == _simulate_ring_reduce_scatter(W, r, d)
    assert rs.arrival[-1] == r


def _check_invariants(desc, t):
    C, T = t.num_chunks, t.num_tiles
    M = desc.world * desc.n if desc.op == P.OP_RING_ATTN else desc.m
    # chunks partition [0, M): contiguous, non-empty
    assert t.chunk_begin[0] == 0 and t.chunk_begin[-1] == M and len(t.chunk_begin) == C + 1
    assert all(t.chunk_begin[c] < t.chunk_begin[c + 1] for c in range(C))
    # arrival is a permutation, chunk_pos its inverse
    assert sorted(t.arrival) == list(range(C))
    assert all(t.chunk_pos[t.arrival[p]] == p for p in range(C))
    assert sorted(t.tile_order) == list(range(T))
    # deps == brute force, row by row
    for tile in range(T):
        i = tile // t.tiles_n
        deps = t.dep_idx[t.dep_ptr[tile]:t.dep_ptr[tile + 1]]
        if desc.op == P.OP_RING_ATTN:
            want = list(range(C))
        else:  # GEMM ops and head-parallel attention: the chunks holding the tile's rows
            rows = range(i * desc.tile_m, min((i + 1) * desc.tile_m, desc.m))
            want = sorted({next(c for c in range(C) if t.chunk_begin[c] <= row < t.chunk_begin[c + 1])
                           for row in rows})
        assert deps == want
    # inv is the transpose of deps
    pairs_dep = {(tile, c) for tile in range(T) for c in t.dep_idx[t.dep_ptr[tile]:t.dep_ptr[tile + 1]]}
    pairs_inv = {(tile, c) for c in range(C) for tile in t.inv_idx[t.inv_ptr[c]:t.inv_ptr[c + 1]]}
    assert pairs_dep == pairs_inv and len(t.dep_idx) == len(t.inv_idx)
    assert all(t.inv_idx[t.inv_ptr[c]:t.inv_ptr[c + 1]] == sorted(t.inv_idx[t.inv_ptr[c]:t.inv_ptr[c + 1]])
               for c in range(C))
    assert t.tiles_in == [t.inv_ptr[c + 1] - t.inv_ptr[c] for c in range(C)]
    # keys: the last (AG) or first (RS) position among a tile's chunks
    for tile in range(T):
        ps = [t.chunk_pos[c] for c in t.dep_idx[t.dep_ptr[tile]:t.dep_ptr[tile + 1]]]
        assert t.tile_key[tile] == (min(ps) if desc.op == P.OP_GEMM_RS else max(ps))
    keys = [t.tile_key[x] for x in t.tile_order]
    if desc.tile_order in (P.ORDER_CHUNK_MAJOR, P.ORDER_SWIZZLED):
        assert keys == sorted(keys)
    else:
        assert t.tile_order == list(range(T))
    # the local shard is resident for AG/attention only
    for c in range(C):
        own = (c // desc.split) == desc.rank
        assert t.resident[c] == int(own and desc.local_resident and desc.op != P.OP_GEMM_RS)
    # aligned case: one dependency per tile, equal tile counts per chunk
    if desc.op != P.OP_RING_ATTN:
        R = desc.m // desc.world  # head-parallel attention: n tokens per peer
        if R % desc.split == 0 and (R // desc.split) % desc.tile_m == 0:
            assert all(t.dep_ptr[x + 1] - t.dep_ptr[x] == 1 for x in range(T))
            assert set(t.tiles_in) == {(R // desc.split // desc.tile_m) * t.tiles_n}


def _enumerate():
    for op in (P.OP_AG_GEMM, P.OP_GEMM_RS):
        for W in (1, 2, 3, 4):
            for rows_per in (1, 2, 3, 5):
                m = W * rows_per
                for s in range(1, min(3, rows_per) + 1):
                    for tm in (1, 2, 3, 4):
                        if -(-m // tm) > 8:
                            continue
                        for order in (0, 1, 2):
                            for d in (1, -1):
                                for r in range(W):
                                    yield P.PlanDesc(op=op, m=m, n=5, k=3, world=W, rank=r, ring_dir=d,
                                                     split=s, tile_m=tm, tile_n=2, tile_order=order,
                                                     group_m=2)
    for W, n, s, tm in itertools.product((1, 2, 3), (2, 3), (1, 2), (1, 3)):
        yield P.PlanDesc(op=P.OP_RING_ATTN, m=5, n=n, k=8, world=W, rank=W - 1, split=s, tile_m=tm,
                         tile_n=1, heads_q=4, heads_kv=2, tile_order=1)
    for W, n, s, tm, order in itertools.product((1, 2, 3, 4), (2, 3, 5), (1, 2), (1, 2, 4), (0, 1, 2)):
        for r in sorted({0, W - 1}):
            yield P.PlanDesc(op=P.OP_HEAD_ATTN, m=W * n, n=n, k=8, world=W, rank=r, split=s, tile_m=tm,
                             heads_q=2, heads_kv=1, tile_order=order, group_m=2)


def test_invariants_brute_force_enumeration():
    count = 0
    for desc in _enumerate():
        _check_invariants(desc, P.plan_ref(desc))
        count += 1
    assert count > 1000


def test_explicit_orders_all_permutations():
    for perm in itertools.permutations(range(4)):
        desc = P.PlanDesc(op=P.OP_AG_GEMM, m=8, n=3, k=2, world=4, rank=2, pattern=P.PAT_EXPLICIT,
                          explicit_order=list(perm), split=2, tile_m=3, tile_n=2)
        t = P.plan_ref(desc)
        _check_invariants(desc, t)
        assert [t.arrival[p] // 2 for p in range(0, 8, 2)] == list(perm)


@pytest.mark.parametrize("bad", [
    dict(m=10, world=4),                       # m % world
    dict(split=0), dict(split=3),             # split out of [1, R]
    dict(rank=4), dict(ring_dir=0), dict(op=9), dict(tile_order=5),
    dict(pattern=1, explicit_order=[0, 0, 1, 2]),
])
def test_rejects_invalid(bad):
    base = dict(op=P.OP_AG_GEMM, m=8, n=4, k=4, world=4, split=1, tile_m=2, tile_n=2)
    base.update(bad)
    with pytest.raises(P.PlanError):
        P.plan_ref(P.PlanDesc(**base))


def test_attention_requires_grouped_heads():
    with pytest.raises(P.PlanError):
        P.plan_ref(P.PlanDesc(op=P.OP_RING_ATTN, m=4, n=4, k=8, world=2, tile_m=2, heads_q=3, heads_kv=2))
    with pytest.raises(P.PlanError):
        P.plan_ref(P.PlanDesc(op=P.OP_HEAD_ATTN, m=8, n=4, k=8, world=2, tile_m=2, heads_q=3, heads_kv=2))


@pytest.mark.parametrize("m", [4, 7, 9])
def test_head_parallel_queries_are_every_token(m):
    """Head-parallel attention: after the all-to-all every token of the head
    group is a query, so m must be world * n."""
    with pytest.raises(P.PlanError):
        P.plan_ref(P.PlanDesc(op=P.OP_HEAD_ATTN, m=m, n=4, k=8, world=2, tile_m=2, heads_q=2, heads_kv=1))


def test_head_parallel_items_start_with_their_queries():
    """Every tile's key is the position of the last chunk holding its query
    rows, so in chunk-major order the tiles whose queries are resident come
    first, and a tile's queries have all arrived by its key."""
    for W in (2, 4, 8):
        for r in range(W):
            t = P.plan_ref(P.PlanDesc(op=P.OP_HEAD_ATTN, m=W * 8, n=8, k=8, world=W, rank=r, split=2, tile_m=4,
                                      heads_q=4, heads_kv=1))
            first = t.tile_order[:(8 // 4) * t.tiles_n]  # the own block's 2 tile rows x 4 heads
            assert all(t.resident[c] for x in first for c in t.dep_idx[t.dep_ptr[x]:t.dep_ptr[x + 1]])
            for x in t.tile_order:
                ps = [t.chunk_pos[c] for c in t.dep_idx[t.dep_ptr[x]:t.dep_ptr[x + 1]]]
                rows = range((x // t.tiles_n) * 4, (x // t.tiles_n) * 4 + 4)
                assert all(any(t.chunk_begin[c] <= q < t.chunk_begin[c + 1] and t.chunk_pos[c] <= t.tile_key[x]
                               for c in range(t.num_chunks)) for q in rows)
                assert max(ps) == t.tile_key[x]


def test_uneven_shards_hand_worked():
    """Three peers send 3, 1 and 4 rows (W = 3, rank 0, split 1, one-row tiles):
    shards start at 0, 3 and 4; the ring brings shard 0 (local), then 2, then 1."""
    t = P.plan_ref(P.PlanDesc(op=P.OP_AG_GEMM, m=8, n=2, k=2, world=3, rank=0, tile_m=1, tile_n=2,
                              shard_rows=[3, 1, 4]))
    assert list(t.chunk_begin) == [0, 3, 4, 8]
    assert list(t.arrival) == [0, 2, 1]
    assert list(t.resident) == [1, 0, 0]
    # one-row tiles: rows 0-2 read chunk 0, row 3 chunk 1, rows 4-7 chunk 2
    assert [t.dep_idx[t.dep_ptr[i]] for i in range(8)] == [0, 0, 0, 1, 2, 2, 2, 2]
    t2 = P.plan_ref(P.PlanDesc(op=P.OP_AG_GEMM, m=8, n=2, k=2, world=3, split=2, tile_m=4, tile_n=2,
                               shard_rows=[3, 2, 3]))
    assert list(t2.chunk_begin) == [0, 1, 3, 4, 5, 6, 8]     # floor(q * R_w / 2) inside each shard
    # a 4-row tile over rows 4-7 meets chunks 3 (row 4), 4 (row 5) and 5 (rows 6-7)
    assert list(t2.dep_idx[t2.dep_ptr[1]:t2.dep_ptr[2]]) == [3, 4, 5]


# ---- hierarchical swizzle and mesh patterns -----------------------------------

def _order(op, W, r, pattern, g=0, d=1, split=1):
    t = P.plan_ref(P.PlanDesc(op=op, m=W * split * 2, n=4, k=4, world=W, rank=r, ring_dir=d, pattern=pattern,
                              hier_group=g, split=split, tile_m=2, tile_n=2))
    return t


@pytest.mark.parametrize("W", [1, 2, 3, 4, 6, 8, 12])
def test_hier_swizzle_steps_are_conflict_free_and_group_first(W):
    """For every group size g dividing W: each rank's order is a permutation
    starting with its own shard and then its own group; at every step the
    ranks pull from distinct shards (a bijection), and the RS send order is
    the all-gather order reversed."""
    for g in [x for x in range(1, W + 1) if W % x == 0]:
        orders = [_order(P.OP_AG_GEMM, W, r, P.PAT_HIER_SWIZZLE, g).arrival for r in range(W)]
        for r, o in enumerate(orders):
            assert sorted(o) == list(range(W)) and o[0] == r
            assert sorted(o[:g]) == list(range((r // g) * g, (r // g) * g + g))
            assert _order(P.OP_GEMM_RS, W, r, P.PAT_HIER_SWIZZLE, g).arrival == o[::-1]
        for k in range(W):
            assert sorted(o[k] for o in orders) == list(range(W)), (g, k)


@pytest.mark.parametrize("W", [1, 2, 4, 5, 8])
def test_hier_swizzle_degenerates_to_the_reverse_ring(W):
    """One group of all ranks, or groups of one rank: both are the ring
    towards rank - 1 (rank r takes r, r+1, r+2, ...)."""
    for r in range(W):
        ring = _order(P.OP_AG_GEMM, W, r, P.PAT_RING, d=-1).arrival
        assert _order(P.OP_AG_GEMM, W, r, P.PAT_HIER_SWIZZLE, W).arrival == ring
        assert _order(P.OP_AG_GEMM, W, r, P.PAT_HIER_SWIZZLE, 1).arrival == ring


@pytest.mark.parametrize("op", [P.OP_AG_GEMM, P.OP_GEMM_RS])
def test_mesh_interleaves_sub_chunks(op):
    """Mesh with split 1 is the ring; with split s the first W positions hold
    sub-chunk 0 of every shard, in ring step order, then sub-chunk 1, ..."""
    W, s = 5, 3
    for r in range(W):
        for d in (1, -1):
            assert _order(op, W, r, P.PAT_MESH, d=d).chunk_pos == _order(op, W, r, P.PAT_RING, d=d).chunk_pos
            ring = _order(op, W, r, P.PAT_RING, d=d, split=s)
            mesh = _order(op, W, r, P.PAT_MESH, d=d, split=s)
            steps = [ring.arrival[k * s] // s for k in range(W)]  # shards in ring step order
            assert mesh.arrival == [steps[k] * s + q for q in range(s) for k in range(W)]


def test_pattern_group_validation():
    for kw in (dict(pattern=P.PAT_HIER_SWIZZLE, hier_group=3), dict(pattern=P.PAT_HIER_SWIZZLE, hier_group=0),
               dict(pattern=P.PAT_RING, hier_group=2), dict(pattern=7)):
        with pytest.raises(P.PlanError):
            P.plan_ref(P.PlanDesc(op=P.OP_AG_GEMM, m=8, n=4, k=4, world=4, tile_m=2, tile_n=2, **kw))
