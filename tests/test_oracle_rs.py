"""Pins for the oracle's reduce-scatter share outputs (oracle/__init__.py:
rs_staging_expected, rs_reduce_staging_expected).

A rank of a ring reduce-scatter sends its chunks in the order the ring needs
them, and with the reduction each sent chunk carries the rank's own partial
result plus the partial sum it received (Syncopate summary page,
"Experiments", paper sec. 6.1: GEMM-RS).  Pinned by a hand-worked two-rank
case and by invariants: with nothing received the reduce step is the plain
send, and every slot is a row block of R + P, each row placed once.
"""
import numpy as np
import pytest

import oracle
from oracle import planner_ref as P


def _plan(m, world, split=1, rank=0, ring_dir=1):
    return P.plan_ref(P.PlanDesc(op=P.OP_GEMM_RS, m=m, n=8, k=8, world=world, rank=rank, ring_dir=ring_dir,
                                 split=split, tile_m=1, tile_n=8))


def test_hand_worked_two_ranks():
    # W = 2, rank 0, ring towards rank 1: the rank first sends the chunk that
    # rank 1 owns (rows 2-3), then its own chunk (rows 0-1) comes last.
    plan = _plan(4, 2)
    r = np.array([[1.0], [2.0], [3.0], [4.0]])
    p = np.array([[10.0], [20.0], [30.0], [40.0]])
    slots, staged = oracle.rs_staging_expected(r, plan)
    assert [s[0] for s in slots] == [1, 0]
    assert staged.ravel().tolist() == [3.0, 4.0, 1.0, 2.0]
    _, red = oracle.rs_reduce_staging_expected(r, p, plan)
    assert red.ravel().tolist() == [33.0, 44.0, 11.0, 22.0]


@pytest.mark.parametrize("m,world,split,rank,d", [(24, 4, 1, 0, 1), (30, 3, 2, 2, -1), (64, 8, 3, 5, 1)])
def test_reduce_step_invariants(m, world, split, rank, d):
    plan = _plan(m, world, split, rank, d)
    rng = np.random.default_rng(7)
    r = rng.standard_normal((m, 5))
    p = rng.standard_normal((m, 5))
    slots, plain = oracle.rs_staging_expected(r, plan)
    _, zero = oracle.rs_reduce_staging_expected(r, np.zeros_like(p), plan)
    assert np.array_equal(plain, zero)                     # nothing received: the plain send
    _, red = oracle.rs_reduce_staging_expected(r, p, plan)
    row = 0
    seen = np.zeros(m, dtype=int)
    for c, b, e in slots:                                  # each slot is the chunk's rows of R + P
        assert np.array_equal(red[row:row + e - b], r[b:e] + p[b:e])
        seen[b:e] += 1
        row += e - b
    assert row == m and np.all(seen == 1)                  # every row sent exactly once
    assert slots[-1][0] in range(rank * split, (rank + 1) * split)  # the rank's own chunks go last


def test_ar_share_hand_worked():
    """W = 2: the own shard's rows end the reduce-scatter as R + P; the other
    rows come from the all-gather."""
    plan = _plan(4, 2)
    r = np.array([[1.0], [2.0], [3.0], [4.0]])
    p = np.array([[10.0], [20.0], [30.0], [40.0]])
    peer = np.array([[100.0], [200.0], [300.0], [400.0]])
    assert oracle.ar_share_expected(r, p, peer, plan, 2, 0).ravel().tolist() == [11.0, 22.0, 300.0, 400.0]
    plan1 = _plan(4, 2, rank=1)
    assert oracle.ar_share_expected(r, p, peer, plan1, 2, 1).ravel().tolist() == [100.0, 200.0, 33.0, 44.0]


def test_ar_share_with_split_keeps_every_own_sub_chunk():
    m, world, split, rank = 48, 4, 3, 2
    plan = _plan(m, world, split, rank)
    rng = np.random.default_rng(3)
    r, p, peer = rng.standard_normal((m, 2)), rng.standard_normal((m, 2)), rng.standard_normal((m, 2))
    out = oracle.ar_share_expected(r, p, peer, plan, world, rank)
    own = np.zeros(m, dtype=bool)
    own[rank * m // world:(rank + 1) * m // world] = True
    assert np.array_equal(out[own], r[own] + p[own]) and np.array_equal(out[~own], peer[~own])
