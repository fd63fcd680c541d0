"""Pins for the head-parallel attention oracle (oracle/head_parallel.py).

Head-parallel attention is among the operators the Syncopate summary page
evaluates ("Experiments", paper sec. 6.1 and Fig. 9); the scheme is the
all-to-all of DeepSpeed-Ulysses (the review page's references).  Pins:
  * the head group a rank holds equals what a message-by-message simulation
    of the all-to-all delivers to it (each peer sends its sequence shard's
    slice of the rank's heads; the rank stacks the messages in peer order);
  * the ranks' shares, concatenated over heads, equal direct attention over
    all heads (so the split keeps every query head with its KV head);
  * uneven head splits are rejected.
Direct attention itself is pinned in test_oracle_attention.py.
"""
import math

import numpy as np
import pytest

import oracle
from communication_overlap_gemm_amd import inputs


def _all_to_all_receive(x, world, rank):
    """Message passing: peer w holds tokens [w*n, (w+1)*n) of every head and
    sends rank `rank` the heads of its group, token by token."""
    s, h, d = x.shape
    n, g = s // world, h // world
    received = []
    for w in range(world):
        shard = x[w * n:(w + 1) * n]                 # peer w's sequence shard
        msg = [[shard[t][rank * g + j] for j in range(g)] for t in range(n)]
        received.extend(msg)
    return np.array(received)


@pytest.mark.parametrize("world,n,h,d", [(1, 3, 2, 4), (2, 3, 4, 2), (4, 2, 8, 3), (3, 1, 6, 1)])
def test_head_group_is_the_all_to_all_receive(world, n, h, d):
    x = np.arange(world * n * h * d, dtype=np.int64).reshape(world * n, h, d)
    for r in range(world):
        assert np.array_equal(oracle.head_group(x, world, r), _all_to_all_receive(x, world, r))


@pytest.mark.parametrize("world,hq,hkv", [(1, 4, 2), (2, 4, 2), (2, 8, 2), (4, 8, 4), (2, 2, 2)])
def test_ranks_together_give_full_attention(world, hq, hkv):
    n, d = 5, 16
    s = world * n
    q, k, v = inputs.attention_operands(s, hq, s, hkv, d, seed_q=world * 10 + hq)
    scale = 1 / math.sqrt(d)
    o_full, lse_full = oracle.attention_f64(q, k, v, scale)
    outs = [oracle.head_parallel_attention_f64(q, k, v, world, r, scale) for r in range(world)]
    o = np.concatenate([x[0] for x in outs], axis=1)
    lse = np.concatenate([x[1] for x in outs], axis=0)
    assert o.shape == o_full.shape and lse.shape == lse_full.shape
    assert np.allclose(o, o_full, rtol=0, atol=1e-12)
    assert np.allclose(lse, lse_full, rtol=0, atol=1e-12)


def test_rejects_uneven_head_groups():
    q, k, v = inputs.attention_operands(4, 6, 4, 3, 8)
    with pytest.raises(ValueError):
        oracle.head_parallel_attention_f64(q, k, v, 4, 0, 0.5)
    with pytest.raises(ValueError):
        oracle.head_parallel_attention_f64(q, k, v, 2, 0, 0.5)   # 3 KV heads over 2 ranks
