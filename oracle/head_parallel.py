"""ORACLE -- head-parallel attention share.  Test infrastructure only: nothing
on the product path imports it; only the tests, the smoke check and the
bench's CPU baseline leg do.

What the pages fix: the Syncopate summary page, "Experiments" (paper sec. 6.1
and Fig. 9), lists head-parallel and sequence-parallel attention among the
operators it evaluates on Llama-3 and Qwen attention shapes; the review page's
reference list names DeepSpeed-Ulysses.  Neither page spells out the scheme.

Reading (the Ulysses scheme, the plainest one the pages support): before
attention, rank w holds a sequence shard, the n tokens [w*n, (w+1)*n) of every
head.  An all-to-all turns sequence shards into head shards: rank r receives
from every peer w the n tokens of w's shard restricted to r's head group, so
afterwards it holds all world*n tokens of heads [r*H/W, (r+1)*H/W) (query
heads and KV heads each split into world equal groups, so a query head's KV
head stays on the same rank).  Attention per head needs nothing from other
heads, so each rank's share is plain softmax attention over every token of its
head group; concatenating the ranks' outputs over heads gives the whole
layer's attention.

Functions:
  head_group(x, world, rank)        what the all-to-all delivers to `rank`
  head_parallel_attention_f64(...)  the share's result: direct attention
                                    (attn_ref.c) on the delivered tensors
"""
from __future__ import annotations

import numpy as np


def head_group(x, world: int, rank: int):
    """Rank `rank`'s head group of a [S][H][d] tensor: heads
    [rank*H/world, (rank+1)*H/world) of every token, as a contiguous array."""
    x = np.asarray(x)
    s, h, d = x.shape
    if world < 1 or not (0 <= rank < world) or h % world:
        raise ValueError("heads must split evenly over world ranks")
    g = h // world
    return np.ascontiguousarray(x[:, rank * g:(rank + 1) * g, :])


def head_parallel_attention_f64(q_bits, k_bits, v_bits, world: int, rank: int, scale: float, threads=None):
    """The head-parallel share of rank `rank` in fp64: Q [S][Hq][d] and K, V
    [S][Hkv][d] (bf16 bits, all S = world*n tokens, all heads) -> (O
    [S][Hq/world][d], LSE [Hq/world][S]) for the rank's head group."""
    from . import attention_f64
    if np.asarray(k_bits).shape[1] % world:
        raise ValueError("KV heads must split evenly over world ranks")
    return attention_f64(head_group(q_bits, world, rank), head_group(k_bits, world, rank),
                         head_group(v_bits, world, rank), scale, threads=threads)
