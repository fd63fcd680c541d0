"""ORACLE -- blockwise online-softmax merge, fp64.  Test infrastructure only.

The ring-attention step (Syncopate summary page, "Experiments", paper sec. 6.1
and Fig. 9: ring attention, with KV blocks passed between ranks) folds each
arriving KV block into a running state (m, l, O) per (query, head):
    m' = max(m, max_j s_j)
    l' = l * exp(m - m') + sum_j exp(s_j - m')
    O' = O * exp(m - m') + sum_j exp(s_j - m') V_j
and at the end O / l is the attention output and m + ln l its log-sum-exp.
This file writes that merge out in fp64 over blocks in a given arrival order,
so the tests can check that it equals the direct form in attn_ref.c (it is a
re-association of the same sums).  Pure numpy; for small shapes only.
"""
from __future__ import annotations

import numpy as np


def _widen(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def attention_online_f64(q_bits, k_bits, v_bits, scale, block_rows, arrival):
    """Q [Sq,Hq,d], K/V [Skv,Hkv,d] bf16 bits.  block_rows[c] = (begin, end) token
    range of KV chunk c; arrival = chunk ids in the order they are merged.
    Returns (O [Sq,Hq,d], LSE [Hq,Sq], m [Hq,Sq], l [Hq,Sq])."""
    q, k, v = _widen(q_bits), _widen(k_bits), _widen(v_bits)
    sq, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    m = np.full((hq, sq), -np.inf)
    l = np.zeros((hq, sq))
    o = np.zeros((hq, sq, d))
    for c in arrival:
        b, e = block_rows[c]
        for h in range(hq):
            g = h // grp
            s = (q[:, h, :] @ k[b:e, g, :].T) * scale            # [sq, e-b]
            m_new = np.maximum(m[h], s.max(axis=1))
            alpha = np.exp(m[h] - m_new)
            p = np.exp(s - m_new[:, None])
            l[h] = l[h] * alpha + p.sum(axis=1)
            o[h] = o[h] * alpha[:, None] + p @ v[b:e, g, :]
            m[h] = m_new
    out = np.transpose(o / l[:, :, None], (1, 0, 2)).copy()
    return out, m + np.log(l), m, l
