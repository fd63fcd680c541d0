"""Pins for the attention oracle (oracle/attn_ref.c direct form and
oracle/attention.py online merge).

Ring attention's local step must equal plain softmax attention over all keys
(Syncopate summary page, "Experiments", paper sec. 6.1 and Fig. 9).  Pins:
a hand-worked two-key example (tests/golden/attention_tiny.json), closed forms
(Q = 0, one key, identical keys), PyTorch's fp64 CPU scaled_dot_product_attention,
and the online merge equal to the direct form for several arrival orders.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from communication_overlap_gemm_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_hand_worked_two_keys():
    g = json.load(open(os.path.join(GOLD, "attention_tiny.json")))
    o, lse = oracle.attention_f64(_bits(g["q"]), _bits(g["k"]), _bits(g["v"]), g["scale"])
    assert np.allclose(o, np.array(g["o"]), atol=g["tol"], rtol=0)
    assert np.allclose(lse, np.array(g["lse"]), atol=g["tol"], rtol=0)


def test_zero_queries_give_mean_of_values():
    sq, hq, hkv, d, skv = 3, 4, 2, 8, 11
    q = np.zeros((sq, hq, d), dtype=np.uint16)
    _, k, v = inputs.attention_operands(sq, hq, skv, hkv, d)
    o, lse = oracle.attention_f64(q, k, v, 1 / math.sqrt(d))
    vf = inputs.bf16_bits_to_f32(v).astype(np.float64)
    for h in range(hq):
        assert np.allclose(o[:, h, :], vf[:, h // 2, :].mean(axis=0), atol=1e-14)
    assert np.allclose(lse, math.log(skv), atol=1e-14)


def test_single_key_returns_its_value():
    q, k, v = inputs.attention_operands(5, 2, 1, 1, 16)
    o, lse = oracle.attention_f64(q, k, v, 0.25)
    vf = inputs.bf16_bits_to_f32(v).astype(np.float64)
    assert np.array_equal(o, np.broadcast_to(vf[0, 0], o.shape))
    qf = inputs.bf16_bits_to_f32(q).astype(np.float64)
    kf = inputs.bf16_bits_to_f32(k).astype(np.float64)
    assert np.allclose(lse, (qf[:, :, :] @ kf[0, 0]).T * 0.25, atol=1e-13)


def test_identical_keys_uniform():
    sq, hq, d, skv = 2, 2, 8, 9
    q, k, v = inputs.attention_operands(sq, hq, skv, hq, d)
    k = np.broadcast_to(k[:1], k.shape).copy()
    o, _ = oracle.attention_f64(q, k, v, 0.3)
    vf = inputs.bf16_bits_to_f32(v).astype(np.float64)
    assert np.allclose(o, np.transpose(vf.mean(axis=0, keepdims=True), (0, 1, 2)), atol=1e-13)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_against_torch_sdpa_fp64(hq, hkv):
    sq, skv, d = 13, 27, 16
    q, k, v = inputs.attention_operands(sq, hq, skv, hkv, d)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention_f64(q, k, v, scale)
    tq = torch.from_numpy(inputs.bf16_bits_to_f32(q).astype(np.float64)).permute(1, 0, 2)
    tk = torch.from_numpy(inputs.bf16_bits_to_f32(k).astype(np.float64)).permute(1, 0, 2)
    tv = torch.from_numpy(inputs.bf16_bits_to_f32(v).astype(np.float64)).permute(1, 0, 2)
    tk = tk.repeat_interleave(hq // hkv, dim=0)
    tv = tv.repeat_interleave(hq // hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
    ref_lse = torch.logsumexp(tq @ tk.transpose(1, 2) * scale, dim=-1)
    assert np.allclose(lse, ref_lse.numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("arrival", [[0, 1, 2, 3], [0, 3, 2, 1], [2, 0, 3, 1]])
def test_online_merge_equals_direct(arrival):
    sq, hq, hkv, d, n = 6, 4, 2, 8, 5
    q, k, v = inputs.attention_operands(sq, hq, 4 * n, hkv, d)
    blocks = [(c * n, (c + 1) * n) for c in range(4)]
    o1, lse1, _, _ = oracle.attention_online_f64(q, k, v, 0.35, blocks, arrival)
    o2, lse2 = oracle.attention_f64(q, k, v, 0.35)
    assert np.allclose(o1, o2, atol=1e-13, rtol=0)
    assert np.allclose(lse1, lse2, atol=1e-13, rtol=0)


def test_sampled_matches_full():
    q, k, v = inputs.attention_operands(7, 4, 10, 2, 8)
    o, lse = oracle.attention_f64(q, k, v, 0.4)
    qi = np.array([0, 6, 3, 3])
    hi = np.array([0, 3, 1, 2])
    os_, ls = oracle.attention_f64_sampled(q, k, v, 0.4, qi, hi)
    assert np.array_equal(os_, o[qi, hi])
    assert np.array_equal(ls, lse[hi, qi])
