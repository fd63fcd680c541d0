"""Ring-attention local step on the GPU, through the C ABI, against the oracle.

The step folds every KV block, in arrival order, into an fp32 online-softmax
state; the result must equal plain softmax attention over all keys (the ring
passes every block to every rank: Syncopate summary page, "Experiments",
paper sec. 6.1, Fig. 9).  Bar: max |O - O_ref| <= 2e-3 and
max |LSE - LSE_ref| <= 2e-3 (a dropped or doubled block moves LSE by
about ln(8/7) ~ 0.13 at 8 blocks).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

from gpu_util import bf16_poison, dev_bits, workspace

pytestmark = pytest.mark.gpu
D = 128
TOL = 2e-3


def run_attn(sq, hq, hkv, world, n, q_bits, k_bits, v_bits, split=1, backend=A.SYNC_COPY_CU, cus=16,
             flags=A.SYNC_ATTN_INIT | A.SYNC_ATTN_FINALIZE, scale=1 / math.sqrt(D), rank=0, state=None, streaming=0,
             teams=0):
    print(f"[attn] sq={sq} hq={hq} hkv={hkv} W={world} n={n} split={split} backend={backend} cus={cus} "
          f"flags={flags} streaming={streaming}", flush=True)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_RING_ATTN, sq, n, D, world, rank=rank, split=split, tile_m=128,
                                   tile_n=1, heads_q=hq, heads_kv=hkv))
    tabs = A.sync_plan_export(plan)
    q = dev_bits(q_bits)
    k_peer, v_peer = dev_bits(k_bits), dev_bits(v_bits)
    if backend == A.SYNC_COPY_PRESET:
        k_local, v_local = k_peer.clone(), v_peer.clone()
    else:
        k_local, v_local = bf16_poison(k_peer.shape), bf16_poison(v_peer.shape)
        for c in range(tabs["num_chunks"]):
            if tabs["resident"][c]:
                r0, r1 = tabs["chunk_begin"][c], tabs["chunk_begin"][c + 1]
                k_local[r0:r1] = k_peer[r0:r1]
                v_local[r0:r1] = v_peer[r0:r1]
    if state is None:
        o = torch.full((sq, hq, D), float("nan"), dtype=torch.float32, device="cuda:0")
        m = torch.full((hq, sq), float("nan"), dtype=torch.float32, device="cuda:0")
        l = torch.full((hq, sq), float("nan"), dtype=torch.float32, device="cuda:0")
    else:
        o, m, l = state
    lse = torch.full((hq, sq), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    cfg = A.make_cfg(backend, copy_cus=cus, copy_streaming=streaming, copy_teams=teams)
    A.sync_ring_attn_step(plan, cfg, q, k_peer, v_peer, k_local, v_local, o, m, l,
                          lse, scale, flags, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    torch.cuda.synchronize()
    return o, m, l, lse


def check(o, lse, ref_o, ref_lse):
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    eo, el = np.max(np.abs(o - ref_o)), np.max(np.abs(lse - ref_lse))
    assert eo <= TOL and el <= TOL, (eo, el)
    return eo, el


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (8, 4), (16, 2)])
@pytest.mark.parametrize("backend,cus", [(A.SYNC_COPY_PRESET, 0), (A.SYNC_COPY_CU, 8), (A.SYNC_COPY_COLOCATED, 0),
                                         (A.SYNC_COPY_SDMA, 0)])
def test_small_heads_and_backends(hq, hkv, backend, cus):
    sq, W, n = 256, 4, 128
    q, k, v = inputs.attention_operands(sq, hq, W * n, hkv, D)
    ref_o, ref_lse = oracle.attention_f64(q, k, v, 1 / math.sqrt(D))
    o, _, _, lse = run_attn(sq, hq, hkv, W, n, q, k, v, backend=backend, cus=cus, rank=1)
    check(o, lse, ref_o, ref_lse)


@pytest.mark.parametrize("sq,n,split,W", [(200, 100, 3, 2), (33, 64, 2, 3), (96, 257, 1, 2)])
def test_ragged(sq, n, split, W):
    hq, hkv = 8, 2
    q, k, v = inputs.attention_operands(sq, hq, W * n, hkv, D)
    ref_o, ref_lse = oracle.attention_f64(q, k, v, 0.1)
    o, _, _, lse = run_attn(sq, hq, hkv, W, n, q, k, v, split=split, scale=0.1, rank=W - 1)
    check(o, lse, ref_o, ref_lse)


def test_zero_queries_closed_form():
    sq, hq, hkv, W, n = 64, 4, 1, 4, 64
    _, k, v = inputs.attention_operands(sq, hq, W * n, hkv, D)
    q = np.zeros((sq, hq, D), dtype=np.uint16)
    o, _, _, lse = run_attn(sq, hq, hkv, W, n, q, k, v)
    vf = inputs.bf16_bits_to_f32(v).astype(np.float64)
    want = np.broadcast_to(vf[:, 0, :].mean(axis=0), (sq, hq, D))
    check(o, lse, want, np.full((hq, sq), math.log(W * n)))


def test_chained_steps_carry_state():
    """Two calls over disjoint KV halves, INIT then FINALIZE, equal one pass over all keys."""
    sq, hq, hkv, n = 128, 8, 2, 192
    q, k, v = inputs.attention_operands(sq, hq, 4 * n, hkv, D)
    ref_o, ref_lse = oracle.attention_f64(q, k, v, 1 / math.sqrt(D))
    half = 2 * n
    o, m, l, _ = run_attn(sq, hq, hkv, 2, n, q, k[:half], v[:half], flags=A.SYNC_ATTN_INIT)
    o2, _, _, lse = run_attn(sq, hq, hkv, 2, n, q, k[half:], v[half:], flags=A.SYNC_ATTN_FINALIZE, state=(o, m, l))
    check(o2, lse, ref_o, ref_lse)


# ---- Qwen-like GQA ring step: Q 4096 x 32 x 128, 8 KV blocks of 4096 x 8 x 128 ----
@pytest.mark.parametrize("backend,cus,teams", [(A.SYNC_COPY_CU, 32, 0), (A.SYNC_COPY_SDMA, 0, 7)])
def test_full_size_sampled(backend, cus, teams):
    sq, hq, hkv, W, n = 4096, 32, 8, 8, 4096
    q, k, v = inputs.attention_operands(sq, hq, W * n, hkv, D)
    o, _, _, lse = run_attn(sq, hq, hkv, W, n, q, k, v, backend=backend, cus=cus, teams=teams)
    rng = np.random.default_rng(5)
    qi = np.concatenate([rng.integers(0, sq, 600), [0, sq - 1]])
    hi = np.concatenate([rng.integers(0, hq, 600), [0, hq - 1]])
    ref_o, ref_lse = oracle.attention_f64_sampled(q, k, v, 1 / math.sqrt(D), qi, hi)
    on, ln_ = o.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(on).all()
    assert np.max(np.abs(on[qi, hi] - ref_o)) <= TOL
    assert np.max(np.abs(ln_[hi, qi] - ref_lse)) <= TOL


@pytest.mark.parametrize("streaming", [1])
@pytest.mark.parametrize("backend,cus", [(A.SYNC_COPY_CU, 8), (A.SYNC_COPY_COLOCATED, 0)])
def test_copy_store_policies(streaming, backend, cus):
    """K and V staged with non-temporal loads and stores: within the
    attention bar of the oracle."""
    sq, hq, hkv, W, n = 256, 8, 2, 4, 128
    q, kk, vv = inputs.attention_operands(sq, hq, W * n, hkv, D)
    ref_o, ref_lse = oracle.attention_f64(q, kk, vv, 1 / math.sqrt(D))
    o, _, _, lse = run_attn(sq, hq, hkv, W, n, q, kk, vv, backend=backend, cus=cus, streaming=streaming)
    check(o, lse, ref_o, ref_lse)
