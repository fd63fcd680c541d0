"""Head-parallel attention share on the GPU, through the C ABI, against the oracle.

The share is the all-to-all receive side (every peer's token block of this
rank's head group: Q, K and V) fused with attention over all world*n tokens
(Syncopate summary page, "Experiments", paper sec. 6.1 and Fig. 9;
DeepSpeed-Ulysses' scheme).  The result must equal direct attention on the
rank's head group of the full tensors (oracle.head_parallel_attention_f64).
Bar: max |O - O_ref| <= 2e-3 and max |LSE - LSE_ref| <= 2e-3 (a query block
read before its chunk landed reads NaN poison; a dropped KV block moves LSE by
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


def query_block(hq, hkv):
    """The kernel's query rows per work item (the plan's tile_m)."""
    return A.sync_attn_query_block(hq, hkv)


def run_head(world, n, rank, qg, kg, vg, split=1, backend=A.SYNC_COPY_CU, cus=16,
             order=A.SYNC_ORDER_CHUNK_MAJOR, scale=1 / math.sqrt(D), teams=0, streaming=0, pattern=A.SYNC_PAT_RING,
             hier_group=0, explicit_order=None, flags=0, withhold_chunk=-1, timeout_ns=0, want_lse=True):
    """qg [world*n][hq][D], kg and vg [world*n][hkv][D]: what the peers send
    this rank (its head group of every token, block w from peer w)."""
    s, hq, hkv = world * n, qg.shape[1], kg.shape[1]
    print(f"[head] W={world} n={n} hq={hq} hkv={hkv} rank={rank} split={split} backend={backend} cus={cus} "
          f"order={order} pattern={pattern} teams={teams} flags={flags}", flush=True)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_HEAD_ATTN, s, n, D, world, rank=rank, split=split,
                                   tile_m=query_block(hq, hkv), tile_n=1, tile_order=order, heads_q=hq,
                                   heads_kv=hkv, pattern=pattern, hier_group=hier_group,
                                   explicit_order=explicit_order))
    tabs = A.sync_plan_export(plan)
    peers = [dev_bits(x) for x in (qg, kg, vg)]
    if backend == A.SYNC_COPY_PRESET:
        local = [p.clone() for p in peers]
    else:
        local = [bf16_poison(p.shape) for p in peers]
        for c in range(tabs["num_chunks"]):
            if tabs["resident"][c]:
                r0, r1 = tabs["chunk_begin"][c], tabs["chunk_begin"][c + 1]
                for dst, src in zip(local, peers):
                    dst[r0:r1] = src[r0:r1]
    o = torch.full((s, hq, D), float("nan"), dtype=torch.float32, device="cuda:0")
    lse = torch.full((hq, s), float("nan"), dtype=torch.float32, device="cuda:0") if want_lse else None
    ws = workspace(plan)
    st = torch.cuda.current_stream()
    cfg = A.make_cfg(backend, copy_cus=cus, copy_streaming=streaming, copy_teams=teams, flags=flags,
                     withhold_chunk=withhold_chunk, timeout_ns=timeout_ns)
    A.sync_head_attn(plan, cfg, *peers, *local, o, lse, scale, ws, st, None)
    rc, chunk = A.sync_workspace_status(ws, st)
    torch.cuda.synchronize()
    return rc, chunk, o, lse, peers, local


def reference(q, k, v, world, rank, scale=1 / math.sqrt(D)):
    return oracle.head_parallel_attention_f64(q, k, v, world, rank, scale)


def group(x, world, rank):
    """The rank's head group of a [S][H][D] tensor (the test's own slicing)."""
    h = x.shape[1] // world
    return np.ascontiguousarray(x[:, rank * h:(rank + 1) * h])


def grouped(q, k, v, world, rank):
    return [group(x, world, rank) for x in (q, k, v)]


def check(o, lse, ref_o, ref_lse):
    o = o.cpu().numpy()
    assert np.isfinite(o).all()
    eo = np.max(np.abs(o - ref_o))
    el = 0.0
    if lse is not None:
        lse = lse.cpu().numpy()
        assert np.isfinite(lse).all()
        el = np.max(np.abs(lse - ref_lse))
    assert eo <= TOL and el <= TOL, (eo, el)
    return eo, el


# heads of the whole layer (query, KV), split over 4 ranks: per rank 8/2, 4/4, 4/2 and 16/1
@pytest.mark.parametrize("hq_all,hkv_all", [(32, 8), (16, 16), (16, 8), (64, 4)])
@pytest.mark.parametrize("backend,cus", [(A.SYNC_COPY_PRESET, 0), (A.SYNC_COPY_CU, 8), (A.SYNC_COPY_COLOCATED, 0),
                                         (A.SYNC_COPY_SDMA, 0)])
def test_small_heads_and_backends(hq_all, hkv_all, backend, cus):
    W, n, rank = 4, 128, 1
    q, k, v = inputs.attention_operands(W * n, hq_all, W * n, hkv_all, D)
    ref_o, ref_lse = reference(q, k, v, W, rank)
    rc, _, o, lse, _, _ = run_head(W, n, rank, *grouped(q, k, v, W, rank), backend=backend, cus=cus)
    assert rc == A.SYNC_OK
    check(o, lse, ref_o, ref_lse)


@pytest.mark.parametrize("W,n,split,order", [(2, 100, 3, A.SYNC_ORDER_CHUNK_MAJOR), (3, 257, 2, A.SYNC_ORDER_SWIZZLED),
                                             (4, 33, 1, A.SYNC_ORDER_ROW_MAJOR), (2, 1, 1, A.SYNC_ORDER_CHUNK_MAJOR)])
def test_ragged_query_blocks_straddle_chunks(W, n, split, order):
    """Token blocks that are not multiples of the 64-row query block: work
    items wait for two chunks (and a last, partial block); single-token
    blocks."""
    hq, hkv = 4, 1
    q, k, v = inputs.attention_operands(W * n, W * hq, W * n, W * hkv, D)
    ref_o, ref_lse = reference(q, k, v, W, W - 1, 0.1)
    rc, _, o, lse, _, _ = run_head(W, n, W - 1, *grouped(q, k, v, W, W - 1), split=split, order=order, scale=0.1,
                                   cus=8)
    assert rc == A.SYNC_OK
    check(o, lse, ref_o, ref_lse)


@pytest.mark.parametrize("pattern,extra", [(A.SYNC_PAT_HIER_SWIZZLE, dict(hier_group=2)),
                                           (A.SYNC_PAT_MESH, {}),
                                           (A.SYNC_PAT_EXPLICIT, dict(explicit_order=[2, 0, 3, 1]))])
def test_arrival_patterns(pattern, extra):
    W, n, rank, hq, hkv = 4, 96, 2, 8, 2
    q, k, v = inputs.attention_operands(W * n, W * hq, W * n, W * hkv, D)
    ref_o, ref_lse = reference(q, k, v, W, rank)
    rc, _, o, lse, _, _ = run_head(W, n, rank, *grouped(q, k, v, W, rank), split=2, pattern=pattern, cus=8, teams=3,
                                   **extra)
    assert rc == A.SYNC_OK
    check(o, lse, ref_o, ref_lse)


def test_lse_optional_and_store_policy():
    W, n, rank, hq, hkv = 2, 192, 0, 8, 1
    q, k, v = inputs.attention_operands(W * n, W * hq, W * n, W * hkv, D)
    ref_o, _ = reference(q, k, v, W, rank)
    rc, _, o, _, _, _ = run_head(W, n, rank, *grouped(q, k, v, W, rank), want_lse=False, streaming=1, cus=8)
    assert rc == A.SYNC_OK
    check(o, None, ref_o, None)


def test_copy_only_stages_every_chunk():
    """COPY_ONLY: the copy agent alone; q, k and v end up equal to what the
    peers sent, bit for bit, and nothing is computed."""
    W, n, rank, hq, hkv = 4, 64, 3, 4, 1
    q, k, v = inputs.attention_operands(W * n, W * hq, W * n, W * hkv, D)
    rc, _, o, _, peers, local = run_head(W, n, rank, *grouped(q, k, v, W, rank), flags=A.SYNC_RUN_COPY_ONLY, cus=8)
    assert rc == A.SYNC_OK
    for p, l in zip(peers, local):
        assert torch.equal(p, l)
    assert torch.isnan(o).all()


def test_withheld_chunk_times_out_and_leaves_outputs():
    """A chunk the copy agent leaves out (forced from the host): every work
    item needs every KV block, so none is written, and the bounded wait
    reports the chunk."""
    W, n, rank, hq, hkv = 4, 64, 0, 4, 1
    q, k, v = inputs.attention_operands(W * n, W * hq, W * n, W * hkv, D)
    rc, chunk, o, lse, _, _ = run_head(W, n, rank, *grouped(q, k, v, W, rank), cus=8, flags=A.SYNC_RUN_WITHHOLD,
                                       withhold_chunk=2, timeout_ns=2_000_000)
    assert rc == A.SYNC_ETIMEOUT and chunk == 2
    assert torch.isnan(o).all() and torch.isnan(lse).all()


# ---- Llama-3-8B-like attention, 8 ranks x 4096 tokens: one rank's 4 query / 1 KV heads over 32768 tokens ----
@pytest.mark.parametrize("backend,cus,teams", [(A.SYNC_COPY_CU, 32, 7), (A.SYNC_COPY_COLOCATED, 0, 0),
                                               (A.SYNC_COPY_SDMA, 0, 7)])
def test_full_size_sampled(backend, cus, teams):
    W, n, rank, hq, hkv = 8, 4096, 3, 4, 1
    s = W * n
    # only this rank's head group is drawn: the other ranks' heads do not enter its share
    q, k, v = inputs.attention_operands(s, hq, s, hkv, D)
    rc, _, o, lse, _, _ = run_head(W, n, rank, q, k, v, backend=backend, cus=cus, teams=teams)
    assert rc == A.SYNC_OK
    rng = np.random.default_rng(11)
    qi = np.concatenate([rng.integers(0, s, 600), [0, n - 1, n, s - 1]])
    hi = np.concatenate([rng.integers(0, hq, 600), [0, hq - 1, 1, hq - 1]])
    ref_o, ref_lse = oracle.attention_f64_sampled(q, k, v, 1 / math.sqrt(D), qi, hi)
    on, ln_ = o.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(on).all() and np.isfinite(ln_).all()
    assert np.max(np.abs(on[qi, hi] - ref_o)) <= TOL
    assert np.max(np.abs(ln_[hi, qi] - ref_lse)) <= TOL


def test_captured_call_replays():
    """A CU-backend head-parallel call is one kernel launch that takes its
    epoch from the workspace, so a captured call can be replayed: each replay
    (with eager work and synchronisation between replays, and different peer
    data) equals the eager result for that data, bit for bit."""
    W, n, rank, hq, hkv = 4, 128, 1, 8, 2
    s_tok = W * n
    datasets = [inputs.attention_operands(s_tok, hq, s_tok, hkv, D, seed_q=inputs.SEED_Q + 11 * x,
                                          seed_k=inputs.SEED_K + 11 * x, seed_v=inputs.SEED_V + 11 * x)
                for x in range(3)]
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_HEAD_ATTN, s_tok, n, D, W, rank=rank, split=2,
                                   tile_m=query_block(hq, hkv), tile_n=1, heads_q=hq, heads_kv=hkv))
    tabs = A.sync_plan_export(plan)
    cfg = A.make_cfg(A.SYNC_COPY_CU, copy_cus=16, copy_teams=3)
    peers = [dev_bits(x) for x in datasets[0]]
    local = [torch.zeros_like(p) for p in peers]
    o = torch.empty((s_tok, hq, D), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((hq, s_tok), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    st = torch.cuda.current_stream()
    scale = 1 / math.sqrt(D)

    def load(x):
        for p, l, src in zip(peers, local, datasets[x]):
            p.copy_(dev_bits(src))
            l.fill_(0x7FC0)  # bf16 NaN: every non-resident row must be staged again
            for c in range(tabs["num_chunks"]):
                if tabs["resident"][c]:
                    r0, r1 = tabs["chunk_begin"][c], tabs["chunk_begin"][c + 1]
                    l[r0:r1] = p[r0:r1]

    eager = []
    for x in range(3):
        load(x)
        A.sync_head_attn(plan, cfg, *peers, *local, o, lse, scale, ws, st, None)
        assert A.sync_workspace_status(ws, st)[0] == A.SYNC_OK
        eager.append((o.clone(), lse.clone()))
        ref_o, ref_lse = oracle.attention_f64(*datasets[x], scale)
        check(o, lse, ref_o, ref_lse)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(st)
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            A.sync_head_attn(plan, cfg, *peers, *local, o, lse, scale, ws, side, None)
    st.wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(6):
        x = rep % 3
        print(f"[head] graph replay {rep} dataset {x}", flush=True)
        load(x)
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert A.sync_workspace_status(ws, st)[0] == A.SYNC_OK
        assert torch.equal(o, eager[x][0]) and torch.equal(lse, eager[x][1]), f"replay {rep} differs"
