"""Arrival and send patterns on the GPU: explicit pull orders, the reverse ring
direction, a single rank, the hierarchical swizzle and the mesh, for AG-GEMM (copy CUs with K-slices, SDMA,
co-located), GEMM-RS (epilogue backend and copy-out) and the GEMM-AR share.

The plan fixes when each chunk arrives or leaves (Syncopate summary page,
"Core method", paper sec. 5.2, Fig. 6: chunks are visited in communication
order); whatever the order, the product must be exact (small-integer
operands), every copied row staged, and the send slots in the oracle
planner's order.
"""
import numpy as np
import pytest
import torch

import oracle
from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

from gpu_util import bf16_poison, dev_bits, host_bits, workspace

pytestmark = pytest.mark.gpu

PATTERNS = [  # (world, rank, ring_dir, order): an explicit order, None (ring), ("hier", g) or ("mesh",)
    (4, 2, 1, [2, 0, 3, 1]),   # explicit: own shard first, then a scattered pull order
    (4, 1, 1, [3, 2, 1, 0]),   # explicit: own shard in the middle of the order
    (4, 1, -1, None),          # ring towards rank - 1
    (1, 0, 1, None),           # one rank: nothing to copy or send
    (8, 5, 1, ("hier", 4)),    # hierarchical swizzle: two groups of four
    (8, 2, 1, ("hier", 2)),    # hierarchical swizzle: four groups of two
    (8, 3, -1, ("mesh",)),     # every peer's link at once, sub-chunks interleaved
]


def _pattern(order):
    """(pattern, explicit order, hier_group) of a PATTERNS entry."""
    if order is None:
        return A.SYNC_PAT_RING, None, 0
    if isinstance(order, tuple):
        return (A.SYNC_PAT_HIER_SWIZZLE, None, order[1]) if order[0] == "hier" else (A.SYNC_PAT_MESH, None, 0)
    return A.SYNC_PAT_EXPLICIT, order, 0


def _desc(op, m, n, k, world, rank, d, order, **kw):
    pat, explicit, g = _pattern(order)
    return A.make_desc(op, m, n, k, world, rank=rank, ring_dir=d, pattern=pat, explicit_order=explicit,
                       hier_group=g, b_layout=A.SYNC_B_NK, **kw)


def _ref_plan(op, m, n, k, world, rank, d, order, split=1, tile=(256, 256)):
    pat, explicit, g = _pattern(order)
    return oracle.plan_ref(oracle.PlanDesc(op=op, m=m, n=n, k=k, world=world, rank=rank, ring_dir=d, pattern=pat,
                                           explicit_order=explicit, hier_group=g, split=split, tile_m=tile[0],
                                           tile_n=tile[1]))


@pytest.mark.parametrize("world,rank,d,order", PATTERNS)
@pytest.mark.parametrize("backend,cus,teams,kslices", [(A.SYNC_COPY_CU, 16, 3, 4), (A.SYNC_COPY_SDMA, 0, 2, 0),
                                                       (A.SYNC_COPY_COLOCATED, 0, 0, 0)])
def test_ag_patterns(world, rank, d, order, backend, cus, teams, kslices):
    m, n, k, split = 2048, 768, 1024, 2
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, rank, d, order, split=split, tile_m=256,
                             tile_n=256))
    tabs = A.sync_plan_export(plan)
    ptab = _ref_plan(oracle.OP_AG_GEMM, m, n, k, world, rank, d, order, split)
    assert list(tabs["arrival"]) == list(ptab.arrival) and list(tabs["resident"]) == list(ptab.resident)
    assert list(tabs["tile_order"]) == list(ptab.tile_order)
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = bf16_poison((m, k))
    for c in range(tabs["num_chunks"]):
        if tabs["resident"][c]:
            r0, r1 = tabs["chunk_begin"][c], tabs["chunk_begin"][c + 1]
            a_local[r0:r1] = a_peer[r0:r1]
    c_out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[pattern ag] W={world} r={rank} d={d} order={order} backend={backend}", flush=True)
    A.sync_ag_gemm(plan, A.make_cfg(backend, copy_cus=cus, copy_teams=min(teams, max(1, world * split - split)),
                                    copy_kslices=kslices), a_peer, a_local, b_d, c_out, A.SYNC_DTYPE_F32, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    assert np.array_equal(host_bits(a_local), a)
    assert np.array_equal(c_out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("world,rank,d,order", PATTERNS)
@pytest.mark.parametrize("backend,cus", [(A.SYNC_COPY_EPILOGUE, 0), (A.SYNC_COPY_CU, 16)])
def test_rs_patterns(world, rank, d, order, backend, cus):
    """Send slots in the oracle planner's send order for every pattern."""
    m, n, k = 2048, 768, 512
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    r = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(_desc(A.SYNC_OP_GEMM_RS, m, n, k, world, rank, d, order, tile_m=256, tile_n=256))
    ptab = _ref_plan(oracle.OP_GEMM_RS, m, n, k, world, rank, d, order)
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    st = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[pattern rs] W={world} r={rank} d={d} order={order} backend={backend}", flush=True)
    A.sync_gemm_rs(plan, A.make_cfg(backend, copy_cus=cus), dev_bits(a), dev_bits(b), c, A.SYNC_DTYPE_F32, st, ws, s,
                   None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    assert np.array_equal(c.cpu().numpy().astype(np.float64), r)
    _, want = oracle.rs_staging_expected(r, ptab)
    assert np.array_equal(st.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("world,rank,d,order", PATTERNS)
def test_ar_patterns(world, rank, d, order):
    """GEMM-AR share for every pattern: the all-gather follows the ring order of
    the descriptor's direction; the output is order-independent."""
    m, n, k = 2048, 768, 512
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    p = inputs.partials_f32(m, n, integer=True)
    peer = inputs.partials_f32(m, n, seed=inputs.SEED_P + inputs.ALT_SEED_OFFSET, integer=True)
    r = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(_desc(A.SYNC_OP_GEMM_RS, m, n, k, world, rank, d, order, tile_m=256, tile_n=256))
    ptab = _ref_plan(oracle.OP_GEMM_RS, m, n, k, world, rank, d, order)
    c, st, out = (torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0") for _ in range(3))
    pd, peer_d = torch.from_numpy(p).to("cuda:0"), torch.from_numpy(peer).to("cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[pattern ar] W={world} r={rank} d={d} order={order}", flush=True)
    A.sync_gemm_ar(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE, 8), dev_bits(a), dev_bits(b), c, pd, peer_d, out, st, ws,
                   s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    _, want_st = oracle.rs_reduce_staging_expected(r, p, ptab)
    assert np.array_equal(st.cpu().numpy().astype(np.float64), want_st)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), oracle.ar_share_expected(r, p, peer, ptab, world, rank))
