"""GEMM-RS share on the GPU, through the C ABI, against the oracle.

The GEMM visits tiles in send order; each stored tile counts toward the
chunks of C it wrote, the last one raises the chunk's done flag, and the copy
agent on dedicated CUs copies each finished chunk, in send order, into its
staging slot (Syncopate summary page, "Experiments": GEMM-RS; Entwine
abstract: reordered tiles feeding fine-grained SM-based communication).
Checks: C within the fp32 parity bar; staging slot p bitwise equal to the rows
of chunk arrival[p] of C (it is a copy); every done and sent flag holds the
call's epoch; every per-chunk counter is back at zero (the tile that
completes a chunk clears its counter for the next call) and so are the
header's exit counter and copy census.
"""
import numpy as np
import pytest
import torch

import oracle
from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

from gpu_util import bf16_poison, check_full_f32, dev_bits, host_bits, shard_frobenius, workspace

pytestmark = pytest.mark.gpu


def ws_arrays(ws, num_chunks):
    w = ws.cpu().numpy().view(np.uint32)
    a = -(-4 * num_chunks // 256) * 256 // 4
    hdr, rest = w[:64], w[64:]
    return hdr, rest[:num_chunks], rest[a:a + num_chunks], rest[2 * a:2 * a + num_chunks], rest[3 * a:3 * a + num_chunks]


def run_rs(m, n, k, world, a_bits, b_bits, split=1, tile=(128, 128), order=A.SYNC_ORDER_CHUNK_MAJOR,
           backend=A.SYNC_COPY_CU, copy_cus=16, c_dtype=A.SYNC_DTYPE_F32, rank=0, layout=A.SYNC_B_KN, teams=0,
           streaming=0):
    print(f"[rs] m={m} n={n} k={k} W={world} split={split} tile={tile} order={order} backend={backend} "
          f"cus={copy_cus} dtype={c_dtype} teams={teams} streaming={streaming}", flush=True)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, world, rank=rank, split=split, tile_m=tile[0],
                                   tile_n=tile[1], tile_order=order, b_layout=layout))
    tabs = A.sync_plan_export(plan)
    a = dev_bits(a_bits)
    b = dev_bits(b_bits)
    if c_dtype == A.SYNC_DTYPE_F32:
        c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
        staging = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    else:
        c = bf16_poison((m, n))
        staging = bf16_poison((m, n))
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    A.sync_gemm_rs(plan, A.make_cfg(backend, copy_cus=copy_cus, copy_teams=teams, copy_streaming=streaming), a, b, c,
                   c_dtype, staging, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    torch.cuda.synchronize()
    hdr, flags, counters, parts, sent = ws_arrays(ws, tabs["num_chunks"])
    assert not counters.any() and not parts.any()
    assert hdr[3] == 0 and not hdr[4:32].any()  # exit counter, copy census
    assert np.all(flags == hdr[0])
    if backend != A.SYNC_COPY_PRESET:
        assert np.all(sent == hdr[0])
    cn = c.cpu().numpy()
    st = staging.cpu().numpy()
    return cn, st, tabs


def check_staging(cn, st, tabs):
    row = 0
    for p in range(tabs["num_chunks"]):
        ch = tabs["arrival"][p]
        r0, r1 = tabs["chunk_begin"][ch], tabs["chunk_begin"][ch + 1]
        assert np.array_equal(st[row:row + r1 - r0].view(np.uint8), cn[r0:r1].view(np.uint8)), f"slot {p}"
        row += r1 - r0
    assert row == cn.shape[0]


@pytest.mark.parametrize("order", [A.SYNC_ORDER_ROW_MAJOR, A.SYNC_ORDER_CHUNK_MAJOR, A.SYNC_ORDER_SWIZZLED])
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_tiny_rs(order, layout):
    m, n, k, W = 1024, 512, 256, 4
    a, b = inputs.gemm_operands(m, n, k, 16.0, b_layout=layout)
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout=layout)
    cn, st, tabs = run_rs(m, n, k, W, a, b, order=order, layout=A.SYNC_B_NK if layout == "nk" else A.SYNC_B_KN)
    assert shard_frobenius(cn.astype(np.float64), ref, W) <= 1e-3
    check_staging(cn, st, tabs)
    assert list(tabs["arrival"]) == [3, 2, 1, 0]  # ring send order of rank 0, own chunk last


@pytest.mark.parametrize("m,n,k,world,split,tile,rank", [
    (1000, 520, 320, 4, 3, (128, 128), 1),   # ragged, chunks of 83/84 rows under 128-row tiles
    (968, 264, 192, 2, 5, (256, 128), 0),
    (512, 256, 128, 8, 2, (256, 256), 5),    # 32-row chunks, 8 per tile
])
def test_ragged_rs(m, n, k, world, split, tile, rank):
    a, b = inputs.gemm_operands(m, n, k, 16.0)
    ref = oracle.gemm_f64(a, b, m, n, k)
    cn, st, tabs = run_rs(m, n, k, world, a, b, split=split, tile=tile, rank=rank, copy_cus=8)
    assert shard_frobenius(cn.astype(np.float64), ref, world) <= 1e-3
    check_staging(cn, st, tabs)


def test_rs_bf16_and_preset():
    m, n, k, W = 1024, 512, 256, 4
    a, b = inputs.gemm_operands(m, n, k, 16.0)
    cn, st, tabs = run_rs(m, n, k, W, a, b, c_dtype=A.SYNC_DTYPE_BF16, copy_cus=32)
    check_staging(cn, st, tabs)
    c32, _, _ = run_rs(m, n, k, W, a, b, backend=A.SYNC_COPY_PRESET)
    want = inputs.f32_to_bf16_bits(c32).view(np.int16)
    assert np.array_equal(cn, want)  # bf16 output is the fp32 result rounded to nearest even


M3, N3, K3, W3 = 8192, 4096, 1792, 8


def test_full_size_rs_exact_integers():
    a, b = inputs.gemm_operands(M3, N3, K3, 1.0, integer=True)
    cn, st, tabs = run_rs(M3, N3, K3, W3, a, b, tile=(256, 256), copy_cus=32)
    assert np.all(cn == np.round(cn))
    rng = np.random.default_rng(3)
    rows, cols = rng.integers(0, M3, 4000), rng.integers(0, N3, 4000)
    assert np.array_equal(cn[rows, cols].astype(np.float64), oracle.gemm_f64_sampled(a, b, M3, N3, K3, rows, cols))
    check_staging(cn, st, tabs)


@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_full_size_rs_normal(cfg3_data, layout):
    """Every element of C against the oracle; every staging slot a copy of its chunk."""
    a, b_kn, ref, absab = cfg3_data
    b = b_kn if layout == "kn" else np.ascontiguousarray(b_kn.T)
    cn, st, tabs = run_rs(M3, N3, K3, W3, a, b, tile=(256, 256), copy_cus=32,
                          layout=A.SYNC_B_NK if layout == "nk" else A.SYNC_B_KN)
    check_full_f32(cn, ref, absab, K3, W3)
    check_staging(cn, st, tabs)


def test_trace_done_and_sent_order():
    """Device trace of an RS call: chunk c's done flag is raised after every
    tile of c started computing, its copy-out after that, and the copy-out
    walks the send order."""
    m, n, k, W = 2048, 1024, 512, 4
    a, b = inputs.gemm_operands(m, n, k, 16.0)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, split=2, tile_m=128, tile_n=128))
    tabs = A.sync_plan_export(plan)
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    staging = torch.empty_like(c)
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    A.sync_gemm_rs(plan, A.make_cfg(A.SYNC_COPY_CU, copy_cus=8, flags=A.SYNC_RUN_TRACE), dev_bits(a), dev_bits(b),
                   c, A.SYNC_DTYPE_F32, staging, ws, s, None)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
    tr = A.sync_trace_export(plan, ws, s)
    assert (tr["chunk_ready"] >= 0).all() and (tr["chunk_sent"] >= 0).all()
    assert (tr["chunk_sent"] >= tr["chunk_ready"]).all()
    sent_in_order = tr["chunk_sent"][tabs["arrival"]]
    assert (np.diff(sent_in_order) >= 0).all()
    for ch in range(tabs["num_chunks"]):
        tiles = tabs["inv_idx"][tabs["inv_ptr"][ch]:tabs["inv_ptr"][ch + 1]]
        assert tr["chunk_ready"][ch] >= tr["tile_wait_end"][tiles].max()


@pytest.mark.parametrize("teams,split", [(3, 1), (4, 1), (5, 2)])
def test_rs_copy_out_teams(teams, split):
    """Copy-out in teams (several chunks in flight): staging still holds every
    chunk's rows in its send slot, bitwise, and the counters come back to zero."""
    m, n, k, W = 1024, 512, 256, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True)
    ref = oracle.gemm_f64(a, b, m, n, k)
    for rep in range(2):
        cn, st, tabs = run_rs(m, n, k, W, a, b, split=split, teams=teams, copy_cus=16)
        assert np.array_equal(cn.astype(np.float64), ref)
        check_staging(cn, st, tabs)


@pytest.mark.parametrize("m,n,k,W,split,tile", [(1024, 512, 256, 4, 1, (128, 128)), (1000, 520, 320, 4, 3, (128, 128)),
                                                 (968, 264, 192, 2, 5, (256, 128)), (1024, 512, 256, 4, 2, (256, 256))])
def test_rs_colocated(m, n, k, W, split, tile):
    """Co-located GEMM-RS: every workgroup stores its tiles, then joins the
    copy-out in send order.  Exact for integer operands; staging bitwise."""
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True)
    ref = oracle.gemm_f64(a, b, m, n, k)
    for teams in (0, W * split):  # one chunk after another; every chunk in its own team
        cn, st, tabs = run_rs(m, n, k, W, a, b, split=split, tile=tile, backend=A.SYNC_COPY_COLOCATED, copy_cus=0,
                              teams=teams)
        assert np.array_equal(cn.astype(np.float64), ref)
        check_staging(cn, st, tabs)


def test_full_size_rs_colocated_exact():
    m, n, k, W = 8192, 4096, 1792, 8
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    cn, st, tabs = run_rs(m, n, k, W, a, b, tile=(256, 256), backend=A.SYNC_COPY_COLOCATED, copy_cus=0,
                          layout=A.SYNC_B_NK, teams=8)
    assert np.all(cn == np.round(cn))
    check_staging(cn, st, tabs)
    rows = np.random.default_rng(3).integers(0, m, 3000)
    cols = np.random.default_rng(4).integers(0, n, 3000)
    exact = oracle.gemm_f64_sampled(a, b, m, n, k, rows, cols, b_layout="nk")
    assert np.array_equal(cn[rows, cols].astype(np.float64), exact)


@pytest.mark.parametrize("streaming", [1])
@pytest.mark.parametrize("backend,cus,teams", [(A.SYNC_COPY_CU, 16, 0), (A.SYNC_COPY_CU, 16, 4),
                                               (A.SYNC_COPY_COLOCATED, 0, 4)])
def test_rs_copy_store_policies(streaming, backend, cus, teams):
    """Copy-out with non-temporal loads and stores: exact C and every chunk
    bitwise in its send slot."""
    m, n, k, W = 1024, 512, 256, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True)
    ref = oracle.gemm_f64(a, b, m, n, k)
    cn, st, tabs = run_rs(m, n, k, W, a, b, split=1, backend=backend, copy_cus=cus, teams=teams, streaming=streaming)
    assert np.array_equal(cn.astype(np.float64), ref)
    check_staging(cn, st, tabs)


@pytest.mark.parametrize("teams", [0, 4])
def test_rs_paced_copy_out(teams):
    """Copy-out paced at 20 GB/s per team: exact C and every chunk bitwise in
    its send slot."""
    m, n, k, W = 1024, 512, 256, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True)
    ref = oracle.gemm_f64(a, b, m, n, k)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, tile_m=128, tile_n=128))
    tabs = A.sync_plan_export(plan)
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    st = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[rs] paced copy-out, teams={teams}", flush=True)
    A.sync_gemm_rs(plan, A.make_cfg(A.SYNC_COPY_CU, copy_cus=16, copy_teams=teams, copy_link_gbps=20.0),
                   dev_bits(a), dev_bits(b), c, A.SYNC_DTYPE_F32, st, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    cn = c.cpu().numpy()
    assert np.array_equal(cn.astype(np.float64), ref)
    check_staging(cn, st.cpu().numpy(), tabs)


# ---- EPILOGUE backend: every tile stores itself into its send slot ----------

@pytest.mark.parametrize("m,n,k,W,split,tile,rank", [(1024, 512, 256, 4, 1, (128, 128), 0),
                                                      (1024, 512, 256, 4, 2, (128, 128), 3),
                                                      (2048, 768, 320, 4, 1, (256, 256), 1),
                                                      (1024, 520, 320, 4, 1, (256, 128), 2)])
@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_rs_epilogue_push(m, n, k, W, split, tile, rank, layout):
    """No copy pass: C exact for small integers, every chunk bitwise in its
    send slot, done and sent flags raised, counters back to zero (a ragged
    last tile column included), with B stored either way."""
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout=layout)
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout=layout)
    for rep in range(2):
        cn, st, tabs = run_rs(m, n, k, W, a, b, split=split, tile=tile, backend=A.SYNC_COPY_EPILOGUE, copy_cus=0,
                              rank=rank, layout=A.SYNC_B_NK if layout == "nk" else A.SYNC_B_KN)
        assert np.array_equal(cn.astype(np.float64), ref)
        check_staging(cn, st, tabs)


def test_rs_epilogue_needs_tiles_inside_chunks():
    """A 256-row tile over 128-row chunks straddles two chunks: EUNSUPPORTED."""
    m, n, k, W = 1024, 512, 256, 4
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, split=2, tile_m=256, tile_n=256,
                                   b_layout=A.SYNC_B_NK))
    ws = workspace(plan)
    t = torch.zeros((m, n), dtype=torch.float32, device="cuda:0")
    ab = torch.zeros((m, k), dtype=torch.int16, device="cuda:0")
    bb = torch.zeros((n, k), dtype=torch.int16, device="cuda:0")
    with pytest.raises(A.SyncError) as ei:
        A.sync_gemm_rs(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), ab, bb, t, A.SYNC_DTYPE_F32, t.clone(), ws,
                       torch.cuda.current_stream(), None)
    assert ei.value.code == A.SYNC_EUNSUPPORTED and "one chunk" in ei.value.message


def test_full_size_rs_epilogue_exact():
    """The Llama-3-8B down-projection share with the epilogue backend: exact
    for small integers on samples, staging bitwise."""
    m, n, k, W = 8192, 4096, 1792, 8
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    cn, st, tabs = run_rs(m, n, k, W, a, b, tile=(256, 256), backend=A.SYNC_COPY_EPILOGUE, copy_cus=0,
                          layout=A.SYNC_B_NK)
    assert np.all(cn == np.round(cn))
    check_staging(cn, st, tabs)
    rows = np.random.default_rng(13).integers(0, m, 3000)
    cols = np.random.default_rng(14).integers(0, n, 3000)
    exact = oracle.gemm_f64_sampled(a, b, m, n, k, rows, cols, b_layout="nk")
    assert np.array_equal(cn[rows, cols].astype(np.float64), exact)


# ---- the reduce-scatter step: send slot = own tile + incoming partial sums ---

def _run_rs_reduce(m, n, k, W, a, b, p, split=1, tile=(128, 128), rank=0):
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, rank=rank, split=split, tile_m=tile[0],
                                   tile_n=tile[1], b_layout=A.SYNC_B_NK))
    tabs = A.sync_plan_export(plan)
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    st = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    pd = torch.from_numpy(p).to("cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[rs-reduce] m={m} n={n} k={k} W={W} split={split} tile={tile} rank={rank}", flush=True)
    A.sync_gemm_rs_reduce(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), dev_bits(a), dev_bits(b), c, pd, st, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    hdr, flags, counters, parts, sent = ws_arrays(ws, tabs["num_chunks"])
    assert np.all(flags == hdr[0]) and np.all(sent == hdr[0]) and not counters.any()
    return c.cpu().numpy(), st.cpu().numpy(), plan


@pytest.mark.parametrize("m,n,k,W,split,tile,rank", [(1024, 512, 256, 4, 1, (128, 128), 0),
                                                      (1024, 520, 320, 4, 2, (128, 128), 3),
                                                      (2048, 768, 320, 4, 1, (256, 256), 1)])
def test_rs_reduce_step_exact(m, n, k, W, split, tile, rank):
    """Small-integer operands and partials: C = R and every send slot = R + P
    over its chunk's rows, exactly, in the oracle's slot order."""
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    p = inputs.partials_f32(m, n, integer=True)
    r = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    cn, st, _ = _run_rs_reduce(m, n, k, W, a, b, p, split, tile, rank)
    assert np.array_equal(cn.astype(np.float64), r)
    ptab = oracle.plan_ref(oracle.PlanDesc(op=oracle.OP_GEMM_RS, m=m, n=n, k=k, world=W, rank=rank, split=split,
                                           tile_m=tile[0], tile_n=tile[1]))
    _, want = oracle.rs_reduce_staging_expected(r, p, ptab)
    assert np.array_equal(st.astype(np.float64), want)


def test_rs_reduce_step_normal_data():
    """N(0,1)/64 operands, N(0,1)/8 partials: every slot within the fp32 bar
    of the fp64 oracle's R + P (relative Frobenius <= 1e-3 per slot)."""
    m, n, k, W = 1024, 512, 1024, 4
    a, b = inputs.gemm_operands(m, n, k, 64.0, b_layout="nk")
    p = inputs.partials_f32(m, n)
    r = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    _, st, _ = _run_rs_reduce(m, n, k, W, a, b, p)
    ptab = oracle.plan_ref(oracle.PlanDesc(op=oracle.OP_GEMM_RS, m=m, n=n, k=k, world=W))
    slots, want = oracle.rs_reduce_staging_expected(r, p, ptab)
    row = 0
    for c, b0, e in slots:
        got, ref = st[row:row + e - b0].astype(np.float64), want[row:row + e - b0]
        assert np.linalg.norm(got - ref) <= 1e-3 * np.linalg.norm(ref), c
        row += e - b0


def test_full_size_rs_reduce_step():
    """The Llama-3-8B down-projection share with its reduce-scatter step:
    sampled C exact against the oracle for small integers, and every send slot
    the fp32 sum of the stored C and the partials, bitwise."""
    m, n, k, W = 8192, 4096, 1792, 8
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    p = inputs.partials_f32(m, n, integer=True)
    cn, st, plan = _run_rs_reduce(m, n, k, W, a, b, p, tile=(256, 256))
    tabs = A.sync_plan_export(plan)
    check_staging((cn + p).astype(np.float32), st, tabs)
    rows = np.random.default_rng(15).integers(0, m, 3000)
    cols = np.random.default_rng(16).integers(0, n, 3000)
    exact = oracle.gemm_f64_sampled(a, b, m, n, k, rows, cols, b_layout="nk")
    assert np.array_equal(cn[rows, cols].astype(np.float64), exact)


def test_rs_reduce_step_validation():
    m, n, k, W = 1024, 512, 256, 4
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, b_layout=A.SYNC_B_NK))
    ws = workspace(plan)
    t = torch.zeros((m, n), dtype=torch.float32, device="cuda:0")
    ab = torch.zeros((m, k), dtype=torch.int16, device="cuda:0")
    bb = torch.zeros((n, k), dtype=torch.int16, device="cuda:0")
    s = torch.cuda.current_stream()
    with pytest.raises(A.SyncError) as ei:
        A.sync_gemm_rs_reduce(plan, A.make_cfg(A.SYNC_COPY_CU, 16), ab, bb, t, t.clone(), t.clone(), ws, s, None)
    assert ei.value.code == A.SYNC_EUNSUPPORTED
    with pytest.raises(A.SyncError) as ei:
        A.sync_gemm_rs_reduce(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), ab, bb, t, None, t.clone(), ws, s, None)
    assert ei.value.code == A.SYNC_EINVAL


# ---- GEMM-AR share: reduce-scatter step, then the all-gather in the same launch

def _run_ar(m, n, k, W, a, b, p, peer, split=1, tile=(128, 128), rank=0, cus=16, with_c=True):
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, rank=rank, split=split, tile_m=tile[0],
                                   tile_n=tile[1], b_layout=A.SYNC_B_NK))
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    st = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    pd, peer_d = torch.from_numpy(p).to("cuda:0"), torch.from_numpy(peer).to("cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[ar] m={m} n={n} k={k} W={W} split={split} tile={tile} rank={rank} cus={cus}", flush=True)
    A.sync_gemm_ar(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE, copy_cus=cus), dev_bits(a), dev_bits(b),
                   c if with_c else None, pd, peer_d, out, st, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    return c.cpu().numpy(), st.cpu().numpy(), out.cpu().numpy(), plan


@pytest.mark.parametrize("m,n,k,W,split,tile,rank,cus", [(1024, 512, 256, 4, 1, (128, 128), 0, 16),
                                                          (1024, 520, 320, 4, 2, (128, 128), 3, 0),
                                                          (2048, 768, 320, 4, 1, (256, 256), 1, 8)])
def test_ar_share_exact(m, n, k, W, split, tile, rank, cus):
    """Small integers: C = R, send slots = R + P, and the all-reduced output
    equals the oracle's (own shard R + P, every other row what the peers sent)."""
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    p = inputs.partials_f32(m, n, integer=True)
    peer = inputs.partials_f32(m, n, seed=inputs.SEED_P + inputs.ALT_SEED_OFFSET, integer=True)
    r = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    for rep in range(2):
        cn, st, out, _ = _run_ar(m, n, k, W, a, b, p, peer, split, tile, rank, cus)
        assert np.array_equal(cn.astype(np.float64), r)
        ptab = oracle.plan_ref(oracle.PlanDesc(op=oracle.OP_GEMM_RS, m=m, n=n, k=k, world=W, rank=rank, split=split,
                                               tile_m=tile[0], tile_n=tile[1]))
        _, want_st = oracle.rs_reduce_staging_expected(r, p, ptab)
        assert np.array_equal(st.astype(np.float64), want_st)
        assert np.array_equal(out.astype(np.float64), oracle.ar_share_expected(r, p, peer, ptab, W, rank))


def test_full_size_ar_share():
    """The Llama-3-8B down-projection shape as a GEMM-AR share: other rows
    bitwise what the peers sent, own rows the fp32 sum of C and P, C exact on
    samples for small integers."""
    m, n, k, W = 8192, 4096, 1792, 8
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    p = inputs.partials_f32(m, n, integer=True)
    peer = inputs.partials_f32(m, n, seed=inputs.SEED_P + inputs.ALT_SEED_OFFSET)
    cn, _, out, _ = _run_ar(m, n, k, W, a, b, p, peer, tile=(256, 256), cus=0)
    own = m // W
    assert np.array_equal(out[own:].view(np.uint32), peer[own:].view(np.uint32))
    assert np.array_equal(out[:own].view(np.uint32), (cn[:own] + p[:own]).astype(np.float32).view(np.uint32))
    rows = np.random.default_rng(17).integers(0, m, 3000)
    cols = np.random.default_rng(18).integers(0, n, 3000)
    exact = oracle.gemm_f64_sampled(a, b, m, n, k, rows, cols, b_layout="nk")
    assert np.array_equal(cn[rows, cols].astype(np.float64), exact)


def test_ar_share_rejects_bad_copy_cus():
    m, n, k, W = 1024, 512, 256, 4
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, b_layout=A.SYNC_B_NK))
    ws = workspace(plan)
    t = torch.zeros((m, n), dtype=torch.float32, device="cuda:0")
    ab = torch.zeros((m, k), dtype=torch.int16, device="cuda:0")
    bb = torch.zeros((n, k), dtype=torch.int16, device="cuda:0")
    with pytest.raises(A.SyncError) as ei:
        A.sync_gemm_ar(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE, 12), ab, bb, t, t.clone(), t.clone(), t.clone(),
                       t.clone(), ws, torch.cuda.current_stream(), None)
    assert ei.value.code == A.SYNC_EINVAL and "copy_cus" in ei.value.message


def test_rs_uneven_shards_copy_out():
    """GEMM-RS over uneven row blocks (an all-to-all's send side): exact C and
    every block bitwise in its send slot."""
    m, n, k, W = 1000, 512, 256, 4
    rows = [100, 400, 150, 350]
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True)
    ref = oracle.gemm_f64(a, b, m, n, k)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, tile_m=128, tile_n=128, shard_rows=rows))
    tabs = A.sync_plan_export(plan)
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    st = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[rs] uneven shards {rows}", flush=True)
    A.sync_gemm_rs(plan, A.make_cfg(A.SYNC_COPY_CU, copy_cus=16, copy_teams=4), dev_bits(a), dev_bits(b), c,
                   A.SYNC_DTYPE_F32, st, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    cn = c.cpu().numpy()
    assert np.array_equal(cn.astype(np.float64), ref)
    check_staging(cn, st.cpu().numpy(), tabs)


@pytest.mark.parametrize("reduce", [False, True])
def test_epilogue_send_without_c(reduce):
    """Epilogue backend with C = NULL: the send slots (plain or with the
    reduce-scatter step) are the only output and match the oracle exactly;
    other backends still need C."""
    m, n, k, W = 1024, 512, 256, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    p = inputs.partials_f32(m, n, integer=True)
    r = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, W, tile_m=128, tile_n=128, b_layout=A.SYNC_B_NK))
    ptab = oracle.plan_ref(oracle.PlanDesc(op=oracle.OP_GEMM_RS, m=m, n=n, k=k, world=W, tile_m=128, tile_n=128))
    st = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[rs] epilogue send without C, reduce={reduce}", flush=True)
    if reduce:
        A.sync_gemm_rs_reduce(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), dev_bits(a), dev_bits(b), None,
                              torch.from_numpy(p).to("cuda:0"), st, ws, s, None)
        _, want = oracle.rs_reduce_staging_expected(r, p, ptab)
    else:
        A.sync_gemm_rs(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), dev_bits(a), dev_bits(b), None, A.SYNC_DTYPE_F32, st,
                       ws, s, None)
        _, want = oracle.rs_staging_expected(r, ptab)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    assert np.array_equal(st.cpu().numpy().astype(np.float64), want)
    with pytest.raises(A.SyncError) as ei:
        A.sync_gemm_rs(plan, A.make_cfg(A.SYNC_COPY_CU, 16), dev_bits(a), dev_bits(b), None, A.SYNC_DTYPE_F32, st, ws,
                       s, None)
    assert ei.value.code == A.SYNC_EINVAL


def test_ar_share_without_c():
    """GEMM-AR share with C = NULL: the reduce step takes the tile from the
    epilogue, so the all-reduced output is exact without C in memory."""
    m, n, k, W = 1024, 512, 256, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    p = inputs.partials_f32(m, n, integer=True)
    peer = inputs.partials_f32(m, n, seed=inputs.SEED_P + inputs.ALT_SEED_OFFSET, integer=True)
    r = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    cn, _, out, _ = _run_ar(m, n, k, W, a, b, p, peer, rank=2, cus=0, with_c=False)
    assert np.isnan(cn).all()  # never written
    ptab = oracle.plan_ref(oracle.PlanDesc(op=oracle.OP_GEMM_RS, m=m, n=n, k=k, world=W, rank=2, tile_m=128,
                                           tile_n=128))
    assert np.array_equal(out.astype(np.float64), oracle.ar_share_expected(r, p, peer, ptab, W, 2))
