"""AG-GEMM share on the GPU, through the C ABI, against the oracle.

Parity bar (per row shard): relative Frobenius error <= 1e-3 for fp32 C;
for bf16 C, |C - bf16(R)| <= 1 bf16 ulp element-wise.  Small-integer inputs
make the product exact in fp32 and give a zero-tolerance check at full size.
Output must be bitwise identical across tile orders, splits and backends
(the per-tile K order is fixed, so the plan changes only *when* a tile runs).
"""
import numpy as np
import pytest
import torch

import oracle
from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

from gpu_util import (bf16_poison, bf16_round, bf16_ulp, check_full_f32, dev_bits, host_bits,
                      shard_frobenius, workspace)

pytestmark = pytest.mark.gpu

LAYOUT = {"kn": A.SYNC_B_KN, "nk": A.SYNC_B_NK}


def run_ag(m, n, k, world, a_bits, b_bits, layout="kn", split=1, tile=(128, 128), order=A.SYNC_ORDER_CHUNK_MAJOR,
           backend=A.SYNC_COPY_SDMA, copy_cus=0, c_dtype=A.SYNC_DTYPE_F32, rank=0, poison=True, flags=0, teams=0,
           kslices=0, streaming=0, calls=1, lead=0):
    print(f"[ag] m={m} n={n} k={k} W={world} split={split} tile={tile} order={order} backend={backend} "
          f"cus={copy_cus} dtype={c_dtype} layout={layout} teams={teams} kslices={kslices} streaming={streaming} "
          f"lead={lead}", flush=True)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, rank=rank, split=split, tile_m=tile[0],
                                   tile_n=tile[1], tile_order=order, b_layout=LAYOUT[layout]))
    tabs = A.sync_plan_export(plan)
    a_peer = dev_bits(a_bits)
    b = dev_bits(b_bits)
    if backend == A.SYNC_COPY_PRESET:
        a_local = a_peer.clone()
    else:
        a_local = bf16_poison((m, k)) if poison else torch.zeros((m, k), dtype=torch.int16, device="cuda:0")
        for c in range(tabs["num_chunks"]):
            if tabs["resident"][c]:
                r0, r1 = tabs["chunk_begin"][c], tabs["chunk_begin"][c + 1]
                a_local[r0:r1] = a_peer[r0:r1]
    if c_dtype == A.SYNC_DTYPE_F32:
        c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    else:
        c = bf16_poison((m, n))
    ws = workspace(plan)
    cfg = A.make_cfg(backend, copy_cus=copy_cus, flags=flags, copy_teams=teams, copy_kslices=kslices,
                     copy_streaming=streaming, copy_lead_slice=lead)
    s = torch.cuda.current_stream()
    for call in range(calls):  # calls > 1: the same workspace again, copied rows and C poisoned in between
        if call:
            c.copy_(torch.full_like(c, float("nan")) if c_dtype == A.SYNC_DTYPE_F32 else bf16_poison((m, n)))
            for ch in range(tabs["num_chunks"]):
                if not tabs["resident"][ch]:
                    r0, r1 = tabs["chunk_begin"][ch], tabs["chunk_begin"][ch + 1]
                    a_local[r0:r1] = bf16_poison((r1 - r0, k))
        A.sync_ag_gemm(plan, cfg, a_peer, a_local, b, c, c_dtype, ws, s, None)
        rc, chunk = A.sync_workspace_status(ws, s)
        assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk} (call {call})"
    torch.cuda.synchronize()
    out = c.cpu().numpy() if c_dtype == A.SYNC_DTYPE_F32 else inputs.bf16_bits_to_f32(host_bits(c))
    return out, host_bits(a_local)


def check_f32(out, ref, world):
    assert np.isfinite(out).all()
    err = shard_frobenius(out.astype(np.float64), ref, world)
    assert err <= 1e-3, err
    return err


# ---- tiny AG-GEMM share: 4 chunks of 256 x 1024, B 1024 x 1024, N(0,1)/32 ----
@pytest.fixture(scope="module")
def tiny():
    m = n = k = 1024
    a, b = inputs.gemm_operands(m, n, k, 32.0)
    return m, n, k, a, b, oracle.gemm_f64(a, b, m, n, k)


@pytest.mark.parametrize("order", [A.SYNC_ORDER_ROW_MAJOR, A.SYNC_ORDER_CHUNK_MAJOR, A.SYNC_ORDER_SWIZZLED])
def test_tiny_sdma_orders(tiny, order):
    m, n, k, a, b, ref = tiny
    out, a_local = run_ag(m, n, k, 4, a, b, order=order)
    check_f32(out, ref, 4)
    assert np.array_equal(a_local, a)  # every peer chunk was staged in


@pytest.mark.parametrize("split,tile", [(1, (128, 128)), (3, (256, 128)), (8, (256, 256))])
def test_tiny_colocated_stages_everything(tiny, split, tile):
    """Co-located backend: the compute workgroups themselves stage every peer
    chunk, then compute."""
    m, n, k, a, b, ref = tiny
    out, a_local = run_ag(m, n, k, 4, a, b, split=split, tile=tile, backend=A.SYNC_COPY_COLOCATED)
    check_f32(out, ref, 4)
    assert np.array_equal(a_local, a)


def test_tiny_bitwise_invariant_across_plans(tiny):
    m, n, k, a, b, ref = tiny
    base, _ = run_ag(m, n, k, 4, a, b, backend=A.SYNC_COPY_PRESET)
    check_f32(base, ref, 4)
    for kw in (dict(order=A.SYNC_ORDER_ROW_MAJOR), dict(order=A.SYNC_ORDER_SWIZZLED, split=3),
               dict(split=2, backend=A.SYNC_COPY_CU, copy_cus=8), dict(backend=A.SYNC_COPY_CU, copy_cus=32),
               dict(split=64), dict(split=4, backend=A.SYNC_COPY_COLOCATED),
               dict(split=3, backend=A.SYNC_COPY_CU, copy_cus=16, teams=9), dict(split=8, backend=A.SYNC_COPY_CU,
                                                                                  copy_cus=24, teams=5)):
        out, _ = run_ag(m, n, k, 4, a, b, **kw)
        assert np.array_equal(out.view(np.uint32), base.view(np.uint32)), kw


@pytest.mark.parametrize("tile", [(128, 128), (256, 128), (256, 256)])
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_tiny_tiles_and_layouts(tiny, tile, layout):
    m, n, k, a, b, ref = tiny
    bb = b if layout == "kn" else np.ascontiguousarray(b.reshape(k, n).T)
    out, _ = run_ag(m, n, k, 4, a, bb, layout=layout, tile=tile)
    check_f32(out, ref, 4)


def test_tiny_bf16_output(tiny):
    """bf16 C = bf16(s) with s the fp32 sum, |s - R| <= K 2^-24 sum|a||b|; so
    |C - bf16(R)| <= ulp(bf16(R)) + K 2^-24 (|A||B|) element-wise."""
    m, n, k, a, b, ref = tiny
    out, _ = run_ag(m, n, k, 4, a, b, c_dtype=A.SYNC_DTYPE_BF16)
    want = bf16_round(ref)
    absab = oracle.gemm_f64(inputs.f32_to_bf16_bits(np.abs(inputs.bf16_bits_to_f32(a))),
                            inputs.f32_to_bf16_bits(np.abs(inputs.bf16_bits_to_f32(b))), m, n, k)
    bound = bf16_ulp(want) + k * 2.0 ** -24 * absab
    bad = ~(np.abs(out - want) <= bound)
    if bad.any():
        idx = np.argwhere(bad)
        raise AssertionError(f"{bad.sum()} elements off by > 1 ulp (nan: {np.isnan(out).sum()}); first "
                             f"{idx[:8].tolist()} got {out[bad][:8]} want {want[bad][:8]}")
    assert shard_frobenius(out.astype(np.float64), want.astype(np.float64), 4) <= 1e-3


@pytest.mark.parametrize("m,n,k,world,split,tile", [
    (1000, 520, 320, 4, 3, (128, 128)),   # ragged M and N, misaligned chunks (83/84 rows)
    (1000, 520, 320, 4, 1, (256, 256)),
    (968, 264, 192, 2, 5, (256, 128)),
    (64, 8, 64, 4, 2, (128, 128)),         # one tile, ragged everywhere, 8-row chunks
])
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_ragged_shapes(m, n, k, world, split, tile, layout):
    a, b = inputs.gemm_operands(m, n, k, 16.0, b_layout=layout)
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout=layout)
    for backend, cus in ((A.SYNC_COPY_SDMA, 0), (A.SYNC_COPY_CU, 16), (A.SYNC_COPY_COLOCATED, 0)):
        out, a_local = run_ag(m, n, k, world, a, b, layout=layout, split=split, tile=tile, backend=backend,
                              copy_cus=cus, rank=world - 1)
        check_f32(out, ref, world)
        assert np.array_equal(a_local, a)


@pytest.mark.parametrize("backend,cus,teams", [(A.SYNC_COPY_CU, 32, 1), (A.SYNC_COPY_CU, 32, 3),
                                               (A.SYNC_COPY_COLOCATED, 0, 1)])
@pytest.mark.parametrize("split", [1, 8])
def test_more_copy_workgroups_than_granules(backend, cus, teams, split):
    """Chunks of 2 rows x 128 B (16 granules of 16 B) against 64 or 256 copy
    workgroups: most workgroups have an empty slice of most chunks and must
    still count toward every chunk's completion exactly once."""
    m, n, k, world = 64, 64, 64, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True)
    ref = oracle.gemm_f64(a, b, m, n, k)
    for rep in range(3):  # repeated calls: the counters must come back to zero each time
        out, a_local = run_ag(m, n, k, world, a, b, split=split, tile=(128, 128), backend=backend, copy_cus=cus,
                              rank=1, teams=teams)
        assert np.array_equal(out.astype(np.float64), ref)
        assert np.array_equal(a_local, a)


def test_epoch_alternating_payloads():
    """Two datasets alternate in the peer region; a tile that read a stale chunk
    (or trusted a flag from the previous call) would mix them."""
    m = n = k = 1024
    a1, b = inputs.gemm_operands(m, n, k, 32.0)
    a2, _ = inputs.gemm_operands(m, n, k, 32.0, seed_a=inputs.SEED_A + inputs.ALT_SEED_OFFSET)
    refs = [oracle.gemm_f64(a, b, m, n, k) for a in (a1, a2)]
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, 4, split=4, tile_m=128, tile_n=128))
    ws = workspace(plan)
    peers = [dev_bits(a1), dev_bits(a2)]
    b_d = dev_bits(b)
    a_local = peers[0].clone()
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.current_stream()
    for it in range(6):
        x = it % 2
        a_local[0:256] = peers[x][0:256]  # the resident shard of rank 0
        cfg = A.make_cfg(A.SYNC_COPY_SDMA if it < 3 else A.SYNC_COPY_CU, copy_cus=16)
        A.sync_ag_gemm(plan, cfg, peers[x], a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
        assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
        check_f32(c.cpu().numpy(), refs[x], 4)


# ---- AG-GEMM share at the Llama-3-8B up-projection size ----------------------
M2, N2, K2, W2 = 8192, 1792, 4096, 8


def _samples(m, n, count, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([rng.integers(0, m, count), np.array([0, m - 1, m // 2])])
    cols = np.concatenate([rng.integers(0, n, count), np.array([0, n - 1, n // 3])])
    return rows, cols




@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_full_size_exact_small_integers(layout):
    a, b = inputs.gemm_operands(M2, N2, K2, 1.0, integer=True, b_layout=layout)
    out, _ = run_ag(M2, N2, K2, W2, a, b, tile=(256, 256), split=2, backend=A.SYNC_COPY_CU, copy_cus=32,
                    layout=layout, teams=7)
    assert np.all(out == np.round(out))  # every element an exact integer
    rows, cols = _samples(M2, N2, 4000)
    exact = oracle.gemm_f64_sampled(a, b, M2, N2, K2, rows, cols, b_layout=layout)
    assert np.array_equal(out[rows, cols].astype(np.float64), exact)


def _b_for(b_kn, layout):
    return b_kn if layout == "kn" else np.ascontiguousarray(b_kn.T)


@pytest.mark.parametrize("backend,cus,split", [
    (A.SYNC_COPY_SDMA, 0, 1), (A.SYNC_COPY_CU, 32, 4),
    (A.SYNC_COPY_CU, 16, 2), (A.SYNC_COPY_PRESET, 0, 1), (A.SYNC_COPY_COLOCATED, 0, 1)])
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_full_size_normal(cfg2_data, backend, cus, split, layout):
    """Every output element of the full-size share against the oracle."""
    a, b_kn, ref, absab = cfg2_data
    out, _ = run_ag(M2, N2, K2, W2, a, _b_for(b_kn, layout), tile=(256, 256), split=split, backend=backend,
                    copy_cus=cus, layout=layout)
    check_full_f32(out, ref, absab, K2, W2)


# ---- one launch per call: failure path and replay ---------------------------

def test_withheld_chunks_time_out_and_error_is_sticky():
    """Chunks that never arrive: the waits expire (2 ms), the call reports the
    timeout with a chunk that was withheld, tiles needing only the resident
    shard are still computed and the others are left untouched; the error
    stays until the workspace is initialised again, after which a normal call
    is exact."""
    m, n, k, world = 1024, 512, 256, 4
    a, b = inputs.gemm_operands(m, n, k, 32.0)
    ref = oracle.gemm_f64(a, b, m, n, k)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, tile_m=128, tile_n=128))
    tabs = A.sync_plan_export(plan)
    resident = [c for c in range(tabs["num_chunks"]) if tabs["resident"][c]]
    assert resident == [0]
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = torch.zeros_like(a_peer)
    a_local[0:256] = a_peer[0:256]
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    withhold = A.make_cfg(A.SYNC_COPY_CU, copy_cus=8, timeout_ns=2_000_000, flags=A.SYNC_RUN_WITHHOLD)
    print("[ag] withheld chunks, 2 ms limit", flush=True)
    A.sync_ag_gemm(plan, withhold, a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_ETIMEOUT and chunk in (1, 2, 3)
    out = c.cpu().numpy()
    assert np.isnan(out[256:]).all()
    check_f32(out[:256], ref[:256], 1)
    # sticky: the next call gives up at once and reports the same error
    A.sync_ag_gemm(plan, A.make_cfg(A.SYNC_COPY_CU, copy_cus=8), a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s,
                   None)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_ETIMEOUT
    A.sync_workspace_init(plan, ws, s)
    c.fill_(float("nan"))
    A.sync_ag_gemm(plan, A.make_cfg(A.SYNC_COPY_CU, copy_cus=8), a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s,
                   None)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
    check_f32(c.cpu().numpy(), ref, world)


def test_captured_call_replays():
    """A CU-backend call is one kernel launch that takes its epoch from the
    workspace, so a captured call can be replayed: each replay (with eager
    work and synchronisation between replays, and different peer data) must
    equal the eager result for that data."""
    m = n = k = 1024
    world = 4
    data = [inputs.gemm_operands(m, n, k, 32.0, seed_a=inputs.SEED_A + 7 * x)[0] for x in range(3)]
    _, b = inputs.gemm_operands(m, n, k, 32.0)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, split=2, tile_m=128, tile_n=128))
    cfg = A.make_cfg(A.SYNC_COPY_CU, copy_cus=16)
    b_d = dev_bits(b)
    a_peer = dev_bits(data[0])
    a_local = torch.zeros_like(a_peer)
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    eager = []
    for x in range(3):  # eager results, one per dataset
        a_peer.copy_(dev_bits(data[x]))
        a_local.zero_()
        a_local[0:256] = a_peer[0:256]
        A.sync_ag_gemm(plan, cfg, a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
        assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
        eager.append(c.clone())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(s)
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            A.sync_ag_gemm(plan, cfg, a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, side, None)
    s.wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(6):
        x = rep % 3
        print(f"[ag] graph replay {rep} dataset {x}", flush=True)
        a_peer.copy_(dev_bits(data[x]))
        a_local.zero_()
        a_local[0:256] = a_peer[0:256]
        c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
        assert torch.equal(c, eager[x]), f"replay {rep} differs from the eager call"


def test_withholding_one_chunk_leaves_exactly_its_tiles():
    """Withhold one copied chunk: exactly the tiles that read it stay unwritten
    (still NaN), every other tile is correct, and the timeout names that chunk."""
    m, n, k, world, split = 1024, 512, 256, 4, 2
    a, b = inputs.gemm_operands(m, n, k, 32.0)
    ref = oracle.gemm_f64(a, b, m, n, k)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, split=split, tile_m=128, tile_n=128))
    tabs = A.sync_plan_export(plan)
    victim = int(tabs["arrival"][3])
    assert not tabs["resident"][victim]
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = torch.zeros_like(a_peer)
    for ch in range(tabs["num_chunks"]):
        if tabs["resident"][ch]:
            r0, r1 = tabs["chunk_begin"][ch], tabs["chunk_begin"][ch + 1]
            a_local[r0:r1] = a_peer[r0:r1]
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    cfg = A.make_cfg(A.SYNC_COPY_CU, copy_cus=8, timeout_ns=2_000_000, flags=A.SYNC_RUN_WITHHOLD,
                     withhold_chunk=victim)
    print(f"[ag] withhold chunk {victim}", flush=True)
    A.sync_ag_gemm(plan, cfg, a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_ETIMEOUT and chunk == victim
    out = c.cpu().numpy()
    skipped = set(tabs["inv_idx"][tabs["inv_ptr"][victim]:tabs["inv_ptr"][victim + 1]].tolist())
    tn = tabs["tiles_n"]
    for t in range(tabs["num_tiles"]):
        i, j = divmod(t, tn)
        blk = out[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
        if t in skipped:
            assert np.isnan(blk).all(), f"tile {t} reads the withheld chunk but was written"
        else:
            r = ref[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert np.isfinite(blk).all() and np.linalg.norm(blk - r) <= 1e-3 * np.linalg.norm(r), f"tile {t}"


@pytest.mark.parametrize("order", [A.SYNC_ORDER_ROW_MAJOR, A.SYNC_ORDER_CHUNK_MAJOR])
def test_trace_tiles_start_after_their_chunks(order):
    """Device trace of one call: slot p ran tile order[p]; every tile's compute
    began after the copy role released each chunk it reads (one device wall
    clock for all XCDs); stamps are ordered within each tile."""
    m, n, k, world, split = 2048, 1024, 512, 4, 2
    a, b = inputs.gemm_operands(m, n, k, 32.0)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, split=split, tile_m=128, tile_n=128,
                                   tile_order=order))
    tabs = A.sync_plan_export(plan)
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = torch.zeros_like(a_peer)
    for ch in range(tabs["num_chunks"]):
        if tabs["resident"][ch]:
            r0, r1 = tabs["chunk_begin"][ch], tabs["chunk_begin"][ch + 1]
            a_local[r0:r1] = a_peer[r0:r1]
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    cfg = A.make_cfg(A.SYNC_COPY_CU, copy_cus=8, flags=A.SYNC_RUN_TRACE)
    A.sync_ag_gemm(plan, cfg, a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
    tr = A.sync_trace_export(plan, ws, s)
    T = tabs["num_tiles"]
    assert (tr["tile_slot"] >= 0).all()
    assert np.array_equal(tabs["tile_order"][tr["tile_slot"]], np.arange(T))
    assert (tr["tile_wait_begin"] <= tr["tile_wait_end"]).all() and (tr["tile_wait_end"] <= tr["tile_end"]).all()
    assert set(tr["tile_xcc"].tolist()) <= set(range(16))
    for ch in range(tabs["num_chunks"]):
        assert (tr["chunk_ready"][ch] < 0) == bool(tabs["resident"][ch])
    worst = 0
    for t in range(T):
        deps = tabs["dep_idx"][tabs["dep_ptr"][t]:tabs["dep_ptr"][t + 1]]
        ready = [tr["chunk_ready"][ch] for ch in deps if not tabs["resident"][ch]]
        if ready:
            worst = min(worst, tr["tile_wait_end"][t] - max(ready))
    assert worst >= 0, f"a tile started {-worst} ns before a chunk it reads was released"


# ---- AG-GEMM share at the 70B-like FFN size --------------------------------------
M4, N4, K4, W4 = 16384, 3584, 8192, 8


@pytest.mark.parametrize("split,teams", [(4, 7), (16, 1)])
def test_full_size_70b_like(split, teams):
    """A 16384x8192 from 8 shards (2048 rows) in 32 or 128 chunks, B 8192x3584
    stored [n][k], N(0,1)/90: sampled outputs against the oracle, per shard."""
    a, b = inputs.gemm_operands(M4, N4, K4, 90.0, b_layout="nk")
    out, a_local = run_ag(M4, N4, K4, W4, a, b, tile=(256, 256), split=split, backend=A.SYNC_COPY_CU, copy_cus=32,
                          layout="nk", teams=teams, poison=False)
    assert np.array_equal(a_local, a)
    rows, cols = _samples(M4, N4, 12000, seed=4)
    ref = oracle.gemm_f64_sampled(a, b, M4, N4, K4, rows, cols, b_layout="nk")
    got = out[rows, cols].astype(np.float64)
    assert np.isfinite(got).all()
    shard = rows // (M4 // W4)
    for s in range(W4):
        sel = shard == s
        assert np.linalg.norm(got[sel] - ref[sel]) <= 1e-3 * np.linalg.norm(ref[sel]), s


# ---- K-sliced copy-in: chunks move as column slices, tiles start on slice 0 --

@pytest.mark.parametrize("backend,cus,teams,kslices,tile,lead", [
    (A.SYNC_COPY_CU, 8, 1, 2, (256, 256), 0), (A.SYNC_COPY_CU, 16, 3, 4, (256, 128), 0),
    (A.SYNC_COPY_CU, 8, 5, 3, (128, 128), 0), (A.SYNC_COPY_COLOCATED, 0, 3, 4, (256, 256), 0),
    (A.SYNC_COPY_COLOCATED, 0, 1, 2, (256, 256), 0), (A.SYNC_COPY_CU, 8, 1, 2, (256, 256), 1),
    (A.SYNC_COPY_CU, 16, 3, 4, (256, 128), 1), (A.SYNC_COPY_CU, 8, 5, 3, (128, 128), 1),
    (A.SYNC_COPY_CU, 16, 3, 4, (256, 256), 2), (A.SYNC_COPY_CU, 8, 5, 3, (128, 128), 2),
    (A.SYNC_COPY_CU, 8, 1, 2, (256, 256), 2), (A.SYNC_COPY_CU, 16, 3, 4, (256, 128), 4),
    (A.SYNC_COPY_CU, 8, 5, 3, (128, 128), 3)])
def test_kslices_parity(backend, cus, teams, kslices, tile, lead):
    """K = 1152 (18 K-steps: uneven slices); the output matches the oracle and
    is bitwise the compute-only output (the copy protocol changes only when
    a K-step's operands are known to be in place)."""
    m, n, k, world, split = 2048, 768, 1152, 4, 2
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    out, a_local = run_ag(m, n, k, world, a, b, layout="nk", split=split, tile=tile, backend=backend,
                          copy_cus=cus, teams=teams, kslices=kslices, lead=lead)
    check_f32(out, ref, world)
    assert np.array_equal(a_local, a)  # every slice of every chunk was staged
    base, _ = run_ag(m, n, k, world, a, b, layout="nk", split=split, tile=tile, backend=A.SYNC_COPY_PRESET)
    assert np.array_equal(out.view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("backend,cus,teams,kslices,tile,lead,n", [
    (A.SYNC_COPY_CU, 8, 1, 2, (256, 256), 1, 768), (A.SYNC_COPY_CU, 16, 3, 4, (256, 128), 2, 768),
    (A.SYNC_COPY_COLOCATED, 0, 3, 4, (256, 256), 0, 768), (A.SYNC_COPY_CU, 8, 5, 3, (128, 128), 3, 768),
    (A.SYNC_COPY_CU, 32, 7, 2, (256, 256), 1, 520), (A.SYNC_COPY_CU, 16, 3, 3, (256, 128), 0, 520)])
def test_kslices_parity_b_kn(backend, cus, teams, kslices, tile, lead, n):
    """The K-sliced copy with B stored [k][n] (the transposing-read path),
    ragged last tile column included: matches the oracle and is bitwise the
    compute-only output."""
    m, k, world, split = 2048, 1152, 4, 2
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="kn")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="kn")
    out, a_local = run_ag(m, n, k, world, a, b, layout="kn", split=split, tile=tile, backend=backend,
                          copy_cus=cus, teams=teams, kslices=kslices, lead=lead)
    check_f32(out, ref, world)
    assert np.array_equal(a_local, a)
    base, _ = run_ag(m, n, k, world, a, b, layout="kn", split=split, tile=tile, backend=A.SYNC_COPY_PRESET)
    assert np.array_equal(out.view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("cus,teams,kslices,tile,rank,lead", [
    (8, 1, 2, (256, 256), 0, 0), (32, 7, 4, (256, 256), 1, 0), (16, 3, 4, (256, 128), 2, 0),
    (8, 5, 3, (128, 128), 3, 0), (32, 7, 4, (256, 256), 1, 1), (8, 5, 3, (128, 128), 3, 1),
    (32, 7, 4, (256, 256), 2, 2), (32, 7, 2, (256, 256), 1, 2), (8, 5, 3, (128, 128), 3, 3)])
def test_kslices_repeated_calls(cus, teams, kslices, tile, rank, lead):
    """Three K-sliced calls on one workspace, the copied rows and C poisoned
    before each: the slice and chunk counters each call leaves cleared let the
    next one stage every slice again and match the oracle, bitwise the
    compute-only output."""
    m, n, k, world, split = 2048, 768, 1152, 4, 2
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    out, a_local = run_ag(m, n, k, world, a, b, layout="nk", split=split, tile=tile, backend=A.SYNC_COPY_CU,
                          copy_cus=cus, teams=teams, kslices=kslices, rank=rank, calls=3, lead=lead)
    check_f32(out, ref, world)
    assert np.array_equal(a_local, a)
    base, _ = run_ag(m, n, k, world, a, b, layout="nk", split=split, tile=tile, backend=A.SYNC_COPY_PRESET,
                     rank=rank)
    assert np.array_equal(out.view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("lead", [0, 1, 2])
def test_kslices_withholding_one_chunk_leaves_exactly_its_tiles(lead):
    """A withheld chunk under a K-sliced copy (with or without the lead slice
    copied by the compute workgroups): none of its slices land, the tiles that
    read it stay unwritten, the others are correct, and the timeout names the
    chunk (not a slice)."""
    m, n, k, world, split = 1024, 512, 512, 4, 2
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, split=split, tile_m=128, tile_n=128,
                                   b_layout=A.SYNC_B_NK))
    tabs = A.sync_plan_export(plan)
    victim = int(tabs["arrival"][4])
    assert not tabs["resident"][victim]
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = torch.zeros_like(a_peer)
    for ch in range(tabs["num_chunks"]):
        if tabs["resident"][ch]:
            r0, r1 = tabs["chunk_begin"][ch], tabs["chunk_begin"][ch + 1]
            a_local[r0:r1] = a_peer[r0:r1]
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    cfg = A.make_cfg(A.SYNC_COPY_CU, copy_cus=8, timeout_ns=2_000_000, flags=A.SYNC_RUN_WITHHOLD,
                     withhold_chunk=victim, copy_teams=3, copy_kslices=2, copy_lead_slice=lead)
    print(f"[ag] kslices=2 withhold chunk {victim}", flush=True)
    A.sync_ag_gemm(plan, cfg, a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_ETIMEOUT and chunk == victim
    out = c.cpu().numpy()
    skipped = set(tabs["inv_idx"][tabs["inv_ptr"][victim]:tabs["inv_ptr"][victim + 1]].tolist())
    tn = tabs["tiles_n"]
    for t in range(tabs["num_tiles"]):
        i, j = divmod(t, tn)
        blk = out[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
        if t in skipped:
            assert np.isnan(blk).all(), f"tile {t} reads the withheld chunk but was written"
        else:
            r = ref[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert np.isfinite(blk).all() and np.linalg.norm(blk - r) <= 1e-3 * np.linalg.norm(r), f"tile {t}"


@pytest.mark.parametrize("backend,cus,teams,kslices,lead", [(A.SYNC_COPY_CU, 32, 7, 4, 0), (A.SYNC_COPY_CU, 32, 7, 8, 0),
                                                            (A.SYNC_COPY_COLOCATED, 0, 7, 4, 0),
                                                            (A.SYNC_COPY_CU, 32, 7, 4, 1), (A.SYNC_COPY_CU, 32, 7, 8, 1),
                                                            (A.SYNC_COPY_CU, 32, 7, 4, 2), (A.SYNC_COPY_CU, 32, 7, 8, 3),
                                                            (A.SYNC_COPY_CU, 32, 7, 2, 2), (A.SYNC_COPY_CU, 32, 7, 4, 4)])
def test_full_size_kslices(cfg2_data, backend, cus, teams, kslices, lead):
    """The Llama-3-8B up-projection share with a K-sliced copy: every output
    element against the oracle."""
    a, b_kn, ref, absab = cfg2_data
    out, a_local = run_ag(M2, N2, K2, W2, a, _b_for(b_kn, "nk"), tile=(256, 256), backend=backend, copy_cus=cus,
                          layout="nk", teams=teams, kslices=kslices, lead=lead)
    assert np.array_equal(a_local, a)
    check_full_f32(out, ref, absab, K2, W2)


# ---- non-temporal loads and stores in the copy role -------------------------

@pytest.mark.parametrize("streaming", [1])
@pytest.mark.parametrize("backend,cus,teams,kslices", [(A.SYNC_COPY_CU, 16, 1, 0), (A.SYNC_COPY_CU, 16, 3, 4),
                                                       (A.SYNC_COPY_COLOCATED, 0, 0, 0)])
def test_copy_store_policies(streaming, backend, cus, teams, kslices):
    """Non-temporal copies stage the same bytes and give the exact output
    (small integers)."""
    m, n, k, world, split = 2048, 768, 1152, 4, 2
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    out, a_local = run_ag(m, n, k, world, a, b, layout="nk", split=split, tile=(256, 256), backend=backend,
                          copy_cus=cus, teams=teams, kslices=kslices, streaming=streaming)
    assert np.array_equal(a_local, a)
    assert np.array_equal(out.astype(np.float64), ref)


@pytest.mark.parametrize("streaming", [1])
def test_full_size_streaming_copy(streaming):
    """The Llama-3-8B up-projection share with the bench's copy (32 copy CUs in
    7 teams, 4 K-slices) with non-temporal copies: exact for small-integer
    operands on sampled outputs, every copied row staged."""
    a, b = inputs.gemm_operands(M2, N2, K2, 1.0, integer=True, b_layout="nk")
    out, a_local = run_ag(M2, N2, K2, W2, a, b, tile=(256, 256), backend=A.SYNC_COPY_CU, copy_cus=32, layout="nk",
                          teams=7, kslices=4, streaming=streaming)
    assert np.array_equal(a_local, a)
    rows, cols = _samples(M2, N2, 4000, seed=5)
    exact = oracle.gemm_f64_sampled(a, b, M2, N2, K2, rows, cols, b_layout="nk")
    assert np.array_equal(out[rows, cols].astype(np.float64), exact)


# ---- SDMA engines driven through HSA: repeated calls, several engines -------

@pytest.mark.parametrize("engines", [1, 7, 14, 16])
def test_full_size_sdma_repeated_calls(engines):
    """Back-to-back SDMA calls at the Llama-3-8B up-projection size, the peer
    region alternating between two datasets: every call's chunks land while
    its GEMM runs, and a tile that trusted a flag of the previous call would
    read the other dataset."""
    a1, b = inputs.gemm_operands(M2, N2, K2, 1.0, integer=True, b_layout="nk")
    a2, _ = inputs.gemm_operands(M2, N2, K2, 1.0, integer=True, b_layout="nk",
                                 seed_a=inputs.SEED_A + inputs.ALT_SEED_OFFSET)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, M2, N2, K2, W2, tile_m=256, tile_n=256, b_layout=A.SYNC_B_NK))
    peers = [dev_bits(a1), dev_bits(a2)]
    b_d = dev_bits(b)
    a_local = bf16_poison((M2, K2))
    c = torch.empty((M2, N2), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    rows, cols = _samples(M2, N2, 3000, seed=9)
    exact = [oracle.gemm_f64_sampled(a, b, M2, N2, K2, rows, cols, b_layout="nk") for a in (a1, a2)]
    cfg = A.make_cfg(A.SYNC_COPY_SDMA, copy_teams=engines)
    for it in range(4):
        x = it % 2
        print(f"[ag] SDMA full size, {engines} engine(s), call {it}", flush=True)
        a_local[:M2 // W2] = peers[x][:M2 // W2]
        c.fill_(float("nan"))
        A.sync_ag_gemm(plan, cfg, peers[x], a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
        rc, chunk = A.sync_workspace_status(ws, s)
        assert rc == A.SYNC_OK, f"call {it}: device wait timed out on chunk {chunk}"
        assert np.array_equal(c[rows, cols].cpu().numpy().astype(np.float64), exact[x]), f"call {it}"
    assert np.array_equal(host_bits(a_local), a2)
    # five calls with no host sync in between, then one check
    a_local[:M2 // W2] = peers[0][:M2 // W2]
    for it in range(5):
        A.sync_ag_gemm(plan, cfg, peers[0], a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    assert np.array_equal(c[rows, cols].cpu().numpy().astype(np.float64), exact[0])


@pytest.mark.parametrize("rows", [[40, 2, 100, 3, 111], [64, 64, 64, 64]])
def test_sdma_chunks_cut_into_row_pieces(rows):
    """SDMA with more engines than copied chunks: every chunk moves as row
    pieces on distinct engines (a chunk with fewer rows than pieces leaves
    some of them empty) and its flag is written once all of them have landed.
    Two calls on one workspace, 16 and 9 engines, copied rows poisoned before
    each: the staged rows and C are exact."""
    m, n, k, world = sum(rows), 256, 512, len(rows)
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, tile_m=128, tile_n=128, b_layout=A.SYNC_B_NK,
                                   shard_rows=rows))
    a_peer, b_d = dev_bits(a), dev_bits(b)
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    for engines in (16, 9):
        print(f"[ag] SDMA row pieces, rows {rows}, {engines} engines", flush=True)
        a_local = bf16_poison((m, k))
        a_local[: rows[0]] = a_peer[: rows[0]]
        c.fill_(float("nan"))
        A.sync_ag_gemm(plan, A.make_cfg(A.SYNC_COPY_SDMA, copy_teams=engines), a_peer, a_local, b_d, c,
                       A.SYNC_DTYPE_F32, ws, s, None)
        rc, chunk = A.sync_workspace_status(ws, s)
        assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
        assert np.array_equal(host_bits(a_local), a)
        assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


def test_sdma_copy_only_advances_the_epoch():
    """SDMA copy-only: the join kernel ends each call once every chunk flag is
    up; the rows are staged and the stored epoch advances once per call."""
    m, n, k, world, split = 1024, 256, 512, 4, 3
    a, _ = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, split=split, tile_m=128, tile_n=128,
                                   b_layout=A.SYNC_B_NK))
    a_peer = dev_bits(a)
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    b_d = torch.zeros((n, k), dtype=torch.int16, device="cuda:0")
    c = torch.zeros((m, n), dtype=torch.float32, device="cuda:0")
    for it in range(3):
        a_local = bf16_poison((m, k))
        a_local[: m // world] = a_peer[: m // world]
        print(f"[ag] SDMA copy-only call {it}", flush=True)
        A.sync_ag_gemm(plan, A.make_cfg(A.SYNC_COPY_SDMA, flags=A.SYNC_RUN_COPY_ONLY, copy_teams=2), a_peer, a_local,
                       b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
        rc, chunk = A.sync_workspace_status(ws, s)
        assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
        assert np.array_equal(host_bits(a_local), a)
        assert int(ws[0].item()) == it + 1


# ---- copy teams paced at a link rate (one team = one link) -------------------

def _paced_call(plan, tabs, a, b, m, n, k, world, flags, teams, kslices, gbps):
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = bf16_poison((m, k))
    for ch in range(tabs["num_chunks"]):
        if tabs["resident"][ch]:
            r0, r1 = tabs["chunk_begin"][ch], tabs["chunk_begin"][ch + 1]
            a_local[r0:r1] = a_peer[r0:r1]
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    A.sync_read_timings(0)
    cfg = A.make_cfg(A.SYNC_COPY_CU, copy_cus=16, flags=flags | A.SYNC_RUN_TIMED, copy_teams=teams,
                     copy_kslices=kslices, copy_link_gbps=gbps)
    print(f"[ag] paced {gbps} GB/s, teams={teams}, kslices={kslices}, flags={flags}", flush=True)
    A.sync_ag_gemm(plan, cfg, a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    (kernel_ms, _), = A.sync_read_timings(16)
    return c.cpu().numpy(), host_bits(a_local), kernel_ms


@pytest.mark.parametrize("teams,kslices", [(1, 0), (3, 0), (1, 2), (3, 4)])
def test_paced_copy_is_exact_and_no_faster_than_its_links(teams, kslices):
    """Three copied chunks of 1 MiB each, every team paced at 10 GB/s: the
    output stays exact and the staged rows complete, and the copy-only call
    lasts at least the busiest link's time (1 team: 3 MiB; 3 teams: 1 MiB)."""
    m, n, k, world, gbps = 2048, 512, 1024, 4, 10.0
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, tile_m=128, tile_n=128, b_layout=A.SYNC_B_NK))
    tabs = A.sync_plan_export(plan)
    out, a_local, _ = _paced_call(plan, tabs, a, b, m, n, k, world, 0, teams, kslices, gbps)
    assert np.array_equal(out.astype(np.float64), ref)
    assert np.array_equal(a_local, a)
    _, a_local, ms = _paced_call(plan, tabs, a, b, m, n, k, world, A.SYNC_RUN_COPY_ONLY, teams, kslices, gbps)
    assert np.array_equal(a_local, a)
    busiest = (3 if teams == 1 else 1) * (m // world) * k * 2
    assert ms * 1e-3 >= 0.95 * busiest / (gbps * 1e9), (ms, busiest)


def test_shutdown_then_calls_again():
    """sync_shutdown releases the library's streams, events and SDMA signals;
    the next SDMA and CU calls re-create what they need and stay exact."""
    m, n, k, world = 1024, 512, 512, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    for backend, cus in ((A.SYNC_COPY_SDMA, 0), (A.SYNC_COPY_CU, 16), (A.SYNC_COPY_SDMA, 0)):
        out, a_local = run_ag(m, n, k, world, a, b, layout="nk", tile=(128, 128), backend=backend, copy_cus=cus,
                              teams=2)
        assert np.array_equal(out.astype(np.float64), ref) and np.array_equal(a_local, a)
        torch.cuda.synchronize()
        A.sync_shutdown()


# ---- uneven shards: the receive side of an all-to-all (A2A-GEMM) ------------

@pytest.mark.parametrize("backend,cus,teams,kslices,split,tile", [
    (A.SYNC_COPY_CU, 16, 3, 0, 1, (128, 128)), (A.SYNC_COPY_CU, 32, 7, 4, 1, (256, 256)),
    (A.SYNC_COPY_SDMA, 0, 3, 0, 2, (256, 128)), (A.SYNC_COPY_COLOCATED, 0, 0, 0, 1, (256, 256))])
def test_a2a_gemm_uneven_shards_exact(backend, cus, teams, kslices, split, tile):
    """Peers send uneven token blocks (tiles straddle shard boundaries): exact
    for small integers, every received row staged."""
    world, n, k = 8, 768, 1024
    rows = inputs.routed_token_counts(2040, world)
    m = sum(rows)
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, split=split, tile_m=tile[0], tile_n=tile[1],
                                   b_layout=A.SYNC_B_NK, shard_rows=rows))
    tabs = A.sync_plan_export(plan)
    ptab = oracle.plan_ref(oracle.PlanDesc(op=oracle.OP_AG_GEMM, m=m, n=n, k=k, world=world, split=split,
                                           tile_m=tile[0], tile_n=tile[1], shard_rows=rows))
    assert list(tabs["chunk_begin"]) == list(ptab.chunk_begin)
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = bf16_poison((m, k))
    a_local[:rows[0]] = a_peer[:rows[0]]
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[a2a] rows={rows} backend={backend} cus={cus} teams={teams} kslices={kslices} split={split} tile={tile}",
          flush=True)
    for rep in range(2):
        c.fill_(float("nan"))
        A.sync_ag_gemm(plan, A.make_cfg(backend, copy_cus=cus, copy_teams=teams, copy_kslices=kslices), a_peer, a_local,
                       b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
        rc, chunk = A.sync_workspace_status(ws, s)
        assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
        assert np.array_equal(host_bits(a_local), a)
        assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


def test_lead_slices_copy_only_stages_everything():
    """COPY_ONLY with lead slices: no compute workgroup runs, so the copy
    workgroups move every slice; every peer row lands and C is untouched."""
    m, n, k, world = 2048, 768, 1152, 4
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk")
    out, a_local = run_ag(m, n, k, world, a, b, layout="nk", split=2, tile=(256, 256), backend=A.SYNC_COPY_CU,
                          copy_cus=16, teams=3, kslices=4, lead=2, flags=A.SYNC_RUN_COPY_ONLY)
    assert np.array_equal(a_local, a)
    assert np.isnan(out).all()


def test_copy_role_refuses_chunks_of_2_gib():
    """The CU and co-located copies store with 32-bit offsets inside one chunk:
    a chunk of 2 GiB (131072 rows of 8192 bf16) is refused before any launch."""
    m, n, k, W = 1 << 20, 256, 8192, 8
    print(f"[ag] refusal m={m} n={n} k={k} W={W}", flush=True)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, W, tile_m=256, tile_n=256, b_layout=A.SYNC_B_NK))
    ws = workspace(plan)
    a_peer = torch.empty((m, k), dtype=torch.int16, device="cuda:0")
    a_local = torch.empty_like(a_peer)
    b = torch.zeros((n, k), dtype=torch.int16, device="cuda:0")
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    for kw in (dict(backend=A.SYNC_COPY_CU, copy_cus=32), dict(backend=A.SYNC_COPY_COLOCATED)):
        with pytest.raises(A.SyncError) as ei:
            A.sync_ag_gemm(plan, A.make_cfg(**kw), a_peer, a_local, b, c, A.SYNC_DTYPE_F32, ws,
                           torch.cuda.current_stream(), None)
        assert ei.value.code == A.SYNC_EUNSUPPORTED and "2 GiB" in ei.value.message
    del a_peer, a_local, c
    torch.cuda.empty_cache()


def test_trace_colocated_tiles_on_an_xcd_multiple():
    """Co-located copy with fewer tiles than workgroups: every workgroup
    copies, and the tiles go to the tile count rounded up to a multiple of the
    XCD count of them.  Trace of one call: slot p ran tile order[p], each tile
    started after the chunks it reads were released, and the XCDs that ran
    tiles ran equally many; C is exact."""
    m, n, k, world = 2048, 1024, 512, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    ref = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, tile_m=256, tile_n=256, b_layout=A.SYNC_B_NK))
    tabs = A.sync_plan_export(plan)
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = bf16_poison((m, k))
    a_local[: m // world] = a_peer[: m // world]
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print("[ag] co-located trace, 32 tiles", flush=True)
    A.sync_ag_gemm(plan, A.make_cfg(A.SYNC_COPY_COLOCATED, flags=A.SYNC_RUN_TRACE), a_peer, a_local, b_d, c,
                   A.SYNC_DTYPE_F32, ws, s, None)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
    tr = A.sync_trace_export(plan, ws, s)
    T = tabs["num_tiles"]
    assert np.array_equal(tabs["tile_order"][tr["tile_slot"]], np.arange(T))
    for t in range(T):
        deps = tabs["dep_idx"][tabs["dep_ptr"][t]:tabs["dep_ptr"][t + 1]]
        ready = [tr["chunk_ready"][ch] for ch in deps if not tabs["resident"][ch]]
        if ready:
            assert tr["tile_wait_end"][t] >= max(ready), f"tile {t} started before its chunks were released"
    per_xcd = np.bincount(tr["tile_xcc"])
    per_xcd = per_xcd[per_xcd > 0]
    assert (per_xcd == per_xcd[0]).all(), f"tiles per XCD {per_xcd.tolist()}"
    assert np.array_equal(host_bits(a_local), a)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)
