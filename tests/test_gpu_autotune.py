"""Autotuner on the GPU: it returns a configuration of the space, that
configuration computes the exact product (small-integer operands), and a
second call is served from the cache (in-process, then from the cache file
in a fresh process)."""
import os

import numpy as np
import pytest
import torch

import oracle
from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

from gpu_util import dev_bits

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def aligned_ws(nbytes):
    raw = torch.zeros(nbytes // 4 + 128, dtype=torch.int32, device="cuda:0")
    off = ((-raw.data_ptr()) % 256) // 4
    return raw[off:off + nbytes // 4 + 1]


@pytest.mark.parametrize("op", [A.SYNC_OP_AG_GEMM, A.SYNC_OP_GEMM_RS])
def test_autotune_picks_a_valid_exact_config(op):
    m, n, k, world = 2048, 1024, 512, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True)
    exact = oracle.gemm_f64(a, b, m, n, k)
    base = A.make_desc(op, m, n, k, world)
    splits, tiles, orders, cus = (1, 2), ((256, 128), (128, 128)), (A.SYNC_ORDER_ROW_MAJOR,
                                                                     A.SYNC_ORDER_CHUNK_MAJOR), (8, 16)
    space = A.make_tune_space(splits=splits, tiles=tiles, orders=orders, copy_cus=cus, warmup=1, iters=3, force=1)
    ws = aligned_ws(A.sync_tune_workspace_size(base, space))
    a_d, b_d = dev_bits(a), dev_bits(b)
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.current_stream()
    print(f"[tune] op={op}", flush=True)
    if op == A.SYNC_OP_AG_GEMM:
        a_local = torch.zeros_like(a_d)
        a_local[0:m // world] = a_d[0:m // world]
        r = A.sync_autotune(base, space, a=a_local, a_peer=a_d, b=b_d, c=c, ws=ws, stream=s)
    else:
        staging = torch.empty_like(c)
        r = A.sync_autotune(base, space, a=a_d, b=b_d, c=c, staging=staging, ws=ws, stream=s)
    assert r["candidates_run"] == 16 and r["candidates_skipped"] == 0
    assert r["split"] in splits and (r["tile_m"], r["tile_n"]) in tiles and r["tile_order"] in orders
    assert r["copy_cus"] in cus and r["best_ms"] > 0
    # the last candidate's output is still in c: exact (integer operands)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), exact)
    # the winner, run on its own, is exact too
    plan = A.sync_plan(A.make_desc(op, m, n, k, world, split=r["split"], tile_m=r["tile_m"], tile_n=r["tile_n"],
                                   tile_order=r["tile_order"]))
    A.sync_workspace_init(plan, ws, s)
    c.fill_(float("nan"))
    cfg = A.make_cfg(A.SYNC_COPY_CU, copy_cus=r["copy_cus"])
    if op == A.SYNC_OP_AG_GEMM:
        A.sync_ag_gemm(plan, cfg, a_d, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    else:
        A.sync_gemm_rs(plan, cfg, a_d, b_d, c, A.SYNC_DTYPE_F32, staging, ws, s, None)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
    assert np.array_equal(c.cpu().numpy().astype(np.float64), exact)
    # cached: same answer, nothing run
    space2 = A.make_tune_space(splits=splits, tiles=tiles, orders=orders, copy_cus=cus, warmup=1, iters=3)
    if op == A.SYNC_OP_AG_GEMM:
        r2 = A.sync_autotune(base, space2, a=a_local, a_peer=a_d, b=b_d, c=c, ws=ws, stream=s)
    else:
        r2 = A.sync_autotune(base, space2, a=a_d, b=b_d, c=c, staging=staging, ws=ws, stream=s)
    assert r2["candidates_run"] == 0 and {k: r2[k] for k in ("split", "tile_m", "tile_n", "tile_order", "copy_cus")} \
        == {k: r[k] for k in ("split", "tile_m", "tile_n", "tile_order", "copy_cus")}
    # tuning cost: the search's wall time is kept with the result; a cache hit costs little
    assert r["from_cache"] == 0 and r["search_wall_ms"] > 0 and r["call_wall_ms"] == r["search_wall_ms"]
    assert r2["from_cache"] == 1 and r2["search_wall_ms"] == r["search_wall_ms"]
    assert 0 <= r2["call_wall_ms"] < r["search_wall_ms"]


def test_cache_file_survives_forgetting(tmp_path, monkeypatch):
    """With SYNC_TUNE_CACHE set, a result is written to the file; after the
    in-process cache is dropped, the file alone serves the same answer."""
    cache = tmp_path / "tune.txt"
    monkeypatch.setenv("SYNC_TUNE_CACHE", str(cache))
    m, n, k = 1024, 512, 256
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True)
    base = A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, 4)
    space = A.make_tune_space(splits=(1, 2), tiles=((128, 128),), copy_cus=(8,), warmup=1, iters=2)
    ws = aligned_ws(A.sync_tune_workspace_size(base, space))
    a_d, b_d = dev_bits(a), dev_bits(b)
    al = torch.zeros_like(a_d)
    al[:256] = a_d[:256]
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.current_stream()
    try:
        r1 = A.sync_autotune(base, space, a=al, a_peer=a_d, b=b_d, c=c, ws=ws, stream=s)
        assert r1["candidates_run"] == 2
        assert cache.read_text().count("\n") == 1
        A.sync_tune_forget()
        r2 = A.sync_autotune(base, space, a=al, a_peer=a_d, b=b_d, c=c, ws=ws, stream=s)
        assert r2["candidates_run"] == 0 and r2["split"] == r1["split"] and r2["from_cache"] == 1
        assert abs(r2["best_ms"] - r1["best_ms"]) <= 1e-3 * r1["best_ms"] + 1e-6
        assert abs(r2["search_wall_ms"] - r1["search_wall_ms"]) <= 1e-3 * r1["search_wall_ms"] + 1e-3
    finally:
        A.sync_tune_forget()


@pytest.mark.parametrize("op", [A.SYNC_OP_AG_GEMM, A.SYNC_OP_GEMM_RS])
def test_autotune_over_copy_agents(op):
    """The copy backend as a tuning dimension: SDMA engines, dedicated copy CUs
    with K-slices, co-located copy, and the RS epilogue backend.  Agents a
    plan cannot use (EPILOGUE for AG; K-slices for RS) are skipped, the winner
    is one of the agents, and running it alone is exact."""
    m, n, k, world = 2048, 1024, 512, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    exact = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    base = A.make_desc(op, m, n, k, world, b_layout=A.SYNC_B_NK)
    agents = (A.make_cfg(A.SYNC_COPY_SDMA, copy_teams=3), A.make_cfg(A.SYNC_COPY_CU, 16, copy_teams=3, copy_kslices=2),
              A.make_cfg(A.SYNC_COPY_COLOCATED, copy_teams=4), A.make_cfg(A.SYNC_COPY_EPILOGUE))
    tiles = ((256, 128), (128, 128))
    space = A.make_tune_space(splits=(1, 2), tiles=tiles, copy_cus=(), agents=agents, warmup=1, iters=3, force=1)
    ws = aligned_ws(A.sync_tune_workspace_size(base, space))
    a_d, b_d = dev_bits(a), dev_bits(b)
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.current_stream()
    print(f"[tune] agents, op={op}", flush=True)
    if op == A.SYNC_OP_AG_GEMM:
        a_local = torch.zeros_like(a_d)
        a_local[0:m // world] = a_d[0:m // world]
        r = A.sync_autotune(base, space, a=a_local, a_peer=a_d, b=b_d, c=c, ws=ws, stream=s)
        usable = (0, 1, 2)  # SDMA, CU, COLOCATED; EPILOGUE sends RS output only
    else:
        staging = torch.empty_like(c)
        r = A.sync_autotune(base, space, a=a_d, b=b_d, c=c, staging=staging, ws=ws, stream=s)
        usable = (2, 3)     # COLOCATED, EPILOGUE; SDMA cannot copy out, K-slices are for AG
    assert r["candidates_run"] == 4 * len(usable) and r["candidates_skipped"] == 4 * (4 - len(usable))
    assert r["agent"] in usable and r["backend"] == agents[r["agent"]].backend and r["best_ms"] > 0
    plan = A.sync_plan(A.make_desc(op, m, n, k, world, split=r["split"], tile_m=r["tile_m"], tile_n=r["tile_n"],
                                   tile_order=r["tile_order"], b_layout=A.SYNC_B_NK))
    A.sync_workspace_init(plan, ws, s)
    c.fill_(float("nan"))
    if op == A.SYNC_OP_AG_GEMM:
        A.sync_ag_gemm(plan, agents[r["agent"]], a_d, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    else:
        A.sync_gemm_rs(plan, agents[r["agent"]], a_d, b_d, c, A.SYNC_DTYPE_F32, staging, ws, s, None)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
    assert np.array_equal(c.cpu().numpy().astype(np.float64), exact)
