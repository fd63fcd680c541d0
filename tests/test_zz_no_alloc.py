"""sync_ag_gemm_noalloc (the AG-GEMM share on the library's static scratch)
against sync_ag_gemm on the same inputs, through the C ABI.

Two no-alloc calls in a row, the second with a smaller plan (fewer chunks and
tiles), after calls of the existing entry point with their own workspaces:
each output is bitwise the existing entry point's (same kernels, same K
order) and within the fp32 bar of the oracle; the static scratch reports no
error.  Also: the calls it refuses.
"""
import numpy as np
import pytest
import torch

import oracle
from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

from gpu_util import dev_bits, shard_frobenius, workspace

pytestmark = pytest.mark.gpu

BIG = dict(m=2048, n=768, k=1152, world=4, split=2, tile=(256, 256))
SMALL = dict(m=1000, n=520, k=576, world=4, split=3, tile=(128, 128))


def _case(shape, seed_off):
    m, n, k = shape["m"], shape["n"], shape["k"]
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk", seed_a=inputs.SEED_A + seed_off,
                                seed_b=inputs.SEED_B + seed_off)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, shape["world"], split=shape["split"],
                                   tile_m=shape["tile"][0], tile_n=shape["tile"][1], b_layout=A.SYNC_B_NK))
    tabs = A.sync_plan_export(plan)
    a_peer, b_d = dev_bits(a), dev_bits(b)

    def fresh_local():
        a_local = torch.full_like(a_peer, 0x7FC0)
        for ch in range(tabs["num_chunks"]):
            if tabs["resident"][ch]:
                r0, r1 = tabs["chunk_begin"][ch], tabs["chunk_begin"][ch + 1]
                a_local[r0:r1] = a_peer[r0:r1]
        return a_local

    return dict(shape=shape, a=a, b=b, plan=plan, a_peer=a_peer, b_d=b_d, fresh_local=fresh_local,
                ref=oracle.gemm_f64(a, b, m, n, k, b_layout="nk"))


@pytest.mark.parametrize("agent", [dict(backend=A.SYNC_COPY_CU, copy_cus=16, copy_teams=3, copy_kslices=2),
                                   dict(backend=A.SYNC_COPY_COLOCATED), dict(backend=A.SYNC_COPY_PRESET)],
                         ids=["cu16_3teams_2slices", "colocated", "preset"])
def test_noalloc_matches_the_workspace_call(agent):
    s = torch.cuda.current_stream()
    cases = [_case(BIG, 0), _case(SMALL, 7)]
    cfg = A.make_cfg(**agent)
    want = []
    for cs in cases:  # the existing entry point, each with its own workspace
        m, n = cs["shape"]["m"], cs["shape"]["n"]
        c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
        a_local = cs["a_peer"].clone() if agent["backend"] == A.SYNC_COPY_PRESET else cs["fresh_local"]()
        print(f"[noalloc] workspace call {cs['shape']} {agent}", flush=True)
        A.sync_ag_gemm(cs["plan"], cfg, cs["a_peer"], a_local, cs["b_d"], c, A.SYNC_DTYPE_F32, workspace(cs["plan"]),
                       s, None)
        want.append(c)
    torch.cuda.synchronize()
    outs, locals_ = [], []
    for cs in cases:  # two no-alloc calls in a row, the larger plan first
        m, n = cs["shape"]["m"], cs["shape"]["n"]
        c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
        a_local = cs["a_peer"].clone() if agent["backend"] == A.SYNC_COPY_PRESET else cs["fresh_local"]()
        print(f"[noalloc] static-scratch call {cs['shape']} {agent}", flush=True)
        A.sync_ag_gemm_noalloc(cs["plan"], cfg, cs["a_peer"], a_local, cs["b_d"], c, A.SYNC_DTYPE_F32, s)
        outs.append(c)
        locals_.append(a_local)
    rc, chunk = A.sync_workspace_status(None, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    for cs, c, w, al in zip(cases, outs, want, locals_):
        got = c.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), w.cpu().numpy().view(np.uint32)), cs["shape"]
        assert np.isfinite(got).all()
        assert shard_frobenius(got.astype(np.float64), cs["ref"], cs["shape"]["world"]) <= 1e-3
        assert np.array_equal(al.cpu().numpy().view(np.uint16), cs["a"])  # every chunk staged


def test_noalloc_refusals():
    s = torch.cuda.current_stream()
    cs = _case(SMALL, 3)
    m, n = SMALL["m"], SMALL["n"]
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")
    a_local = cs["fresh_local"]()
    args = (cs["a_peer"], a_local, cs["b_d"], c, A.SYNC_DTYPE_F32, s)
    # the plan's tables are not on the device yet
    with pytest.raises(A.SyncError) as ei:
        A.sync_ag_gemm_noalloc(cs["plan"], A.make_cfg(A.SYNC_COPY_CU, 16), *args)
    assert ei.value.code == A.SYNC_EINVAL and "sync_workspace_init" in ei.value.message
    workspace(cs["plan"])  # set-up: puts the tables on the device
    for bad, msg in ((A.make_cfg(A.SYNC_COPY_SDMA), "backends"),
                     (A.make_cfg(A.SYNC_COPY_CU, 16, flags=A.SYNC_RUN_TIMED), "TIMED"),
                     (A.make_cfg(A.SYNC_COPY_CU, 16, flags=A.SYNC_RUN_TRACE), "TRACE")):
        with pytest.raises(A.SyncError) as ei:
            A.sync_ag_gemm_noalloc(cs["plan"], bad, *args)
        assert ei.value.code == A.SYNC_EUNSUPPORTED and msg in ei.value.message
    rc = A.lib().sync_ag_gemm_noalloc(cs["plan"].handle, None, 0, 0, 0, 0, 0, None)
    assert rc == A.SYNC_EINVAL
    # a plan whose workspace exceeds the static scratch (2048 chunks)
    big = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 2048, 128, 64, 8, split=256, tile_m=128, tile_n=128,
                                  b_layout=A.SYNC_B_NK))
    workspace(big)
    ab = torch.zeros((2048, 64), dtype=torch.int16, device="cuda:0")
    bb = torch.zeros((128, 64), dtype=torch.int16, device="cuda:0")
    cb = torch.empty((2048, 128), dtype=torch.float32, device="cuda:0")
    with pytest.raises(A.SyncError) as ei:
        A.sync_ag_gemm_noalloc(big, A.make_cfg(A.SYNC_COPY_CU, 16), ab, ab.clone(), bb, cb, A.SYNC_DTYPE_F32, s)
    assert ei.value.code == A.SYNC_EINVAL and "static scratch" in ei.value.message
    torch.cuda.synchronize()
