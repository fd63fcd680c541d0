"""The kernel-level overlap baseline (sync_gemm_split) on the GPU.

The baseline splits the share into per-chunk runtime copies and per-chunk GEMM
launches joined by events (Syncopate summary page, "Key observations",
observation 1, Fig. 2(a)-(b)).  Its GEMM is the fused calls' kernel with the
same per-tile K order, so its output must be bitwise the compute-only output,
every copied row staged, every send slot its chunk; at full size every
element within the fp32 bar of the oracle.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

from gpu_util import bf16_poison, check_full_f32, dev_bits, host_bits, workspace

pytestmark = pytest.mark.gpu


def _split_ag(m, n, k, world, a, b, split, tile, backend, c_dtype=A.SYNC_DTYPE_F32, rank=0):
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, world, rank=rank, split=split, tile_m=tile[0],
                                   tile_n=tile[1], b_layout=A.SYNC_B_NK))
    tabs = A.sync_plan_export(plan)
    a_peer, b_d = dev_bits(a), dev_bits(b)
    a_local = bf16_poison((m, k))
    for c in range(tabs["num_chunks"]):
        if tabs["resident"][c]:
            r0, r1 = tabs["chunk_begin"][c], tabs["chunk_begin"][c + 1]
            a_local[r0:r1] = a_peer[r0:r1]
    out = (torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0") if c_dtype == A.SYNC_DTYPE_F32
           else bf16_poison((m, n)))
    ws = workspace(plan)
    s, x = torch.cuda.current_stream(), torch.cuda.Stream()
    print(f"[split ag] m={m} n={n} k={k} W={world} split={split} tile={tile} backend={backend}", flush=True)
    A.sync_gemm_split(plan, A.make_cfg(backend), a_peer, a_local, b_d, out, c_dtype, None, ws, s, x)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, chunk
    torch.cuda.synchronize()
    base = a_peer.clone()  # the fused compute-only call on the gathered A
    ref = torch.full_like(out, float("nan")) if c_dtype == A.SYNC_DTYPE_F32 else bf16_poison((m, n))
    A.sync_ag_gemm(plan, A.make_cfg(A.SYNC_COPY_PRESET), None, base, b_d, ref, c_dtype, ws, s, None)
    torch.cuda.synchronize()
    return out, ref, host_bits(a_local)


@pytest.mark.parametrize("split,tile,backend", [(1, (256, 256), A.SYNC_COPY_CU), (3, (128, 128), A.SYNC_COPY_CU),
                                                (2, (256, 128), A.SYNC_COPY_SDMA)])
def test_split_ag_is_bitwise_the_fused_kernel(split, tile, backend):
    m, n, k, world = 2048, 768, 1024, 4
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk")
    out, ref, a_local = _split_ag(m, n, k, world, a, b, split, tile, backend, rank=1)
    assert np.array_equal(a_local, a)
    o, r = out.cpu().numpy(), ref.cpu().numpy()
    assert np.isfinite(o).all()
    assert np.array_equal(o.view(np.uint32), r.view(np.uint32))


def test_split_ag_bf16():
    m, n, k, world = 1000, 520, 576, 4
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk")
    out, ref, _ = _split_ag(m, n, k, world, a, b, 3, (128, 128), A.SYNC_COPY_CU, c_dtype=A.SYNC_DTYPE_BF16)
    assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy())


@pytest.mark.parametrize("split,backend", [(1, A.SYNC_COPY_CU), (2, A.SYNC_COPY_SDMA)])
def test_split_rs_slots_and_output(split, backend):
    m, n, k, world = 2048, 768, 512, 4
    a, b = inputs.gemm_operands(m, n, k, 1.0, integer=True, b_layout="nk")
    r = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, world, split=split, tile_m=256, tile_n=256,
                                   b_layout=A.SYNC_B_NK))
    ptab = oracle.plan_ref(oracle.PlanDesc(op=oracle.OP_GEMM_RS, m=m, n=n, k=k, world=world, split=split,
                                           tile_m=256, tile_n=256))
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    st = torch.full_like(c, float("nan"))
    ws = workspace(plan)
    s, x = torch.cuda.current_stream(), torch.cuda.Stream()
    print(f"[split rs] split={split} backend={backend}", flush=True)
    A.sync_gemm_split(plan, A.make_cfg(backend), None, dev_bits(a), dev_bits(b), c, A.SYNC_DTYPE_F32, st, ws, s, x)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy().astype(np.float64), r)
    _, want = oracle.rs_staging_expected(r, ptab)
    assert np.array_equal(st.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("name", sorted(bench.SPLIT_AGENTS))
def test_full_size_split_ag(cfg2_data, name):
    """The Llama-3-8B up-projection share through the baseline, with each copy
    the bench times: every element against the oracle."""
    a, b_kn, ref, absab = cfg2_data
    out, fused, a_local = _split_ag(8192, 1792, 4096, 8, a, np.ascontiguousarray(b_kn.T), 1, (256, 256),
                                    bench.SPLIT_AGENTS[name]["backend"])
    assert np.array_equal(a_local, a)
    o = out.cpu().numpy()
    check_full_f32(o, ref, absab, 4096, 8)
    assert np.array_equal(o.view(np.uint32), fused.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("name", sorted(bench.SPLIT_AGENTS))
def test_full_size_split_rs(cfg3_data, name):
    a, b_kn, ref, absab = cfg3_data
    m, n, k, world = 8192, 4096, 1792, 8
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, world, b_layout=A.SYNC_B_NK))
    tabs = A.sync_plan_export(plan)
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    st = torch.full_like(c, float("nan"))
    ws = workspace(plan)
    s, x = torch.cuda.current_stream(), torch.cuda.Stream()
    print(f"[split rs] full size {name}", flush=True)
    A.sync_gemm_split(plan, A.make_cfg(**bench.SPLIT_AGENTS[name]), None, dev_bits(a),
                      dev_bits(np.ascontiguousarray(b_kn.T)), c, A.SYNC_DTYPE_F32, st, ws, s, x)
    assert A.sync_workspace_status(ws, s)[0] == A.SYNC_OK
    torch.cuda.synchronize()
    cn = c.cpu().numpy()
    check_full_f32(cn, ref, absab, k, world)
    stn, row = st.cpu().numpy(), 0
    for p in range(tabs["num_chunks"]):
        ch = tabs["arrival"][p]
        r0, r1 = tabs["chunk_begin"][ch], tabs["chunk_begin"][ch + 1]
        assert np.array_equal(stn[row:row + r1 - r0].view(np.uint32), cn[r0:r1].view(np.uint32)), p
        row += r1 - r0
