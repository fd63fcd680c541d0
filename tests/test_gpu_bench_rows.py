"""Parity at the exact configuration of every row bench.py reports.

Each bench row names a workload and the copy agents it times (bench.py's
module constants, imported here, so a row cannot report an agent that is not
tested at its shape).  Inputs and outputs are poisoned before each call
(bf16 NaN in the rows the copy agent must write, NaN in C and staging).
Bars: the Llama-3-8B shares and the MoE-like A2A share compare every output
element with the oracle's whole product (fp32 accumulation bound element-wise,
relative Frobenius <= 1e-3 per row shard); the 70B-like share and ring
attention compare sampled outputs (the oracle's whole product would take
minutes there).
"""
import math

import numpy as np
import pytest
import torch

import bench
import oracle
from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

from gpu_util import check_full_f32, dev_bits, workspace
from test_gpu_ag_gemm import _samples, run_ag
from test_gpu_gemm_rs import check_staging, run_rs
from test_gpu_head_attn import run_head
from test_gpu_ring_attn import TOL, run_attn

pytestmark = pytest.mark.gpu

M2, N2, K2, W2 = bench.M, bench.N, bench.K, bench.WORLD


def _ag_kwargs(ag):
    return dict(backend=ag["backend"], copy_cus=ag.get("copy_cus", 0), teams=ag.get("copy_teams", 0),
                kslices=ag.get("copy_kslices", 0), lead=ag.get("copy_lead_slice", 0))


def _paced(ag):
    """Paced copies run through run_ag's own configuration; they take the
    link rate as well."""
    return ag.get("copy_link_gbps", 0.0)


HEADLINE_CASES = [("headline", 1, bench.HEADLINE_AGENT)] + \
    [(f"sweep_{nm}", 1, ag) for nm, ag in bench.SWEEP_AGENTS.items()] + \
    [(f"split{sp}_{nm}", sp, ag) for sp in (2, 4) for nm, ag in bench.SPLIT_SWEEP_AGENTS.items()]


@pytest.mark.parametrize("name,split,ag", HEADLINE_CASES, ids=[c[0] for c in HEADLINE_CASES])
def test_headline_workload_agents(cfg2_data, name, split, ag):
    """The Llama-3-8B up-projection share (B stored [n][k], fp32 C) with each
    copy agent the headline, the copy-backend sweep and the split sweep time:
    every output element against the oracle; every copied row staged."""
    a, b_kn, ref, absab = cfg2_data
    b_nk = np.ascontiguousarray(b_kn.T)
    gbps = _paced(ag)
    if gbps:
        out, a_local = _run_ag_paced(a, b_nk, split, ag)
    else:
        out, a_local = run_ag(M2, N2, K2, W2, a, b_nk, layout="nk", split=split, tile=bench.HEADLINE["tile"],
                              **_ag_kwargs(ag))
    assert np.array_equal(a_local, a)
    check_full_f32(out, ref, absab, K2, W2)


@pytest.mark.parametrize("tile", [t for t in bench.TILE_SWEEP if t != bench.HEADLINE["tile"]],
                         ids=[f"{t[0]}x{t[1]}" for t in bench.TILE_SWEEP if t != bench.HEADLINE["tile"]])
def test_tile_sweep_agent(cfg2_data, tile):
    """The tile sweep's other shapes with the headline agent: every output
    element against the oracle; every copied row staged."""
    a, b_kn, ref, absab = cfg2_data
    out, a_local = run_ag(M2, N2, K2, W2, a, np.ascontiguousarray(b_kn.T), layout="nk", split=1, tile=tile,
                          **_ag_kwargs(bench.HEADLINE_AGENT))
    assert np.array_equal(a_local, a)
    check_full_f32(out, ref, absab, K2, W2)


def _run_ag_paced(a, b_nk, split, ag):
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, M2, N2, K2, W2, split=split, tile_m=256, tile_n=256,
                                   b_layout=A.SYNC_B_NK))
    a_peer, b = dev_bits(a), dev_bits(b_nk)
    a_local = torch.full_like(a_peer, 0x7FC0)
    a_local[: M2 // W2] = a_peer[: M2 // W2]
    c = torch.full((M2, N2), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[bench-row] paced {ag}", flush=True)
    A.sync_ag_gemm(plan, A.make_cfg(**ag), a_peer, a_local, b, c, A.SYNC_DTYPE_F32, ws, s, None)
    rc, chunk = A.sync_workspace_status(ws, s)
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"
    return c.cpu().numpy(), a_local.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", sorted(bench.KN_AGENTS))
def test_layout_kn_row(cfg2_data, name):
    """The headline share with B stored [k][n] (the bench's [k][n] row, its
    tile and agents): every output element against the oracle."""
    a, b_kn, ref, absab = cfg2_data
    out, _ = run_ag(M2, N2, K2, W2, a, b_kn, layout="kn", tile=bench.KN_TILE, **_ag_kwargs(bench.KN_AGENTS[name]))
    check_full_f32(out, ref, absab, K2, W2)


# ---- GEMM-RS row: Llama-3-8B down-projection ---------------------------------
M3, N3, K3, W3 = (bench.RS_SHAPE[x] for x in ("m", "n", "k", "world"))


@pytest.mark.parametrize("name", sorted(bench.RS_AGENTS))
def test_rs_row_agents(cfg3_data, name):
    """Every agent of the GEMM-RS row: C against the oracle element by element,
    each staging slot bitwise its chunk (PRESET sends nothing)."""
    ag = bench.RS_AGENTS[name]
    a, b_kn, ref, absab = cfg3_data
    cn, st, tabs = run_rs(M3, N3, K3, W3, a, np.ascontiguousarray(b_kn.T), tile=(256, 256), backend=ag["backend"],
                          copy_cus=ag.get("copy_cus", 0), teams=ag.get("copy_teams", 0), layout=A.SYNC_B_NK)
    check_full_f32(cn, ref, absab, K3, W3)
    if ag["backend"] != bench.PRESET:
        check_staging(cn, st, tabs)


def _rs_buffers(plan, a, b_nk, p=None, peer=None):
    t = dict(a=dev_bits(a), b=dev_bits(b_nk),
             c=torch.full((M3, N3), float("nan"), dtype=torch.float32, device="cuda:0"),
             st=torch.full((M3, N3), float("nan"), dtype=torch.float32, device="cuda:0"),
             out=torch.full((M3, N3), float("nan"), dtype=torch.float32, device="cuda:0"), ws=workspace(plan))
    if p is not None:
        t["p"] = torch.from_numpy(p).to("cuda:0")
    if peer is not None:
        t["peer"] = torch.from_numpy(peer).to("cuda:0")
    return t


def _ok(ws):
    rc, chunk = A.sync_workspace_status(ws, torch.cuda.current_stream())
    assert rc == A.SYNC_OK, f"device wait timed out on chunk {chunk}"


def test_rs_row_send_only_and_reduce_step(cfg3_data):
    """The RS row's epilogue variants: send slots only (C never written), and
    the reduce-scatter step (slot = stored C + incoming partials, fp32)."""
    a, b_kn, ref, absab = cfg3_data
    b_nk = np.ascontiguousarray(b_kn.T)
    p = inputs.partials_f32(M3, N3)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, M3, N3, K3, W3, b_layout=A.SYNC_B_NK))
    tabs = A.sync_plan_export(plan)
    s = torch.cuda.current_stream()
    t = _rs_buffers(plan, a, b_nk, p)
    print("[bench-row] rs send only", flush=True)
    A.sync_gemm_rs(plan, A.make_cfg(bench.EPI), t["a"], t["b"], None, A.SYNC_DTYPE_F32, t["st"], t["ws"], s, None)
    _ok(t["ws"])
    assert np.isnan(t["c"].cpu().numpy()).all()
    st = t["st"].cpu().numpy()
    slots = np.concatenate([ref[tabs["chunk_begin"][ch]:tabs["chunk_begin"][ch + 1]] for ch in tabs["arrival"]])
    sab = np.concatenate([absab[tabs["chunk_begin"][ch]:tabs["chunk_begin"][ch + 1]] for ch in tabs["arrival"]])
    check_full_f32(st, slots, sab, K3, W3)
    t = _rs_buffers(plan, a, b_nk, p)
    print("[bench-row] rs reduce step", flush=True)
    A.sync_gemm_rs_reduce(plan, A.make_cfg(bench.EPI), t["a"], t["b"], t["c"], t["p"], t["st"], t["ws"], s, None)
    _ok(t["ws"])
    cn = t["c"].cpu().numpy()
    check_full_f32(cn, ref, absab, K3, W3)
    check_staging((cn + p).astype(np.float32), t["st"].cpu().numpy(), tabs)


@pytest.mark.parametrize("split", bench.AR_SPLITS)
@pytest.mark.parametrize("with_c", [True, False])
def test_ar_row_splits(cfg3_data, split, with_c):
    """The GEMM-AR split sweep: own rows the fp32 sum of the tile and the
    partials (against the oracle's R + P), every other row bitwise what the
    peers sent; C (when kept) against the oracle element by element."""
    a, b_kn, ref, absab = cfg3_data
    p = inputs.partials_f32(M3, N3)
    peer = inputs.partials_f32(M3, N3, seed=inputs.SEED_P + inputs.ALT_SEED_OFFSET)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, M3, N3, K3, W3, split=split, b_layout=A.SYNC_B_NK))
    t = _rs_buffers(plan, a, np.ascontiguousarray(b_kn.T), p, peer)
    s = torch.cuda.current_stream()
    print(f"[bench-row] gemm-ar split={split} with_c={with_c}", flush=True)
    A.sync_gemm_ar(plan, A.make_cfg(bench.EPI), t["a"], t["b"], t["c"] if with_c else None, t["p"], t["peer"],
                   t["out"], t["st"], t["ws"], s, None)
    _ok(t["ws"])
    out = t["out"].cpu().numpy()
    own = M3 // W3
    assert np.array_equal(out[own:].view(np.uint32), peer[own:].view(np.uint32))
    want = ref[:own] + p[:own].astype(np.float64)
    check_full_f32(out[:own], want, absab[:own] + np.abs(p[:own]), K3 + 1, 1)
    if with_c:
        cn = t["c"].cpu().numpy()
        check_full_f32(cn, ref, absab, K3, W3)
        assert np.array_equal(out[:own].view(np.uint32), (cn[:own] + p[:own]).astype(np.float32).view(np.uint32))


# ---- 70B-like AG row ------------------------------------------------------------
M4, N4, K4, W4 = (bench.AG70_SHAPE[x] for x in ("m", "n", "k", "world"))


@pytest.fixture(scope="module")
def ag70():
    a, b = inputs.gemm_operands(M4, N4, K4, bench.AG70_SHAPE["divisor"], b_layout="nk")
    rows, cols = _samples(M4, N4, 12000, seed=4)
    return a, b, rows, cols, oracle.gemm_f64_sampled(a, b, M4, N4, K4, rows, cols, b_layout="nk")


AG70_CASES = [(nm, sp, "chunk_major", ag) for nm, (sp, ag) in bench.AG70_AGENTS.items()] + \
    [(f"sweep_split{sp}_{o}", sp, o, bench.AG70_SWEEP_AGENT) for sp, o in
     ((64, "row_major"), (64, "chunk_major"), (16, "swizzled"), (2, "row_major"), (32, "swizzled"))]


@pytest.mark.parametrize("name,split,order,ag", AG70_CASES, ids=[c[0] for c in AG70_CASES])
def test_70b_row_agents(ag70, name, split, order, ag):
    """The 70B-like share with each agent and split the row times (and sweep
    points across chunk size and tile order): sampled outputs per row shard
    against the oracle, every copied row staged."""
    a, b, rows, cols, ref = ag70
    out, a_local = run_ag(M4, N4, K4, W4, a, b, layout="nk", split=split, tile=(256, 256),
                          order=bench.ORDERS[order], **_ag_kwargs(ag))
    assert np.array_equal(a_local, a)
    got = out[rows, cols].astype(np.float64)
    assert np.isfinite(got).all()
    shard = rows // (M4 // W4)
    for s in range(W4):
        sel = shard == s
        assert np.linalg.norm(got[sel] - ref[sel]) <= 1e-3 * np.linalg.norm(ref[sel]), s
    assert not np.isnan(out).any()  # every tile stored


# ---- MoE-like A2A row -----------------------------------------------------------
M5, N5, K5, W5 = (bench.A2A_SHAPE[x] for x in ("m", "n", "k", "world"))


@pytest.fixture(scope="module")
def a2a():
    rows = inputs.routed_token_counts(M5, W5)
    a, b = inputs.gemm_operands(M5, N5, K5, bench.A2A_SHAPE["divisor"], b_layout="nk")
    ref = oracle.gemm_f64(a, b, M5, N5, K5, b_layout="nk")
    absab = oracle.gemm_f64(a & 0x7FFF, b & 0x7FFF, M5, N5, K5, b_layout="nk")
    return rows, a, b, ref, absab


@pytest.mark.parametrize("name", sorted(bench.A2A_AGENTS) + ["compute_only"])
def test_a2a_row_agents(a2a, name):
    """The MoE-like receive side (8192 tokens in Dirichlet-skewed blocks) with
    each agent of the row: every output element against the oracle, every
    received row staged."""
    rows, a, b, ref, absab = a2a
    ag = bench.A2A_AGENTS.get(name, dict(backend=bench.PRESET))
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, M5, N5, K5, W5, b_layout=A.SYNC_B_NK, shard_rows=rows))
    a_peer, b_d = dev_bits(a), dev_bits(b)
    if ag["backend"] == bench.PRESET:
        a_local = a_peer.clone()
    else:
        a_local = torch.full_like(a_peer, 0x7FC0)
        a_local[: rows[0]] = a_peer[: rows[0]]
    c = torch.full((M5, N5), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan)
    s = torch.cuda.current_stream()
    print(f"[bench-row] a2a {name} rows={rows}", flush=True)
    A.sync_ag_gemm(plan, A.make_cfg(**ag), a_peer, a_local, b_d, c, A.SYNC_DTYPE_F32, ws, s, None)
    _ok(ws)
    assert np.array_equal(a_local.cpu().numpy().view(np.uint16), a)
    check_full_f32(c.cpu().numpy(), ref, absab, K5, W5)


# ---- ring-attention row -----------------------------------------------------------

@pytest.mark.parametrize("name", sorted(bench.ATTN_AGENTS))
def test_attention_row_agents(name):
    """The Qwen-like ring step (Q 4096x32x128, 8 KV blocks of 4096x8x128) with
    each agent the row times: sampled (query, head) rows of O and LSE within
    2e-3 of the oracle."""
    ag = bench.ATTN_AGENTS[name]
    sq, hq, hkv, d, n, w = (bench.ATTN_SHAPE[x] for x in ("sq", "hq", "hkv", "d", "n", "world"))
    q, k, v = inputs.attention_operands(sq, hq, w * n, hkv, d)
    o, _, _, lse = run_attn(sq, hq, hkv, w, n, q, k, v, backend=ag["backend"], cus=ag.get("copy_cus", 0),
                            teams=ag.get("copy_teams", 0))
    rng = np.random.default_rng(6)
    qi = np.concatenate([rng.integers(0, sq, 600), [0, sq - 1]])
    hi = np.concatenate([rng.integers(0, hq, 600), [0, hq - 1]])
    ref_o, ref_lse = oracle.attention_f64_sampled(q, k, v, 1 / math.sqrt(d), qi, hi)
    on, ln_ = o.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(on).all() and np.isfinite(ln_).all()
    assert np.max(np.abs(on[qi, hi] - ref_o)) <= TOL
    assert np.max(np.abs(ln_[hi, qi] - ref_lse)) <= TOL


# ---- head-parallel attention row ----------------------------------------------------

@pytest.mark.parametrize("name", sorted(bench.HEAD_AGENTS))
def test_head_attention_row_agents(name):
    """The Llama-3-8B-like head-parallel share (one rank's 4 query / 1 KV
    heads over 8 x 4096 tokens, rank 0) with each agent the row times:
    sampled (query, head) rows of O and LSE within 2e-3 of the oracle."""
    ag = bench.HEAD_AGENTS[name]
    w, n, hq, hkv, d = (bench.HEAD_SHAPE[x] for x in ("world", "n", "hq", "hkv", "d"))
    s = w * n
    q, k, v = inputs.attention_operands(s, hq, s, hkv, d)
    rc, _, o, lse, _, _ = run_head(w, n, 0, q, k, v, backend=ag["backend"], cus=ag.get("copy_cus", 0),
                                   teams=ag.get("copy_teams", 0))
    assert rc == A.SYNC_OK
    rng = np.random.default_rng(7)
    qi = np.concatenate([rng.integers(0, s, 600), [0, n, s - 1]])
    hi = np.concatenate([rng.integers(0, hq, 600), [0, 1, hq - 1]])
    ref_o, ref_lse = oracle.attention_f64_sampled(q, k, v, 1 / math.sqrt(d), qi, hi)
    on, ln_ = o.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(on).all() and np.isfinite(ln_).all()
    assert np.max(np.abs(on[qi, hi] - ref_o)) <= TOL
    assert np.max(np.abs(ln_[hi, qi] - ref_lse)) <= TOL


def test_head_attention_row_copy_only():
    """The row's copy-only agent stages Q, K and V bit for bit."""
    ag = bench.HEAD_COPY_ONLY
    w, n, hq, hkv, d = (bench.HEAD_SHAPE[x] for x in ("world", "n", "hq", "hkv", "d"))
    s = w * n
    q, k, v = inputs.attention_operands(s, hq, s, hkv, d)
    rc, _, _, _, peers, local = run_head(w, n, 0, q, k, v, backend=ag["backend"], cus=ag["copy_cus"],
                                         teams=ag["copy_teams"], flags=ag["flags"])
    assert rc == A.SYNC_OK
    for p, l in zip(peers, local):
        assert torch.equal(p, l)
