"""Benchmark: AG-GEMM share, Llama-3-8B FFN up-projection at TP=8, on one MI355X.

One step = one sync_ag_gemm call, which is one kernel launch: its first
workgroups (the copy role, on 32 CUs) stage the 7 peer chunks of A
(8192 x 4096 bf16, 8 shards of 1024 rows, N(0,1)/64) from the peer HBM region,
all 7 at once in 7 teams (as pulls from every peer over a full xGMI mesh), in 2
K-slices each (the compute workgroups copy the first slice of the chunk their
first tile reads), while the other workgroups run the persistent MFMA GEMM of the
gathered A with B (4096 x 1792 bf16, stored [n][k] like a linear layer's
weight) into C (8192 x 1792 fp32), each tile waiting on the chunks it reads.
Inputs are resident in HBM before the timed region.

Timing.  Every call is bracketed by device events on the stream it is
launched on.  The headline is cold-cache: before each timed call (outside
its events) a 512 MiB scratch buffer is written, which evicts the inputs from
the L2s and the 256 MB Infinity Cache, and then read back, so that the dirty
lines the write leaves are written to HBM before the timed call rather than
during it; a warm series (calls back to back, wall clock over the K steps)
and a cold series with the write alone (the call then also pays for writing
back the flush's dirty lines) are reported beside it.  Every series gives
mean, median, p10 and p90.

Printed: one JSON line with the metric (TFLOP/s of the overlapped call), the
overlap efficiency (overlapped time / max(compute-only, copy-only)), the
roofline of the dominant kernel (the call's launch), the other rows of the hot
path (GEMM-RS, the 70B-like AG with its chunk-size and tile-order sweep, the
MoE-like A2A, ring attention, head-parallel attention, the GEMM-AR split
sweep, the split multi-kernel baseline), and the CPU oracle timed on the host
on the same products.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from communication_overlap_gemm_amd import _abi as A  # noqa: E402  (ctypes binding; the library loads on first call)

METRIC = "AG-GEMM TFLOP/s (bf16, % MFMA peak) + overlap efficiency, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
M, N, K, WORLD = 8192, 1792, 4096, 8
DIVISOR = 64.0
FLUSH_BYTES = 512 << 20       # written (and read back) between cold-cache calls: twice the Infinity Cache

# ---- copy agents of every reported row (sync_copy_cfg keyword sets) ---------
# The parity tests import these, so every agent a row reports is tested at
# that row's shape.
CU, COLOC, SDMA, PRESET, EPI = (A.SYNC_COPY_CU, A.SYNC_COPY_COLOCATED, A.SYNC_COPY_SDMA, A.SYNC_COPY_PRESET,
                                A.SYNC_COPY_EPILOGUE)
HEADLINE = dict(split=1, tile=(256, 256), order="chunk_major", layout="nk", c_dtype="f32")
HEADLINE_AGENT = dict(backend=CU, copy_cus=32, copy_teams=7, copy_kslices=2, copy_lead_slice=1)
BACKENDS = {"sdma": dict(backend=SDMA, copy_teams=7), "cu8": dict(backend=CU, copy_cus=8),
            "cu16": dict(backend=CU, copy_cus=16), "cu24": dict(backend=CU, copy_cus=24),
            "cu32": dict(backend=CU, copy_cus=32), "cu40": dict(backend=CU, copy_cus=40),
            "cu64": dict(backend=CU, copy_cus=64), "colocated": dict(backend=COLOC)}
SWEEP_AGENTS = {
    "sdma_1_engine": dict(backend=SDMA, copy_teams=1), "sdma_7_engines": dict(backend=SDMA, copy_teams=7),
    # 14 engines for 7 copied chunks: every chunk moves as two row pieces on two engines
    "sdma_14_engines": dict(backend=SDMA, copy_teams=14),
    "cu32_4slices_lead2": dict(backend=CU, copy_cus=32, copy_teams=7, copy_kslices=4, copy_lead_slice=2),
    # every slice by the compute workgroups whose first tile reads the chunk: the per-tile co-located form
    "cu32_2slices_lead_all": dict(backend=CU, copy_cus=32, copy_teams=7, copy_kslices=2, copy_lead_slice=2),
    "cu32_2slices_no_lead": dict(backend=CU, copy_cus=32, copy_teams=7, copy_kslices=2),
    "cu8": dict(backend=CU, copy_cus=8, copy_teams=7, copy_kslices=4),
    "cu16": dict(backend=CU, copy_cus=16, copy_teams=7, copy_kslices=4),
    "cu32": dict(backend=CU, copy_cus=32, copy_teams=7, copy_kslices=4),
    "colocated": dict(backend=COLOC),
    "cu32_xgmi_ring_153": dict(backend=CU, copy_cus=32, copy_teams=1, copy_kslices=4, copy_link_gbps=153.0),
    "cu32_xgmi_mesh_153": dict(backend=CU, copy_cus=32, copy_teams=7, copy_kslices=4, copy_link_gbps=153.0)}
SPLIT_SWEEP_AGENTS = {"cu32": dict(backend=CU, copy_cus=32, copy_teams=7, copy_kslices=2, copy_lead_slice=1),
                      "sdma_7_engines": dict(backend=SDMA, copy_teams=7),
                      "sdma_14_engines": dict(backend=SDMA, copy_teams=14)}
# GEMM-RS, Llama-3-8B down-projection
RS_SHAPE = dict(m=8192, n=4096, k=1792, world=8, divisor=64.0)
RS_AGENTS = {"overlapped": dict(backend=EPI), "overlapped_colocated": dict(backend=COLOC, copy_teams=8),
             "overlapped_32_copy_cus": dict(backend=CU, copy_cus=32), "compute_only": dict(backend=PRESET)}
AR_SPLITS = (1, 2, 4)
# AG-GEMM, 70B-like
AG70_SHAPE = dict(m=16384, n=3584, k=8192, world=8, divisor=90.0)
AG70_AGENTS = {"split4_cu32_7teams": (4, dict(backend=CU, copy_cus=32, copy_teams=7)),
               "split4_cu16_7teams": (4, dict(backend=CU, copy_cus=16, copy_teams=7)),
               "split4_colocated": (4, dict(backend=COLOC)),
               "split1_colocated": (1, dict(backend=COLOC))}
AG70_SWEEP_SPLITS = (1, 2, 4, 8, 16, 32, 64)        # chunks of 32 MiB down to 0.5 MiB
AG70_SWEEP_ORDERS = ("row_major", "chunk_major", "swizzled")
AG70_SWEEP_AGENT = dict(backend=COLOC)
# A2A-GEMM receive side, MoE-like
A2A_SHAPE = dict(m=8192, n=1792, k=4096, world=8, divisor=64.0)
A2A_AGENTS = {"cu32_7teams_4slices": dict(backend=CU, copy_cus=32, copy_teams=7, copy_kslices=4),
              "cu32_1team_4slices": dict(backend=CU, copy_cus=32, copy_teams=1, copy_kslices=4),
              "colocated": dict(backend=COLOC), "colocated_4slices": dict(backend=COLOC, copy_kslices=4)}
# ring attention, Qwen-like GQA
ATTN_SHAPE = dict(sq=4096, hq=32, hkv=8, d=128, n=4096, world=8)
ATTN_AGENTS = {"colocated": dict(backend=COLOC), "cu32_7teams": dict(backend=CU, copy_cus=32, copy_teams=7),
               "sdma_14_engines": dict(backend=SDMA, copy_teams=14), "compute_only": dict(backend=PRESET)}

# head-parallel attention share, Llama-3-8B-like (32 query / 8 KV heads): 8 ranks x 4096 tokens, one
# rank's head group of 4 query heads and 1 KV head over all 32768 tokens
HEAD_SHAPE = dict(world=8, n=4096, hq=4, hkv=1, d=128)
HEAD_AGENTS = {"colocated": dict(backend=COLOC), "cu32_7teams": dict(backend=CU, copy_cus=32, copy_teams=7),
               "sdma_14_engines": dict(backend=A.SYNC_COPY_SDMA, copy_teams=14), "compute_only": dict(backend=PRESET)}
HEAD_COPY_ONLY = dict(backend=CU, copy_cus=32, copy_teams=7, flags=A.SYNC_RUN_COPY_ONLY)

ORDERS = {"row_major": A.SYNC_ORDER_ROW_MAJOR, "chunk_major": A.SYNC_ORDER_CHUNK_MAJOR,
          "swizzled": A.SYNC_ORDER_SWIZZLED}
TUNE_AGENTS = (("sdma_7_engines", "sdma", 7, 1, 0), ("cu16", "cu16", 7, 4, 0), ("cu32", "cu32", 7, 4, 0),
               ("cu32_lead", "cu32", 7, 2, 1), ("colocated", "colocated", 0, 1, 0))

PROFILE = os.path.join(ROOT, "profiles", "gemm_dma_ag_llama8b_up.md")
KERNEL_SOURCES = ["gemm_persistent.hip", "copy_role.hpp", "device_common.hpp", "launch_args.hpp"]
PROFILED = {"tile": "256x256", "split": 1, "order": "chunk_major", "backend": "cu32", "c_dtype": "f32", "layout": "nk",
            "teams": 7, "kslices": 2, "lead": 1, "copy_store": "plain"}


def cfg(flags=0, **kw):
    return A.make_cfg(flags=flags, **kw)


def agent_for(name, teams, kslices, lead=0):
    """Copy configuration of a command-line backend name: SDMA takes the engine
    count (teams); the CU and co-located backends take teams and K-slices; the
    CU backend with K-slices also the lead slices its compute workgroups copy."""
    kw = dict(BACKENDS[name])
    if kw["backend"] in (CU, SDMA, COLOC):
        kw["copy_teams"] = teams
    if kw["backend"] in (CU, COLOC):
        kw["copy_kslices"] = kslices
    if kw["backend"] == CU and kslices > 1:
        kw["copy_lead_slice"] = lead
    return kw


def profiled_traffic(args):
    """Bytes between the L2s and the memory fabric per overlapped launch, from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a
    copy-kernel calibration), or None when the configuration differs from the
    profiled one or the kernel sources have changed since the counters were taken."""
    import hashlib

    if any(getattr(args, k) != v for k, v in PROFILED.items()) or not os.path.exists(PROFILE):
        return None
    h = hashlib.sha256()
    kdir = os.path.join(ROOT, "communication_overlap_gemm_amd", "csrc", "kernels")
    for f in KERNEL_SOURCES:
        with open(os.path.join(kdir, f), "rb") as fh:
            h.update(fh.read())
    vals = {}
    with open(PROFILE) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch_overlapped", "kernel_sources_sha256"):
                k, v = line.split(":", 1)
                vals[k] = v.strip()
    if vals.get("kernel_sources_sha256") != h.hexdigest():
        return None
    return int(vals["traffic_bytes_per_launch_overlapped"])


def parse(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--backend", default="cu32", choices=sorted(BACKENDS))
    p.add_argument("--split", type=int, default=HEADLINE["split"])
    p.add_argument("--tile", default="256x256")
    p.add_argument("--order", default=HEADLINE["order"], choices=sorted(ORDERS))
    p.add_argument("--c-dtype", default="f32", choices=["f32", "bf16"])
    p.add_argument("--layout", default="nk", choices=["nk", "kn"], help="B stored [n][k] or [k][n]")
    p.add_argument("--teams", type=int, default=7,
                   help="copied chunks in flight at once (1: one after another, as along a ring; 7: all, as "
                        "pulls from every peer over a full mesh)")
    p.add_argument("--kslices", type=int, default=2,
                   help="K-slices per copied chunk (1: whole chunks; >1: slice 0 of every chunk first, tiles start "
                        "on it and wait in-kernel for the later slices)")
    p.add_argument("--lead", type=int, default=1,
                   help="CU backend with K-slices: leading slices of each chunk copied by the compute workgroups "
                        "whose first tile reads it (0: the copy workgroups move every slice)")
    p.add_argument("--copy-store", default="plain", choices=["plain", "stream"],
                   help="loads and stores of the copy role: plain or non-temporal (stream)")
    p.add_argument("--cache", default="cold", choices=["cold", "warm"],
                   help="headline series: cold (512 MiB written and read back between calls) or warm (back to back)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-other-rows", action="store_true", help="only the headline workload")
    p.add_argument("--attention-only", action="store_true",
                   help="time only the ring-attention and head-parallel attention rows (--steps/--warmup calls "
                        "per agent) and print them as one JSON object (a profiling aid, not the bench line)")
    p.add_argument("--row", default=None, choices=["rs", "ag70", "a2a", "attention"],
                   help="time only one of the other rows (GEMM-RS and GEMM-AR, 70B-like AG, A2A receive side, or "
                        "attention), --steps/--warmup calls per series, and print it as one JSON object (a "
                        "profiling aid, not the bench line)")
    p.add_argument("--tune", action="store_true",
                   help="run the autotuner over split {1,2,4} x tile {256x256, 256x128} x copy agent (SDMA on 7 "
                        "engines, 16 or 32 copy CUs with 4 K-slices, co-located) first and bench its choice")
    return p.parse_args(argv)


def progress(msg):
    """One line per finished row on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---- timing ------------------------------------------------------------------
class Timer:
    """Device-event timing of calls on the current stream (the stream every
    library call here is launched on), cold or warm."""

    def __init__(self, torch):
        self.torch = torch
        self.flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0")
        self.sink = torch.empty(1, dtype=torch.int64, device="cuda:0")

    def evict(self, i, clean=True):
        """Outside the timed events: write the scratch buffer, which evicts the
        inputs from every cache level; with `clean`, read it back, so that the
        dirty lines the write left are written back now and not by the next
        timed call."""
        self.flush.fill_(i)
        if clean:
            self.sink.copy_(self.flush.sum(dtype=self.torch.int64).view(1))

    def series(self, fn, steps, warmup, cold, clean=True):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            if cold:
                self.evict(i, clean)
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        return stats([a.elapsed_time(b) * 1e-3 for a, b in ev], wall if not cold else None)


def stats(xs, wall=None):
    import numpy as np

    x = np.asarray(xs, dtype=np.float64)
    out = {"mean_s": float(x.mean()), "median_s": float(np.median(x)), "p10_s": float(np.percentile(x, 10)),
           "p90_s": float(np.percentile(x, 90)), "n": int(x.size), "samples": [float(v) for v in x]}
    if wall is not None:
        out["wall_s_per_step"] = wall
    return out


def us(st, key="median_s"):
    return round(st[key] * 1e6, 1)


def brief(st):
    return {"median_us": us(st), "p10_us": us(st, "p10_s"), "p90_us": us(st, "p90_s"), "mean_us": us(st, "mean_s")}


def check(ws, stream):
    rc, ch = A.sync_workspace_status(ws, stream)
    if rc != A.SYNC_OK:
        raise SystemExit(f"device wait timed out on chunk {ch}")


def workspace(plan, torch):
    n = A.sync_workspace_size(plan)
    raw = torch.zeros(n // 4 + 64, dtype=torch.int32, device="cuda:0")
    ws = raw[((-raw.data_ptr()) % 256) // 4:]
    ws = ws[: (n + 3) // 4]
    A.sync_workspace_init(plan, ws, torch.cuda.current_stream())
    return ws


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported on this single-GPU "
              "build (the multi-GPU exchange is not part of it).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from communication_overlap_gemm_amd import inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    timer = Timer(torch)
    row = "attention" if args.attention_only else args.row
    if row:
        fn = {"rs": rs_rows, "ag70": ag70_row, "a2a": a2a_row, "attention": attention_rows}[row]
        print(json.dumps(fn(timer, torch, inputs, stream, args.steps, args.warmup)), flush=True)
        return
    cold = args.cache == "cold"
    tuned = None
    if args.tune:
        tuned = tune(args)
        args.split, args.tile = tuned["split"], f'{tuned["tile_m"]}x{tuned["tile_n"]}'
        args.backend, args.teams, args.kslices, args.lead = TUNE_AGENTS[tuned["agent"]][1:]
    tm, tn = (int(x) for x in args.tile.split("x"))
    order = ORDERS[args.order]
    c_dtype = A.SYNC_DTYPE_F32 if args.c_dtype == "f32" else A.SYNC_DTYPE_BF16
    b_layout = A.SYNC_B_NK if args.layout == "nk" else A.SYNC_B_KN
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, M, N, K, WORLD, split=args.split, tile_m=tm, tile_n=tn,
                                   tile_order=order, b_layout=b_layout))
    tabs = A.sync_plan_export(plan)

    a_bits, b_bits = inputs.gemm_operands(M, N, K, DIVISOR, b_layout=args.layout)
    a_peer = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    a_local = torch.zeros_like(a_peer)
    for c in range(tabs["num_chunks"]):
        if tabs["resident"][c]:
            r0, r1 = tabs["chunk_begin"][c], tabs["chunk_begin"][c + 1]
            a_local[r0:r1] = a_peer[r0:r1]
    c_out = torch.empty((M, N), dtype=torch.float32 if c_dtype == A.SYNC_DTYPE_F32 else torch.int16, device=dev)
    ws = workspace(plan, torch)

    agent = agent_for(args.backend, args.teams, args.kslices, args.lead)
    agent["copy_streaming"] = 1 if args.copy_store == "stream" else 0

    def ag_call(c_cfg, pl=plan, w=ws):
        return lambda: A.sync_ag_gemm(pl, c_cfg, a_peer, a_local, b, c_out, c_dtype, w, stream, None)

    def series(c_cfg, steps, warmup, is_cold, pl=plan, w=ws, clean=True):
        st = timer.series(ag_call(c_cfg, pl, w), steps, warmup, is_cold, clean)
        check(w, stream)
        return st

    # headline: overlapped, compute-only on the full chip, copy-only; cold and warm
    res = {}
    for mode in ("cold", "warm"):
        res[mode] = {
            "overlapped": series(cfg(**agent), args.steps, args.warmup, mode == "cold"),
            "compute_only": series(cfg(backend=PRESET), args.steps, args.warmup, mode == "cold"),
            "copy_only": series(cfg(flags=A.SYNC_RUN_COPY_ONLY, **agent), args.steps, args.warmup, mode == "cold")}
    dirty = {"overlapped": series(cfg(**agent), args.steps, args.warmup, True, clean=False),
             "compute_only": series(cfg(backend=PRESET), args.steps, args.warmup, True, clean=False)}
    # compute-only on the workgroups the CU split leaves the GEMM (the copy CUs idle), cold
    same_mask = series(cfg(flags=A.SYNC_RUN_COMPUTE_ONLY, backend=CU, copy_cus=agent["copy_cus"]), args.steps,
                       args.warmup, True) if agent["backend"] == CU else None
    progress("headline series done")
    head = res[args.cache]
    flops = 2.0 * M * N * K
    t_ovl = head["overlapped"]["mean_s"]
    value = flops / t_ovl / 1e12
    copied = sum(int(tabs["chunk_begin"][c + 1] - tabs["chunk_begin"][c]) for c in range(tabs["num_chunks"])
                 if not tabs["resident"][c]) * K * 2

    def overlap_block(r):
        t_o, t_c, t_p = (r[x]["median_s"] for x in ("overlapped", "compute_only", "copy_only"))
        return {"t_overlap_us": round(t_o * 1e6, 1), "t_compute_only_us": round(t_c * 1e6, 1),
                "t_copy_only_us": round(t_p * 1e6, 1), "ratio": round(t_o / max(t_c, t_p), 4),
                "tflops": round(flops / t_o / 1e12, 1),
                "copy_GBps": round(2 * copied / t_p / 1e9, 1),
                "series": {x: brief(r[x]) for x in r}}

    kname = f"gemm_dma<{tm},{tn},{args.c_dtype},AG,B {args.layout}>" + (
        f" with {agent.get('copy_cus')} copy workgroups" if agent["backend"] == CU else
        " with co-located copy" if agent["backend"] == COLOC else "")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_ovl * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "AG-GEMM share, Llama-3-8B FFN up-projection at TP=8: A 8192x4096 bf16 gathered from "
                        "8 row chunks (N(0,1)/64), B 4096x1792 bf16, C 8192x1792 " + args.c_dtype,
            "m": M, "n": N, "k": K, "world": WORLD, "split": args.split, "tile": args.tile,
            "tile_order": args.order, "copy_backend": args.backend, "copy_teams": args.teams,
            "copy_kslices": args.kslices, "copy_lead_slices": agent.get("copy_lead_slice", 0),
            "copy_store": args.copy_store, "b_layout": args.layout,
            "cache": args.cache,
            "timing": "value = 2MNK / mean per-call duration; each call bracketed by device events on its launch "
                      "stream" + ("; 512 MiB written and read back between calls, outside the events" if cold else
                                  "; calls back to back"),
        },
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "overlap": {"cold": overlap_block(res["cold"]), "warm": overlap_block(res["warm"]),
                    "cold_write_only_flush": {
                        "note": "the 512 MiB flush written but not read back: the timed call also writes back "
                                "the flush's dirty lines",
                        "t_overlap_us": us(dirty["overlapped"]), "t_compute_only_us": us(dirty["compute_only"]),
                        "series": {x: brief(dirty[x]) for x in dirty}},
                    "warm_wall_ms_per_step": round(res["warm"]["overlapped"]["wall_s_per_step"] * 1e3, 4)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(value, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(value / PEAK_BF16_TFLOPS, 4),
            "traffic": profiled_traffic(args),
            "traffic_note": "FETCH_SIZE + WRITE_SIZE per launch: bytes between the L2s and the memory fabric "
                            "(Infinity Cache hits included), cold overlapped series, scaled by a copy-only calibration",
            "kernel": kname,
            "flops_per_launch": flops,
            "launch_mean_us": round(t_ovl * 1e6, 2),
        },
    }
    if same_mask is not None:
        t_sm, t_o, t_p = same_mask["median_s"], res["cold"]["overlapped"]["median_s"], res["cold"]["copy_only"]["median_s"]
        line["overlap"]["cold_same_cu_mask"] = {
            "note": "compute-only on the workgroups the copy CUs leave the GEMM (the copy CUs idle)",
            "t_compute_only_us": round(t_sm * 1e6, 1), "ratio": round(t_o / max(t_sm, t_p), 4),
            "series": brief(same_mask)}
    if tuned is not None:
        line["autotune"] = tuned
    if not args.no_other_rows:
        line["copy_backend_sweep"] = backend_sweep(series, flops)
        progress("copy backend sweep done")
        line["split_sweep"] = split_sweep(series, torch, tm, tn, order, b_layout)
        progress("split sweep done")
        line["tile_sweep"] = tile_sweep(series, torch, order, b_layout, agent)
        progress("tile sweep done")
        line["trace_headline"] = trace_headline(plan, agent, a_peer, a_local, b, c_out, c_dtype, ws, stream, tabs)
        line["layout_kn_row"] = layout_kn_row(timer, torch, inputs, stream)
        line["split_baseline"] = {"ag_llama8b_up": split_baseline_ag(timer, plan, a_peer, a_local, b, c_out, c_dtype, ws,
                                                                     stream, torch, res["cold"]["overlapped"])}
        progress("trace, B-layout and split-baseline rows done")
        del a_peer, a_local, b, c_out
        torch.cuda.empty_cache()
        line["other_rows"] = other_rows(timer, torch, inputs, stream)
        progress("other rows done")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a_bits, b_bits, args.layout)
        progress("CPU baseline done")
        if not args.no_other_rows:
            line["cpu_baseline_by_config"] = cpu_baseline_by_config(inputs)
            progress("CPU baseline by configuration done")
    print(json.dumps(line), flush=True)


def backend_sweep(series, flops, steps=10, warmup=3):
    """The same workload with other copy agents: SDMA on one engine (one ring
    link) and on seven (pulls from seven peers), 8/16/32 dedicated copy CUs
    (7 teams, 4 K-slices), co-located copy, and 32 copy CUs paced as xGMI
    links of 153 GB/s: one link carrying every chunk (ring) or seven links at
    once (mesh).  Cold cache."""
    comp = series(cfg(backend=PRESET), steps, warmup, True)["median_s"]
    out = {}
    for name, ag in SWEEP_AGENTS.items():
        t_o = series(cfg(**ag), steps, warmup, True)["median_s"]
        t_c = series(cfg(flags=A.SYNC_RUN_COPY_ONLY, **ag), steps, warmup, True)["median_s"]
        out[name] = {"t_overlap_us": round(t_o * 1e6, 1), "t_copy_only_us": round(t_c * 1e6, 1),
                     "tflops": round(flops / t_o / 1e12, 1), "ratio": round(t_o / max(comp, t_c), 4)}
    out["t_compute_only_us"] = round(comp * 1e6, 1)
    return out


def split_sweep(series, torch, tm, tn, order, b_layout, steps=10, warmup=3):
    """Split factor (sub-chunks per peer shard: chunks of 8, 4 and 2 MiB), cold cache."""
    out = {}
    comp = None
    for sp in (1, 2, 4):
        pl = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, M, N, K, WORLD, split=sp, tile_m=tm, tile_n=tn,
                                     tile_order=order, b_layout=b_layout))
        w = workspace(pl, torch)
        if comp is None:
            comp = series(cfg(backend=PRESET), steps, warmup, True, pl, w)["median_s"]
        for name, ag in SPLIT_SWEEP_AGENTS.items():
            t_o = series(cfg(**ag), steps, warmup, True, pl, w)["median_s"]
            t_c = series(cfg(flags=A.SYNC_RUN_COPY_ONLY, **ag), steps, warmup, True, pl, w)["median_s"]
            out[f"split{sp}_{name}"] = {"chunk_mib": round(8.0 / sp, 2), "t_overlap_us": round(t_o * 1e6, 1),
                                        "t_copy_only_us": round(t_c * 1e6, 1), "ratio": round(t_o / max(comp, t_c), 4)}
    return out


TILE_SWEEP = ((256, 256), (256, 128), (128, 128))  # the kernel's tile shapes (256x224 splits no wave grid in 32s)
WG_PER_CU = {(128, 128): 2}  # workgroups per CU each tile shape runs with (others: 1)


def tile_sweep(series, torch, order, b_layout, agent, steps=10, warmup=3):
    """Tile shape x mode on the headline workload (split 1), cold cache, with
    the wave efficiency T / (P ceil(T / P)) of T tiles on P resident compute
    workgroups (all CUs for compute-only, all but the 32 copy CUs overlapped)."""
    import math

    out = {}
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    for tm, tn in TILE_SWEEP:
        pl = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, M, N, K, WORLD, tile_m=tm, tile_n=tn, tile_order=order,
                                     b_layout=b_layout))
        w = workspace(pl, torch)
        t_c = series(cfg(backend=PRESET), steps, warmup, True, pl, w)["median_s"]
        t_o = series(cfg(**agent), steps, warmup, True, pl, w)["median_s"]
        tiles = math.ceil(M / tm) * math.ceil(N / tn)
        wpc = WG_PER_CU.get((tm, tn), 1)
        eff = {}
        for mode, cus in (("compute_only", num_cus), ("overlapped", num_cus - agent.get("copy_cus", 0))):
            p = cus * wpc
            eff[mode] = round(tiles / (p * math.ceil(tiles / p)), 4)
        out[f"{tm}x{tn}"] = {"tiles": tiles, "workgroups_per_cu": wpc, "t_compute_only_us": round(t_c * 1e6, 1),
                             "t_overlap_us": round(t_o * 1e6, 1), "tflops_overlap": round(2.0 * M * N * K / t_o / 1e12, 1),
                             "wave_efficiency": eff}
    return out


def trace_headline(plan, agent, a_peer, a_local, b, c_out, c_dtype, ws, stream, tabs):
    """One traced call of the headline: exposed wait (time tiles spent waiting
    for their chunks) and the chunks' ready times."""
    import numpy as np

    A.sync_ag_gemm(plan, cfg(flags=A.SYNC_RUN_TRACE, **agent), a_peer, a_local, b, c_out, c_dtype, ws, stream, None)
    check(ws, stream)
    tr = A.sync_trace_export(plan, ws, stream)
    waits = (tr["tile_wait_end"] - tr["tile_wait_begin"]).astype(np.float64)
    ready = sorted(int(tr["chunk_ready"][c]) for c in range(tabs["num_chunks"]) if tr["chunk_ready"][c] >= 0)
    return {"exposed_wait_us_total": round(waits.sum() / 1e3, 1), "exposed_wait_us_mean_per_tile":
            round(waits.mean() / 1e3, 2), "exposed_wait_us_max": round(waits.max() / 1e3, 1),
            "chunk_ready_us": [round(x / 1e3, 1) for x in ready],
            "last_tile_end_us": round(float(tr["tile_end"].max()) / 1e3, 1)}


SPLIT_AGENTS = {"runtime_copy_blit": dict(backend=CU), "runtime_copy_sdma": dict(backend=SDMA)}


def split_baseline_ag(timer, plan, a_peer, a_local, b, c_out, c_dtype, ws, stream, torch, fused, steps=10, warmup=3):
    """The kernel-level overlap baseline on the headline workload (per-chunk
    runtime copies on a second stream, per-chunk GEMM launches joined by
    events), cold cache, against the fused call: the fusion gain."""
    x = torch.cuda.Stream()
    out = {}
    for name, ag in SPLIT_AGENTS.items():
        st = timer.series(lambda: A.sync_gemm_split(plan, cfg(**ag), a_peer, a_local, b, c_out, c_dtype, None, ws,
                                                    stream, x), steps, warmup, True)
        check(ws, stream)
        out[name] = {"t_us": us(st), "tflops": round(2.0 * M * N * K / st["median_s"] / 1e12, 1),
                     "fusion_gain": round(st["median_s"] / fused["median_s"], 3)}
    out["t_fused_us"] = us(fused)
    out["workload"] = "the headline share split into 8 per-chunk copies and GEMM launches (7 copied)"
    return out


KN_TILE = HEADLINE["tile"]  # B [k][n] runs the headline's kernel, with transposing B reads
KN_AGENTS = {"overlapped_headline_agent": HEADLINE_AGENT, "overlapped_colocated": dict(backend=COLOC),
             "compute_only": dict(backend=PRESET)}


def layout_kn_row(timer, torch, inputs, stream, steps=10, warmup=3):
    """The headline workload with B stored [k][n] (the kernel for that layout), cold cache."""
    import numpy as np

    a_bits, b_bits = inputs.gemm_operands(M, N, K, DIVISOR, b_layout="kn")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, M, N, K, WORLD, tile_m=KN_TILE[0], tile_n=KN_TILE[1],
                                   b_layout=A.SYNC_B_KN))
    ap = torch.from_numpy(a_bits.view(np.int16)).to("cuda:0")
    b = torch.from_numpy(b_bits.view(np.int16)).to("cuda:0")
    al = torch.zeros_like(ap)
    al[: M // WORLD] = ap[: M // WORLD]
    c = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    ws = workspace(plan, torch)
    out = {}
    for name, ag in KN_AGENTS.items():
        st = timer.series(lambda: A.sync_ag_gemm(plan, cfg(**ag), ap, al, b, c, A.SYNC_DTYPE_F32, ws, stream, None),
                          steps, warmup, True)
        check(ws, stream)
        out[name] = {"median_us": us(st), "tflops": round(2.0 * M * N * K / st["median_s"] / 1e12, 1)}
    out["workload"] = (f"the headline share with B stored [k][n] (gemm_dma<{KN_TILE[0]},{KN_TILE[1]}>), "
                       "fp32 C, cold cache")
    return out


def _interleaved_medians(timer, stream, calls, steps, warmup):
    """Cold medians of several calls on one workload (name -> (call, workspace)),
    timed in two rounds, the second in reverse order, so that a drift of the
    chip's clock over the row (long attention launches warm it) weighs on
    every call alike."""
    import numpy as np

    samples = {k: [] for k in calls}
    order = list(calls)
    for rnd, seq in enumerate((order, order[::-1])):
        for k in seq:
            fn, ws = calls[k]
            st = timer.series(fn, steps, warmup if rnd == 0 else 1, True)
            check(ws, stream)
            samples[k] += st["samples"]
    return {k: float(np.median(v)) for k, v in samples.items()}


def _cold_median(timer, stream, steps, warmup):
    """A timer of one call: its median over `steps` cold launches after `warmup`, the workspace checked."""
    def t_of(fn, ws):
        st = timer.series(fn, steps, warmup, True)
        check(ws, stream)
        return st["median_s"]
    return t_of


def other_rows(timer, torch, inputs, stream, steps=5, warmup=2):
    """The other rows of the hot path on their configurations, cold cache."""
    out = rs_rows(timer, torch, inputs, stream, steps, warmup)
    progress("GEMM-RS and GEMM-AR rows done")
    out.update(ag70_row(timer, torch, inputs, stream, steps, warmup))
    progress("70B-like AG row done")
    out.update(a2a_row(timer, torch, inputs, stream, steps, warmup))
    out.update(attention_rows(timer, torch, inputs, stream, steps, warmup))
    return out


def rs_rows(timer, torch, inputs, stream, steps=5, warmup=2):
    """GEMM-RS on the Llama-3-8B down-projection (copy agents, send slots only,
    the reduce-scatter step, the split baseline, emission cadence) and the
    GEMM-AR share by split, cold cache."""
    import numpy as np

    dev = torch.device("cuda:0")
    out = {}
    t_of = _cold_median(timer, stream, steps, warmup)

    # GEMM-RS, Llama-3-8B down-projection (B stored [n][k], C fp32)
    m, n, k, w = (RS_SHAPE[x] for x in ("m", "n", "k", "world"))
    a_bits, b_bits = inputs.gemm_operands(m, n, k, RS_SHAPE["divisor"], b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, w, b_layout=A.SYNC_B_NK))
    a = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    c = torch.empty((m, n), dtype=torch.float32, device=dev)
    st = torch.empty_like(c)
    ws = workspace(plan, torch)
    calls = {name: ((lambda ag=ag: A.sync_gemm_rs(plan, cfg(**ag), a, b, c, A.SYNC_DTYPE_F32, st, ws, stream, None)), ws)
             for name, ag in RS_AGENTS.items()}
    calls["send_only"] = (lambda: A.sync_gemm_rs(plan, cfg(backend=EPI), a, b, None, A.SYNC_DTYPE_F32, st, ws, stream,
                                                 None), ws)
    t = _interleaved_medians(timer, stream, calls, steps, warmup)
    part = torch.from_numpy(inputs.partials_f32(m, n)).to(dev)
    t["overlapped_reduce_step"] = t_of(lambda: A.sync_gemm_rs_reduce(plan, cfg(backend=EPI), a, b, c, part, st, ws,
                                                                     stream, None), ws)
    # the kernel-level overlap baseline: per-chunk GEMM launches, each chunk copied out after its launch
    x = torch.cuda.Stream()
    for name, ag in SPLIT_AGENTS.items():
        t["split_" + name] = t_of(lambda: A.sync_gemm_split(plan, cfg(**ag), None, a, b, c, A.SYNC_DTYPE_F32, st, ws,
                                                            stream, x), ws)
    # emission cadence: done-flag times of one traced call, in send order
    A.sync_gemm_rs(plan, cfg(backend=EPI, flags=A.SYNC_RUN_TRACE), a, b, c, A.SYNC_DTYPE_F32, st, ws, stream, None)
    check(ws, stream)
    tr = A.sync_trace_export(plan, ws, stream)
    tabs = A.sync_plan_export(plan)
    done = np.array([tr["chunk_ready"][tabs["arrival"][p]] for p in range(tabs["num_chunks"])], dtype=np.float64)
    gaps = np.diff(done)
    # GEMM-AR share: that reduce-scatter step, then the all-gather of the reduced chunks, at several splits
    peer = torch.from_numpy(inputs.partials_f32(m, n, seed=inputs.SEED_P + inputs.ALT_SEED_OFFSET)).to(dev)
    out_ar = torch.empty_like(c)
    ar = {}
    for sp in AR_SPLITS:
        pl = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, w, split=sp, b_layout=A.SYNC_B_NK))
        wsp = workspace(pl, torch)
        ar[f"split{sp}"] = {
            "chunk_mib": round(m // w // sp * n * 4 / 2 ** 20, 2),
            "t_us": round(1e6 * t_of(lambda: A.sync_gemm_ar(pl, cfg(backend=EPI), a, b, c, part, peer, out_ar, st, wsp,
                                                            stream, None), wsp), 1),
            "t_without_c_us": round(1e6 * t_of(lambda: A.sync_gemm_ar(pl, cfg(backend=EPI), a, b, None, part, peer,
                                                                      out_ar, st, wsp, stream, None), wsp), 1)}
    del part, peer, out_ar
    flops = 2.0 * m * n * k
    hbm = (m * k + k * n) * 2 + m * n * 4 * 2  # A, B, then C and staging each written once
    out["gemm_rs_llama8b_down"] = {
        "workload": "GEMM-RS share: A 8192x1792 bf16, B 1792x4096 bf16, C 8192x4096 fp32 in 8 row chunks, each "
                    "sent to its staging slot in send order; epilogue backend (every tile stores itself into C and "
                    "into its send slot; the tile completing a chunk raises its done and sent flags)",
        "tflops": round(flops / t["overlapped"] / 1e12, 1),
        "t_overlap_us": round(t["overlapped"] * 1e6, 1), "t_compute_only_us": round(t["compute_only"] * 1e6, 1),
        "t_overlap_colocated_us": round(t["overlapped_colocated"] * 1e6, 1),
        "t_overlap_32_copy_cus_us": round(t["overlapped_32_copy_cus"] * 1e6, 1),
        "t_overlap_send_slots_only_us": round(t["send_only"] * 1e6, 1),
        "t_overlap_with_reduce_step_us": round(t["overlapped_reduce_step"] * 1e6, 1),
        "gemm_ar_share_by_split": ar,
        "split_baseline": {nm: {"t_us": round(t["split_" + nm] * 1e6, 1),
                                "fusion_gain": round(t["split_" + nm] / t["overlapped"], 3)} for nm in SPLIT_AGENTS},
        "ratio_to_compute_only": round(t["overlapped"] / t["compute_only"], 4),
        "frac_mfma_peak": round(flops / t["overlapped"] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "hbm_bound_us": round(hbm / 8e12 * 1e6, 1), "frac_hbm_roofline": round(hbm / 8e12 / t["overlapped"], 4),
        "emission_cadence": {"done_us_in_send_order": [round(x / 1e3, 1) for x in done],
                             "gap_mean_us": round(float(gaps.mean()) / 1e3, 2),
                             "gap_cv": round(float(gaps.std() / gaps.mean()), 3) if gaps.mean() > 0 else None}}
    del a, b, c, st

    return out


def ag70_row(timer, torch, inputs, stream, steps=5, warmup=2):
    """AG-GEMM on the 70B-like FFN shape: copy agents and the chunk-size x
    tile-order sweep, cold cache."""
    import numpy as np

    dev = torch.device("cuda:0")
    out = {}
    t_of = _cold_median(timer, stream, steps, warmup)

    # AG-GEMM 70B-like: A 16384x8192 (8 shards of 2048 rows), B 8192x3584 stored [n][k], C fp32
    m, n, k, w = (AG70_SHAPE[x] for x in ("m", "n", "k", "world"))
    a_bits, b_bits = inputs.gemm_operands(m, n, k, AG70_SHAPE["divisor"], b_layout="nk")
    ap = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    al = torch.zeros_like(ap)
    al[: m // w] = ap[: m // w]
    c = torch.empty((m, n), dtype=torch.float32, device=dev)
    plans = {(sp, o): A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, w, split=sp, tile_order=ORDERS[o],
                                              b_layout=A.SYNC_B_NK))
             for sp in AG70_SWEEP_SPLITS for o in AG70_SWEEP_ORDERS}
    wss = {key: workspace(pl, torch) for key, pl in plans.items()}

    def ag70(key, ag):
        return lambda: A.sync_ag_gemm(plans[key], cfg(**ag), ap, al, b, c, A.SYNC_DTYPE_F32, wss[key], stream, None)

    calls = {"compute_only": (ag70((4, "chunk_major"), dict(backend=PRESET)), wss[(4, "chunk_major")])}
    for name, (split, ag) in AG70_AGENTS.items():
        calls[name] = (ag70((split, "chunk_major"), ag), wss[(split, "chunk_major")])
    t = _interleaved_medians(timer, stream, calls, steps, warmup)
    best = min(AG70_AGENTS, key=lambda nm: t[nm])
    split, ag = AG70_AGENTS[best]
    t["copy_only"] = t_of(lambda: A.sync_ag_gemm(plans[(split, "chunk_major")], cfg(flags=A.SYNC_RUN_COPY_ONLY, **ag),
                                                 ap, al, b, c, A.SYNC_DTYPE_F32, wss[(split, "chunk_major")], stream,
                                                 None), wss[(split, "chunk_major")])
    sweep = {}
    for sp in AG70_SWEEP_SPLITS:
        for o in AG70_SWEEP_ORDERS:
            tt = t_of(ag70((sp, o), AG70_SWEEP_AGENT), wss[(sp, o)])
            sweep[f"split{sp}_{o}"] = {"chunk_mib": round(32.0 / sp, 2), "t_us": round(tt * 1e6, 1)}
    flops = 2.0 * m * n * k
    out["ag_gemm_70b_like"] = {
        "workload": "AG-GEMM share: A 16384x8192 bf16 from 8 shards of 2048 rows (split 1: 32 MiB chunks, split 4: "
                    "8 MiB), B 8192x3584 bf16, C fp32; fastest of the agents timed", "agent": best,
        "chunks": int(A.sync_plan_export(plans[(split, "chunk_major")])["num_chunks"]),
        "tflops": round(flops / t[best] / 1e12, 1), "t_overlap_us": round(t[best] * 1e6, 1),
        "t_compute_only_us": round(t["compute_only"] * 1e6, 1), "t_copy_only_us": round(t["copy_only"] * 1e6, 1),
        "ratio": round(t[best] / max(t["compute_only"], t["copy_only"]), 4),
        "frac_mfma_peak": round(flops / t[best] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "t_overlap_us_by_agent": {nm: round(t[nm] * 1e6, 1) for nm in AG70_AGENTS},
        "chunk_size_x_tile_order_sweep": {"agent": "colocated", "by_split_order": sweep}}
    del ap, b, al, c, wss, plans

    return out


def a2a_row(timer, torch, inputs, stream, steps=5, warmup=2):
    """The A2A-GEMM receive side with uneven token blocks, cold cache."""
    import numpy as np

    dev = torch.device("cuda:0")
    out = {}
    t_of = _cold_median(timer, stream, steps, warmup)

    # A2A-GEMM receive side, MoE-like: 8 peers send uneven token blocks to this rank's expert
    m, n, k, w = (A2A_SHAPE[x] for x in ("m", "n", "k", "world"))
    rows = inputs.routed_token_counts(m, w)
    a_bits, b_bits = inputs.gemm_operands(m, n, k, A2A_SHAPE["divisor"], b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, w, b_layout=A.SYNC_B_NK, shard_rows=rows))
    ap = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    al = torch.zeros_like(ap)
    al[: rows[0]] = ap[: rows[0]]
    c = torch.empty((m, n), dtype=torch.float32, device=dev)
    ws = workspace(plan, torch)
    calls = {name: ((lambda ag=ag: A.sync_ag_gemm(plan, cfg(**ag), ap, al, b, c, A.SYNC_DTYPE_F32, ws, stream, None)),
                    ws) for name, ag in list(A2A_AGENTS.items()) + [("compute_only", dict(backend=PRESET))]}
    t = _interleaved_medians(timer, stream, calls, steps, warmup)
    best = min(A2A_AGENTS, key=lambda nm: t[nm])
    ag = A2A_AGENTS[best]
    t["copy_only"] = t_of(lambda: A.sync_ag_gemm(plan, cfg(flags=A.SYNC_RUN_COPY_ONLY, **ag), ap, al, b, c,
                                                 A.SYNC_DTYPE_F32, ws, stream, None), ws)
    flops = 2.0 * m * n * k
    out["a2a_gemm_moe_like"] = {
        "workload": "A2A-GEMM receive side: 8 peers send uneven token blocks " + str(rows) + " (8192 tokens, "
                    "d 4096, bf16), GEMM with B 4096x1792, C fp32; fastest of the agents timed", "agent": best,
        "tflops": round(flops / t[best] / 1e12, 1), "t_overlap_us": round(t[best] * 1e6, 1),
        "t_compute_only_us": round(t["compute_only"] * 1e6, 1), "t_copy_only_us": round(t["copy_only"] * 1e6, 1),
        "ratio": round(t[best] / max(t["compute_only"], t["copy_only"]), 4),
        "frac_mfma_peak": round(flops / t[best] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "t_overlap_us_by_agent": {nm: round(t[nm] * 1e6, 1) for nm in A2A_AGENTS}}
    del ap, b, al, c
    return out


def attention_rows(timer, torch, inputs, stream, steps=5, warmup=2):
    """The ring-attention step and the head-parallel share, cold cache."""
    import numpy as np

    dev = torch.device("cuda:0")
    out = {}

    # Ring attention: Q 4096x32x128, K/V 8 blocks of 4096 tokens x 8 heads x 128, non-causal
    sq, hq, hkv, d, nb, w = (ATTN_SHAPE[x] for x in ("sq", "hq", "hkv", "d", "n", "world"))
    q_bits, k_bits, v_bits = inputs.attention_operands(sq, hq, w * nb, hkv, d)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_RING_ATTN, sq, nb, d, w, tile_m=128, tile_n=1, heads_q=hq, heads_kv=hkv))
    q = torch.from_numpy(q_bits.view(np.int16)).to(dev)
    kp = torch.from_numpy(k_bits.view(np.int16)).to(dev)
    vp = torch.from_numpy(v_bits.view(np.int16)).to(dev)
    kl, vl = torch.zeros_like(kp), torch.zeros_like(vp)
    kl[:nb], vl[:nb] = kp[:nb], vp[:nb]
    o = torch.empty((sq, hq, d), dtype=torch.float32, device=dev)
    ms, ls, lse = (torch.empty((hq, sq), dtype=torch.float32, device=dev) for _ in range(3))
    ws = workspace(plan, torch)
    fl = A.SYNC_ATTN_INIT | A.SYNC_ATTN_FINALIZE
    calls = {name: ((lambda ag=ag: A.sync_ring_attn_step(plan, cfg(**ag), q, kp, vp, kl, vl, o, ms, ls, lse,
                                                         1.0 / d ** 0.5, fl, ws, stream, None)), ws)
             for name, ag in ATTN_AGENTS.items()}
    t = _interleaved_medians(timer, stream, calls, steps, warmup)
    best = min((x for x in ATTN_AGENTS if x != "compute_only"), key=lambda x: t[x])
    flops = 4.0 * sq * (w * nb) * hq * d
    out["ring_attention_qwen_like"] = {
        "workload": "Ring-attention local step: Q 4096x32x128 bf16, K/V 8 blocks of 4096x8x128 bf16 (7 copied), "
                    "fp32 (m, l, O); fastest of the copy agents timed",
        "best_agent": best, "tflops": round(flops / t[best] / 1e12, 1), "t_overlap_us": round(t[best] * 1e6, 1),
        "t_compute_only_us": round(t["compute_only"] * 1e6, 1),
        "ratio": round(t[best] / t["compute_only"], 4),
        "frac_mfma_peak": round(flops / t[best] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "t_us_by_agent": {nm: round(t[nm] * 1e6, 1) for nm in t}}
    del q, kp, vp, kl, vl, o, ms, ls, lse

    progress("ring attention row done")
    # Head-parallel share: Q, K, V of one head group arrive as 8 token blocks (7 from peers)
    w, nb, hq, hkv, d = (HEAD_SHAPE[x] for x in ("world", "n", "hq", "hkv", "d"))
    s = w * nb
    q_bits, k_bits, v_bits = inputs.attention_operands(s, hq, s, hkv, d)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_HEAD_ATTN, s, nb, d, w, tile_m=A.sync_attn_query_block(hq, hkv), tile_n=1,
                                   heads_q=hq, heads_kv=hkv))
    peers = [torch.from_numpy(x.view(np.int16)).to(dev) for x in (q_bits, k_bits, v_bits)]
    local = [torch.zeros_like(x) for x in peers]
    for lo, pe in zip(local, peers):
        lo[:nb] = pe[:nb]  # rank 0's own block
    o = torch.empty((s, hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((hq, s), dtype=torch.float32, device=dev)
    ws = workspace(plan, torch)
    calls = {name: ((lambda ag=ag: A.sync_head_attn(plan, cfg(**ag), *peers, *local, o, lse, 1.0 / d ** 0.5, ws,
                                                    stream, None)), ws)
             for name, ag in list(HEAD_AGENTS.items()) + [("copy_only", HEAD_COPY_ONLY)]}
    t = _interleaved_medians(timer, stream, calls, steps, warmup)
    best = min((x for x in HEAD_AGENTS if x != "compute_only"), key=lambda x: t[x])
    flops = 4.0 * s * s * hq * d
    out["head_parallel_attention_llama8b_like"] = {
        "workload": "Head-parallel attention share: 8 ranks x 4096 tokens; this rank's head group (4 query heads, "
                    "1 KV head, d 128) of all 32768 tokens arrives as 8 token blocks of Q, K and V (7 copied), "
                    "non-causal attention over all 32768 tokens, fp32 O and LSE",
        "best_agent": best, "tflops": round(flops / t[best] / 1e12, 1), "t_overlap_us": round(t[best] * 1e6, 1),
        "t_compute_only_us": round(t["compute_only"] * 1e6, 1), "t_copy_only_us": round(t["copy_only"] * 1e6, 1),
        "ratio": round(t[best] / max(t["compute_only"], t["copy_only"]), 4),
        "frac_mfma_peak": round(flops / t[best] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "t_us_by_agent": {nm: round(t[nm] * 1e6, 1) for nm in t}}
    return out


def tune(args):
    """sync_autotune on the headline workload (chunk-major order, copy teams as given)."""
    import numpy as np
    import torch

    from communication_overlap_gemm_amd import inputs

    dev = torch.device("cuda:0")
    b_layout = A.SYNC_B_NK if args.layout == "nk" else A.SYNC_B_KN
    base = A.make_desc(A.SYNC_OP_AG_GEMM, M, N, K, WORLD, b_layout=b_layout)
    agents = [A.make_cfg(**agent_for(be, teams, ks, ld)) for _, be, teams, ks, ld in TUNE_AGENTS]
    space = A.make_tune_space(splits=(1, 2, 4), tiles=((256, 256), (256, 128)), orders=(A.SYNC_ORDER_CHUNK_MAJOR,),
                              copy_cus=(), agents=agents, warmup=2, iters=5)
    a_bits, b_bits = inputs.gemm_operands(M, N, K, DIVISOR, b_layout=args.layout)
    a_peer = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    a_local = torch.zeros_like(a_peer)
    a_local[:M // WORLD] = a_peer[:M // WORLD]
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    nb = A.sync_tune_workspace_size(base, space)
    raw = torch.zeros(nb // 4 + 64, dtype=torch.int32, device=dev)
    ws = raw[((-raw.data_ptr()) % 256) // 4:]
    return A.sync_autotune(base, space, a=a_local, a_peer=a_peer, b=b, c=c, ws=ws,
                           stream=torch.cuda.current_stream())


# ---- the oracle on the host ---------------------------------------------------
def host_facts():
    """Threads the oracle runs with and what the host is."""
    import oracle

    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"threads": oracle.default_threads(), "host_cpus": os.cpu_count(), "cpu_model": model}


def cpu_baseline(a_bits, b_bits, layout):
    """The fp64 oracle on the headline product itself (all of A . B, B in the
    layout the bench used), on the host."""
    import oracle

    h = host_facts()
    t0 = time.perf_counter()
    oracle.gemm_f64(a_bits, b_bits, M, N, K, b_layout=layout, threads=h["threads"])
    dt = time.perf_counter() - t0
    return {"value": round(2.0 * M * N * K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": h["threads"],
            "kind": "oracle", "host_cpus": h["host_cpus"], "cpu_model": h["cpu_model"],
            "sample": f"the whole headline product: fp64 oracle GEMM {M}x{N}x{K} with B [{layout[0]}][{layout[1]}] "
                      f"on {h['threads']} threads, {dt:.2f} s"}


def cpu_baseline_by_config(inputs):
    """The oracle on every configuration: the whole product for the tiny AG,
    the up-projection AG (timed above) and the down-projection RS; sampled
    output rows (70B-like AG) or sampled (query, head) pairs (attention),
    scaled to the full work, for the two large ones."""
    import numpy as np

    import oracle

    h = host_facts()
    th = h["threads"]
    out = {"threads": th, "host_cpus": h["host_cpus"], "cpu_model": h["cpu_model"]}

    def gemm_row(name, m, n, k, div, sample_rows=None, reps=1):
        a, b = inputs.gemm_operands(m, n, k, div, b_layout="nk")
        rows = m if sample_rows is None else sample_rows
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.gemm_f64(np.ascontiguousarray(a[:rows]), b, rows, n, k, b_layout="nk", threads=th)
            ts.append(time.perf_counter() - t0)
        dt = float(np.median(ts))
        full = dt * m / rows
        out[name] = {"seconds": round(full, 3), "gflops": round(2.0 * m * n * k / full / 1e9, 2),
                     "measured": "whole product" + (f", median of {reps}" if reps > 1 else "") if sample_rows is None
                     else f"{rows} of {m} output rows ({dt:.2f} s), scaled by {m / rows:.0f}"}

    gemm_row("1_tiny_ag_1024", 1024, 1024, 1024, 32.0, reps=5)
    gemm_row("3_rs_llama8b_down", RS_SHAPE["m"], RS_SHAPE["n"], RS_SHAPE["k"], RS_SHAPE["divisor"])
    gemm_row("4_ag_70b_like", AG70_SHAPE["m"], AG70_SHAPE["n"], AG70_SHAPE["k"], AG70_SHAPE["divisor"],
             sample_rows=1024)
    sq, hq, hkv, d, nb, w = (ATTN_SHAPE[x] for x in ("sq", "hq", "hkv", "d", "n", "world"))
    q, kk, vv = inputs.attention_operands(sq, hq, w * nb, hkv, d)
    rng = np.random.default_rng(0)
    count = 2048
    qi, hi = rng.integers(0, sq, count), rng.integers(0, hq, count)
    t0 = time.perf_counter()
    oracle.attention_f64_sampled(q, kk, vv, 1.0 / d ** 0.5, qi, hi, threads=th)
    dt = time.perf_counter() - t0
    full = dt * sq * hq / count
    out["5_ring_attention_qwen_like"] = {"seconds": round(full, 2),
                                         "gflops": round(4.0 * sq * w * nb * hq * d / full / 1e9, 2),
                                         "measured": f"{count} of {sq * hq} (query, head) rows ({dt:.2f} s), scaled "
                                                     f"by {sq * hq / count:.0f}"}
    del q, kk, vv
    w, nb, hq, hkv, d = (HEAD_SHAPE[x] for x in ("world", "n", "hq", "hkv", "d"))
    s = w * nb
    q, kk, vv = inputs.attention_operands(s, hq, s, hkv, d)
    qi, hi = rng.integers(0, s, count), rng.integers(0, hq, count)
    t0 = time.perf_counter()
    oracle.attention_f64_sampled(q, kk, vv, 1.0 / d ** 0.5, qi, hi, threads=th)
    dt = time.perf_counter() - t0
    full = dt * s * hq / count
    out["6_head_parallel_attention_llama8b_like"] = {
        "seconds": round(full, 2), "gflops": round(4.0 * s * s * hq * d / full / 1e9, 2),
        "measured": f"{count} of {s * hq} (query, head) rows ({dt:.2f} s), scaled by {s * hq / count:.0f}"}
    return out


if __name__ == "__main__":
    main()
