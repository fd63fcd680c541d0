"""Benchmark: AG-GEMM share, Llama-3-8B FFN up-projection at TP=8, on one MI355X.

One step = one sync_ag_gemm call, which is one kernel launch: its first
workgroups (the copy role, on 32 CUs) stage the 7 peer chunks of A
(8192 x 4096 bf16, 8 shards of 1024 rows, N(0,1)/64) from the peer HBM region,
all 7 at once in 7 teams (as pulls from every peer over a full xGMI mesh; --teams 1
copies them one after another, as along a ring), while the other workgroups
run the persistent MFMA GEMM of the gathered A
with B (4096 x 1792 bf16, stored [n][k] like a linear layer's weight by
default) into C (8192 x 1792 fp32), each tile waiting on the chunks it reads.
Inputs are resident in HBM before the timed region.

Printed: one JSON line with the metric (TFLOP/s of the overlapped call), the
overlap efficiency (overlapped time / max(compute-only, copy-only)), the
roofline of the dominant kernel (the call's kernel; its launch duration from
HIP events recorded by the library on the launch stream during the timed
steps), and the CPU oracle's throughput on a bounded sample of the same
product.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "AG-GEMM TFLOP/s (bf16, % MFMA peak) + overlap efficiency, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
M, N, K, WORLD = 8192, 1792, 4096, 8
DIVISOR = 64.0

STORE_POLICIES = {"plain": 0, "stream": 1}
# copy agents the autotuner tries: (label, bench backend, copy teams, K-slices)
TUNE_AGENTS = (("sdma_7_engines", "sdma", 7, 1), ("cu16", "cu16", 7, 4), ("cu32", "cu32", 7, 4),
               ("colocated", "colocated", 0, 1))
BACKENDS = {"sdma": (1, 0), "cu8": (2, 8), "cu16": (2, 16), "cu24": (2, 24), "cu32": (2, 32), "cu40": (2, 40),
            "cu64": (2, 64), "colocated": (4, 0)}
PROFILE = os.path.join(ROOT, "profiles", "gemm_dma_ag_llama8b_up.md")
KERNEL_SOURCES = ["gemm_persistent.hip", "copy_role.hpp", "device_common.hpp", "launch_args.hpp"]
PROFILED = {"tile": "256x256", "split": 1, "order": "chunk_major", "backend": "cu32", "c_dtype": "f32", "layout": "nk",
            "teams": 7, "kslices": 4, "copy_store": "plain"}


def profiled_traffic(args):
    """HBM bytes per overlapped launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), or None when
    the configuration differs from the profiled one or the kernel sources have
    changed since the counters were taken."""
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


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--backend", default="cu32", choices=sorted(BACKENDS))
    p.add_argument("--split", type=int, default=1)
    p.add_argument("--tile", default="256x256")
    p.add_argument("--order", default="chunk_major", choices=["row_major", "chunk_major", "swizzled"])
    p.add_argument("--c-dtype", default="f32", choices=["f32", "bf16"])
    p.add_argument("--layout", default="nk", choices=["nk", "kn"], help="B stored [n][k] or [k][n]")
    p.add_argument("--teams", type=int, default=7,
                   help="copied chunks in flight at once (1: one after another, as along a ring; 7: all, as "
                        "pulls from every peer over a full mesh)")
    p.add_argument("--kslices", type=int, default=4,
                   help="K-slices per copied chunk (1: whole chunks; >1: slice 0 of every chunk first, tiles start "
                        "on it and wait in-kernel for the later slices)")
    p.add_argument("--copy-store", default="plain", choices=sorted(STORE_POLICIES),
                   help="loads and stores of the copy role: plain or non-temporal (stream)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-other-rows", action="store_true", help="skip the RS, 70B-like AG and attention rows")
    p.add_argument("--tune", action="store_true",
                   help="run the autotuner over split {1,2,4} x tile {256x256, 256x128} x copy agent (SDMA on 7 "
                        "engines, 16 or 32 copy CUs with 4 K-slices, co-located) first and bench its choice")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported on this single-GPU "
              "build (the multi-GPU exchange is not part of it).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from communication_overlap_gemm_amd import _abi as A
    from communication_overlap_gemm_amd import inputs

    dev = torch.device("cuda:0")
    tuned = None
    if args.tune:
        tuned = tune(args)
        args.split, args.tile = tuned["split"], f'{tuned["tile_m"]}x{tuned["tile_n"]}'
        args.backend, args.teams, args.kslices = TUNE_AGENTS[tuned["agent"]][1:]
    tm, tn = (int(x) for x in args.tile.split("x"))
    order = {"row_major": A.SYNC_ORDER_ROW_MAJOR, "chunk_major": A.SYNC_ORDER_CHUNK_MAJOR,
             "swizzled": A.SYNC_ORDER_SWIZZLED}[args.order]
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
    nws = A.sync_workspace_size(plan)
    ws_raw = torch.zeros(nws // 4 + 64, dtype=torch.int32, device=dev)
    ws = ws_raw[((-ws_raw.data_ptr()) % 256) // 4:]
    stream = torch.cuda.current_stream()
    A.sync_workspace_init(plan, ws, stream)

    backend, cus = BACKENDS[args.backend]

    def timed_loop(cfg, steps, warmup, plan=plan, ws=ws):
        for _ in range(warmup):
            A.sync_ag_gemm(plan, cfg, a_peer, a_local, b, c_out, c_dtype, ws, stream, None)
        torch.cuda.synchronize()
        A.sync_read_timings(0)  # drop warm-up records
        cfg_t = A.make_cfg(cfg.backend, cfg.copy_cus, cfg.timeout_ns, None, cfg.flags | A.SYNC_RUN_TIMED,
                           copy_streaming=cfg.copy_streaming, copy_link_gbps=cfg.copy_link_gbps,
                           copy_teams=cfg.copy_teams, copy_kslices=cfg.copy_kslices)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            A.sync_ag_gemm(plan, cfg_t, a_peer, a_local, b, c_out, c_dtype, ws, stream, None)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        rc, chunk = A.sync_workspace_status(ws, stream)
        if rc != A.SYNC_OK:
            raise SystemExit(f"device wait timed out on chunk {chunk}")
        recs = A.sync_read_timings(4096)
        return wall, recs

    # overlapped (the metric), compute-only on the full chip, copy-only
    pol = STORE_POLICIES[args.copy_store]
    t_ovl, recs = timed_loop(A.make_cfg(backend, cus, copy_teams=args.teams, copy_kslices=args.kslices,
                                        copy_streaming=pol), args.steps,
                             args.warmup)
    k_ms = float(np.mean([r[0] for r in recs]))
    t_comp, recs_c = timed_loop(A.make_cfg(A.SYNC_COPY_PRESET), args.steps, args.warmup)
    k_comp_ms = float(np.mean([r[0] for r in recs_c]))
    t_copy, recs_p = timed_loop(A.make_cfg(backend, cus, flags=A.SYNC_RUN_COPY_ONLY, copy_teams=args.teams,
                                           copy_streaming=pol,
                                           copy_kslices=args.kslices), args.steps, args.warmup)
    # CU backend: the copy-only launch is the copy role alone; SDMA: the copies' span
    copy_only_ms = float(np.mean([r[1] if backend == A.SYNC_COPY_SDMA else r[0] for r in recs_p]))
    # (co-located: the copy-only launch is every workgroup copying, none computing)

    # copy-backend sweep on the same workload (a few timed calls each): SDMA on
    # one engine (as one ring link) and on seven (as pulls from seven peers),
    # 8/16/32 dedicated copy CUs (7 teams, 4 K-slices), co-located copy, and
    # 32 copy CUs paced as xGMI links of 153 GB/s: one link carrying every
    # chunk (ring) or seven links at once (mesh)
    sweep = {}
    if not args.no_other_rows:
        for sname, (sb, scus, steams, sks, gbps) in (("sdma_1_engine", (A.SYNC_COPY_SDMA, 0, 1, 1, 0.0)),
                                                      ("sdma_7_engines", (A.SYNC_COPY_SDMA, 0, 7, 1, 0.0)),
                                                      ("cu8", (A.SYNC_COPY_CU, 8, 7, 4, 0.0)),
                                                      ("cu16", (A.SYNC_COPY_CU, 16, 7, 4, 0.0)),
                                                      ("cu32", (A.SYNC_COPY_CU, 32, 7, 4, 0.0)),
                                                      ("colocated", (A.SYNC_COPY_COLOCATED, 0, 0, 1, 0.0)),
                                                      ("cu32_xgmi_ring_153", (A.SYNC_COPY_CU, 32, 1, 4, 153.0)),
                                                      ("cu32_xgmi_mesh_153", (A.SYNC_COPY_CU, 32, 7, 4, 153.0))):
            t_o, _ = timed_loop(A.make_cfg(sb, scus, copy_teams=steams, copy_kslices=sks, copy_link_gbps=gbps), 10, 3)
            t_c, _ = timed_loop(A.make_cfg(sb, scus, flags=A.SYNC_RUN_COPY_ONLY, copy_teams=steams,
                                           copy_kslices=sks, copy_link_gbps=gbps), 10, 3)
            sweep[sname] = {"t_overlap_us": round(t_o * 1e6, 1), "t_copy_only_us": round(t_c * 1e6, 1),
                            "tflops": round(2.0 * M * N * K / t_o / 1e12, 1),
                            "ratio": round(t_o / max(t_comp, t_c), 4)}

    flops = 2.0 * M * N * K
    value = flops / t_ovl / 1e12
    achieved = flops / (k_ms * 1e-3) / 1e12
    copied = sum(int(tabs["chunk_begin"][c + 1] - tabs["chunk_begin"][c]) for c in range(tabs["num_chunks"])
                 if not tabs["resident"][c]) * K * 2
    kname = ("gemm_dma" if args.layout == "nk" else "gemm_persistent") + \
        f"<{tm},{tn},{args.c_dtype},AG>" + (f" with {cus} copy workgroups" if backend == A.SYNC_COPY_CU else
                                              " with co-located copy" if backend == A.SYNC_COPY_COLOCATED else "")
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
            "copy_kslices": args.kslices, "copy_store": args.copy_store, "b_layout": args.layout,
        },
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "overlap": {
            "t_overlap_ms": round(t_ovl * 1e3, 4),
            "t_compute_only_ms": round(t_comp * 1e3, 4),
            "t_copy_only_ms": round(t_copy * 1e3, 4),
            "ratio": round(t_ovl / max(t_comp, t_copy), 4),
            "kernel_ms_overlapped": round(k_ms, 4),
            "gemm_kernel_ms_compute_only": round(k_comp_ms, 4),
            "copy_ms": round(copy_only_ms, 4),
            "copy_GBps": round(2 * copied / (copy_only_ms * 1e-3) / 1e9, 1),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": profiled_traffic(args),
            "kernel": kname,
            "flops_per_launch": flops,
        },
    }
    if tuned is not None:
        line["autotune"] = tuned
    if sweep:
        line["copy_backend_sweep"] = sweep
    if not args.no_other_rows:
        # split factor (sub-chunks per peer shard: chunks of 8, 4 and 2 MiB)
        split_sweep = {}
        for sp in (1, 2, 4):
            pl = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, M, N, K, WORLD, split=sp, tile_m=tm, tile_n=tn,
                                         tile_order=order, b_layout=b_layout))
            w_raw = torch.zeros(A.sync_workspace_size(pl) // 4 + 64, dtype=torch.int32, device=dev)
            w = w_raw[((-w_raw.data_ptr()) % 256) // 4:]
            A.sync_workspace_init(pl, w, stream)
            for sname, (sb, scus, steams, sks) in (("cu32", (A.SYNC_COPY_CU, 32, 7, 4)),
                                                    ("sdma_7_engines", (A.SYNC_COPY_SDMA, 0, 7, 1))):
                t_o, _ = timed_loop(A.make_cfg(sb, scus, copy_teams=steams, copy_kslices=sks), 10, 3, pl, w)
                t_c, _ = timed_loop(A.make_cfg(sb, scus, flags=A.SYNC_RUN_COPY_ONLY, copy_teams=steams,
                                               copy_kslices=sks), 10, 3, pl, w)
                split_sweep[f"split{sp}_{sname}"] = {"chunk_mib": round(8.0 / sp, 2),
                                                     "t_overlap_us": round(t_o * 1e6, 1),
                                                     "t_copy_only_us": round(t_c * 1e6, 1),
                                                     "ratio": round(t_o / max(t_comp, t_c), 4)}
            del w_raw
        line["split_sweep"] = split_sweep
    if not args.no_other_rows:
        del a_peer, a_local, b, c_out
        line["other_rows"] = other_rows(pol=pol)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a_bits, b_bits, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def tune(args):
    """sync_autotune on the headline workload (chunk-major order, copy teams as given)."""
    import numpy as np
    import torch

    from communication_overlap_gemm_amd import _abi as A
    from communication_overlap_gemm_amd import inputs

    dev = torch.device("cuda:0")
    b_layout = A.SYNC_B_NK if args.layout == "nk" else A.SYNC_B_KN
    base = A.make_desc(A.SYNC_OP_AG_GEMM, M, N, K, WORLD, b_layout=b_layout)
    agents = [A.make_cfg(BACKENDS[be][0], BACKENDS[be][1], copy_teams=teams, copy_kslices=ks)
              for _, be, teams, ks in TUNE_AGENTS]
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


def _time_calls(fn, steps, warmup):
    """Mean seconds per call of fn() on the current stream (device events), after warm-up."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e-3


def _ws(plan, torch, A):
    n = A.sync_workspace_size(plan)
    raw = torch.zeros(n // 4 + 64, dtype=torch.int32, device="cuda:0")
    ws = raw[((-raw.data_ptr()) % 256) // 4:]
    A.sync_workspace_init(plan, ws, torch.cuda.current_stream())
    return ws


def other_rows(steps=5, warmup=2, pol=0):
    """The other rows of the hot path on their configurations (one line each in
    the output): GEMM-RS share (Llama-3-8B down-projection), AG-GEMM share
    (70B-like FFN), A2A-GEMM receive side (MoE-like uneven token blocks),
    ring-attention local step (Qwen-like GQA)."""
    import numpy as np
    import torch

    from communication_overlap_gemm_amd import _abi as A
    from communication_overlap_gemm_amd import inputs

    dev = torch.device("cuda:0")
    s = torch.cuda.current_stream()
    out = {}

    def check(ws):
        rc, ch = A.sync_workspace_status(ws, s)
        if rc != A.SYNC_OK:
            raise SystemExit(f"device wait timed out on chunk {ch}")

    # GEMM-RS: A 8192x1792, B 1792x4096 (stored [n][k]), C fp32, copy-out on 32 CUs in send order
    m, n, k, w = 8192, 4096, 1792, 8
    a_bits, b_bits = inputs.gemm_operands(m, n, k, 64.0, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, m, n, k, w, b_layout=A.SYNC_B_NK))
    a = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    c = torch.empty((m, n), dtype=torch.float32, device=dev)
    st = torch.empty_like(c)
    ws = _ws(plan, torch, A)
    t = {}
    for name, cfg in (("overlapped", A.make_cfg(A.SYNC_COPY_EPILOGUE)),
                      ("overlapped_colocated", A.make_cfg(A.SYNC_COPY_COLOCATED, copy_teams=8, copy_streaming=pol)),
                      ("overlapped_32_copy_cus", A.make_cfg(A.SYNC_COPY_CU, 32, copy_streaming=pol)),
                      ("compute_only", A.make_cfg(A.SYNC_COPY_PRESET))):
        t[name] = _time_calls(lambda: A.sync_gemm_rs(plan, cfg, a, b, c, A.SYNC_DTYPE_F32, st, ws, s, None), steps,
                              warmup)
        check(ws)
    # epilogue backend with C left unwritten: the send slots are the only output
    t["send_only"] = _time_calls(
        lambda: A.sync_gemm_rs(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), a, b, None, A.SYNC_DTYPE_F32, st, ws, s, None),
        steps, warmup)
    check(ws)
    # the same with its reduce-scatter step: each send slot = own tile + incoming partial sums
    part = torch.from_numpy(inputs.partials_f32(m, n)).to(dev)
    t["overlapped_reduce_step"] = _time_calls(
        lambda: A.sync_gemm_rs_reduce(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), a, b, c, part, st, ws, s, None), steps,
        warmup)
    check(ws)
    # GEMM-AR share: that reduce-scatter step, then the all-gather of the reduced chunks (every
    # workgroup joins it once its tiles are stored)
    peer = torch.from_numpy(inputs.partials_f32(m, n, seed=inputs.SEED_P + inputs.ALT_SEED_OFFSET)).to(dev)
    out_ar = torch.empty_like(c)
    t["gemm_ar"] = _time_calls(
        lambda: A.sync_gemm_ar(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), a, b, c, part, peer, out_ar, st, ws, s, None),
        steps, warmup)
    check(ws)
    t["gemm_ar_no_c"] = _time_calls(
        lambda: A.sync_gemm_ar(plan, A.make_cfg(A.SYNC_COPY_EPILOGUE), a, b, None, part, peer, out_ar, st, ws, s, None),
        steps, warmup)
    check(ws)
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
        "t_overlap_send_slots_only_us": round(t["send_only"] * 1e6, 1),
        "t_overlap_with_reduce_step_us": round(t["overlapped_reduce_step"] * 1e6, 1),
        "t_gemm_ar_share_us": round(t["gemm_ar"] * 1e6, 1),
        "t_gemm_ar_share_without_c_us": round(t["gemm_ar_no_c"] * 1e6, 1),
        "t_overlap_32_copy_cus_us": round(t["overlapped_32_copy_cus"] * 1e6, 1),
        "ratio_to_compute_only": round(t["overlapped"] / t["compute_only"], 4),
        "frac_mfma_peak": round(flops / t["overlapped"] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "hbm_bound_us": round(hbm / 8e12 * 1e6, 1), "frac_hbm_roofline": round(hbm / 8e12 / t["overlapped"], 4)}
    del a, b, c, st

    # AG-GEMM 70B-like: A 16384x8192 (8 shards of 2048 rows), B 8192x3584, C fp32; a few copy agents and
    # splits timed live, the fastest reported as the row's figure
    m, n, k = 16384, 3584, 8192
    a_bits, b_bits = inputs.gemm_operands(m, n, k, 90.0, b_layout="nk")
    ap = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    al = torch.zeros_like(ap)
    r = m // w
    al[:r] = ap[:r]
    c = torch.empty((m, n), dtype=torch.float32, device=dev)
    agents = {"split4_cu32_7teams": (4, A.make_cfg(A.SYNC_COPY_CU, 32, copy_teams=7, copy_streaming=pol)),
              "split4_cu16_7teams": (4, A.make_cfg(A.SYNC_COPY_CU, 16, copy_teams=7, copy_streaming=pol)),
              "split4_colocated": (4, A.make_cfg(A.SYNC_COPY_COLOCATED, copy_streaming=pol)),
              "split1_colocated": (1, A.make_cfg(A.SYNC_COPY_COLOCATED, copy_streaming=pol))}
    t, plans = {}, {}
    for split in (1, 4):
        plans[split] = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, w, split=split, b_layout=A.SYNC_B_NK))
    wss = {sp: _ws(plans[sp], torch, A) for sp in plans}  # one workspace per plan
    ws = wss[4]
    t["compute_only"] = _time_calls(lambda: A.sync_ag_gemm(plans[4], A.make_cfg(A.SYNC_COPY_PRESET), ap, al, b, c,
                                                           A.SYNC_DTYPE_F32, ws, s, None), steps, warmup)
    check(ws)
    for name, (split, cfg) in agents.items():
        t[name] = _time_calls(lambda: A.sync_ag_gemm(plans[split], cfg, ap, al, b, c, A.SYNC_DTYPE_F32, wss[split], s,
                                                     None), steps, warmup)
        check(wss[split])
    best = min(agents, key=lambda nm: t[nm])
    split, cfg = agents[best]
    cfg_copy = A.make_cfg(cfg.backend, cfg.copy_cus, flags=A.SYNC_RUN_COPY_ONLY, copy_teams=cfg.copy_teams,
                          copy_streaming=pol)
    t["copy_only"] = _time_calls(lambda: A.sync_ag_gemm(plans[split], cfg_copy, ap, al, b, c, A.SYNC_DTYPE_F32,
                                                        wss[split], s, None), steps, warmup)
    check(wss[split])
    flops = 2.0 * m * n * k
    out["ag_gemm_70b_like"] = {
        "workload": "AG-GEMM share: A 16384x8192 bf16 from 8 shards of 2048 rows (split 1: 32 MiB chunks, split 4: "
                    "8 MiB), B 8192x3584 bf16, C fp32; fastest of the agents timed", "agent": best,
        "chunks": int(A.sync_plan_export(plans[split])["num_chunks"]),
        "tflops": round(flops / t[best] / 1e12, 1), "t_overlap_us": round(t[best] * 1e6, 1),
        "t_compute_only_us": round(t["compute_only"] * 1e6, 1), "t_copy_only_us": round(t["copy_only"] * 1e6, 1),
        "ratio": round(t[best] / max(t["compute_only"], t["copy_only"]), 4),
        "frac_mfma_peak": round(flops / t[best] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "t_overlap_us_by_agent": {nm: round(t[nm] * 1e6, 1) for nm in agents}}
    del ap, b, al, c, ws, wss

    # A2A-GEMM receive side, MoE-like: 8 peers send uneven token blocks (seeded Dirichlet(2) routing skew,
    # 8192 tokens in all) of d_model 4096 to this rank's expert, up-projection to 1792, C fp32
    m, n, k = 8192, 1792, 4096
    rng = np.random.default_rng(21)
    rows = np.maximum(1, np.floor(rng.dirichlet(np.full(w, 2.0)) * m).astype(np.int64))
    rows[-1] += m - rows.sum()
    rows = [int(x) for x in rows]
    a_bits, b_bits = inputs.gemm_operands(m, n, k, 64.0, b_layout="nk")
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, m, n, k, w, b_layout=A.SYNC_B_NK, shard_rows=rows))
    ap = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    b = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    al = torch.zeros_like(ap)
    al[:rows[0]] = ap[:rows[0]]
    c = torch.empty((m, n), dtype=torch.float32, device=dev)
    ws = _ws(plan, torch, A)
    # copy agents timed live, the fastest reported: 7 teams (one block per team, so the largest block sets the
    # copy time), one team (all copy workgroups on each block in turn), co-located copy
    agents = {"cu32_7teams_4slices": A.make_cfg(A.SYNC_COPY_CU, 32, copy_teams=7, copy_kslices=4),
              "cu32_1team_4slices": A.make_cfg(A.SYNC_COPY_CU, 32, copy_teams=1, copy_kslices=4),
              "colocated": A.make_cfg(A.SYNC_COPY_COLOCATED),
              "colocated_4slices": A.make_cfg(A.SYNC_COPY_COLOCATED, copy_kslices=4)}
    t = {}
    for name, cfg in list(agents.items()) + [("compute_only", A.make_cfg(A.SYNC_COPY_PRESET))]:
        t[name] = _time_calls(lambda: A.sync_ag_gemm(plan, cfg, ap, al, b, c, A.SYNC_DTYPE_F32, ws, s, None), steps,
                              warmup)
        check(ws)
    best = min(agents, key=lambda nm: t[nm])
    cfg = agents[best]
    cfg_copy = A.make_cfg(cfg.backend, cfg.copy_cus, flags=A.SYNC_RUN_COPY_ONLY, copy_teams=cfg.copy_teams,
                          copy_kslices=cfg.copy_kslices)
    t["copy_only"] = _time_calls(lambda: A.sync_ag_gemm(plan, cfg_copy, ap, al, b, c, A.SYNC_DTYPE_F32, ws, s, None),
                                 steps, warmup)
    check(ws)
    flops = 2.0 * m * n * k
    out["a2a_gemm_moe_like"] = {
        "workload": "A2A-GEMM receive side: 8 peers send uneven token blocks " + str(rows) + " (8192 tokens, "
                    "d 4096, bf16), GEMM with B 4096x1792, C fp32; fastest of the agents timed", "agent": best,
        "tflops": round(flops / t[best] / 1e12, 1), "t_overlap_us": round(t[best] * 1e6, 1),
        "t_compute_only_us": round(t["compute_only"] * 1e6, 1), "t_copy_only_us": round(t["copy_only"] * 1e6, 1),
        "ratio": round(t[best] / max(t["compute_only"], t["copy_only"]), 4),
        "frac_mfma_peak": round(flops / t[best] / 1e12 / PEAK_BF16_TFLOPS, 4),
        "t_overlap_us_by_agent": {nm: round(t[nm] * 1e6, 1) for nm in agents}}
    del ap, b, al, c

    # Ring attention: Q 4096x32x128, K/V 8 blocks of 4096 tokens x 8 heads x 128, non-causal
    sq, hq, hkv, d, nb = 4096, 32, 8, 128, 4096
    q_bits, k_bits, v_bits = inputs.attention_operands(sq, hq, w * nb, hkv, d)
    plan = A.sync_plan(A.make_desc(A.SYNC_OP_RING_ATTN, sq, nb, d, w, tile_m=128, tile_n=1, heads_q=hq, heads_kv=hkv))
    q = torch.from_numpy(q_bits.view(np.int16)).to(dev)
    kp = torch.from_numpy(k_bits.view(np.int16)).to(dev)
    vp = torch.from_numpy(v_bits.view(np.int16)).to(dev)
    kl, vl = torch.zeros_like(kp), torch.zeros_like(vp)
    kl[:nb], vl[:nb] = kp[:nb], vp[:nb]
    o = torch.empty((sq, hq, d), dtype=torch.float32, device=dev)
    ms, ls, lse = (torch.empty((hq, sq), dtype=torch.float32, device=dev) for _ in range(3))
    ws = _ws(plan, torch, A)
    t = {}
    fl = A.SYNC_ATTN_INIT | A.SYNC_ATTN_FINALIZE
    for name, cfg in (("overlapped", A.make_cfg(A.SYNC_COPY_COLOCATED, copy_streaming=pol)),
                      ("overlapped_32_copy_cus", A.make_cfg(A.SYNC_COPY_CU, 32, copy_teams=7, copy_streaming=pol)),
                      ("compute_only", A.make_cfg(A.SYNC_COPY_PRESET))):
        t[name] = _time_calls(lambda: A.sync_ring_attn_step(plan, cfg, q, kp, vp, kl, vl, o, ms, ls, lse,
                                                            1.0 / d ** 0.5, fl, ws, s, None), steps, warmup)
        check(ws)
    flops = 4.0 * sq * (w * nb) * hq * d
    out["ring_attention_qwen_like"] = {
        "workload": "Ring-attention local step: Q 4096x32x128 bf16, K/V 8 blocks of 4096x8x128 bf16, fp32 (m, l, O), "
                    "co-located copy (every workgroup pulls its share of K and V, then computes)",
        "tflops": round(flops / t["overlapped"] / 1e12, 1), "t_overlap_us": round(t["overlapped"] * 1e6, 1),
        "t_overlap_32_copy_cus_us": round(t["overlapped_32_copy_cus"] * 1e6, 1),
        "t_compute_only_us": round(t["compute_only"] * 1e6, 1),
        "ratio": round(t["overlapped"] / t["compute_only"], 4),
        "frac_mfma_peak": round(flops / t["overlapped"] / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return out


def cpu_baseline(a_bits, b_bits, target_s):
    """The fp64 oracle on the first R rows of A (R sized for ~target_s seconds)."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    rows = 16
    t0 = time.perf_counter()
    oracle.gemm_f64(a_bits[:rows], b_bits, rows, N, K, threads=threads)
    probe = time.perf_counter() - t0
    rows = int(max(16, min(M, rows * target_s / max(probe, 1e-3))))
    rows -= rows % 16
    t0 = time.perf_counter()
    oracle.gemm_f64(np.ascontiguousarray(a_bits[:rows]), b_bits, rows, N, K, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 oracle GEMM on the first {rows} of {M} rows of A (full N={N}, K={K}); {dt:.1f} s"}


if __name__ == "__main__":
    main()
