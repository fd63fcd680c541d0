"""Helpers for the GPU tests: device buffers for bf16 bit arrays, plans,
workspaces and the error metrics the parity tests use."""
from __future__ import annotations

import numpy as np
import torch

from communication_overlap_gemm_amd import _abi as A
from communication_overlap_gemm_amd import inputs

DEV = "cuda:0"


def dev_bits(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits -> int16 device tensor with the same bytes."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_poison(shape) -> torch.Tensor:
    """int16 tensor holding bf16 quiet NaNs."""
    return torch.full(shape, 0x7FC0, dtype=torch.int16, device=DEV)


def workspace(plan) -> torch.Tensor:
    n = A.sync_workspace_size(plan)
    ws = torch.empty((n + 255) // 4 + 64, dtype=torch.int32, device=DEV)
    off = (-ws.data_ptr()) % 256
    ws = ws[off // 4: off // 4 + n // 4]
    A.sync_workspace_init(plan, ws, torch.cuda.current_stream())
    return ws


def shard_frobenius(c: np.ndarray, r: np.ndarray, world: int) -> float:
    """max over row shards of ||C_s - R_s||_F / ||R_s||_F."""
    worst = 0.0
    for s in np.array_split(np.arange(c.shape[0]), world):
        num = np.linalg.norm((c[s] - r[s]).ravel())
        den = np.linalg.norm(r[s].ravel())
        worst = max(worst, num / den if den > 0 else num)
    return worst


def bf16_round(x: np.ndarray) -> np.ndarray:
    return inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(x.astype(np.float32)))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (x already a bf16 value)."""
    ax = np.abs(x.astype(np.float32))
    e = np.floor(np.log2(np.maximum(ax, np.float32(2.0 ** -126))))
    return np.float32(2.0) ** (e - 7)


def check_full_f32(out: np.ndarray, ref: np.ndarray, absab: np.ndarray, k: int, world: int) -> float:
    """Whole-output parity of an fp32-accumulated product against the fp64
    oracle R: every element within the worst-case bound of a K-term fp32 sum
    in any order, |C - R| <= K 2^-24 (|A||B|) (plus one fp32 ulp of slack for
    the final rounding), and the per-row-shard relative Frobenius error at
    most 1e-3.  A stale, missing or misplaced tile fails the first check."""
    assert out.shape == ref.shape
    assert np.isfinite(out).all(), f"{(~np.isfinite(out)).sum()} non-finite outputs"
    o = out.astype(np.float64)
    bound = k * 2.0 ** -24 * absab + np.abs(ref) * 2.0 ** -23
    bad = np.abs(o - ref) > bound
    if bad.any():
        idx = np.argwhere(bad)
        raise AssertionError(f"{bad.sum()} outputs outside the fp32 accumulation bound; first {idx[:6].tolist()} "
                             f"got {o[bad][:6]} want {ref[bad][:6]}")
    err = shard_frobenius(o, ref, world)
    assert err <= 1e-3, err
    return err
