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
