"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only draws numbers and encodes them as bfloat16 bit patterns; it
holds none of the method's arithmetic.  Recipe: a float32 standard normal from
``numpy.random.default_rng(seed)``, divided in float32 by the workload's scale
divisor, then rounded to bfloat16 with round-to-nearest-even.  Arrays are in
their logical row-major shape.  The result is a ``uint16`` array of bf16 bits.

Seeds used across the repository: A=1, B=2, Q=3, K=4, V=5; the alternate
("other epoch") dataset adds 100 to a seed.
"""
from __future__ import annotations

import numpy as np

SEED_A, SEED_B, SEED_Q, SEED_K, SEED_V = 1, 2, 3, 4, 5
SEED_P = 6
ALT_SEED_OFFSET = 100


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) and return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    out = ((u + bias) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, shape, divisor: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0,1)/divisor drawn with a seeded PCG64 generator."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if divisor != 1.0:
        x = x / np.float32(divisor)
    return f32_to_bf16_bits(x)


def small_int_bf16(seed: int, shape, lo: int = -2, hi: int = 2) -> np.ndarray:
    """bf16 bits of integers drawn uniformly from [lo, hi] (exact in bf16)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=tuple(shape)).astype(np.float32)
    return f32_to_bf16_bits(x)


def gemm_operands(m: int, n: int, k: int, divisor: float, b_layout: str = "kn",
                  seed_a: int = SEED_A, seed_b: int = SEED_B, integer: bool = False):
    """A [m,k] and B as bf16 bits.  B is drawn as the logical K x N matrix and
    returned either row-major [k,n] ("kn") or transposed to [n,k] ("nk")."""
    if integer:
        a = small_int_bf16(seed_a, (m, k))
        b = small_int_bf16(seed_b, (k, n))
    else:
        a = normal_bf16(seed_a, (m, k), divisor)
        b = normal_bf16(seed_b, (k, n), divisor)
    if b_layout == "nk":
        b = np.ascontiguousarray(b.T)
    elif b_layout != "kn":
        raise ValueError(f"unknown B layout {b_layout!r}")
    return a, b


def attention_operands(sq: int, hq: int, skv: int, hkv: int, d: int,
                       seed_q: int = SEED_Q, seed_k: int = SEED_K, seed_v: int = SEED_V):
    """Q [sq,hq,d], K and V [skv,hkv,d] as bf16 bits of N(0,1)."""
    q = normal_bf16(seed_q, (sq, hq, d))
    k = normal_bf16(seed_k, (skv, hkv, d))
    v = normal_bf16(seed_v, (skv, hkv, d))
    return q, k, v


def partials_f32(m: int, n: int, seed: int = SEED_P, integer: bool = False) -> np.ndarray:
    """[m, n] float32 stand-in for the partial sums a rank receives in a ring
    reduce-scatter: small integers in [-8, 8] (exact sums) or N(0,1)/8."""
    rng = np.random.default_rng(seed)
    if integer:
        return rng.integers(-8, 9, size=(m, n)).astype(np.float32)
    return (rng.standard_normal((m, n), dtype=np.float32) / np.float32(8.0)).astype(np.float32)


SEED_ROUTING = 21


def routed_token_counts(total: int, world: int, seed: int = SEED_ROUTING, alpha: float = 2.0) -> list:
    """Uneven token counts per peer for an all-to-all (MoE-like routing skew):
    a seeded Dirichlet(alpha) split of `total` tokens, each count at least 1,
    the last absorbing the rounding so that they sum to `total`."""
    rng = np.random.default_rng(seed)
    w = rng.dirichlet(np.full(world, alpha))
    rows = np.maximum(1, np.floor(w * total).astype(np.int64))
    rows[-1] += total - rows.sum()
    if rows.min() < 1 or rows.sum() != total:
        raise ValueError("cannot split the tokens into positive counts")
    return [int(x) for x in rows]
