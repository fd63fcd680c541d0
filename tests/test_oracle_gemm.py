"""Pins for the fp64 GEMM oracle (oracle/gemm_ref.c).

The oracle is the definition of a matrix product (the overlapped kernel keeps
the local kernel's semantics: Syncopate review page, "Core claim").  It is
pinned here to things other than itself: exact integer arithmetic, the
identity and permutation special cases, and numpy's float64 matmul.  Shapes are
non-square so a transposed operand or a swapped index fails.
"""
import numpy as np
import pytest

import oracle
from communication_overlap_gemm_amd import inputs


def _exact_int_product(a_bits, b_kn_bits):
    a = inputs.bf16_bits_to_f32(a_bits).astype(np.int64)
    b = inputs.bf16_bits_to_f32(b_kn_bits).astype(np.int64)
    return a @ b  # integer matmul: exact


@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_small_integer_inputs_are_exact(layout):
    m, n, k = 37, 29, 53
    a, b = inputs.gemm_operands(m, n, k, 1.0, b_layout=layout, integer=True)
    b_kn = b if layout == "kn" else np.ascontiguousarray(b.T)
    r = oracle.gemm_f64(a, b, m, n, k, b_layout=layout)
    exact = _exact_int_product(a, b_kn)
    assert np.array_equal(r, exact.astype(np.float64))


def test_identity_and_permutation():
    m, k = 19, 24
    a = inputs.normal_bf16(7, (m, k), 3.0)
    eye = inputs.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    r = oracle.gemm_f64(a, eye, m, k, k)
    assert np.array_equal(r, inputs.bf16_bits_to_f32(a).astype(np.float64))
    perm = np.random.default_rng(3).permutation(k)
    pmat = np.zeros((k, k), dtype=np.float32)
    pmat[perm, np.arange(k)] = 1.0   # column j of A.P is column perm[j] of A
    r2 = oracle.gemm_f64(a, inputs.f32_to_bf16_bits(pmat), m, k, k)
    assert np.array_equal(r2, inputs.bf16_bits_to_f32(a).astype(np.float64)[:, perm])


def test_against_numpy_float64_matmul():
    m, n, k = 96, 80, 200
    a, b = inputs.gemm_operands(m, n, k, 32.0)
    r = oracle.gemm_f64(a, b, m, n, k)
    ref = inputs.bf16_bits_to_f32(a).astype(np.float64) @ inputs.bf16_bits_to_f32(b).astype(np.float64)
    assert np.max(np.abs(r - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_sampled_matches_full():
    m, n, k = 64, 48, 96
    a, b = inputs.gemm_operands(m, n, k, 32.0, b_layout="nk")
    full = oracle.gemm_f64(a, b, m, n, k, b_layout="nk")
    rng = np.random.default_rng(0)
    rows = rng.integers(0, m, 50)
    cols = rng.integers(0, n, 50)
    s = oracle.gemm_f64_sampled(a, b, m, n, k, rows, cols, b_layout="nk")
    assert np.array_equal(s, full[rows, cols])


def test_rejects_out_of_range_samples():
    a, b = inputs.gemm_operands(4, 4, 4, 1.0)
    with pytest.raises(ValueError):
        oracle.gemm_f64_sampled(a, b, 4, 4, 4, [0, 4], [0, 0])


def test_empty_dimension():
    a = np.zeros((0, 8), dtype=np.uint16)
    b = inputs.normal_bf16(1, (8, 5))
    r = oracle.gemm_f64(a, b, 0, 5, 8)
    assert r.shape == (0, 5)
