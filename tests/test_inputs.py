"""The seeded input generator (shared by both sides) is pinned to PyTorch's
float32 -> bfloat16 rounding and to its own determinism."""
import numpy as np
import torch

from communication_overlap_gemm_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 37,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0,
                                  3.0e38, 1e-40], dtype=np.float32)])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_roundtrip_exact_for_bf16_values():
    b = inputs.normal_bf16(5, (1000,), 64.0)
    assert np.array_equal(inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(b)), b)


def test_deterministic_and_seed_sensitive():
    a1 = inputs.normal_bf16(1, (64, 32), 32.0)
    a2 = inputs.normal_bf16(1, (64, 32), 32.0)
    a3 = inputs.normal_bf16(101, (64, 32), 32.0)
    assert np.array_equal(a1, a2) and not np.array_equal(a1, a3)


def test_nk_layout_is_transpose():
    a, b_kn = inputs.gemm_operands(8, 6, 4, 1.0, b_layout="kn")
    _, b_nk = inputs.gemm_operands(8, 6, 4, 1.0, b_layout="nk")
    assert np.array_equal(b_kn.T, b_nk)
