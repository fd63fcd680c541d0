import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _whole_product(m, n, k, divisor):
    """Operands of a full-size GEMM share (B drawn as the logical K x N matrix)
    with the oracle's whole product R and |A||B| (the latter bounds the fp32
    accumulation error element by element)."""
    import oracle
    from communication_overlap_gemm_amd import inputs

    a, b_kn = inputs.gemm_operands(m, n, k, divisor, b_layout="kn")
    ref = oracle.gemm_f64(a, b_kn, m, n, k)
    absab = oracle.gemm_f64(a & 0x7FFF, b_kn & 0x7FFF, m, n, k)
    return a, b_kn, ref, absab


@pytest.fixture(scope="session")
def cfg2_data():
    """Llama-3-8B up-projection AG share: A 8192x4096, B 4096x1792, N(0,1)/64."""
    return _whole_product(8192, 1792, 4096, 64.0)


@pytest.fixture(scope="session")
def cfg3_data():
    """Llama-3-8B down-projection RS share: A 8192x1792, B 1792x4096, N(0,1)/64."""
    return _whole_product(8192, 4096, 1792, 64.0)
