"""Static checks of the GEMM's gfx950 assembly (CPU only: hipcc cross-compiles).

The direct-to-LDS GEMM issues its fragment reads as inline asm and waits for
them explicitly; the check fails if any compiler-generated instruction touches
a fragment register while its LDS read may still be in flight, following
branches through the control-flow graph.  A kernel variant that uses a
fragment before its wait is planted to show that the check catches the
hazard.
"""
import os
import shutil

import pytest

from communication_overlap_gemm_amd import asm_check

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def asm():
    return asm_check.device_assembly()


def test_no_pending_fragment_register_is_touched(asm):
    n, found = asm_check.hazards(asm)
    assert n >= 12, n  # 3 tiles x 2 C dtypes x AG/RS
    assert not found, "\n".join(found[:20])


def test_check_catches_a_use_before_the_wait(tmp_path):
    """Plant an instruction that reads a just-requested fragment register
    before the lgkmcnt wait (a VALU use of nxt[0]); the check must flag it."""
    with open(asm_check.KERNEL) as f:
        src = f.read()
    old = """      wait_lgkmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
    };"""
    new = """      acc[0][0][0] += static_cast<float>(nxt[0][0]);
      wait_lgkmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
    };"""
    assert src.count(old) == 1, "kernel text changed: update the planted variant"
    bad = src.replace(old, new)
    kdir = os.path.dirname(asm_check.KERNEL)
    for name in os.listdir(kdir):
        if name.endswith(".hpp"):
            shutil.copy(os.path.join(kdir, name), tmp_path / name)
    path = tmp_path / "gemm_persistent.hip"
    path.write_text(bad)
    n, found = asm_check.hazards(asm_check.device_assembly(str(path)))
    assert n >= 12 and len(found) >= n  # at least one per kernel
