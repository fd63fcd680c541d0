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
    old = """      if constexpr (REG)
        wait_lgkmcnt<PPW>();
      else
        wait_lgkmcnt<0>();"""
    new = """      acc[0][0][0] += static_cast<float>(nxt[0][0]);
      __builtin_amdgcn_sched_barrier(0);  // keep the planted use ahead of the wait
      if constexpr (REG)
        wait_lgkmcnt<PPW>();
      else
        wait_lgkmcnt<0>();"""
    assert src.count(old) == 1, "kernel text changed: update the planted variant"
    bad = src.replace(old, new)
    kdir = os.path.dirname(asm_check.KERNEL)
    for name in os.listdir(kdir):
        if name.endswith(".hpp"):
            shutil.copy(os.path.join(kdir, name), tmp_path / name)
    path = tmp_path / "gemm_persistent.hip"
    path.write_text(bad)
    n, found = asm_check.hazards(asm_check.device_assembly(str(path)))
    flagged = {f.split(":")[0] for f in found}
    # the compiler may place a wait of its own ahead of the planted use in an
    # instance (then that use is no hazard); nearly every instance must flag it
    assert n >= 12 and len(flagged) >= n - 2, (n, sorted(flagged))
