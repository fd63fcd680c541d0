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
    assert n >= 24, n  # 3 tiles x 2 C dtypes x AG/RS x 2 B layouts
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
    new = """      acc[0][0][0] += static_cast<float>(nxt.a[0][0]);
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
    assert n >= 24 and len(flagged) >= n - 4, (n, sorted(flagged))


def _resources(asm):
    """name -> (total VGPRs incl. AGPRs, LDS bytes) of every kernel in the assembly."""
    import re
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S):
        body = m.group(2)
        vgpr = int(re.search(r"\.amdhsa_next_free_vgpr\s+(\d+)", body).group(1))
        lds = int(re.search(r"\.amdhsa_group_segment_fixed_size\s+(\d+)", body).group(1))
        out[m.group(1)] = (vgpr, lds)
    return out


def test_occupancy_the_launcher_assumes(asm):
    """128x128 tiles run two workgroups of four waves per CU (two waves per
    SIMD); the co-located backend needs every workgroup of the grid resident
    at once, so those kernels must stay within 256 VGPRs per wave and half the
    LDS.  Eight-wave 256x256 kernels must also fit two waves per SIMD."""
    res = _resources(asm)
    assert res
    checked = 0
    for name, (vgpr, lds) in res.items():
        if "ILi128ELi128E" in name:  # gemm_dma<128, 128, ...>
            assert vgpr <= 256 and 2 * lds <= 160 * 1024, (name, vgpr, lds)
            checked += 1
        if "gemm_dmaILi256ELi256E" in name:
            assert vgpr <= 256, (name, vgpr)
            checked += 1
    assert checked >= 12, checked


def test_no_scratch_in_the_gemm_kernels(asm):
    """Every gemm_dma instance (the one GEMM kernel: B stored [n][k] or [k][n],
    AG and RS, fp32 and bf16 C, all three tiles) keeps its state in registers:
    no private segment.  An out-of-line copy role once left the bf16-C
    256x256 instances with 588 bytes of scratch and 15 % slower."""
    import re
    checked = 0
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S):
        if "gemm_dma" not in m.group(1):
            continue
        scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", m.group(2)).group(1))
        assert scratch == 0, (m.group(1), scratch)
        checked += 1
    assert checked == 24, checked
