"""Static checks of the GEMM's gfx950 assembly (CPU only: hipcc cross-compiles).

The direct-to-LDS GEMM issues its fragment reads as inline asm and waits for
them explicitly; the check fails if any compiler-generated instruction touches
a fragment register while its LDS read may still be in flight.  A kernel
variant with a runtime-conditional read (which makes the compiler emit select
code on those registers) is planted to show that the check catches the
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


def test_check_catches_conditional_reads(tmp_path):
    with open(asm_check.KERNEL) as f:
        src = f.read()
    edits = [
        ("if (x < NFRAG) nxt[x] = read_frag(nst, nkk, x);",
         "if (x < NFRAG && (nkk != 0 || live)) nxt[x] = read_frag(nst, nkk, x);"),
        ("auto mma = [&](bf16x8_t (&cur)[NFRAG], bf16x8_t (&nxt)[NFRAG], uint32_t nst, int nkk) {",
         "auto mma = [&](bf16x8_t (&cur)[NFRAG], bf16x8_t (&nxt)[NFRAG], uint32_t nst, int nkk, bool live = true) {"),
        ("mma(fq, fp, ring + ((kt + 1) % NS) * STAGE, 0);", "mma(fq, fp, ring + ((kt + 1) % NS) * STAGE, 0, kt + 1 < nk);"),
    ]
    bad = src
    for old, new in edits:
        assert old in bad, "kernel text changed: update the planted variant"
        bad = bad.replace(old, new)
    kdir = os.path.dirname(asm_check.KERNEL)
    for name in os.listdir(kdir):
        if name.endswith(".hpp"):
            shutil.copy(os.path.join(kdir, name), tmp_path / name)
    path = tmp_path / "gemm_persistent.hip"
    path.write_text(bad)
    _, found = asm_check.hazards(asm_check.device_assembly(str(path)))
    assert found
