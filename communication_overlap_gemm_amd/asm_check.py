"""Static check of the direct-to-LDS GEMM's device assembly.

The GEMM reads its MFMA fragments from LDS with inline-asm ds_read_b128 and
waits for them itself (lgkmcnt), so the compiler believes each destination
register holds its value as soon as the asm statement issues.  Any
compiler-generated instruction that reads or writes such a register before
the next lgkmcnt(0) wait would see or clobber a value the LDS has not yet
returned.  This module compiles the kernel source to gfx950 assembly and
reports every such instruction; the kernels are correct only if it reports
none.

    python -m communication_overlap_gemm_amd.asm_check   # exit status 1 on a hazard
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL = os.path.join(HERE, "csrc", "kernels", "gemm_persistent.hip")
_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(text: str) -> set[int]:
    out: set[int] = set()
    for m in _REG.finditer(text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def device_assembly(source: str = KERNEL) -> str:
    """gfx950 assembly of one kernel source, compiled as the library does."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", os.path.dirname(source), source, "-o", out],
                       check=True, capture_output=True)
        with open(out) as f:
            return f.read()


def hazards(asm: str, kernel_prefix: str = "_ZN6syncov8gemm_dma") -> tuple[int, list[str]]:
    """(kernels scanned, hazard descriptions) for kernels whose symbol starts with kernel_prefix."""
    found: list[str] = []
    kernels = 0
    kern = None
    pending: set[int] = set()
    in_asm = False
    for ln, line in enumerate(asm.split("\n"), 1):
        m = re.match(rf"^({kernel_prefix}\w*):", line)
        if m:
            kern, pending, kernels = m.group(1), set(), kernels + 1
            continue
        if kern is None:
            continue
        if line.startswith(".Lfunc_end"):
            kern = None
            continue
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        if t.startswith("s_waitcnt"):
            if "lgkmcnt(0)" in t:
                pending = set()
            continue
        if in_asm and t.startswith("ds_read_b128"):
            dst, addr = t.split(None, 1)[1].split(",", 1)
            if _regs(addr) & pending:
                found.append(f"{kern}:{ln}: address register still pending: {t}")
            pending |= _regs(dst)
            continue
        hit = _regs(t) & pending
        if hit:
            found.append(f"{kern}:{ln}: {t} touches {sorted(hit)}")
    return kernels, found


def main() -> int:
    n, found = hazards(device_assembly())
    for f in found[:50]:
        print(f)
    print(f"{n} kernels scanned, {len(found)} hazards")
    return 1 if found or n == 0 else 0


if __name__ == "__main__":
    sys.exit(main())
