"""Static check of the direct-to-LDS GEMM's device assembly.

The GEMM reads its MFMA fragments from LDS with inline-asm ds_read_b128 (and,
for B stored [k][n], the transposing ds_read_b64_tr_b16) and waits for them
itself (lgkmcnt), so the compiler believes each destination
register holds its value as soon as the asm statement issues.  Any
compiler-generated instruction that reads or writes such a register before a
wait that covers the read would see or clobber a value the LDS has not yet
returned.  LDS operations of one wave complete in issue order, so
lgkmcnt(N) covers a read once N or more LDS operations were issued after it.
This module compiles the kernel source to gfx950 assembly and reports every
such instruction; the kernels are correct only if it reports none.

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


def _kernels(asm: str, kernel_prefix: str):
    """(name, [lines]) of every kernel whose symbol starts with kernel_prefix."""
    out, cur, name = [], None, None
    for line in asm.split("\n"):
        m = re.match(rf"^({kernel_prefix}\w*):", line)
        if m:
            name, cur = m.group(1), []
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            out.append((name, cur))
            cur = None
            continue
        cur.append(line)
    return out


def _blocks(lines: list[str]):
    """Basic blocks [label, [(line index, instruction, is_asm)], successor labels].
    A block ends at a label, a branch or a terminator; it falls through to the
    next block unless it ends in an unconditional branch or a terminator."""
    blocks: list = []
    in_asm = False
    counter = 0

    def new_block(label):
        blocks.append([label, [], []])

    new_block("<entry>")
    for i, line in enumerate(lines):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^(\.L\w+):", t)
        if m:
            new_block(m.group(1))
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        blocks[-1][1].append((i, t, in_asm))
        bm = re.match(r"^s_(c?branch\w*)\s+(\.L\w+)", t)
        if bm or re.match(r"^(s_endpgm|s_setpc|s_trap)", t):
            if bm:
                blocks[-1][2].append(bm.group(2))
            counter += 1
            new_block(f"<after {counter}>")
    for k, blk in enumerate(blocks[:-1]):
        last = blk[1][-1][1] if blk[1] else ""
        if not _ends_block(last):
            blk[2].append(blocks[k + 1][0])  # fall through
    return blocks


def _ends_block(instr: str) -> bool:
    """Unconditional transfer: no fall-through."""
    return bool(re.match(r"^(s_branch\s|s_endpgm|s_setpc|s_trap)", instr))


_LGKM = re.compile(r"lgkmcnt\((\d+)\)")
_ASM_READS = ("ds_read_b128", "ds_read_b64_tr_b16")  # the kernel's inline-asm fragment reads
_CAP = 16  # LDS operations issued after a read, counted up to this


def _transfer(block, pending: frozenset, report=None, name=""):
    """pending: frozenset of (register, LDS operations issued since its read)."""
    pend = dict()
    for r, n in pending:  # a register pending along several paths keeps its smallest count
        pend[r] = min(n, pend.get(r, _CAP))
    for i, t, is_asm in block[1]:
        if t.startswith("s_waitcnt"):
            m = _LGKM.search(t)
            if m:
                n = int(m.group(1))
                pend = {r: c for r, c in pend.items() if c < n}
            continue
        if t.startswith("ds_"):
            if is_asm and t.startswith(_ASM_READS):
                dst, addr = t.split(None, 1)[1].split(",", 1)
                if report is not None and _regs(addr) & set(pend):
                    report.append(f"{name}:{i}: address register still pending: {t}")
            else:
                dst = ""
            hit = _regs(t) & set(pend) if not is_asm else set()
            if hit and report is not None:
                report.append(f"{name}:{i}: {t} touches {sorted(hit)}")
            pend = {r: min(c + 1, _CAP) for r, c in pend.items()}
            for r in _regs(dst):
                pend[r] = 0
            continue
        hit = _regs(t) & set(pend)
        if hit and report is not None:
            report.append(f"{name}:{i}: {t} touches {sorted(hit)}")
    return frozenset(pend.items())


def hazards(asm: str, kernel_prefix: str = "_ZN6syncov8gemm_dma") -> tuple[int, list[str]]:
    """(kernels scanned, hazard descriptions) for kernels whose symbol starts with
    kernel_prefix.  Pending fragment registers are propagated along the
    control-flow graph (branches and fall-through) to a fixpoint, so a read
    whose wait sits in another block is followed through the branch."""
    found: list[str] = []
    kernels = _kernels(asm, kernel_prefix)
    for name, lines in kernels:
        blocks = _blocks(lines)
        index = {b[0]: k for k, b in enumerate(blocks)}
        entry = [frozenset() for _ in blocks]
        work = list(range(len(blocks)))
        while work:
            k = work.pop()
            out = _transfer(blocks[k], entry[k])
            for succ in blocks[k][2]:
                j = index.get(succ)
                if j is None:
                    continue
                merged = entry[j] | out
                if merged != entry[j]:
                    entry[j] = merged
                    work.append(j)
        for k, blk in enumerate(blocks):
            _transfer(blk, entry[k], found, name)
    return len(kernels), found


def main() -> int:
    n, found = hazards(device_assembly())
    for f in found[:50]:
        print(f)
    print(f"{n} kernels scanned, {len(found)} hazards")
    return 1 if found or n == 0 else 0


if __name__ == "__main__":
    sys.exit(main())
