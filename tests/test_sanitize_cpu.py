"""The host runtime and planner under AddressSanitizer and UBSan (no GPU).

The library's host sources (runtime, autotuner, SDMA agent, planner) are
built with both sanitizers on the host side only, the kernel launchers are
replaced by stand-ins that are never reached, and tests/sanitize/host_checks.cpp
drives the C ABI: plans over a wide enumeration (valid and invalid, every op
and pattern, uneven shards), the bounds of their exported tables, and every
entry point's argument checks.  Any sanitizer report fails the run.
"""
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
from communication_overlap_gemm_amd import build as B  # noqa: E402

SAN = os.path.join(HERE, "sanitize")
OUT = os.path.join(SAN, "_build")
CLANG = "/opt/rocm/llvm/bin/clang++"
HIP_HOST = ["runtime.cpp", "autotune.cpp", "sdma_engine.cpp"]
CXX = [os.path.join(B.CSRC, "planner.cpp"), os.path.join(SAN, "no_kernels.cpp"), os.path.join(SAN, "host_checks.cpp")]
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _inputs_hash():
    h = hashlib.sha256()
    srcs = [os.path.join(B.CSRC, s) for s in HIP_HOST] + CXX
    for d in (B.CSRC, os.path.join(B.CSRC, "kernels"), os.path.join(ROOT, "include")):
        srcs += sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith((".h", ".hpp")))
    for s in srcs:
        h.update(open(s, "rb").read())
    return h.hexdigest()[:16]


def _build():
    exe = os.path.join(OUT, f"host_checks_{_inputs_hash()}")
    if os.path.exists(exe):
        return exe
    shutil.rmtree(OUT, ignore_errors=True)
    os.makedirs(OUT)
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{B.CSRC}"]
    objs, procs = [], []
    for s in HIP_HOST:
        o = os.path.join(OUT, s + ".o")
        host_san = [x for f in SAN_FLAGS for x in ("-Xarch_host", f)]
        cmd = [B.HIPCC, "-O1", "-g", "-std=c++17", "-fPIC"] + inc + B.HIP_FLAGS + host_san + \
            ["-c", os.path.join(B.CSRC, s), "-o", o]
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(o)
    for s in CXX:
        o = os.path.join(OUT, os.path.basename(s) + ".o")
        cmd = [CLANG, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"] + inc + SAN_FLAGS + \
            ["-c", s, "-o", o]
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(o)
    for s, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"compile {s}:\n{out[-4000:]}"
    tmp = exe + ".tmp"
    link = [CLANG] + SAN_FLAGS + ["-o", tmp] + objs + ["-L/opt/rocm/lib", "-lamdhip64", "-lhsa-runtime64",
                                                        "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    os.replace(tmp, exe)
    return exe


@pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(B.HIPCC)), reason="ROCm clang/hipcc not found")
def test_host_runtime_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations: leak reports are left out
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # no device, also on a machine that has one
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    assert "0 failures" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    print(r.stdout.strip())
