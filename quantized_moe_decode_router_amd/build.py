"""Compile the HIP library (libmoe_amd.so) for gfx950 with hipcc, in-tree.

Every kernel and the C ABI live under csrc/; the result is a plain C-ABI shared object that the
ctypes binding loads. Compiled with packed-FP32 instructions disabled.

build(phase_timer=True) compiles the same sources with MOE_PHASE_TIMER into libmoe_amd_phase.so:
the decode kernel then stamps the real-time counter at the phase marks of every layer into the
workspace (bench.py --phases loads that library and summarises the stamps)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libmoe_amd.so")
PHASE_LIB = os.path.join(LIBDIR, "libmoe_amd_phase.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
SOURCES = ["moe_abi.cpp", "residency.cpp", "decode.hip", "route.hip", "batched.hip", "static_scratch.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def build(verbose: bool = False, phase_timer: bool = False) -> str:
    """Compile every source (always; callers rely on this being a real build check) and link."""
    objdir = os.path.join(LIBDIR, "phase") if phase_timer else LIBDIR
    lib = PHASE_LIB if phase_timer else LIB
    extra = ["-DMOE_PHASE_TIMER"] if phase_timer else []
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [_hipcc()] + HIPCC_FLAGS + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out = pr.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "not a recognized feature" not in l)
        if pr.returncode != 0:
            failed.append(src)
            print(out, file=sys.stderr)
        elif verbose and out.strip():
            print(out, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_timer="--phase-timer" in sys.argv))
