"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the C oracle (gcc, one thread)
and the expert-residency policy of the library's host code (ROCm's clang as a plain host C++
compiler: no device code is built). Each driver under tests/c/ allocates every array to its exact
size, checks the invariants of what it calls, and must end with status 0 and no sanitizer report,
leaks included."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")


def _run(exe, marker):
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
    assert marker in out.stdout
    assert "Sanitizer" not in out.stderr, out.stderr


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "sanitize_oracle")
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Wno-unknown-pragmas", *SAN,
                           os.path.join(ROOT, "tests", "c", "sanitize_oracle.c"), "-lm", "-o", exe])
    _run(exe, "oracle sanitizer checks passed")


def test_residency_policy_under_sanitizers(tmp_path):
    if not os.path.exists(CLANGXX) or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("no ROCm clang++ / HIP runtime to link against")
    exe = str(tmp_path / "sanitize_policy")
    csrc = os.path.join(ROOT, "quantized_moe_decode_router_amd", "csrc")
    built = subprocess.run([CLANGXX, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
                           os.path.join(csrc, "residency.cpp"), os.path.join(ROOT, "tests", "c", "sanitize_policy.cpp"),
                           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
                           "-o", exe], capture_output=True, text=True)
    assert built.returncode == 0, built.stderr[-4000:]
    _run(exe, "policy sanitizer checks passed")
