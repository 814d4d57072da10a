"""The C ABI from plain C: tests/c/abi_consumer.c is compiled with gcc against include/moe.h,
linked to the built library and run (host-only calls and argument checks; no device needed)."""
import os
import shutil
import subprocess

import pytest

from quantized_moe_decode_router_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_uses_the_abi(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    if not os.path.exists(binding.LIB_PATH):
        from quantized_moe_decode_router_amd import build
        build.build()
    libdir = os.path.dirname(binding.LIB_PATH)
    exe = str(tmp_path / "abi_consumer")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I" + os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-L" + libdir, "-lmoe_amd",
                           "-Wl,-rpath," + libdir, "-o", exe])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "all C-ABI checks passed" in out.stdout
