"""The C-ABI library without a GPU: it loads, exports every symbol include/moe.h declares, and
its host-side checks reject bad arguments before anything is enqueued (no kernel is launched)."""
import ctypes
import os
import re

import pytest

import quantized_moe_decode_router_amd as moe
from quantized_moe_decode_router_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from quantized_moe_decode_router_amd import build
        build.build()
    return moe.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 7, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding.EXPORTED)


def test_status_strings(L):
    assert moe.status_string(0) == "MOE_OK"
    assert moe.status_string(5) == "MOE_ERR_TIMEOUT"
    assert moe.status_string(99) == "MOE_ERR_UNKNOWN"


def S(**kw):
    d = dict(hidden=2048, num_experts=256, top_k=8, inter=512, shared_inter=512, bits=4, group_size=64)
    d.update(kw)
    return binding.MoeShape(**d)


def ws(shape, T=1, kind=0, L=1):
    return binding.lib().moe_workspace_bytes(ctypes.byref(shape), T, L, kind)


def test_workspace_bytes_and_shape_checks(L):
    assert ws(S()) > 0
    assert ws(S(), T=8) > ws(S(), T=1)
    assert ws(S(), T=9, kind=0) == 0  # decode takes at most 8 tokens
    assert ws(S(), T=512, kind=1) > 0
    assert ws(S(), kind=2, L=40) > ws(S(), kind=2, L=1) == ws(S(), kind=0)
    assert ws(S(), kind=2, L=0) == 0
    assert ws(S(bits=3)) == 0
    assert ws(S(group_size=32)) == 0
    assert ws(S(top_k=300)) == 0  # K > E
    assert ws(S(hidden=2000)) == 0
    assert ws(S(hidden=1984)) == 0  # multiple of 64 but not a power of two: unsupported
    assert ws(S(inter=0)) == 0


def _call_decode(shape, layer, x=1 << 20, T=1, y=1 << 20, ws_ptr=1 << 20, ws_bytes=1 << 24):
    return binding.lib().moe_layer_decode(ctypes.byref(shape), ctypes.byref(layer) if layer else None,
                                          x, T, y, None, None, None, ws_ptr, ws_bytes, None)


def _fake_layer(align=16, shared=True):
    a = 1 << 24
    q = lambda base: binding.MoeQWeight(base, base + a, base + 2 * a)
    return binding.MoeLayer(a * 10 + align % 16, None, a * 11 if shared else None, q(a * 20), q(a * 30),
                            q(a * 40) if shared else binding.MoeQWeight(), q(a * 50) if shared else binding.MoeQWeight())


def test_decode_argument_errors_are_caught_on_host(L):
    # every case fails a host-side check, so no kernel is launched and no device is needed
    assert _call_decode(S(), None) == moe.MOE_ERR_INVALID_ARG
    assert _call_decode(S(bits=3), _fake_layer()) == moe.MOE_ERR_UNSUPPORTED
    assert _call_decode(S(bits=0), _fake_layer()) == moe.MOE_ERR_INVALID_ARG
    assert _call_decode(S(top_k=257), _fake_layer()) == moe.MOE_ERR_INVALID_ARG
    assert _call_decode(S(top_k=17), _fake_layer()) == moe.MOE_ERR_UNSUPPORTED
    assert _call_decode(S(hidden=2000), _fake_layer()) == moe.MOE_ERR_INVALID_ARG
    assert _call_decode(S(group_size=128), _fake_layer()) == moe.MOE_ERR_UNSUPPORTED
    assert _call_decode(S(), _fake_layer(align=4)) == moe.MOE_ERR_INVALID_ARG  # misaligned router
    assert _call_decode(S(), _fake_layer(shared=False)) == moe.MOE_ERR_INVALID_ARG  # shared missing
    assert _call_decode(S(), _fake_layer(), T=0) == moe.MOE_ERR_INVALID_ARG
    assert _call_decode(S(), _fake_layer(), T=9) == moe.MOE_ERR_INVALID_ARG
    assert _call_decode(S(), _fake_layer(), x=None) == moe.MOE_ERR_INVALID_ARG
    assert _call_decode(S(), _fake_layer(), x=(1 << 20) + 2) == moe.MOE_ERR_INVALID_ARG
    assert _call_decode(S(), _fake_layer(), ws_ptr=None) == moe.MOE_ERR_WORKSPACE
    assert _call_decode(S(), _fake_layer(), ws_bytes=16) == moe.MOE_ERR_WORKSPACE


def test_route_argument_errors(L):
    s = S()
    lay = _fake_layer()
    r = binding.lib().moe_route
    ok_ptr = 1 << 20
    assert r(ctypes.byref(s), ctypes.byref(lay), ok_ptr, 0, ok_ptr, ok_ptr, ok_ptr, None, 0, None) == 1
    assert r(ctypes.byref(s), ctypes.byref(lay), ok_ptr, 1, None, ok_ptr, ok_ptr, None, 0, None) == 1
    assert r(ctypes.byref(s), ctypes.byref(lay), ok_ptr, 1, ok_ptr, ok_ptr, ok_ptr, None, 2, None) == 1
    # gamma cannot be produced from given logits
    assert r(ctypes.byref(s), None, None, 1, ok_ptr, ok_ptr, ok_ptr, ok_ptr, 1, None) == 1


def test_binding_refuses_host_tensors(L):
    import torch
    import synth
    st = synth.make_stack(synth.TINY.shape, 1, 1)
    x = synth.make_x(synth.TINY.shape, 1, 1)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_layer_decode(synth.TINY.shape, st.layer(0), x, 1, torch.empty(1, 256),
                             workspace=torch.empty(16, dtype=torch.uint8))


def test_layer_path_boundary(L):
    """moe_layer_path (host-only): decode for T up to the crossover (default 1, the measured
    boundary) when the decode call takes the shape, batched above it, above T = 8, or for shapes
    the decode kernel does not take."""
    path = lambda shape, T, c=0: binding.lib().moe_layer_path(ctypes.byref(shape), T, c)
    s = S()
    assert moe.MOE_DEFAULT_CROSSOVER == 1
    assert path(s, 1) == moe.MOE_PATH_DECODE
    assert [path(s, T) for T in (2, 3, 8, 9, 16, 512, 65536)] == [moe.MOE_PATH_BATCHED] * 7
    assert [path(s, T, 8) for T in (1, 7, 8)] == [moe.MOE_PATH_DECODE] * 3
    assert path(s, 3, 2) == moe.MOE_PATH_BATCHED and path(s, 2, 2) == moe.MOE_PATH_DECODE
    assert path(s, 9, 100) == moe.MOE_PATH_BATCHED  # the decode path takes at most 8 tokens
    assert path(s, 1, -1) == moe.MOE_PATH_DECODE == path(s, moe.MOE_DEFAULT_CROSSOVER)
    assert path(s, 2, -1) == moe.MOE_PATH_BATCHED
    assert path(S(hidden=4096), 1) == moe.MOE_PATH_BATCHED  # beyond the decode limits
    assert path(S(inter=64), 1) == moe.MOE_PATH_BATCHED
    assert path(s, 0) == -1 and path(s, 65537) == -1 and path(S(bits=3), 1) == -1
    assert moe.moe_layer_path(synth_tiny_shape(), 1) == moe.MOE_PATH_DECODE
    assert moe.moe_layer_path(synth_tiny_shape(), 4, 8) == moe.MOE_PATH_DECODE


def synth_tiny_shape():
    import synth
    return synth.TINY.shape


def test_forward_workspace_and_host_checks(L):
    s = S()
    fwd = ws(s, T=512, kind=moe.MOE_WS_FORWARD)
    # a decode part for 8 tokens (independent of T), then a batched part for T
    assert fwd >= ws(s, T=8, kind=0) + ws(s, T=512, kind=1)
    assert ws(s, T=1, kind=moe.MOE_WS_FORWARD) - ws(s, T=1, kind=1) == fwd - ws(s, T=512, kind=1)
    assert ws(s, T=65537, kind=moe.MOE_WS_FORWARD) == 0
    f = binding.lib().moe_layer_forward
    lay, p = _fake_layer(), 1 << 20
    assert f(ctypes.byref(s), ctypes.byref(lay), p, 0, 0, p, None, None, None, p, fwd, None) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(s), ctypes.byref(lay), p, 4, 0, p, None, None, None, p, 64, None) == moe.MOE_ERR_WORKSPACE
    assert f(ctypes.byref(s), ctypes.byref(lay), p, 4, 0, p, None, None, None, None, fwd, None) == moe.MOE_ERR_WORKSPACE
    assert f(ctypes.byref(S(bits=3)), ctypes.byref(lay), p, 4, 0, p, None, None, None, p, fwd, None) == \
        moe.MOE_ERR_UNSUPPORTED


def test_library_override_selects_the_named_build(tmp_path):
    """MOE_AMD_LIB names another build of the library (a same-machine A/B of kernel variants): the
    binding loads that file, and MOE_AMD_PHASE_TIMER=1 alone selects the phase-timer build."""
    import subprocess
    import sys
    code = "from quantized_moe_decode_router_amd import binding; print(binding.LIB_PATH)"
    env = dict(os.environ)
    env.pop("MOE_AMD_PHASE_TIMER", None)
    env["MOE_AMD_LIB"] = str(tmp_path / "libvariant.so")
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == str(tmp_path / "libvariant.so")
    env.pop("MOE_AMD_LIB")
    env["MOE_AMD_PHASE_TIMER"] = "1"
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, check=True)
    assert out.stdout.strip().endswith(os.path.join("_lib", "libmoe_amd_phase.so"))
