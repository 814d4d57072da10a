"""fp64 CPU oracle of the quantised MoE FFN layer (ctypes wrapper around moe_oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package. It shares no code with the HIP library or its Python binding and
imports neither.

Parity pins (tests/test_oracle_*.py): brute-force top-k over all subsets, closed forms of the
renormalised weights, hand-packed dequantisation fixtures (tests/golden/), exactly-zero and
closed-form layers, expert-permutation and token-independence invariances, and the textbook
SwiGLU MLP through torch's own linear/silu routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIBDIR = os.path.join(_HERE, "_lib")
_LIB = os.path.join(_LIBDIR, "libmoe_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over independent output rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(_LIBDIR, exist_ok=True)
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OrcShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "num_experts", "top_k", "inter", "shared_inter", "bits", "group")]


_P = ctypes.c_void_p


class OrcLayer(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "router", "router_bias", "shared_gate",
        "w13_codes", "w13_scales", "w13_biases",
        "w2_codes", "w2_scales", "w2_biases",
        "s13_codes", "s13_scales", "s13_biases",
        "s2_codes", "s2_scales", "s2_biases")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_double_to_bf16.restype = ctypes.c_uint16
        L.orc_double_to_bf16.argtypes = [ctypes.c_double]
        L.orc_sigmoid.restype = ctypes.c_double
        L.orc_sigmoid.argtypes = [ctypes.c_double]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        L.orc_dequant_row.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, _P]
        L.orc_qmatvec.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, _P, _P]
        L.orc_router_logits.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, _P]
        L.orc_topk.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P]
        L.orc_route_weights.argtypes = [_P, ctypes.c_int, _P, ctypes.c_int, _P]
        L.orc_gate_up.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, _P, _P, _P]
        L.orc_swiglu.argtypes = [_P, _P, ctypes.c_int, _P]
        L.orc_expert.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, _P, _P, _P]
        L.orc_layer_forward.restype = ctypes.c_int
        L.orc_layer_forward.argtypes = [ctypes.POINTER(OrcShape), ctypes.POINTER(OrcLayer), _P,
                                ctypes.c_int, _P, _P, _P, _P, _P, _P]
        L.orc_rms_glue.argtypes = [_P, ctypes.c_int, ctypes.c_double, _P]
        del dp
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---- element functions -------------------------------------------------------------------

def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(bits)


def double_to_bf16(v: float) -> int:
    return lib().orc_double_to_bf16(v)


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(n)


def num_threads() -> int:
    return lib().orc_num_threads()


def dequant_row(codes, scales, biases, cols: int, bits: int, group: int, row: int) -> np.ndarray:
    codes, scales, biases = _c(codes, np.uint8), _c(scales, np.uint16), _c(biases, np.uint16)
    out = np.empty(cols, np.float64)
    lib().orc_dequant_row(_ptr(codes), _ptr(scales), _ptr(biases), cols, bits, group, row, _ptr(out))
    return out


def qmatvec(codes, scales, biases, rows: int, cols: int, bits: int, group: int, v) -> np.ndarray:
    codes, scales, biases = _c(codes, np.uint8), _c(scales, np.uint16), _c(biases, np.uint16)
    v = _c(v, np.float64)
    out = np.empty(rows, np.float64)
    lib().orc_qmatvec(_ptr(codes), _ptr(scales), _ptr(biases), rows, cols, bits, group, _ptr(v),
                      _ptr(out))
    return out


def router_logits(x, R, bias=None) -> np.ndarray:
    x, R, bias = _c(x, np.float64), _c(R, np.float32), _c(bias, np.float32)
    E, H = R.shape
    out = np.empty(E, np.float64)
    lib().orc_router_logits(_ptr(x), _ptr(R), _ptr(bias), E, H, _ptr(out))
    return out


def topk(logits, K: int) -> np.ndarray:
    logits = _c(logits, np.float64)
    idx = np.empty(K, np.int32)
    lib().orc_topk(_ptr(logits), logits.shape[0], K, _ptr(idx))
    return idx


def route_weights(logits, idx) -> np.ndarray:
    logits, idx = _c(logits, np.float64), _c(idx, np.int32)
    w = np.empty(idx.shape[0], np.float64)
    lib().orc_route_weights(_ptr(logits), logits.shape[0], _ptr(idx), idx.shape[0], _ptr(w))
    return w


def gate_up(c13, s13, b13, H: int, I: int, bits: int, group: int, x):
    c13, s13, b13 = _c(c13, np.uint8), _c(s13, np.uint16), _c(b13, np.uint16)
    x = _c(x, np.float64)
    g, u = np.empty(I, np.float64), np.empty(I, np.float64)
    lib().orc_gate_up(_ptr(c13), _ptr(s13), _ptr(b13), H, I, bits, group, _ptr(x), _ptr(g), _ptr(u))
    return g, u


def swiglu(g, u) -> np.ndarray:
    g, u = _c(g, np.float64), _c(u, np.float64)
    h = np.empty(g.shape[0], np.float64)
    lib().orc_swiglu(_ptr(g), _ptr(u), g.shape[0], _ptr(h))
    return h


def expert(c13, s13, b13, c2, s2, b2, H: int, I: int, bits: int, group: int, x):
    arrs = [_c(c13, np.uint8), _c(s13, np.uint16), _c(b13, np.uint16),
            _c(c2, np.uint8), _c(s2, np.uint16), _c(b2, np.uint16)]
    x = _c(x, np.float64)
    h, d = np.empty(I, np.float64), np.empty(H, np.float64)
    lib().orc_expert(*[_ptr(a) for a in arrs], H, I, bits, group, _ptr(x), _ptr(h), _ptr(d))
    return h, d


def rms_glue(y, eps: float = 1e-6) -> np.ndarray:
    y = _c(y, np.float64)
    out = np.empty(y.shape[0], np.uint16)
    lib().orc_rms_glue(_ptr(y), y.shape[0], eps, _ptr(out))
    return out


# ---- whole layer -----------------------------------------------------------------------------

class HostLayer:
    """Numpy (host) arrays of one layer, in the stacked layout with the layer dim removed.

    bf16 tensors are held as their uint16 bit patterns."""

    FIELDS = OrcLayer._fields_

    def __init__(self, shape, arrays: dict):
        self.shape = shape
        self.arrays = {}
        for name, _ in self.FIELDS:
            a = arrays.get(name)
            if a is None:
                self.arrays[name] = None
                continue
            dt = {"router": np.float32, "router_bias": np.float32, "shared_gate": np.float32}.get(name)
            if dt is None:
                dt = np.uint8 if name.endswith("codes") else np.uint16
            self.arrays[name] = np.ascontiguousarray(a, dtype=dt)

    def c_struct(self) -> OrcLayer:
        return OrcLayer(**{n: _ptr(a) for n, a in self.arrays.items()})

    def c_shape(self) -> OrcShape:
        s = self.shape
        return OrcShape(s.hidden, s.num_experts, s.top_k, s.inter, s.shared_inter, s.bits, s.group_size)


def layer_forward(layer: HostLayer, x_bf16_bits, logits_in=None):
    """Run the layer on [T][H] bf16 input bits. Returns dict(logits, idx, w, gamma, y)."""
    s = layer.shape
    x = _c(x_bf16_bits, np.uint16)
    T = x.shape[0]
    li = _c(logits_in, np.float32)
    out = dict(logits=np.empty((T, s.num_experts), np.float64),
               idx=np.empty((T, s.top_k), np.int32),
               w=np.empty((T, s.top_k), np.float64),
               gamma=np.empty(T, np.float64),
               y=np.empty((T, s.hidden), np.float64))
    cs, cl = layer.c_shape(), layer.c_struct()
    rc = lib().orc_layer_forward(ctypes.byref(cs), ctypes.byref(cl), _ptr(x), T, _ptr(li),
                         _ptr(out["logits"]), _ptr(out["idx"]), _ptr(out["w"]), _ptr(out["gamma"]),
                         _ptr(out["y"]))
    if rc != 0:
        raise ValueError("oracle rejected the layer shape")
    return out


# ---- grouping of (token, slot) pairs by expert ------------------------------------------------

def group_pairs(idx, E: int):
    """Plain definition of the expert grouping used by a batched layer (no arithmetic of the
    method; a bookkeeping step of the grouped evaluation the spec layer describes):
    pairs q = t*K + k are ordered by (expert idx[t, k], q) with a stable sort.
    Returns counts[E], offsets[E+1] (exclusive prefix sums), perm[T*K] (pair at each row) and
    pos[T*K] (row of each pair)."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return counts, offsets, perm, pos
