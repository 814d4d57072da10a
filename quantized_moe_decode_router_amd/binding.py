"""ctypes binding of libmoe_amd.so (include/moe.h): argument marshalling only.

Every function has the C entry point's name and argument order, takes torch tensors for the
pointer arguments, and raises MoeError on a non-OK status. All compute happens in the HIP
library; torch only provides device memory and the current stream. Tensors must be contiguous
and on the GPU: a host pointer handed to a kernel would fault the device, so that is checked
here before the call.

Layer arguments are duck-typed: any object with the attributes router, router_bias,
shared_gate and {w13,w2,s13,s2}_{codes,scales,biases} (torch tensors or None). For the stack
call the tensors carry a leading layer dimension and the base pointers describe layer 0.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_AMD_PHASE_TIMER=1 loads the phase-timer build of the same sources (build.py, phase_timer);
# MOE_AMD_LIB names another build of the library to load instead (an A/B comparison of kernel
# variants built from other sources on one machine)
LIB_PATH = os.environ.get("MOE_AMD_LIB") or os.path.join(
    _HERE, "_lib", "libmoe_amd_phase.so" if os.environ.get("MOE_AMD_PHASE_TIMER") == "1" else "libmoe_amd.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_TIMEOUT = range(6)
MOE_ROUTE_LOGITS_IN = 1
MOE_WS_DECODE, MOE_WS_BATCHED, MOE_WS_STACK, MOE_WS_FORWARD = 0, 1, 2, 3
MOE_PATH_DECODE, MOE_PATH_BATCHED = 0, 1
MOE_DEFAULT_CROSSOVER = 1

MOE_STACK_INDEPENDENT = 1
MOE_STATIC_RESET = 2

EXPORTED = ("moe_route", "moe_layer_decode", "moe_stack_decode", "moe_layer_batched", "moe_group_pairs",
            "moe_layer_path", "moe_layer_forward", "moe_workspace_bytes", "moe_read_status", "moe_status_string",
            "moe_expert_stride", "moe_pack_experts", "moe_stack_decode_table", "moe_layer_batched_table", "moe_cache_create",
            "moe_cache_update", "moe_cache_admit", "moe_cache_stats", "moe_cache_owners", "moe_cache_destroy", "moe_cache_policy_run",
            "moe_stack_decode_static")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class MoeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "num_experts", "top_k", "inter", "shared_inter", "bits", "group_size")]


class MoeQWeight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class MoeLayer(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("shared_gate", ctypes.c_void_p), ("w13", MoeQWeight), ("w2", MoeQWeight),
                ("s13", MoeQWeight), ("s2", MoeQWeight)]


_lib = None


def lib():
    """Load the built library; fails loudly if it is missing (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run quantized_moe_decode_router_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        PS, PL = ctypes.POINTER(MoeShape), ctypes.POINTER(MoeLayer)
        L.moe_route.argtypes = [PS, PL, P, I32, P, P, P, P, U32, P]
        L.moe_layer_decode.argtypes = [PS, PL, P, I32, P, P, P, P, P, SZ, P]
        L.moe_layer_batched.argtypes = [PS, PL, P, I32, P, P, P, P, P, SZ, P]
        L.moe_group_pairs.argtypes = [PS, P, I32, P, P, P, P, P, SZ, P]
        L.moe_layer_path.argtypes = [PS, I32, I32]
        L.moe_layer_path.restype = I32
        L.moe_layer_forward.argtypes = [PS, PL, P, I32, I32, P, P, P, P, P, SZ, P]
        L.moe_stack_decode.argtypes = [PS, PL, I32, U32, P, I32, P, P, P, P, P, P, P, SZ, P]
        L.moe_stack_decode_static.argtypes = [PS, PL, I32, U32, P, I32, P, P, P, P, P, P, P]
        L.moe_stack_decode_table.argtypes = [PS, PL, I32, P, P, SZ, U32, P, I32, P, P, P, P, P, P, P, SZ, P]
        L.moe_layer_batched_table.argtypes = [PS, PL, P, P, I32, P, P, P, P, P, SZ, P]
        L.moe_expert_stride.argtypes = [PS]
        L.moe_expert_stride.restype = SZ
        L.moe_pack_experts.argtypes = [PS, PL, I32, P, SZ, P]
        L.moe_cache_create.argtypes = [PS, I32, P, SZ, P, SZ, I32, P, SZ, P, SZ, P, ctypes.POINTER(P)]
        L.moe_cache_update.argtypes = [P, P, I32, I32, P, ctypes.POINTER(I32), ctypes.POINTER(I32)]
        L.moe_cache_admit.argtypes = [P, P, ctypes.c_int64, P, ctypes.POINTER(I32), ctypes.POINTER(I32)]
        U64P = ctypes.POINTER(ctypes.c_uint64)
        L.moe_cache_stats.argtypes = [P, U64P, U64P, U64P]
        L.moe_cache_owners.argtypes = [P, P]
        L.moe_cache_destroy.argtypes = [P]
        L.moe_cache_destroy.restype = None
        L.moe_cache_policy_run.argtypes = [I32, I32, P, ctypes.c_int64, P, P, P]
        L.moe_workspace_bytes.argtypes = [PS, I32, I32, I32]
        L.moe_workspace_bytes.restype = SZ
        L.moe_read_status.argtypes = [P, P, ctypes.POINTER(I32)]
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        for name in ("moe_route", "moe_layer_decode", "moe_layer_batched", "moe_stack_decode",
                     "moe_layer_forward", "moe_group_pairs", "moe_read_status"):
            if name != "moe_cache_destroy":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (the library takes device pointers)")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _dptr(t, name: str) -> int:
    """Address the device can read: a GPU tensor, a pinned (page-locked) host tensor, or a raw
    (address, nbytes) pair of such memory allocated elsewhere (e.g. hipHostMalloc)."""
    if isinstance(t, tuple):
        return int(t[0])
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name}: must be a GPU tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _nbytes(t) -> int:
    if isinstance(t, tuple):
        return int(t[1])
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def shape_struct(shape) -> MoeShape:
    return MoeShape(shape.hidden, shape.num_experts, shape.top_k, shape.inter, shape.shared_inter,
                    shape.bits, getattr(shape, "group_size", 64))


_BF16_BITS = (torch.bfloat16, torch.int16, torch.uint16)


def layer_struct(layer) -> MoeLayer:
    def q(prefix):
        c = getattr(layer, prefix + "_codes", None)
        if c is None:
            return MoeQWeight(None, None, None)
        return MoeQWeight(_ptr(c, prefix + "_codes", torch.uint8),
                          _ptr(getattr(layer, prefix + "_scales"), prefix + "_scales", _BF16_BITS),
                          _ptr(getattr(layer, prefix + "_biases"), prefix + "_biases", _BF16_BITS))
    return MoeLayer(_ptr(getattr(layer, "router", None), "router", torch.float32),
                    _ptr(getattr(layer, "router_bias", None), "router_bias", torch.float32),
                    _ptr(getattr(layer, "shared_gate", None), "shared_gate", torch.float32),
                    q("w13"), q("w2"), q("s13"), q("s2"))


# ---- entry points ----------------------------------------------------------------------------

def moe_workspace_bytes(shape, T: int, kind: int, n_layers: int = 1) -> int:
    s = shape_struct(shape)
    return int(lib().moe_workspace_bytes(ctypes.byref(s), int(T), int(n_layers), int(kind)))


def moe_route(shape, layer, x, T: int, logits, topk_idx, topk_w, gamma=None, flags: int = 0,
              stream=None) -> None:
    s = shape_struct(shape)
    L = layer_struct(layer) if layer is not None else None
    st = lib().moe_route(ctypes.byref(s), ctypes.byref(L) if L is not None else None,
                         _ptr(x, "x", _BF16_BITS), int(T), _ptr(logits, "logits", torch.float32),
                         _ptr(topk_idx, "topk_idx", torch.int32), _ptr(topk_w, "topk_w", torch.float32),
                         _ptr(gamma, "gamma", torch.float32), int(flags), _stream(stream))
    _check(st, "moe_route")


def moe_layer_decode(shape, layer, x, T: int, y, topk_idx=None, topk_w=None, logits=None,
                     workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    s, L = shape_struct(shape), layer_struct(layer)
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = lib().moe_layer_decode(ctypes.byref(s), ctypes.byref(L), _ptr(x, "x", _BF16_BITS), int(T),
                                _ptr(y, "y", torch.float32), _ptr(topk_idx, "topk_idx", torch.int32),
                                _ptr(topk_w, "topk_w", torch.float32), _ptr(logits, "logits", torch.float32),
                                _ptr(workspace, "workspace"), int(wsb), _stream(stream))
    _check(st, "moe_layer_decode")


def moe_stack_decode(shape, stack, n_layers: int, x, T: int, y, x_all=None, y_all=None, topk_idx_all=None,
                     topk_w_all=None, logits_all=None, workspace=None, workspace_bytes=None, stream=None,
                     flags: int = 0) -> None:
    s, L = shape_struct(shape), layer_struct(stack)
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = lib().moe_stack_decode(ctypes.byref(s), ctypes.byref(L), int(n_layers), int(flags),
                                _ptr(x, "x", _BF16_BITS), int(T), _ptr(y, "y", torch.float32),
                                _ptr(x_all, "x_all", _BF16_BITS), _ptr(y_all, "y_all", torch.float32),
                                _ptr(topk_idx_all, "topk_idx_all", torch.int32),
                                _ptr(topk_w_all, "topk_w_all", torch.float32),
                                _ptr(logits_all, "logits_all", torch.float32), _ptr(workspace, "workspace"),
                                int(wsb), _stream(stream))
    _check(st, "moe_stack_decode")


def moe_stack_decode_static(shape, stack, n_layers: int, x, T: int, y, x_all=None, y_all=None, topk_idx_all=None,
                            topk_w_all=None, logits_all=None, stream=None, flags: int = 0) -> None:
    s, L = shape_struct(shape), layer_struct(stack)
    st = lib().moe_stack_decode_static(ctypes.byref(s), ctypes.byref(L), int(n_layers), int(flags),
                                       _ptr(x, "x", _BF16_BITS), int(T), _ptr(y, "y", torch.float32),
                                       _ptr(x_all, "x_all", _BF16_BITS), _ptr(y_all, "y_all", torch.float32),
                                       _ptr(topk_idx_all, "topk_idx_all", torch.int32),
                                       _ptr(topk_w_all, "topk_w_all", torch.float32),
                                       _ptr(logits_all, "logits_all", torch.float32), _stream(stream))
    _check(st, "moe_stack_decode_static")


def moe_layer_batched(shape, layer, x, T: int, y, topk_idx=None, topk_w=None, logits=None,
                      workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    s, L = shape_struct(shape), layer_struct(layer)
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = lib().moe_layer_batched(ctypes.byref(s), ctypes.byref(L), _ptr(x, "x", _BF16_BITS), int(T),
                                 _ptr(y, "y", torch.float32), _ptr(topk_idx, "topk_idx", torch.int32),
                                 _ptr(topk_w, "topk_w", torch.float32), _ptr(logits, "logits", torch.float32),
                                 _ptr(workspace, "workspace"), int(wsb), _stream(stream))
    _check(st, "moe_layer_batched")


def moe_layer_path(shape, T: int, crossover: int = 0) -> int:
    s = shape_struct(shape)
    return int(lib().moe_layer_path(ctypes.byref(s), int(T), int(crossover)))


def moe_layer_forward(shape, layer, x, T: int, y, topk_idx=None, topk_w=None, logits=None,
                      workspace=None, workspace_bytes: Optional[int] = None, stream=None,
                      crossover: int = 0) -> None:
    s, L = shape_struct(shape), layer_struct(layer)
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = lib().moe_layer_forward(ctypes.byref(s), ctypes.byref(L), _ptr(x, "x", _BF16_BITS), int(T),
                                 int(crossover), _ptr(y, "y", torch.float32),
                                 _ptr(topk_idx, "topk_idx", torch.int32), _ptr(topk_w, "topk_w", torch.float32),
                                 _ptr(logits, "logits", torch.float32), _ptr(workspace, "workspace"), int(wsb),
                                 _stream(stream))
    _check(st, "moe_layer_forward")


def moe_group_pairs(shape, topk_idx, T: int, counts, offsets, perm, pos, workspace=None,
                    workspace_bytes: Optional[int] = None, stream=None) -> None:
    s = shape_struct(shape)
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = lib().moe_group_pairs(ctypes.byref(s), _ptr(topk_idx, "topk_idx", torch.int32), int(T),
                               _ptr(counts, "counts", torch.int32), _ptr(offsets, "offsets", torch.int32),
                               _ptr(perm, "perm", torch.int32), _ptr(pos, "pos", torch.int32),
                               _ptr(workspace, "workspace"), int(wsb), _stream(stream))
    _check(st, "moe_group_pairs")


def moe_expert_stride(shape) -> int:
    s = shape_struct(shape)
    return int(lib().moe_expert_stride(ctypes.byref(s)))


def moe_pack_experts(shape, stack, n_layers: int, container, stream=None) -> None:
    s, L = shape_struct(shape), layer_struct(stack)
    st = lib().moe_pack_experts(ctypes.byref(s), ctypes.byref(L), int(n_layers), _dptr(container, "container"),
                                _nbytes(container), _stream(stream))
    _check(st, "moe_pack_experts")


def moe_stack_decode_table(shape, stack, n_layers: int, expert_table, x, T: int, y, x_all=None, y_all=None,
                           topk_idx_all=None, topk_w_all=None, logits_all=None, workspace=None,
                           workspace_bytes=None, stream=None, flags: int = 0, landing=None) -> None:
    s, L = shape_struct(shape), layer_struct(stack)
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = lib().moe_stack_decode_table(ctypes.byref(s), ctypes.byref(L), int(n_layers),
                                      _ptr(expert_table, "expert_table", (torch.int64, torch.uint64)),
                                      _ptr(landing, "landing"), _nbytes(landing) if landing is not None else 0, int(flags),
                                      _ptr(x, "x", _BF16_BITS), int(T), _ptr(y, "y", torch.float32),
                                      _ptr(x_all, "x_all", _BF16_BITS), _ptr(y_all, "y_all", torch.float32),
                                      _ptr(topk_idx_all, "topk_idx_all", torch.int32),
                                      _ptr(topk_w_all, "topk_w_all", torch.float32),
                                      _ptr(logits_all, "logits_all", torch.float32), _ptr(workspace, "workspace"),
                                      int(wsb), _stream(stream))
    _check(st, "moe_stack_decode_table")


def moe_layer_batched_table(shape, layer, expert_table, x, T: int, y, topk_idx=None, topk_w=None, logits=None,
                            workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    s, L = shape_struct(shape), layer_struct(layer)
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = lib().moe_layer_batched_table(ctypes.byref(s), ctypes.byref(L),
                                       _ptr(expert_table, "expert_table", (torch.int64, torch.uint64)),
                                       _ptr(x, "x", _BF16_BITS), int(T), _ptr(y, "y", torch.float32),
                                       _ptr(topk_idx, "topk_idx", torch.int32), _ptr(topk_w, "topk_w", torch.float32),
                                       _ptr(logits, "logits", torch.float32), _ptr(workspace, "workspace"), int(wsb),
                                       _stream(stream))
    _check(st, "moe_layer_batched_table")


class MoeCache:
    """moe_cache_* over caller-owned tensors: a packed container (GPU or pinned host uint8), a GPU
    pool of `slots` strides and a GPU int64 [L][E] expert table."""

    def __init__(self, shape, n_layers: int, container, pool, slots: int, table, stream=None, landing=None):
        s = shape_struct(shape)
        self._h = ctypes.c_void_p()
        self._keep = (container, pool, table, landing)
        self.slots = int(slots)
        st = lib().moe_cache_create(ctypes.byref(s), int(n_layers), _dptr(container, "container"),
                                    _nbytes(container), _ptr(pool, "pool") if pool is not None else None,
                                    _nbytes(pool) if pool is not None else 0, self.slots,
                                    _ptr(table, "table", (torch.int64, torch.uint64)), _nbytes(table),
                                    _ptr(landing, "landing") if landing is not None else None,
                                    _nbytes(landing) if landing is not None else 0, _stream(stream),
                                    ctypes.byref(self._h))
        _check(st, "moe_cache_create")

    def update(self, topk_idx_all, T: int, top_k: int, stream=None):
        """topk_idx_all: host int32 [L][T][K] (tensor or array). Returns (hits, misses) of the call."""
        a = np.ascontiguousarray(topk_idx_all.cpu().numpy() if isinstance(topk_idx_all, torch.Tensor)
                                 else topk_idx_all, dtype=np.int32)
        h, m = ctypes.c_int32(0), ctypes.c_int32(0)
        st = lib().moe_cache_update(self._h, a.ctypes.data, int(T), int(top_k), _stream(stream), ctypes.byref(h),
                                    ctypes.byref(m))
        _check(st, "moe_cache_update")
        return int(h.value), int(m.value)

    def admit(self, keys, stream=None):
        """Feed keys (l * E + e) through the policy and admit them; returns (hits, misses)."""
        k = np.ascontiguousarray(keys, dtype=np.int32)
        h, m = ctypes.c_int32(0), ctypes.c_int32(0)
        st = lib().moe_cache_admit(self._h, k.ctypes.data if k.size else None, int(k.size), _stream(stream),
                                   ctypes.byref(h), ctypes.byref(m))
        _check(st, "moe_cache_admit")
        return int(h.value), int(m.value)

    def stats(self):
        h, m, b = ctypes.c_uint64(0), ctypes.c_uint64(0), ctypes.c_uint64(0)
        _check(lib().moe_cache_stats(self._h, ctypes.byref(h), ctypes.byref(m), ctypes.byref(b)), "moe_cache_stats")
        return int(h.value), int(m.value), int(b.value)

    def owners(self) -> np.ndarray:
        out = np.full(max(self.slots, 1), -1, dtype=np.int32)
        _check(lib().moe_cache_owners(self._h, out.ctypes.data), "moe_cache_owners")
        return out[:self.slots]

    def close(self) -> None:
        if self._h:
            lib().moe_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_cache_policy_run(slots: int, n_keys: int, keys):
    """The cache policy on the host: per access (hit, slot, evicted) as int32 arrays."""
    k = np.ascontiguousarray(keys, dtype=np.int32)
    n = k.size
    hit, slot, ev = (np.zeros(max(n, 1), dtype=np.int32) for _ in range(3))
    st = lib().moe_cache_policy_run(int(slots), int(n_keys), k.ctypes.data if n else None, int(n),
                                    hit.ctypes.data, slot.ctypes.data, ev.ctypes.data)
    _check(st, "moe_cache_policy_run")
    return hit[:n], slot[:n], ev[:n]


def moe_read_status(workspace, stream=None) -> int:
    out = ctypes.c_int32(-1)
    st = lib().moe_read_status(_ptr(workspace, "workspace"), _stream(stream), ctypes.byref(out))
    _check(st, "moe_read_status")
    return int(out.value)


def workspace(shape, T: int, kind: int, device="cuda", n_layers: int = 1) -> torch.Tensor:
    """Allocate (through torch) a zero-filled workspace of moe_workspace_bytes() bytes."""
    n = moe_workspace_bytes(shape, T, kind, n_layers)
    if n == 0:
        raise MoeError(MOE_ERR_UNSUPPORTED, "moe_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)
