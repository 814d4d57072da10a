"""Quantised sparse MoE FFN layer for MI355X (gfx950): HIP kernels behind a C ABI.

The Python surface is the ctypes binding of include/moe.h (same names, marshalling only).
Build the library with `quantized_moe_decode_router_amd.build.build()`."""
from .binding import (LIB_PATH, MOE_DEFAULT_CROSSOVER, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_TIMEOUT,  # noqa: F401
                      MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_OK, MOE_PATH_BATCHED, MOE_PATH_DECODE,
                      MOE_ROUTE_LOGITS_IN, MOE_STACK_INDEPENDENT, MOE_STATIC_RESET, MOE_WS_BATCHED, MOE_WS_DECODE,
                      MOE_WS_FORWARD, MOE_WS_STACK, MoeError, lib, moe_group_pairs, moe_layer_batched,
                      moe_layer_decode, moe_layer_forward, moe_layer_path, moe_read_status, moe_route,
                      moe_stack_decode, moe_workspace_bytes, status_string, workspace, MoeCache,
                      moe_cache_policy_run, moe_expert_stride, moe_layer_batched_table, moe_pack_experts,
                      moe_stack_decode_table, moe_stack_decode_static)
