// moe_abi.cpp -- the extern "C" entry points of include/moe.h: host-side argument checks,
// workspace carving and kernel dispatch. Nothing here allocates device memory or synchronises,
// except moe_read_status, which exists to read the device status word.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/moe.h"
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace {

using moe::align_up;

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int kMaxDecodeT = 8;
constexpr int kMaxLayers = 4096;
constexpr int kMaxBatchT = 65536;

// Shape checks shared by every entry point.
moe_status check_shape(const moe_shape *s) {
    if (!s) return MOE_ERR_INVALID_ARG;
    if (s->hidden <= 0 || s->num_experts <= 0 || s->top_k <= 0 || s->inter <= 0 ||
        s->shared_inter < 0 || s->bits <= 0 || s->group_size <= 0)
        return MOE_ERR_INVALID_ARG;
    if (s->top_k > s->num_experts) return MOE_ERR_INVALID_ARG;
    if (s->hidden % s->group_size || s->inter % s->group_size ||
        (s->shared_inter && s->shared_inter % s->group_size))
        return MOE_ERR_INVALID_ARG;
    if (s->bits != 4 && s->bits != 8) return MOE_ERR_UNSUPPORTED;
    if (s->group_size != 64) return MOE_ERR_UNSUPPORTED;
    if (!pow2(s->hidden) || s->hidden < 256 || s->hidden > 4096) return MOE_ERR_UNSUPPORTED;
    if (!pow2(s->inter) || s->inter < 64 || s->inter > 4096) return MOE_ERR_UNSUPPORTED;
    if (s->shared_inter && (!pow2(s->shared_inter) || s->shared_inter < 64 || s->shared_inter > 4096))
        return MOE_ERR_UNSUPPORTED;
    if (s->top_k > 16 || s->num_experts > 1024) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_qweight(const moe_qweight &q) {
    if (!q.codes || !q.scales || !q.biases) return MOE_ERR_INVALID_ARG;
    if (!al16(q.codes) || !al16(q.scales) || !al16(q.biases)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// routed = false: the routed experts come from an expert table, so w13 and w2 are not read.
moe_status check_layer(const moe_shape *s, const moe_layer *L, bool routed = true) {
    if (!L || !L->router || !al16(L->router)) return MOE_ERR_INVALID_ARG;
    if (L->router_bias && !al4(L->router_bias)) return MOE_ERR_INVALID_ARG;
    moe_status st;
    if (routed && (st = check_qweight(L->w13)) != MOE_OK) return st;
    if (routed && (st = check_qweight(L->w2)) != MOE_OK) return st;
    if (s->shared_inter) {
        if (!L->shared_gate || !al16(L->shared_gate)) return MOE_ERR_INVALID_ARG;
        if ((st = check_qweight(L->s13)) != MOE_OK) return st;
        if ((st = check_qweight(L->s2)) != MOE_OK) return st;
    }
    return MOE_OK;
}

size_t decode_ws_bytes(const moe_shape *s, int T, int L) {
    return moe::decode_ws_layout(L, T, s->hidden, s->num_experts, s->top_k, s->inter, s->shared_inter).total;
}

size_t batched_ws_bytes(const moe_shape *s, int T) {
    return moe::batched_ws_layout(T, s->hidden, s->num_experts, s->top_k, s->inter, s->shared_inter).total;
}

// LDS available to the decode kernel's dynamic plan (the rest of the 160 KiB holds its small
// static arrays).
constexpr int kDecodeLdsBudget = 160 * 1024 - 1024;

int decode_chunk(const moe_shape *s, int T, int grid, bool xt = false) {
    return moe::decode_chunk_pairs(T, s->hidden, s->num_experts, s->top_k, s->inter, s->shared_inter, s->bits, grid,
                                   kDecodeLdsBudget, xt);
}

int rows_per_wg(int H, int grid) { return (H + grid - 1) / grid; }

// Compute units assumed by moe_layer_path when no device is visible (MI355X).
constexpr int kAssumedCus = 256;

// Decode part of a moe_layer_forward workspace: a decode workspace for the largest decode T (its
// status word at byte 0), rounded up so that the batched part after it stays aligned. Its size does
// not depend on T, so calls with any T that share the workspace keep the decode exchange words
// and the batched scratch apart (a batched call never writes where a later decode call looks for
// words of its epoch).
size_t forward_decode_part(const moe_shape *s) { return align_up(decode_ws_bytes(s, kMaxDecodeT, 1), 256); }

// Shapes the decode kernel handles (beyond check_shape): rows of at most 64 slices of 32 columns,
// intermediates of at least 128 columns (whole dwords of scales per row for the LDS staging),
// and an LDS plan within the compute unit's 160 KiB.
moe_status decode_supported(const moe_shape *s, int T, int grid, bool xt = false) {
    if (s->hidden > 2048 || s->inter > 2048 || s->shared_inter > 2048) return MOE_ERR_UNSUPPORTED;
    if (s->inter < 128 || (s->shared_inter && s->shared_inter < 128)) return MOE_ERR_UNSUPPORTED;
    if (decode_chunk(s, T, grid, xt) == 0) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status decode_common(const moe_shape *s, const moe_layer *L, int32_t n_layers, uint32_t flags,
                         const uint16_t *x, int32_t T, float *y, uint16_t *x_all, float *y_all,
                         int32_t *idx_all, float *w_all, float *logits_all, void *ws, size_t ws_bytes,
                         void *stream, const uint64_t *xtab = nullptr, void *landing = nullptr,
                         size_t landing_bytes = 0) {
    moe_status st = check_shape(s);
    if (st != MOE_OK) return st;
    if ((st = check_layer(s, L, xtab == nullptr)) != MOE_OK) return st;
    if (xtab && (reinterpret_cast<uintptr_t>(xtab) & 15u)) return MOE_ERR_INVALID_ARG;
    if (landing && (!xtab || (reinterpret_cast<uintptr_t>(landing) & 4095u) ||
                    landing_bytes < (size_t)n_layers * T * s->top_k *
                                        moe::expert_block(s->hidden, s->inter, s->bits).stride))
        return MOE_ERR_INVALID_ARG;
    if (flags & ~MOE_STACK_INDEPENDENT) return MOE_ERR_INVALID_ARG;
    if (n_layers < 1 || n_layers > kMaxLayers || T < 1 || T > kMaxDecodeT) return MOE_ERR_INVALID_ARG;
    if (!x || !y || !al16(x) || !al16(y)) return MOE_ERR_INVALID_ARG;
    if ((x_all && !al16(x_all)) || (y_all && !al16(y_all)) || (idx_all && !al4(idx_all)) ||
        (w_all && !al4(w_all)) || (logits_all && !al4(logits_all)))
        return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < decode_ws_bytes(s, T, n_layers) || !al16(ws)) return MOE_ERR_WORKSPACE;
    const int grid = moe::device_cu_count();
    if (grid <= 0) return MOE_ERR_HIP;
    if (grid > moe::kMaxGrid) return MOE_ERR_UNSUPPORTED;
    const bool xt = xtab != nullptr;
    if ((st = decode_supported(s, T, grid, xt)) != MOE_OK) return st;

    const size_t H = s->hidden, E = s->num_experts, I = s->inter, Is = s->shared_inter;
    const size_t bits = s->bits;
    moe::DecodeParams p;
    memset(&p, 0, sizeof p);
    p.H = s->hidden; p.E = s->num_experts; p.K = s->top_k; p.I = s->inter; p.Is = s->shared_inter;
    p.bits = s->bits; p.T = T; p.L = n_layers;
    p.chained = (flags & MOE_STACK_INDEPENDENT) ? 0 : 1;
    p.rows_per_wg = rows_per_wg(s->hidden, grid);
    p.nrr = (s->num_experts + (Is ? 1 : 0) + grid - 1) / grid;
    p.nps = Is ? ((int)Is + grid - 1) / grid : 0;
    p.log2I = 0;
    while ((1 << p.log2I) < s->inter) ++p.log2I;
    p.kdiv = moe::div_magic((unsigned)s->top_k);
    p.tdiv = moe::div_magic((unsigned)T);
    p.cp = decode_chunk(s, T, grid, xt);
    p.lds = moe::decode_lds_plan(T, s->hidden, s->num_experts, s->top_k, s->inter, s->shared_inter, s->bits, grid,
                                 p.cp, xt);
    p.spin_limit = 1u << 20;
    p.eps = 1e-6f;
    p.router = L->router; p.rbias = L->router_bias; p.sgate = Is ? L->shared_gate : nullptr;
    if (xtab) {
        const moe::ExpertBlock xb = moe::expert_block(s->hidden, s->inter, s->bits);
        p.xtab = xtab;
        p.xo13s = (uint32_t)xb.o13s; p.xo13b = (uint32_t)xb.o13b;
        p.xo2c = (uint32_t)xb.o2c; p.xo2s = (uint32_t)xb.o2s; p.xo2b = (uint32_t)xb.o2b;
        p.xstride = xb.stride;
        p.landing = static_cast<char *>(landing);
    } else {
        p.w13 = {L->w13.codes, L->w13.scales, L->w13.biases};
        p.w2 = {L->w2.codes, L->w2.scales, L->w2.biases};
    }
    if (Is) {
        p.s13 = {L->s13.codes, L->s13.scales, L->s13.biases};
        p.s2 = {L->s2.codes, L->s2.scales, L->s2.biases};
    }
    p.x_in = x; p.y_out = y;
    p.x_all = x_all; p.y_all = y_all; p.idx_all = idx_all; p.w_all = w_all; p.logits_all = logits_all;
    char *w = static_cast<char *>(ws);
    const moe::DecodeWs lay = moe::decode_ws_layout(n_layers, T, s->hidden, s->num_experts, s->top_k, s->inter,
                                                    s->shared_inter);
    p.ctrl = reinterpret_cast<int *>(w);
    p.phase = lay.phase ? reinterpret_cast<uint64_t *>(w + lay.phase) : nullptr;
    p.ll_start = reinterpret_cast<uint64_t *>(w + lay.start);
    p.ll_logits = reinterpret_cast<uint64_t *>(w + lay.logits);
    p.ll_h = reinterpret_cast<uint64_t *>(w + lay.h);
    p.ll_y = reinterpret_cast<uint64_t *>(w + lay.y);
    hipError_t err = moe::launch_decode(p, grid, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

namespace moe {

int device_cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64) cache[dev] = n;
    return n;
}

}  // namespace moe

extern "C" {

const char *moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        case MOE_ERR_TIMEOUT: return "MOE_ERR_TIMEOUT";
    }
    return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_bytes(const moe_shape *s, int32_t T, int32_t n_layers, int32_t kind) {
    if (check_shape(s) != MOE_OK || T < 1) return 0;
    if (kind == MOE_WS_FORWARD) {
        if (T > kMaxBatchT) return 0;
        return forward_decode_part(s) + batched_ws_bytes(s, T);
    }
    if (kind == MOE_WS_DECODE || kind == MOE_WS_STACK) {
        const int L = kind == MOE_WS_DECODE ? 1 : n_layers;
        if (T > kMaxDecodeT || L < 1 || L > kMaxLayers) return 0;
        return decode_ws_bytes(s, T, L);
    }
    if (kind == MOE_WS_BATCHED) {
        if (T > kMaxBatchT) return 0;
        return batched_ws_bytes(s, T);
    }
    return 0;
}

moe_status moe_read_status(const void *ws, void *stream, int32_t *status) {
    if (!ws || !status) return MOE_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_HIP;
    if (hipMemcpy(status, ws, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status moe_route(const moe_shape *s, const moe_layer *L, const uint16_t *x, int32_t T,
                     float *logits, int32_t *topk_idx, float *topk_w, float *gamma, uint32_t flags,
                     void *stream) {
    moe_status st = check_shape(s);
    if (st != MOE_OK) return st;
    if (flags & ~MOE_ROUTE_LOGITS_IN) return MOE_ERR_INVALID_ARG;
    const bool lin = (flags & MOE_ROUTE_LOGITS_IN) != 0;
    if (T < 1 || T > kMaxBatchT) return MOE_ERR_INVALID_ARG;
    if (!logits || !topk_idx || !topk_w || !al4(logits) || !al4(topk_idx) || !al4(topk_w))
        return MOE_ERR_INVALID_ARG;
    if (gamma && (lin || !s->shared_inter || !al4(gamma))) return MOE_ERR_INVALID_ARG;
    if (!lin) {
        if (!L || !L->router || !al16(L->router) || !x || !al16(x)) return MOE_ERR_INVALID_ARG;
        if (L->router_bias && !al4(L->router_bias)) return MOE_ERR_INVALID_ARG;
        if (gamma && (!L->shared_gate || !al16(L->shared_gate))) return MOE_ERR_INVALID_ARG;
    }
    moe::RouteParams p;
    memset(&p, 0, sizeof p);
    p.H = s->hidden; p.E = s->num_experts; p.K = s->top_k; p.T = T;
    p.logits_in = lin ? 1 : 0;
    p.has_gate = gamma ? 1 : 0;
    p.x = x;
    if (!lin) {
        p.router = L->router;
        p.rbias = L->router_bias;
        p.sgate = gamma ? L->shared_gate : nullptr;
    }
    p.logits = logits; p.idx = topk_idx; p.w = topk_w; p.gamma = gamma;
    hipError_t err = moe::launch_route(p, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_layer_decode(const moe_shape *s, const moe_layer *L, const uint16_t *x, int32_t T,
                            float *y, int32_t *topk_idx_opt, float *topk_w_opt, float *logits_opt,
                            void *ws, size_t ws_bytes, void *stream) {
    return decode_common(s, L, 1, 0, x, T, y, nullptr, nullptr, topk_idx_opt, topk_w_opt, logits_opt, ws,
                         ws_bytes, stream);
}

moe_status moe_stack_decode(const moe_shape *s, const moe_layer *stack, int32_t n_layers, uint32_t flags,
                            const uint16_t *x, int32_t T, float *y, uint16_t *x_all_opt,
                            float *y_all_opt, int32_t *idx_all_opt, float *w_all_opt,
                            float *logits_all_opt, void *ws, size_t ws_bytes, void *stream) {
    return decode_common(s, stack, n_layers, flags, x, T, y, x_all_opt, y_all_opt, idx_all_opt, w_all_opt,
                         logits_all_opt, ws, ws_bytes, stream);
}

moe_status moe_stack_decode_static(const moe_shape *s, const moe_layer *stack, int32_t n_layers, uint32_t flags,
                                   const uint16_t *x, int32_t T, float *y, uint16_t *x_all_opt, float *y_all_opt,
                                   int32_t *idx_all_opt, float *w_all_opt, float *logits_all_opt, void *stream) {
    if (flags & ~(MOE_STACK_INDEPENDENT | MOE_STATIC_RESET)) return MOE_ERR_INVALID_ARG;
    moe_status st = check_shape(s);
    if (st != MOE_OK) return st;
    if (n_layers < 1 || n_layers > kMaxLayers || T < 1 || T > kMaxDecodeT) return MOE_ERR_INVALID_ARG;
    const size_t need = decode_ws_bytes(s, T, n_layers);
    if (need > moe::kStaticScratchBytes) return MOE_ERR_WORKSPACE;
    void *ws = nullptr;
    if (moe::static_scratch(need, (flags & MOE_STATIC_RESET) != 0, static_cast<hipStream_t>(stream), &ws) !=
        hipSuccess)
        return MOE_ERR_HIP;
    return decode_common(s, stack, n_layers, flags & MOE_STACK_INDEPENDENT, x, T, y, x_all_opt, y_all_opt,
                         idx_all_opt, w_all_opt, logits_all_opt, ws, need, stream);
}

moe_status moe_stack_decode_table(const moe_shape *s, const moe_layer *stack, int32_t n_layers,
                                  const uint64_t *expert_table, void *landing_opt, size_t landing_bytes,
                                  uint32_t flags,
                                  const uint16_t *x, int32_t T,
                                  float *y, uint16_t *x_all_opt, float *y_all_opt, int32_t *idx_all_opt,
                                  float *w_all_opt, float *logits_all_opt, void *ws, size_t ws_bytes,
                                  void *stream) {
    if (!expert_table) return MOE_ERR_INVALID_ARG;
    return decode_common(s, stack, n_layers, flags, x, T, y, x_all_opt, y_all_opt, idx_all_opt, w_all_opt,
                         logits_all_opt, ws, ws_bytes, stream, expert_table, landing_opt, landing_bytes);
}

size_t moe_expert_stride(const moe_shape *s) {
    if (check_shape(s) != MOE_OK) return 0;
    return moe::expert_block(s->hidden, s->inter, s->bits).stride;
}

moe_status moe_pack_experts(const moe_shape *s, const moe_layer *stack, int32_t n_layers, void *container,
                            size_t container_bytes, void *stream) {
    moe_status st = check_shape(s);
    if (st != MOE_OK) return st;
    if (!stack || check_qweight(stack->w13) != MOE_OK || check_qweight(stack->w2) != MOE_OK)
        return MOE_ERR_INVALID_ARG;
    if (n_layers < 1 || n_layers > kMaxLayers || !container || (reinterpret_cast<uintptr_t>(container) & 4095u))
        return MOE_ERR_INVALID_ARG;
    const moe::ExpertBlock xb = moe::expert_block(s->hidden, s->inter, s->bits);
    const size_t n = (size_t)n_layers * s->num_experts;
    if (container_bytes < n * xb.stride) return MOE_ERR_INVALID_ARG;
    char *dst = static_cast<char *>(container);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // six strided copies: piece p of every expert, source rows of piece-size bytes, destination
    // rows one block apart
    const struct {
        const void *src;
        size_t off, bytes;
    } piece[6] = {{stack->w13.codes, 0, xb.c13},   {stack->w13.scales, xb.o13s, xb.s13},
                  {stack->w13.biases, xb.o13b, xb.s13}, {stack->w2.codes, xb.o2c, xb.c2},
                  {stack->w2.scales, xb.o2s, xb.s2},     {stack->w2.biases, xb.o2b, xb.s2}};
    for (const auto &pc : piece)
        if (hipMemcpy2DAsync(dst + pc.off, xb.stride, pc.src, pc.bytes, pc.bytes, n, hipMemcpyDefault, hs) !=
            hipSuccess)
            return MOE_ERR_HIP;
    return MOE_OK;
}

namespace {
moe_status batched_common(const moe_shape *s, const moe_layer *L, const uint16_t *x, int32_t T, float *y,
                          int32_t *topk_idx_opt, float *topk_w_opt, float *logits_opt, void *ws, size_t ws_bytes,
                          void *stream, const uint64_t *xtab, int *status_word = nullptr) {
    moe_status st = check_shape(s);
    if (st != MOE_OK) return st;
    if ((st = check_layer(s, L, xtab == nullptr)) != MOE_OK) return st;
    if (xtab && (reinterpret_cast<uintptr_t>(xtab) & 7u)) return MOE_ERR_INVALID_ARG;
    if (T < 1 || T > kMaxBatchT) return MOE_ERR_INVALID_ARG;
    // gate|up work items span 128 intermediate columns, and a k-step's scale DMA reads a dword
    // (two groups) of every row
    if (s->inter < 128 || (s->shared_inter && s->shared_inter < 128)) return MOE_ERR_UNSUPPORTED;
    // a grouped-GEMM workgroup stages every scale and bias of its rows in LDS (at most 32 groups)
    if (s->hidden > 2048 || s->inter > 2048 || s->shared_inter > 2048) return MOE_ERR_UNSUPPORTED;
    if (!x || !y || !al16(x) || !al16(y)) return MOE_ERR_INVALID_ARG;
    if ((topk_idx_opt && !al4(topk_idx_opt)) || (topk_w_opt && !al4(topk_w_opt)) ||
        (logits_opt && !al4(logits_opt)))
        return MOE_ERR_INVALID_ARG;
    if (!ws || !al16(ws) || ws_bytes < batched_ws_bytes(s, T)) return MOE_ERR_WORKSPACE;
    const moe::BatchedWs lay = moe::batched_ws_layout(T, s->hidden, s->num_experts, s->top_k, s->inter,
                                                      s->shared_inter);
    char *w = static_cast<char *>(ws);
    moe::BatchedParams p;
    memset(&p, 0, sizeof p);
    p.H = s->hidden; p.E = s->num_experts; p.K = s->top_k; p.I = s->inter; p.Is = s->shared_inter;
    p.Imax = p.I > p.Is ? p.I : p.Is;
    p.bits = s->bits; p.T = T;
    p.x = x;
    p.router = L->router; p.rbias = L->router_bias;
    p.sgate = p.Is ? L->shared_gate : nullptr;
    if (xtab) {
        const moe::ExpertBlock xb = moe::expert_block(s->hidden, s->inter, s->bits);
        p.xtab = xtab;
        p.xo13s = (uint32_t)xb.o13s; p.xo13b = (uint32_t)xb.o13b;
        p.xo2c = (uint32_t)xb.o2c; p.xo2s = (uint32_t)xb.o2s; p.xo2b = (uint32_t)xb.o2b;
    } else {
        p.w13 = {L->w13.codes, L->w13.scales, L->w13.biases};
        p.w2 = {L->w2.codes, L->w2.scales, L->w2.biases};
    }
    if (p.Is) {
        p.s13 = {L->s13.codes, L->s13.scales, L->s13.biases};
        p.s2 = {L->s2.codes, L->s2.scales, L->s2.biases};
    }
    p.logits = logits_opt ? logits_opt : reinterpret_cast<float *>(w + lay.logits);
    p.gate = reinterpret_cast<float *>(w + lay.gate);
    p.idx = topk_idx_opt ? topk_idx_opt : reinterpret_cast<int *>(w + lay.idx);
    p.w = topk_w_opt ? topk_w_opt : reinterpret_cast<float *>(w + lay.w);
    p.gamma = reinterpret_cast<float *>(w + lay.gamma);
    p.blkcnt = reinterpret_cast<int *>(w + lay.blkcnt);
    p.rank = reinterpret_cast<int *>(w + lay.rank);
    p.gcnt = reinterpret_cast<int *>(w + lay.gcnt);
    p.goff = reinterpret_cast<int *>(w + lay.goff);
    p.ntiles = reinterpret_cast<int *>(w + lay.ntiles);
    p.tiles = reinterpret_cast<int2 *>(w + lay.tiles);
    p.perm = reinterpret_cast<int *>(w + lay.perm);
    p.pos = reinterpret_cast<int *>(w + lay.pos);
    p.hh = reinterpret_cast<_Float16 *>(w + lay.hh);
    p.hl = reinterpret_cast<_Float16 *>(w + lay.hl);
    p.out = reinterpret_cast<float *>(w + lay.out);
    p.rhi = reinterpret_cast<uint16_t *>(w + lay.rhi);
    p.rlo = reinterpret_cast<uint16_t *>(w + lay.rlo);
    p.lpart = reinterpret_cast<float *>(w + lay.lpart);
    p.wgu = reinterpret_cast<int4 *>(w + lay.wgu);
    p.wdn = reinterpret_cast<int4 *>(w + lay.wdn);
    p.max_wgu = lay.max_wgu;
    p.max_wdn = lay.max_wdn;
    p.x16 = reinterpret_cast<_Float16 *>(w + lay.x16);
    p.xe = reinterpret_cast<int *>(w + lay.xe);
    p.hexp = reinterpret_cast<int *>(w + lay.hexp);
    p.y = y;
    p.status = status_word ? status_word : reinterpret_cast<int *>(w);
    hipError_t err = moe::launch_batched(p, lay, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
}  // namespace

moe_status moe_layer_batched(const moe_shape *s, const moe_layer *L, const uint16_t *x, int32_t T,
                             float *y, int32_t *topk_idx_opt, float *topk_w_opt, float *logits_opt,
                             void *ws, size_t ws_bytes, void *stream) {
    return batched_common(s, L, x, T, y, topk_idx_opt, topk_w_opt, logits_opt, ws, ws_bytes, stream, nullptr);
}

moe_status moe_layer_batched_table(const moe_shape *s, const moe_layer *L, const uint64_t *expert_table,
                                   const uint16_t *x, int32_t T, float *y, int32_t *topk_idx_opt,
                                   float *topk_w_opt, float *logits_opt, void *ws, size_t ws_bytes,
                                   void *stream) {
    if (!expert_table) return MOE_ERR_INVALID_ARG;
    return batched_common(s, L, x, T, y, topk_idx_opt, topk_w_opt, logits_opt, ws, ws_bytes, stream,
                          expert_table);
}

int32_t moe_layer_path(const moe_shape *s, int32_t T, int32_t crossover) {
    if (check_shape(s) != MOE_OK || T < 1 || T > kMaxBatchT) return -1;
    const int cross = crossover > 0 ? crossover : MOE_DEFAULT_CROSSOVER;
    if (T > cross || T > kMaxDecodeT) return MOE_PATH_BATCHED;
    int grid = moe::device_cu_count();
    if (grid <= 0) grid = kAssumedCus;
    if (grid > moe::kMaxGrid || decode_supported(s, T, grid) != MOE_OK) return MOE_PATH_BATCHED;
    return MOE_PATH_DECODE;
}

moe_status moe_layer_forward(const moe_shape *s, const moe_layer *L, const uint16_t *x, int32_t T,
                             int32_t crossover, float *y, int32_t *topk_idx_opt, float *topk_w_opt,
                             float *logits_opt, void *ws, size_t ws_bytes, void *stream) {
    moe_status st = check_shape(s);
    if (st != MOE_OK) return st;
    if (T < 1 || T > kMaxBatchT) return MOE_ERR_INVALID_ARG;
    if (!ws || !al16(ws) || ws_bytes < moe_workspace_bytes(s, T, 0, MOE_WS_FORWARD)) return MOE_ERR_WORKSPACE;
    const size_t dpart = forward_decode_part(s);
    if (moe_layer_path(s, T, crossover) == MOE_PATH_DECODE)
        return moe_layer_decode(s, L, x, T, y, topk_idx_opt, topk_w_opt, logits_opt, ws, dpart, stream);
    // the batched part reports through the workspace's first word, as the decode part does
    return batched_common(s, L, x, T, y, topk_idx_opt, topk_w_opt, logits_opt, static_cast<char *>(ws) + dpart,
                          ws_bytes - dpart, stream, nullptr, static_cast<int *>(ws));
}

moe_status moe_group_pairs(const moe_shape *s, const int32_t *topk_idx, int32_t T, int32_t *counts,
                           int32_t *offsets, int32_t *perm, int32_t *pos, void *ws, size_t ws_bytes,
                           void *stream) {
    moe_status st = check_shape(s);
    if (st != MOE_OK) return st;
    if (T < 1 || T > kMaxBatchT) return MOE_ERR_INVALID_ARG;
    if (!topk_idx || !counts || !offsets || !perm || !pos) return MOE_ERR_INVALID_ARG;
    if (!al4(topk_idx) || !al4(counts) || !al4(offsets) || !al4(perm) || !al4(pos)) return MOE_ERR_INVALID_ARG;
    if (!ws || !al16(ws) || ws_bytes < batched_ws_bytes(s, T)) return MOE_ERR_WORKSPACE;
    const moe::BatchedWs lay = moe::batched_ws_layout(T, s->hidden, s->num_experts, s->top_k, s->inter,
                                                      s->shared_inter);
    char *w = static_cast<char *>(ws);
    moe::BatchedParams p;
    memset(&p, 0, sizeof p);
    p.H = s->hidden; p.E = s->num_experts; p.K = s->top_k; p.I = s->inter; p.Is = 0;
    p.Imax = p.I; p.bits = s->bits; p.T = T;
    p.idx = const_cast<int *>(topk_idx);
    p.blkcnt = reinterpret_cast<int *>(w + lay.blkcnt);
    p.rank = reinterpret_cast<int *>(w + lay.rank);
    p.gcnt = counts;
    p.goff = offsets;
    p.ntiles = reinterpret_cast<int *>(w + lay.ntiles);
    p.tiles = reinterpret_cast<int2 *>(w + lay.tiles);
    p.perm = perm;
    p.pos = pos;
    hipError_t err = moe::launch_bucket(p, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
