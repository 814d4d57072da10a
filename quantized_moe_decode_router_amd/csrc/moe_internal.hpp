// moe_internal.hpp -- parameter blocks and launchers shared between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct QMat {
    const uint8_t *c;   // codes
    const uint16_t *s;  // bf16 scales
    const uint16_t *b;  // bf16 biases
};

// Decode of L layers (L = 1 for a single layer). Every weight pointer is the layer-0 base of an
// [L]-stacked array; ls_* are the per-layer strides in elements.
struct DecodeParams {
    int H, E, K, I, Is, bits, T, L;
    int chained;          // layer l+1 takes the RMS glue of y_l (else every layer takes x_in)
    int rows_per_wg;      // rows of y owned by each workgroup
    unsigned spin_limit;  // bound on every wait
    float eps;
    const float *router, *rbias, *sgate;
    QMat w13, w2, s13, s2;
    long long ls_router, ls_rbias, ls_sgate;
    long long ls_w13c, ls_w13s, ls_w2c, ls_w2s, ls_s13c, ls_s13s, ls_s2c, ls_s2s;
    const uint16_t *x_in;  // [T][H] bf16
    float *y_out;          // [T][H] fp32, last layer
    uint16_t *x_all;       // [L][T][H] or null
    float *y_all;          // [L][T][H] or null
    int *idx_all;          // [L][T][K] or null
    float *w_all;          // [L][T][K] or null
    float *logits_all;     // [L][T][E] or null
    // workspace (zero-filled before first use)
    int *ctrl;               // [0] status, [1] call sequence number
    uint64_t *ll_start;      // [grid]            one word per workgroup: "this call has started"
    uint64_t *ll_logits;     // [L][T][E+1]       router logits, column E = shared-gate logit
    uint64_t *ll_h;          // [L][T][K][I]      routed h
    uint64_t *ll_hs;         // [L][T][Is]        shared-expert h
    uint64_t *ll_y;          // [L][T][H]
};

constexpr int kDecodeThreads = 512;
constexpr size_t kCtrlBytes = 256;

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout of the decode kernel (bytes from the workspace base).
struct DecodeWs {
    size_t start, logits, h, hs, y, total;
};
constexpr int kMaxGrid = 1024;
__host__ __device__ inline DecodeWs decode_ws_layout(int L, int T, int H, int E, int K, int I, int Is) {
    DecodeWs w;
    size_t o = kCtrlBytes;
    w.start = o;  o = align_up(o + 8 * (size_t)kMaxGrid, 256);
    w.logits = o; o = align_up(o + 8 * (size_t)L * T * (E + 1), 256);
    w.h = o;      o = align_up(o + 8 * (size_t)L * T * K * I, 256);
    w.hs = o;     o = align_up(o + 8 * (size_t)L * T * (Is > 0 ? Is : 1), 256);
    w.y = o;      o = align_up(o + 8 * (size_t)L * T * H, 256);
    w.total = o;
    return w;
}

// Enqueue the decode kernel. Returns a hipError_t.
hipError_t launch_decode(const DecodeParams &p, int grid, hipStream_t stream);
// Dynamic LDS bytes the decode kernel needs (0 if the shape does not fit).
size_t decode_lds_bytes(int T, int H, int E, int K, int I, int Is, int bits, int rows_per_wg);

// Router for T tokens: logits (or given logits), top-k, renormalised weights, optional gamma.
struct RouteParams {
    int H, E, K, T, has_gate, logits_in;
    const uint16_t *x;
    const float *router, *rbias, *sgate;
    float *logits;  // [T][E]
    int *idx;       // [T][K]
    float *w;       // [T][K]
    float *gamma;   // [T] or null
};
hipError_t launch_route(const RouteParams &p, hipStream_t stream);

// One batched layer (T tokens). Pointers into the workspace are carved by the host.
struct BatchedParams {
    int H, E, K, I, Is, Imax, bits, T;
    const uint16_t *x;  // [T][H] bf16
    const float *router, *rbias, *sgate;
    QMat w13, w2, s13, s2;
    float *logits;      // [T][E]
    float *gate;        // [T] shared-gate logit
    int *idx;           // [T][K]
    float *w;           // [T][K]
    float *gamma;       // [T]
    int *blkcnt;        // [ceil(T/64)][E] per-block counts, then per-block exclusive prefixes
    int *rank;          // [T*K] rank of a pair among its 64-token block's pairs of the same expert
    int *gcnt;          // [E+1] rows per group (group E = shared expert, T rows)
    int *goff;          // [E+2] first row of each group
    int *ntiles;        // [1]
    int2 *tiles;        // [max_tiles] (group, first row in group)
    int *perm;          // [R] pair index t*K+k of each row (shared rows: t*K)
    int *pos;           // [T*K] row of each pair
    _Float16 *hh, *hl;  // [R][Imax] SwiGLU output, fp16 hi and lo halves
    float *out;         // [R][H] scaled down-projection rows
    float *y;           // [T][H]
};

// Workspace layout of the batched path (bytes from the workspace base); R = T*K (+ T with a
// shared expert) rows.
struct BatchedWs {
    size_t logits, gate, idx, w, gamma, blkcnt, rank, gcnt, goff, ntiles, tiles, perm, pos, hh, hl, out, total;
    int max_tiles;
};
__host__ inline BatchedWs batched_ws_layout(int T, int H, int E, int K, int I, int Is) {
    BatchedWs w;
    const size_t TK = (size_t)T * K, R = TK + (Is ? (size_t)T : 0);
    const size_t Imax = I > Is ? I : Is, nblk = ((size_t)T + 63) / 64;
    const size_t touched = TK < (size_t)E ? TK : (size_t)E;
    w.max_tiles = (int)(TK / 64 + touched + (Is ? ((size_t)T + 63) / 64 : 0) + 1);
    size_t o = kCtrlBytes;
    w.logits = o; o = align_up(o + 4 * (size_t)T * E, 256);
    w.gate = o;   o = align_up(o + 4 * (size_t)T, 256);
    w.idx = o;    o = align_up(o + 4 * TK, 256);
    w.w = o;      o = align_up(o + 4 * TK, 256);
    w.gamma = o;  o = align_up(o + 4 * (size_t)T, 256);
    w.blkcnt = o; o = align_up(o + 4 * nblk * E, 256);
    w.rank = o;   o = align_up(o + 4 * TK, 256);
    w.gcnt = o;   o = align_up(o + 4 * ((size_t)E + 2), 256);
    w.goff = o;   o = align_up(o + 4 * ((size_t)E + 2), 256);
    w.ntiles = o; o = align_up(o + 16, 256);
    w.tiles = o;  o = align_up(o + 8 * (size_t)w.max_tiles, 256);
    w.perm = o;   o = align_up(o + 4 * R, 256);
    w.pos = o;    o = align_up(o + 4 * TK, 256);
    w.hh = o;     o = align_up(o + 2 * R * Imax, 256);
    w.hl = o;     o = align_up(o + 2 * R * Imax, 256);
    w.out = o;    o = align_up(o + 4 * R * (size_t)H, 256);
    w.total = o;
    return w;
}
hipError_t launch_batched(const BatchedParams &p, int max_tiles, hipStream_t stream);
// Histogram / scan / stable scatter of the batched path (fills gcnt, goff, tiles, perm, pos).
hipError_t launch_bucket(const BatchedParams &p, hipStream_t stream);
// Router GEMM + per-token top-k of the batched path (fills logits, gate, idx, w, gamma).
hipError_t launch_router_topk(const BatchedParams &p, hipStream_t stream);

// Query (and cache per device) the compute-unit count.
int device_cu_count();

}  // namespace moe
