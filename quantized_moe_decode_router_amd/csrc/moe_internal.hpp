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

// Decode of L chained layers (L = 1 for a single layer). Every weight pointer is the layer-0
// base of an [L]-stacked array; ls_* are the per-layer strides in elements.
struct DecodeParams {
    int H, E, K, I, Is, bits, T, L, glue;
    int Imax;         // max(I, Is): row stride of the h buffer
    int rows_per_wg;  // down-projection rows owned by each workgroup
    unsigned spin_limit;
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
    // workspace
    int *ctrl;      // [0] status, [1] barrier arrivals, [2] barrier generation
    float *logits;  // [T][E+1]: router logits, column E = shared-gate logit
    float *hbuf;    // [T][K+1][Imax]: routed h at slot k, shared h at slot K
    float *ybuf;    // [T][H]
};

struct DecodeLds {
    size_t xs, lg, sidx, sw, gam, part, red, total;
};

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

__host__ __device__ inline DecodeLds decode_lds_layout(int T, int H, int E, int K, int rows_per_wg) {
    DecodeLds d;
    size_t o = 0;
    d.xs = o;   o = align_up(o + sizeof(float) * (size_t)T * H, 16);
    d.lg = o;   o = align_up(o + sizeof(float) * (size_t)T * (E + 1), 16);
    d.sidx = o; o = align_up(o + sizeof(int) * (size_t)T * K, 16);
    d.sw = o;   o = align_up(o + sizeof(float) * (size_t)T * K, 16);
    d.gam = o;  o = align_up(o + sizeof(float) * (size_t)T, 16);
    d.part = o; o = align_up(o + sizeof(float) * (size_t)T * (K + 1) * rows_per_wg, 16);
    d.red = o;  o = align_up(o + sizeof(float) * 64, 16);
    d.total = o;
    return d;
}

constexpr int kDecodeThreads = 512;

// Enqueue the decode kernel(s). persistent != 0: one cooperative launch with grid barriers;
// persistent == 0: one launch per phase (3 per layer). Returns a hipError_t.
hipError_t launch_decode(const DecodeParams &p, int grid, hipStream_t stream, int persistent);

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

// Query (and cache per device) the compute-unit count.
int device_cu_count();

}  // namespace moe
