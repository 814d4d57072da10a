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

// LDS plan of the decode kernel: byte offsets of every region (computed once on the host).
struct DecodeLds {
    int xp, lg, sidx, sw, gam, rt, sg, sd, rd, rg, hp, part, red, xq, xsx, hq, hsx, xt;
    int total;
};

// Decode of L layers (L = 1 for a single layer). Every weight pointer is the layer-0 base of an
// [L]-stacked array (each layer one contiguous block of the shape's size).
struct DecodeParams {
    int H, E, K, I, Is, bits, T, L;
    int chained;          // layer l+1 takes the RMS glue of y_l (else every layer takes x_in)
    int rows_per_wg;      // rows of y owned by each workgroup
    int nrr;              // router rows per workgroup (rows e = b + r * grid, r < nrr; row E = shared gate)
    int nps;              // shared-expert pairs per workgroup (j = b + r * grid, r < nps)
    int cp;               // routed gate|up pairs staged in LDS at once
    int log2I;            // log2(I)
    unsigned kdiv, tdiv;  // div_magic(K), div_magic(T)
    unsigned spin_limit;  // bound on every wait
    float eps;
    DecodeLds lds;
    const float *router, *rbias, *sgate;
    QMat w13, w2, s13, s2;
    const uint16_t *x_in;  // [T][H] bf16
    float *y_out;          // [T][H] fp32, last layer
    uint16_t *x_all;       // [L][T][H] or null
    float *y_all;          // [L][T][H] or null
    int *idx_all;          // [L][T][K] or null
    float *w_all;          // [L][T][K] or null
    float *logits_all;     // [L][T][E] or null
    // expert-table mode: routed expert (l, e) is the fixed-stride block at xtab[l * E + e] (device
    // or device-visible host memory), pieces at these byte offsets (gate|up codes at 0); w13 and w2
    // are then unused
    const uint64_t *xtab;  // bit 0 of an entry: the block is outside HBM (written through, below)
    uint32_t xo13s, xo13b, xo2c, xo2s, xo2b;
    uint64_t xstride;      // block bytes
    char *landing;         // or null: [L][T][K] blocks; rows staged from a marked block are stored
                           // to the block of their (layer, token, slot)
    // phase-timer build only (MOE_PHASE_TIMER): [L][grid][kPhaseMarks] real-time stamps, else null
    uint64_t *phase;
    // workspace (zero-filled before first use)
    int *ctrl;               // [0] status, [1] call sequence number, [2] wait bound (0 = default)
    uint64_t *ll_start;      // [grid]               one word per workgroup: "this call has started"
    uint64_t *ll_logits;     // [L][T][E+1]          router logits, column E = shared-gate logit
    uint64_t *ll_h;          // [L][T][K*I + Is]     routed h of slots 0..K-1, then the shared expert's h
    uint64_t *ll_y;          // [L][T][H]
};

// Fixed-stride expert container: routed expert (l, e) is one block of `stride` bytes holding its
// gate|up codes, scales, biases, then its down codes, scales, biases, each piece at a 256-byte
// aligned offset (the block size rounded up to 4 KiB).
struct ExpertBlock {
    size_t o13s, o13b, o2c, o2s, o2b, stride;
    size_t c13, s13, c2, s2;  // piece sizes in bytes (scales and biases alike)
};
__host__ inline ExpertBlock expert_block(int H, int I, int bits) {
    ExpertBlock x;
    x.c13 = (size_t)2 * I * H * bits / 8;
    x.s13 = (size_t)2 * I * (H / 64) * 2;
    x.c2 = (size_t)H * I * bits / 8;
    x.s2 = (size_t)H * (I / 64) * 2;
    auto a = [](size_t v) { return (v + 255) / 256 * 256; };
    x.o13s = a(x.c13);
    x.o13b = x.o13s + a(x.s13);
    x.o2c = x.o13b + a(x.s13);
    x.o2s = x.o2c + a(x.c2);
    x.o2b = x.o2s + a(x.s2);
    x.stride = (x.o2b + x.s2 + 4095) / 4096 * 4096;
    return x;
}

constexpr int kDecodeThreads = 512;
constexpr size_t kCtrlBytes = 256;

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout of the decode kernel (bytes from the workspace base). A library built with
// MOE_PHASE_TIMER keeps the per-layer phase stamps of every workgroup right after the control block.
struct DecodeWs {
    size_t phase, start, logits, h, y, total;
};
constexpr int kMaxGrid = 1024;
constexpr int kPhaseMarks = 21;
__host__ __device__ inline DecodeWs decode_ws_layout(int L, int T, int H, int E, int K, int I, int Is) {
    DecodeWs w;
    size_t o = kCtrlBytes;
#ifdef MOE_PHASE_TIMER
    w.phase = o;  o = align_up(o + 8 * (size_t)L * kMaxGrid * kPhaseMarks, 256);
#else
    w.phase = 0;
#endif
    w.start = o;  o = align_up(o + 8 * (size_t)kMaxGrid, 256);
    w.logits = o; o = align_up(o + 8 * (size_t)L * T * (E + 1), 256);
    w.h = o;      o = align_up(o + 8 * (size_t)L * T * ((size_t)K * I + Is), 256);
    w.y = o;      o = align_up(o + 8 * (size_t)L * T * H, 256);
    w.total = o;
    return w;
}

// LDS plan for a shape, token count and grid (router rows and shared pairs per workgroup and
// the y rows per workgroup follow from the grid); cp = routed gate|up pairs per LDS chunk.
__host__ inline DecodeLds decode_lds_plan(int T, int H, int E, int K, int I, int Is, int bits, int grid, int cp,
                                          bool xt = false) {
    DecodeLds d;
    const size_t RB = ((size_t)H + grid - 1) / grid;
    const size_t nrr = ((size_t)E + (Is ? 1 : 0) + grid - 1) / grid;
    const size_t nps = Is ? ((size_t)Is + grid - 1) / grid : 0;
    const size_t cbH = (size_t)H * bits / 8, sbH = (size_t)H / 32;
    const size_t cbS = (size_t)Is * bits / 8, sbS = (size_t)Is / 32;
    const size_t cbI = (size_t)I * bits / 8, sbI = (size_t)I / 32;
    const size_t nh = (size_t)K * I + Is;
    // hp: gathered h (fp32), the y gather buffer, the exchange-start gather and the gate|up partial
    // sums ([ranges][tokens][rows], ranges x tiles <= 8 or one range)
    size_t hp = nh * 4;
    if ((size_t)H * 4 > hp) hp = (size_t)H * 4;
    if ((size_t)kMaxGrid * 4 > hp) hp = (size_t)kMaxGrid * 4;
    const size_t gpart = 4 * (size_t)T * (128 > 2 * cp ? 128 : 2 * cp) + 8 * (size_t)T * nps;
    if (gpart > hp) hp = gpart;
    // the x pairs, the x limbs and the h limbs share one region (disjoint lifetimes), as do the two
    // limb-group tables
    size_t xp = 4 * (size_t)T * (H / 32) * 20;
    if (3 * (size_t)T * H > xp) xp = 3 * (size_t)T * H;
    if (3 * nh > xp) xp = 3 * nh;
    size_t gsx = 8 * (size_t)T * (H / 64);
    if (8 * (nh / 64) > gsx) gsx = 8 * (nh / 64);
    const size_t sz[15] = {
        xp,                              // xp (also xq and hq)
        4 * (size_t)T * (E + 1),         // lg
        4 * (size_t)T * K,               // sidx
        4 * (size_t)T * K,               // sw
        4 * (size_t)T,                   // gam
        4 * nrr * H,                     // rt
        2 * nps * (cbH + 2 * sbH),       // sg
        RB * (cbS + 2 * sbS),            // sd
        (size_t)K * RB * (cbI + 2 * sbI),  // rd
        2 * (size_t)cp * (cbH + 2 * sbH),  // rg
        hp,                              // hp
        4 * (size_t)T * (K + 1) * RB,    // part
        4 * 64,                          // red
        gsx,                             // xsx (also hsx)
        xt ? 16 * (size_t)E : 0};        // xt: two layers' rows of the expert table (expert-table mode)
    int *o[15] = {&d.xp, &d.lg, &d.sidx, &d.sw, &d.gam, &d.rt, &d.sg, &d.sd, &d.rd, &d.rg, &d.hp, &d.part, &d.red,
                  &d.xsx, &d.xt};
    size_t off = 0;
    for (int i = 0; i < 15; ++i) {
        *o[i] = (int)off;
        off = align_up(off + sz[i], 16);
    }
    d.xq = d.hq = d.xp;
    d.hsx = d.xsx;
    d.total = off > (size_t)0x7fffffff ? 0x7fffffff : (int)off;
    return d;
}
// Routed gate|up pairs per LDS chunk: every pair of the workgroup's share if that fits in
// `budget` bytes of LDS, else the largest power of two that does (0 if not even one pair fits).
__host__ inline int decode_chunk_pairs(int T, int H, int E, int K, int I, int Is, int bits, int grid, int budget,
                                      bool xt = false) {
    const long long total = (long long)T * K * I;
    int cp = (int)((total + grid - 1) / grid);
    int p2 = 1;
    while (p2 < cp) p2 <<= 1;
    for (int c = cp; c >= 1; c = (c == cp && cp != p2) ? p2 / 2 : c / 2)
        if (decode_lds_plan(T, H, E, K, I, Is, bits, grid, c, xt).total <= budget) return c;
    return 0;
}

// Enqueue the decode kernel. Returns a hipError_t.
hipError_t launch_decode(const DecodeParams &p, int grid, hipStream_t stream);

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
    int *ntiles;        // [4]: tiles, gate|up work items, down work items
    int2 *tiles;        // [max_tiles] (group, first row in group)
    int4 *wgu, *wdn;    // work items of the grouped GEMMs: {group, first row P0, rows | first column << 16,
                        // tile index}, ordered by group, then column block, then row tile
    int max_wgu, max_wdn;  // the lists' capacities (the GEMM grids); slots past the items hold rows = 0
    _Float16 *x16;      // [T][H] x as fp16 in pair order, scaled by 2^-xe[t]
    int *xe;            // [T] per-token exponent of that scaling
    int *hexp;          // [max_tiles][Imax/64] exponent e of h's fp16 halves in (tile, 64-column group):
                        // they hold h * 2^-e
    int *perm;          // [R] pair index t*K+k of each row (shared rows: t*K)
    int *pos;           // [T*K] row of each pair
    _Float16 *hh, *hl;  // [R][Imax] SwiGLU output, fp16 hi and lo halves
    float *out;         // [R][H] scaled down-projection rows
    float *y;           // [T][H]
    uint16_t *rhi, *rlo;  // [E+1][H] bf16 hi / lo halves of the router rows (row E = shared gate)
    float *lpart;         // [kRouterSplitK][T][E+1] router partial sums over quarters of H
    // expert-table mode: routed expert e is the fixed-stride block at xtab[e] (bit 0 ignored),
    // pieces at these byte offsets (gate|up codes at 0); w13 and w2 are then unused
    const uint64_t *xtab;
    uint32_t xo13s, xo13b, xo2c, xo2s, xo2b;
    // status word (the workspace's first word, or the decode part's in a moe_layer_forward
    // workspace): set to MOE_ERR_UNSUPPORTED (2) when a grouped-GEMM accumulator is not finite, i.e.
    // an fp16 operand (x, s*q + b or h) was beyond fp16's range
    int *status;
};
// The batched router GEMM splits H into this many contiguous ranges (fewer when H has fewer
// 64-column steps); the top-k kernel adds the partial sums in range order.
constexpr int kRouterSplitK = 4;

// Workspace layout of the batched path (bytes from the workspace base); R = T*K (+ T with a
// shared expert) rows.
struct BatchedWs {
    size_t logits, gate, idx, w, gamma, blkcnt, rank, gcnt, goff, ntiles, tiles, perm, pos, hh, hl, out, rhi, rlo,
        lpart, wgu, wdn, x16, xe, hexp, total;
    int max_tiles, max_wgu, max_wdn;
};
// Rows per tile of the grouped GEMMs, and the column blocks of one gate|up (j) and down (output row)
// work item.
constexpr int kTileRows = 128;
constexpr int kGuCols = 128;     // gate|up work item: 128 j (8 waves x 16)
constexpr int kDnCols = 256;     // down work item: 256 output rows (8 waves x 32)
constexpr int kGemmWavesG = 8;   // waves per grouped-GEMM workgroup
__host__ inline BatchedWs batched_ws_layout(int T, int H, int E, int K, int I, int Is) {
    BatchedWs w;
    const size_t TK = (size_t)T * K, R = TK + (Is ? (size_t)T : 0);
    const size_t Imax = I > Is ? I : Is, nblk = ((size_t)T + 63) / 64;
    const size_t touched = TK < (size_t)E ? TK : (size_t)E;
    w.max_tiles = (int)(TK / kTileRows + touched + (Is ? ((size_t)T + kTileRows - 1) / kTileRows : 0) + 1);
    w.max_wgu = w.max_tiles * (int)(Imax / kGuCols);
    w.max_wdn = w.max_tiles * (int)((size_t)H / kDnCols);
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
    w.rhi = o;    o = align_up(o + 2 * ((size_t)E + 1) * H, 256);
    w.rlo = o;    o = align_up(o + 2 * ((size_t)E + 1) * H, 256);
    w.lpart = o;  o = align_up(o + 4 * (size_t)kRouterSplitK * T * ((size_t)E + 1), 256);
    w.wgu = o;    o = align_up(o + 16 * (size_t)w.max_wgu, 256);
    w.wdn = o;    o = align_up(o + 16 * (size_t)w.max_wdn, 256);
    w.x16 = o;    o = align_up(o + 2 * (size_t)T * H, 256);
    w.xe = o;     o = align_up(o + 4 * (size_t)T, 256);
    w.hexp = o;   o = align_up(o + 4 * (size_t)w.max_tiles * (Imax / 64), 256);
    w.total = o;
    return w;
}
hipError_t launch_batched(const BatchedParams &p, const BatchedWs &lay, hipStream_t stream);
// Histogram / scan / stable scatter of the batched path (fills gcnt, goff, tiles, perm, pos).
hipError_t launch_bucket(const BatchedParams &p, hipStream_t stream);
// Router GEMM + per-token top-k of the batched path (fills logits, gate, idx, w, gamma).
hipError_t launch_router_topk(const BatchedParams &p, hipStream_t stream);

// Query (and cache per device) the compute-unit count.
int device_cu_count();

// The fixed device scratch of moe_stack_decode_static (one per device, held until the process
// ends): its device address on the current device, cleared on the stream on its first use on that
// device or when `reset` is set. hipErrorInvalidValue if `need` exceeds it. Allocates nothing.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(size_t need, bool reset, hipStream_t stream, void **out);

}  // namespace moe
