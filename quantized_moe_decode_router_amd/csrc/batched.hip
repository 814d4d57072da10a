// batched.hip -- one MoE layer for a batch of T tokens (prefill / batched decode) on gfx950.
//
// Six launches on one stream (seven when step 3 takes two), no host synchronisation:
//   1. router_gemm   logits[T][E] (+ shared-gate logit) = x . R^T on v_mfma_f32_16x16x32_bf16, the
//                    fp32 router split into bf16 hi + lo halves on its way into LDS (x is bf16,
//                    exact)
//   2. topk_kernel   per token one wave: top-k by (logit desc, index asc), renormalised weights
//                    (softmax of the kept logits), gamma = sigmoid(gate logit); beside it another
//                    wave: x as scaled fp16
//   3. bucket_small  (T <= 1024, E <= 512) the two steps below in one workgroup, counts in LDS
//      bucket_count  per block of 64 tokens: per-expert counts and every pair's rank in its block
//      bucket_plan   one workgroup: exclusive scans, stable scatter (pairs of one expert stay in
//                    pair order), the inverse map, the list of 128-row tiles of every group
//                    (routed experts, then the shared expert as group E with one row per token)
//                    and the two GEMMs' work lists, longest first
//   4. gu_gemm       per item: [<=128 pairs x H] . [H x (128 gate + 128 up) rows] on
//                    v_mfma_f32_16x16x32_f16, codes dequantised to fp16 in registers, SwiGLU
//                    epilogue; h is stored as fp16 hi + lo halves (22 significant bits)
//   5. dn_gemm       per item: [<=128 pairs x I] . [I x 256 output rows], once with h hi and once
//                    with h lo; epilogue scales by the routing weight (gamma for the shared group)
//   6. combine       y[t] = sum_k out[pos(t, k)] + out[shared row of t], k = 0..K-1 in order
//
// MFMA operands are fp16, products exact in the fp32 accumulators: x scaled by a power of two per
// token (any bf16 x fits), the dequantised weights s * q + b rounded once, and h as fp16
// hi + lo halves scaled down by a power of two per tile and 64-column group where its magnitude
// needs it (the down GEMM scales that k-step's dequantised weights up by the same power, so each
// product is unchanged). So s, b and s * q + b must lie within fp16's range (+-65504), and so must a
// down weight times that power (|W2| max|h| below ~2^31); a weight beyond it becomes infinite, the
// accumulators it reaches are not finite, and the epilogues then set the status word to
// MOE_ERR_UNSUPPORTED (the outputs are then undefined). Weights and h below 2^-14 in magnitude are
// held as fp16 subnormals.
#include <type_traits>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;         // pair rows of an A stage in LDS
constexpr int kXcds = 8;         // XCDs of the device: workgroup b of a launch runs on XCD b mod 8
static_assert(kTileRows <= kBM, "a tile's rows fit one A stage");
constexpr int kGemmThreads = 256;
constexpr int kLdsK = 72;        // fp16 per LDS tile row: 64 + 8 padding (16 bytes)

__device__ __forceinline__ _Float16 bf16_to_f16(uint16_t b) { return (_Float16)bf16_to_f32(b); }

// ---- 1. router GEMM ------------------------------------------------------------------------------
// logits = x . R^T on bf16 MFMA: x is bf16 (exact), every fp32 router weight is split into
// bf16 hi = rne(R) and lo = rne(R - hi), so R - hi - lo is below 2^-17 |R|; both products are exact
// in the fp32 accumulators. Rows E+1: the router, then the shared gate.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Tile: 32 tokens x 32 router rows x one of ks contiguous ranges of H (blockIdx.z), k-steps of 64;
// wave w: tokens 16 (w & 1) .., rows 16 (w >> 1) ... The range's partial sums go to lpart; the
// top-k kernel adds the ranges in order (the ranges keep the k-loop of a workgroup short, so
// that many workgroups hide each other's load latency).
constexpr int kRtT = 32, kRtN = 32;
constexpr int kRtSteps = 8;  // k-steps per range: H / 64 / router_ksplit(H) <= 2048 / 64 / 4
__host__ __device__ inline int router_ksplit(int H) { return H / 64 < kRouterSplitK ? H / 64 : kRouterSplitK; }

__global__ void __launch_bounds__(kGemmThreads) router_gemm(BatchedParams p) {
    __shared__ __align__(16) uint16_t xs[2][kRtT][kLdsK];
    __shared__ __align__(16) uint16_t rh[2][kRtN][kLdsK];
    __shared__ __align__(16) uint16_t rl[2][kRtN][kLdsK];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int t0 = blockIdx.x * kRtT, n0 = blockIdx.y * kRtN;
    const int H = p.H, E = p.E, T = p.T;
    const int N = E + (p.sgate ? 1 : 0);
    // loads: row r (8 bf16 at c) of the x tile and of both router tiles
    const int r = tid / 8, c = (tid % 8) * 8;
    const bool xok = t0 + r < T, rok = n0 + r < N;
    const uint16_t *xrow = p.x + (size_t)(xok ? t0 + r : 0) * H;
    const float *frow = !rok ? p.router : (n0 + r < E ? p.router + (size_t)(n0 + r) * H : p.sgate);
    struct St {
        uint4 x;
        float4 f0, f1;
    };
    // rows past T or N read row 0 (their results are not stored), so every load is unconditional
    auto load = [&](int kb) {
        St st;
        st.x = *reinterpret_cast<const uint4 *>(xrow + kb * 64 + c);
        st.f0 = *reinterpret_cast<const float4 *>(frow + kb * 64 + c);
        st.f1 = *reinterpret_cast<const float4 *>(frow + kb * 64 + c + 4);
        return st;
    };
    // the fp32 router weights split into bf16 hi = rne(R) and lo = rne(R - hi) on the way into LDS
    auto store = [&](const St &st, int bf) {
        *reinterpret_cast<uint4 *>(&xs[bf][r][c]) = st.x;
        auto split2 = [](float a, float b, uint32_t &hi, uint32_t &lo) __attribute__((always_inline)) {
            const uint16_t h0 = f32_to_bf16_rne(a), h1 = f32_to_bf16_rne(b);
            hi = h0 | (uint32_t)h1 << 16;
            lo = f32_to_bf16_rne(a - bf16_to_f32(h0)) | (uint32_t)f32_to_bf16_rne(b - bf16_to_f32(h1)) << 16;
        };
        uint4 hi, lo;
        split2(st.f0.x, st.f0.y, hi.x, lo.x);
        split2(st.f0.z, st.f0.w, hi.y, lo.y);
        split2(st.f1.x, st.f1.y, hi.z, lo.z);
        split2(st.f1.z, st.f1.w, hi.w, lo.w);
        *reinterpret_cast<uint4 *>(&rh[bf][r][c]) = hi;
        *reinterpret_cast<uint4 *>(&rl[bf][r][c]) = lo;
    };
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const int th = wave & 1, nh = wave >> 1;
    auto mfma_step = [&](int bf) {
#pragma unroll
        for (int ks = 0; ks < 64; ks += 32) {
            const int kc = ks + 8 * (lane / 16);
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(&xs[bf][16 * th + lane % 16][kc]);
            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&rh[bf][16 * nh + lane % 16][kc]);
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&rl[bf][16 * nh + lane % 16][kc]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc, 0, 0, 0);
        }
    };
    // this range's k-steps (at most kRtSteps: H <= 2048, H / 4 per range): every load is
    // issued up front, then each k-step goes through one of two LDS buffers (k-step j + 1 is stored
    // while k-step j's MFMAs run: one barrier per k-step); the barriers are LDS-only, so that the
    // loads of later k-steps stay in flight
    const int nk = H / 64 / router_ksplit(H), k0 = blockIdx.z * nk;
    St S[kRtSteps];
#pragma unroll
    for (int j = 0; j < kRtSteps; ++j) S[j] = load(k0 + min(j, nk - 1));
    store(S[0], 0);
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kRtSteps; ++j) {
        if (j < nk) {  // nk is uniform
            if (j + 1 < nk) store(S[j + 1], (j + 1) & 1);
            mfma_step(j & 1);
            lds_barrier();
        }
    }
    // lane l, register q -> token t0 + 16 th + 4 (l / 16) + q, row n0 + 16 nh + l % 16
    const int n = n0 + 16 * nh + lane % 16;
    float *part = p.lpart + (size_t)blockIdx.z * T * N;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int t = t0 + 16 * th + 4 * (lane / 16) + q;
        if (t < T && n < N) part[(size_t)t * N + n] = acc[q];
    }
}

// ---- 2. top-k per token, x as fp16 -------------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
template <int BITS>
__device__ void act16_to_pairs8(const uint4 r, int sh, half2_t *out);

// x16[t] = x[t] * 2^-xe[t] in fp16, columns in pair order (see the grouped GEMMs), with xe[t] =
// E - 15 for the token's largest magnitude in [2^(E-1), 2^E): the token's values fill fp16's range
// up to 2^15 whatever their bf16 magnitude (only values more than 2^29 below the token's largest
// become fp16 subnormals); the power-of-two scaling is exact and the gate|up epilogue multiplies
// it back. One wave per token.
template <int BITS>
__device__ __forceinline__ void wave_x16(const BatchedParams &p, int t) {
    const int lane = threadIdx.x % kWave, H = p.H;
    const uint16_t *xr = p.x + (size_t)t * H;
    constexpr int NC = 4;  // H <= 2048: at most 4 chunks of 8 columns per lane
    uint4 v[NC];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = (i * kWave + lane) * 8;
        v[i] = c < H ? *reinterpret_cast<const uint4 *>(xr + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(w[k] & 0xFFFF)), fabsf(bf16_to_f32(w[k] >> 16))));
    }
    amax = __int_as_float((int)wave_max_u32(__float_as_uint(amax)));  // non-negative floats order as integers
    int e = 0;
    if (amax > 0.0f) {
        frexpf(amax, &e);
        e -= 15;
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = (i * kWave + lane) * 8;
        if (c >= H) break;
        half2_t hv[4];
        act16_to_pairs8<BITS>(v[i], -e, hv);
        *reinterpret_cast<uint4 *>(p.x16 + (size_t)t * H + c) = __builtin_bit_cast(uint4, hv);
    }
    if (lane == 0) p.xe[t] = e;
}

// kTopkTokens tokens per workgroup: wave w < kTopkTokens selects token w's experts while wave
// kTopkTokens + w scales its x, so the two latency chains of a token run side by side.
constexpr int kTopkTokens = 2;
__global__ void __launch_bounds__(2 * kTopkTokens * kWave) topk_kernel(BatchedParams p) {
    extern __shared__ __align__(16) char smem[];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int E = p.E, K = p.K;
    const int t = blockIdx.x * kTopkTokens + wave % kTopkTokens;
    if (t >= p.T) return;  // whole wave leaves together; no workgroup barrier follows
    if (wave >= kTopkTokens) {
        if (p.x16) {
            if (p.bits == 4) wave_x16<4>(p, t);
            else wave_x16<8>(p, t);
        }
        return;
    }
    float *lt = reinterpret_cast<float *>(smem) + (size_t)wave * E;
    // logits: the router GEMM's range partial sums added in range order, then the bias
    const int N = E + (p.sgate ? 1 : 0), ks = router_ksplit(p.H);
    const float *part = p.lpart + (size_t)t * N;
    const size_t zs = (size_t)p.T * N;
    // every partial sum of this lane's logits, their biases and the gate partials in flight at
    // once (E <= 1024, ks <= 4)
    float g[kRouterSplitK];
#pragma unroll
    for (int z = 0; z < kRouterSplitK; ++z) g[z] = p.sgate && z < ks ? part[z * zs + E] : 0.0f;
    for (int e0 = 0; e0 < E; e0 += 4 * kWave) {
        float v[4][kRouterSplitK], bias[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = min(e0 + u * kWave + lane, E - 1);
#pragma unroll
            for (int z = 0; z < kRouterSplitK; ++z) v[u][z] = z < ks ? part[z * zs + e] : 0.0f;
            bias[u] = p.rbias ? p.rbias[e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * kWave + lane;
            if (e >= E) break;
            float a = v[u][0];
            for (int z = 1; z < ks; ++z) a += v[u][z];
            if (p.rbias) a += bias[u];
            lt[e] = a;
            p.logits[(size_t)t * E + e] = a;
        }
    }
    float gate = 0.0f;
    if (p.sgate) {
        gate = g[0];
        for (int z = 1; z < ks; ++z) gate += g[z];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    wave_topk(lt, E, K, p.idx + (size_t)t * K, p.w + (size_t)t * K);
    if (lane == 0 && p.gamma) p.gamma[t] = p.sgate ? 1.0f / (1.0f + expf(-gate)) : 0.0f;
}

// ---- 3. histogram, exclusive scan, stable scatter, tile list -------------------------------------
// Two launches. bucket_count: one wave per block of 64 tokens (one lane each), four blocks per
// workgroup; wave-private LDS holds one 64-bit mask per expert with bit l set when token (block, l)
// selected that expert. popcount(mask) is the block's count for the expert and popcount(mask &
// lanes below) the pair's rank among the block's pairs of the same expert. bucket_plan: one
// workgroup: per-expert exclusive prefixes over blocks, the scans of the group sizes, tile counts
// and work items, the tile list, the work lists, then every pair's place: expert offset + its
// block's prefix + its rank, so pairs of one expert stay in token order, which is pair order (a
// token selects an expert at most once). The shared expert is group E with one row per token.
constexpr int kCountWaves = 4;
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kMaxGroups = 1025;  // experts (<= 1024) and the shared expert

__global__ void __launch_bounds__(kCountWaves * kWave) bucket_count(BatchedParams p) {
    extern __shared__ __align__(16) char smem[];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int T = p.T, K = p.K, E = p.E;
    const int blk = blockIdx.x * kCountWaves + wave;
    if (blk * kWave >= T) return;  // whole wave leaves together; no workgroup barrier follows
    unsigned long long *masks = reinterpret_cast<unsigned long long *>(smem) + (size_t)wave * E;
    const unsigned long long below = (1ull << lane) - 1ull;
    const int t = blk * kWave + lane;
    const bool valid = t < T;
    for (int e = lane; e < E; e += kWave) masks[e] = 0ull;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int ex[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) ex[k] = k < K && valid ? min((unsigned)p.idx[(size_t)t * K + k], (unsigned)(E - 1)) : -1;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (ex[k] >= 0) atomicOr(&masks[ex[k]], 1ull << lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (ex[k] >= 0) p.rank[(size_t)t * K + k] = __popcll(masks[ex[k]] & below);
    for (int e = lane; e < E; e += kWave) p.blkcnt[(size_t)blk * E + e] = __popcll(masks[e]);
}

// From the group sizes gcnt[0..E) (per-block prefixes already in place): the shared group's size,
// the scans of the group sizes, tile counts and work items (goff, gtoff, the totals in p.ntiles),
// p.gcnt / p.goff, the tile list and, when p.wgu is set, both GEMMs' work lists, longest first.
// Called by the whole workgroup of kPlanThreads; the arrays live in the caller's LDS.
__device__ void plan_groups(const BatchedParams &p, int *gcnt, int *goff, int *gtoff, int *hgu, int *hdn, int *hds,
                            int *hdc) {
    const int tid = threadIdx.x;
    const int T = p.T, E = p.E;
    const int ng = E + (p.Is ? 1 : 0);  // groups: experts, then the shared expert
    if (tid == 0 && p.Is) gcnt[E] = T;
    // every slot of both work lists starts as an empty item (rows = 0), the real items overwrite
    // theirs below: a GEMM workgroup reads its slot directly, with no load of the item count first
    if (p.wgu) {
        for (int i = tid; i < p.max_wgu; i += kPlanThreads) p.wgu[i] = make_int4(0, 0, 0, 0);
        for (int i = tid; i < p.max_wdn; i += kPlanThreads) p.wdn[i] = make_int4(0, 0, 0, 0);
    }
    __syncthreads();
    // exclusive scans of the group sizes, their tile counts and their gate|up and down work items
    const int ndn = p.H / kDnCols;
    auto ngu_of = [&](int g) { return (g < E ? p.I : p.Is) / kGuCols; };
    if (tid < kWave) {
        // one wave: lane l sums the run of groups [l G, l G + G), G = ceil(ng / 64), in order; a wave
        // scan of the runs' totals; then the run's exclusive offsets, group by group
        const int G = (ng + kWave - 1) / kWave, g0 = tid * G, g1 = min(g0 + G, ng);
        int v[4] = {0, 0, 0, 0};
        for (int g = g0; g < g1; ++g) {
            const int nt = (gcnt[g] + kTileRows - 1) / kTileRows;
            v[0] += gcnt[g];
            v[1] += nt;
            v[2] += nt * ngu_of(g);
            v[3] += nt * ndn;
        }
        int inc[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int x = __shfl_up(inc[i], o, kWave);
                if (tid >= o) inc[i] += x;
            }
        }
        int e0 = inc[0] - v[0], e1 = inc[1] - v[1];
        for (int g = g0; g < g1; ++g) {
            const int c = gcnt[g];
            goff[g] = e0;
            gtoff[g] = e1;
            e0 += c;
            e1 += (c + kTileRows - 1) / kTileRows;
        }
        if (tid == kWave - 1) {
            goff[ng] = inc[0];
            gtoff[ng] = inc[1];
            p.ntiles[0] = inc[1];
            p.ntiles[1] = inc[2];
            p.ntiles[2] = inc[3];
        }
    }
    __syncthreads();
    for (int g = tid; g <= ng; g += kPlanThreads) {
        p.goff[g] = goff[g];
        if (g < ng) p.gcnt[g] = gcnt[g];
    }
    for (int g = tid; g < ng; g += kPlanThreads) {
        const int nt = (gcnt[g] + kTileRows - 1) / kTileRows;
        for (int i = 0; i < nt; ++i) p.tiles[gtoff[g] + i] = make_int2(g, i * kTileRows);
    }
    // work items of the grouped GEMMs, longest first: a counting sort of the tiles by row count
    // (128 rows down to 1), so that the workgroups taken in list order fill the compute units
    // greedily and the heavy tiles do not form the tail. Within a bucket the order is arbitrary
    // (each item writes its own block of the output, so it does not change any result).
    if (p.wgu) {
        for (int i = tid; i <= kTileRows; i += kPlanThreads) hgu[i] = hdn[i] = 0;
        __syncthreads();
        const int ntile = gtoff[ng];
        // tile i: its group by binary search over the tile offsets
        auto tile_group = [&](int i) {
            int lo = 0, hi = ng - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (gtoff[mid] <= i) lo = mid;
                else hi = mid - 1;
            }
            return lo;
        };
        const int gfirst = tid < ntile ? tile_group(tid) : 0;  // this thread's first tile, used twice
        for (int i = tid; i < ntile; i += kPlanThreads) {
            const int g = i == tid ? gfirst : tile_group(i), m0 = (i - gtoff[g]) * kTileRows, rows = min(kTileRows, gcnt[g] - m0);
            atomicAdd(&hgu[rows], ngu_of(g));
            atomicAdd(&hdn[rows], ndn);
        }
        __syncthreads();
        if (tid < kWave) {  // exclusive prefix from kTileRows rows down: lane l owns rows kTileRows - RPL l - j
            constexpr int RPL = kTileRows / kWave;  // row counts per lane, j = 0 .. RPL-1
            static_assert(kTileRows % kWave == 0, "whole row counts per lane");
            int cu = 0, cd = 0;
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const int r = kTileRows - RPL * tid - j;  // >= 1
                cu += hgu[r];
                cd += hdn[r];
            }
            int iu = cu, id = cd;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int a = __shfl_up(iu, o, kWave), b = __shfl_up(id, o, kWave);
                if (tid >= o) {
                    iu += a;
                    id += b;
                }
            }
            int eu = iu - cu, ed = id - cd;
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const int r = kTileRows - RPL * tid - j;
                const int hu = hgu[r], hd = hdn[r];
                hgu[r] = eu;
                hdn[r] = ed;
                hds[r] = ed;  // the down bucket's first slot and its item count
                hdc[r] = hd;
                eu += hu;
                ed += hd;
            }
        }
        __syncthreads();
        for (int i = tid; i < ntile; i += kPlanThreads) {
            const int g = i == tid ? gfirst : tile_group(i), mi = i - gtoff[g], m0 = mi * kTileRows,
                      rows = min(kTileRows, gcnt[g] - m0);
            const int nu = ngu_of(g);
            const int bu = atomicAdd(&hgu[rows], nu), bd = atomicAdd(&hdn[rows], ndn);
            for (int c = 0; c < nu; ++c)
                p.wgu[bu + c] = make_int4(g, goff[g] + m0, rows | (c * kGuCols) << 16, i);
            // The down items of one tile all read the tile's h rows: within each whole group of
            // kXcds tiles of a bucket, tile q's items take the slots of one residue mod kXcds
            // (workgroup b runs on XCD b mod kXcds), so they run on one XCD and share its L2's copy
            // of those rows; the bucket's last, partial group keeps consecutive slots.
            const int B = hds[rows], nb = hdc[rows] / ndn, q = (bd - B) / ndn, full = nb / kXcds * kXcds;
            for (int c = 0; c < ndn; ++c) {
                const int slot = q < full ? B + (q / kXcds) * kXcds * ndn + c * kXcds + q % kXcds : bd + c;
                p.wdn[slot] = make_int4(g, goff[g] + m0, rows | (c * kDnCols) << 16, i);
            }
        }
    }
}

__global__ void __launch_bounds__(kPlanThreads) bucket_plan(BatchedParams p) {
    __shared__ int gcnt[kMaxGroups], goff[kMaxGroups + 1], gtoff[kMaxGroups + 1];
    __shared__ int hgu[kTileRows + 1], hdn[kTileRows + 1], hds[kTileRows + 1], hdc[kTileRows + 1];
    const int tid = threadIdx.x;
    const int T = p.T, K = p.K, E = p.E;
    const int nblk = (T + kWave - 1) / kWave;
    // per expert: exclusive prefix over blocks (in place) and the total; the counts of eight blocks
    // are loaded before any is rewritten, so that a chunk costs one memory round trip
    if (tid < E) {
        const int e = tid;
        int run = 0;
        for (int b0 = 0; b0 < nblk; b0 += 8) {
            int c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = b0 + i < nblk ? p.blkcnt[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (b0 + i < nblk) p.blkcnt[(size_t)(b0 + i) * E + e] = run;
                run += c[i];
            }
        }
        gcnt[e] = run;
    }
    plan_groups(p, gcnt, goff, gtoff, hgu, hdn, hds, hdc);
    // scatter: four pairs per thread in flight at once
    const int TK = T * K;
    for (int q0 = tid; q0 < TK; q0 += 4 * kPlanThreads) {
        int e[4], r[4], c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = q0 + u * kPlanThreads;
            e[u] = q < TK ? min((unsigned)p.idx[q], (unsigned)(E - 1)) : 0;
            r[u] = q < TK ? p.rank[q] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = q0 + u * kPlanThreads;
            c[u] = q < TK ? p.blkcnt[(size_t)(q / K / kWave) * E + e[u]] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = q0 + u * kPlanThreads;
            if (q < TK) {
                const int P = goff[e[u]] + c[u] + r[u];
                p.perm[P] = q;
                p.pos[q] = P;
            }
        }
    }
    if (p.Is)
        for (int t = tid; t < T; t += kPlanThreads) p.perm[(size_t)TK + t] = t * K;
}

// Both bucket steps in one workgroup, for T <= 64 kPlanWaves tokens and E <= kSmallBucketE: wave w
// builds block w's lane masks as bucket_count does, but the counts and the per-block prefixes stay
// in LDS and every pair's rank stays in the register of the lane that scatters it, so that no
// count, rank or index goes back through memory between the steps. The results are those of the
// two-launch form.
constexpr int kSmallBucketE = 512;
__host__ __device__ inline size_t bucket_small_lds_bytes(int E) { return 12 * (size_t)kPlanWaves * E; }
__global__ void __launch_bounds__(kPlanThreads) bucket_small(BatchedParams p) {
    extern __shared__ __align__(16) char smem[];
    __shared__ int gcnt[kMaxGroups], goff[kMaxGroups + 1], gtoff[kMaxGroups + 1];
    __shared__ int hgu[kTileRows + 1], hdn[kTileRows + 1], hds[kTileRows + 1], hdc[kTileRows + 1];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int T = p.T, K = p.K, E = p.E;
    const int nblk = (T + kWave - 1) / kWave;  // <= kPlanWaves
    unsigned long long *masks = reinterpret_cast<unsigned long long *>(smem) + (size_t)wave * E;
    int *cnt = reinterpret_cast<int *>(smem + 8 * (size_t)kPlanWaves * E);  // [block][E]
    const unsigned long long below = (1ull << lane) - 1ull;
    const int t = wave * kWave + lane;
    const bool valid = wave < nblk && t < T;
    int ex[16], rk[16];
    // the selections are loaded first, so that their latency covers the mask clearing
#pragma unroll
    for (int k = 0; k < 16; ++k) ex[k] = k < K && valid ? min((unsigned)p.idx[(size_t)t * K + k], (unsigned)(E - 1)) : -1;
    for (int e = lane; e < E; e += kWave) masks[e] = 0ull;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (ex[k] >= 0) atomicOr(&masks[ex[k]], 1ull << lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < 16; ++k) rk[k] = ex[k] >= 0 ? __popcll(masks[ex[k]] & below) : 0;
    if (wave < nblk)
        for (int e = lane; e < E; e += kWave) cnt[wave * E + e] = __popcll(masks[e]);
    __syncthreads();
    // per expert: exclusive prefix over blocks (in place) and the total
    for (int e = tid; e < E; e += kPlanThreads) {
        int run = 0;
        for (int b = 0; b < nblk; ++b) {
            const int c = cnt[b * E + e];
            cnt[b * E + e] = run;
            run += c;
        }
        gcnt[e] = run;
    }
    plan_groups(p, gcnt, goff, gtoff, hgu, hdn, hds, hdc);
    // scatter by the lane that ranked the pair: expert offset + block prefix + rank
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (ex[k] >= 0) {
            const int q = t * K + k, P = goff[ex[k]] + cnt[wave * E + ex[k]] + rk[k];
            p.perm[P] = q;
            p.pos[q] = P;
        }
    if (p.Is)
        for (int u = tid; u < T; u += kPlanThreads) p.perm[(size_t)T * K + u] = u * K;
}

// ---- shared pieces of the grouped GEMMs -------------------------------------------------------------
struct GroupW {
    const uint8_t *c;
    const uint16_t *s, *b;
    int inter;
};
// Weights of group g of a matrix family: routed expert g < E, or the shared expert (g == E).
__device__ __forceinline__ GroupW group_w13(const BatchedParams &p, int g) {
    const size_t H = p.H;
    if (g < p.E && p.xtab) {
        const uint64_t blk = p.xtab[g] & ~1ull;
        return {reinterpret_cast<const uint8_t *>(blk), reinterpret_cast<const uint16_t *>(blk + p.xo13s),
                reinterpret_cast<const uint16_t *>(blk + p.xo13b), p.I};
    }
    if (g < p.E) {
        const size_t rows = 2 * (size_t)p.I;
        return {p.w13.c + g * rows * H * p.bits / 8, p.w13.s + g * rows * (H / 64), p.w13.b + g * rows * (H / 64),
                p.I};
    }
    return {p.s13.c, p.s13.s, p.s13.b, p.Is};
}
__device__ __forceinline__ GroupW group_w2(const BatchedParams &p, int g) {
    const size_t H = p.H;
    if (g < p.E && p.xtab) {
        const uint64_t blk = p.xtab[g] & ~1ull;
        return {reinterpret_cast<const uint8_t *>(blk + p.xo2c), reinterpret_cast<const uint16_t *>(blk + p.xo2s),
                reinterpret_cast<const uint16_t *>(blk + p.xo2b), p.I};
    }
    if (g < p.E) {
        const size_t cols = p.I;
        return {p.w2.c + g * H * cols * p.bits / 8, p.w2.s + g * H * (cols / 64), p.w2.b + g * H * (cols / 64), p.I};
    }
    return {p.s2.c, p.s2.s, p.s2.b, p.Is};
}

// Global-memory view of a pointer: loads through it compile to global (not flat) instructions,
// which count against the vector-memory counter only, so waiting for a load never also waits for
// LDS traffic (and LDS waits never wait for the weight loads in flight).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *gp(const T *p) {
    return (const __attribute__((address_space(1))) T *)p;
}

// A 16-byte global load (through a native vector type: HIP's uint4 has no address-space load).
typedef unsigned int u32x4n_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(const void *p) {
    const u32x4n_t v = *(const __attribute__((address_space(1))) u32x4n_t *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A non-finite accumulator: an fp16 operand was out of range (see the file header).
__device__ __forceinline__ void flag_unsupported(int *status) {
    __hip_atomic_store(status, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- fp16 tiles: column order --------------------------------------------------------------------
// Inside every 8-column block (4-bit) or 4-column block (8-bit) the A operands of the grouped GEMMs
// (x for gate|up, h for down) hold their columns in the order the packed dequantisation produces
// them: 4-bit (0,4,1,5,2,6,3,7), 8-bit (0,2,1,3). Both operands of every MFMA use the same order,
// so each product and each k-sum is that of the natural order.
template <int BITS>
__device__ __forceinline__ int pair_pos(int c) {  // stored position of column c (blocks stay in place)
    if constexpr (BITS == 4) return (c & ~7) + 2 * (c & 3) + ((c >> 2) & 1);
    else return (c & ~3) + 2 * (c & 1) + ((c >> 1) & 1);
}

// 8 bf16 activations (natural order) times 2^sh -> 8 fp16 in pair order (4-bit: one block of 8;
// 8-bit: two blocks of 4).
template <int BITS>
__device__ void act16_to_pairs8(const uint4 r, int sh, half2_t *out) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = ldexpf(bf16_to_f32(w[i] & 0xFFFF), sh);
        v[2 * i + 1] = ldexpf(bf16_to_f32(w[i] >> 16), sh);
    }
    if constexpr (BITS == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = half2_t{(_Float16)v[q], (_Float16)v[q + 4]};
    } else {
        out[0] = half2_t{(_Float16)v[0], (_Float16)v[2]};
        out[1] = half2_t{(_Float16)v[1], (_Float16)v[3]};
        out[2] = half2_t{(_Float16)v[4], (_Float16)v[6]};
        out[3] = half2_t{(_Float16)v[5], (_Float16)v[7]};
    }
}

// ---- 4 / 5. grouped GEMMs --------------------------------------------------------------------------
// Both GEMMs run one work item per workgroup of 512 threads (8 waves, one workgroup per compute
// unit): a tile of up to 128 pair rows of one group (A, fp16) against a block of the group's weight
// rows (B), in k-steps of 64 columns (one quantisation group). Each wave owns 32 weight rows and
// every row of the tile; a lane holds the MFMA B fragments of one weight row (row l % 16 of a
// 16-row block): the 16 columns [16 (l / 16), +16) of the group, which in pair order are its k
// values of both 32-column fragments. It dequantises them in registers, one k-step ahead of the
// MFMAs, so each code is dequantised once per tile and the dequantised weights never pass through
// LDS.
//
// Every operand reaches LDS through the LDS-DMA form of the global load, issued from inline
// assembly: per k-step the tile's A rows (shared by the waves; chunk c of row r stored at
// c ^ (r & 7), so the 16 rows of a fragment read spread over the banks), and each wave's own
// weight codes (whole 64-column groups of its 32 rows) with their scales and biases. The
// loop therefore holds no load the compiler tracks: the vector-memory counter completes in issue
// order, so a compiler wait for one load would also wait for every DMA issued before it. Batch kb
// = {A(kb), B(kb + 1)} is issued L k-steps ahead into rings of L + 1 stages; at the top of k-step
// kb each wave waits until only the L - 1 younger batches are outstanding, then an LDS-only
// barrier makes every wave's A(kb) visible and frees the stages read in k-step kb - 1. Loads past
// the last k-step are clamped to it, so that every batch has the same number of DMAs and the
// counts in the waits hold; the workgroup drains its DMAs before it leaves.
//
// The k-loop is compiled once per count MT of 16-row subtiles that hold rows of the tile, so that
// a k-step has no branches inside and the MFMAs of one k-step interleave with the dequantisation of
// the next. Block b runs slot b of a work list ordered longest first (see plan_groups); the
// slots past the list's items hold rows = 0, and their blocks return at once.
__device__ __forceinline__ int chunk_pos(int row, int c) { return c ^ (row & 7); }

constexpr int kGW = kGemmWavesG;           // waves per grouped-GEMM workgroup
constexpr int kGT = kGW * kWave;           // threads per grouped-GEMM workgroup

// ---- LDS DMA --------------------------------------------------------------------------------------
// The LDS-DMA load writes lane l's 16 (4) bytes to LDS address M0 + 16 l (4 l), M0 wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    // a generic pointer into LDS converted to its 32-bit LDS address (address space 3)
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)p));
}
// The scalar copy of a value the caller knows to be wave-uniform (for scalar-register operands).
// (readfirstlane returns int: each half goes through uint32_t so that the low half is not
// sign-extended into the high one)
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const void *uniform(const void *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void *>(lo | hi << 32);
}
// 16 bytes per lane from the wave-uniform base sbase plus the lane's 32-bit byte offset voff.
__device__ __forceinline__ void dma16s(uint32_t voff, const void *sbase, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform(sbase)),
                 "s"(uniform(m0))
                 : "memory", "m0");
}
// 4 bytes per lane from the lane's own address.
__device__ __forceinline__ void dma4v(const void *g, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(uniform(m0))
                 : "memory", "m0");
}
// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// (a & m) | o in one instruction (for constant operands the compiler emits an AND and an OR)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(o));
    return d;
}

// Codes -> fp16 s q + b, two per packed instruction: a code masked into the mantissa of the fp16
// constant 1024 reads as 1024 + q; the subtraction of 1024 is exact and one packed fma rounds
// s q + b once. 4-bit: a dword holds columns 0..7 of a block, giving pairs (0,4) (1,5) (2,6) (3,7);
// 8-bit: a dword holds columns 0..3, giving pairs (0,2) (1,3) -- the pair order of the A tiles.
// One fragment (8 columns): 4-bit from one dword, 8-bit from two.
template <int BITS>
__device__ __forceinline__ half8_t dequant_frag(uint32_t d0, uint32_t d1, half2_t s2, half2_t b2) {
    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    half2_t h0, h1, h2, h3;
    if constexpr (BITS == 4) {
        const uint32_t M = 0x64006400u;
        h0 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(d0, 0x000F000Fu, M)) - k1024, s2, b2);
        h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(d0 >> 4, 0x000F000Fu, M)) - k1024, s2, b2);
        h2 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(d0 >> 8, 0x000F000Fu, M)) - k1024, s2, b2);
        h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(d0 >> 12, 0x000F000Fu, M)) - k1024, s2, b2);
    } else {
        const uint32_t K64 = 0x64646464u;
        h0 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(K64, d0, 0x04020400u)) - k1024, s2, b2);
        h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(K64, d0, 0x04030401u)) - k1024, s2, b2);
        h2 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(K64, d1, 0x04020400u)) - k1024, s2, b2);
        h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(K64, d1, 0x04030401u)) - k1024, s2, b2);
    }
    return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}
__device__ __forceinline__ half2_t f16_splat(uint16_t bf, float f) {
    const _Float16 h = (_Float16)(bf16_to_f32(bf) * f);
    return half2_t{h, h};
}

// Pipeline parameters of the grouped GEMMs (gate|up: DN = false; down: DN = true).
//   BB    bytes of a weight row per B block (a whole 128-byte cache line for gate|up)
//   SB    k-steps per B block
//   L     k-steps of lookahead: batch t = {A(t + L), and every SB k-steps one B block} is issued at
//         k-step t, and k-step kb waits for the batches issued up to k-step kb - L
//   NBUF  B block buffers per wave, (NBUF - 1) SB >= L so that a block's buffer is free when the
//         block two (or three) ahead is issued into it
//   RA    A stages (L + 1)
//   NBC   DMAs per B block and wave (32 rows x BB bytes)
//   LO    a lookahead other than the default L0 for some items (their k-loop only: the LDS layout,
//         i.e. the A region, the per-wave B ring stride and the scale quarters, is the default's)
template <int BITS, bool DN, int LO = 0>
struct GCfg {
    static constexpr int BB = DN ? 64 : 128;
    static constexpr int SB = BB / (8 * BITS);
    static constexpr int L0 = DN ? (BITS == 4 ? 2 : 1) : (BITS == 4 ? 3 : 2);
    static constexpr int L = LO ? LO : L0;
    static constexpr int NBUF0 = (L0 + SB - 1) / SB + 1;
    static constexpr int NBUF = (L + SB - 1) / SB + 1;
    static constexpr int RA0 = L0 + 1;
    static constexpr int RA = L + 1;
    static constexpr int NBC = 32 * BB / 1024;
    static constexpr int A_STAGE = (DN ? 2 : 1) * kBM * 128;  // A bytes per stage (h: hi and lo)
    static constexpr int B_BLOCK = 32 * BB;                    // B bytes per block and wave
    static_assert(NBUF <= NBUF0, "a B ring within the default's");
    // LDS bytes for ng groups per weight row: A stages, B buffers, then each wave's scale and bias
    // quarters (16 rows x ng groups x 2 bytes each)
    __host__ __device__ static constexpr int lds_bytes(int ng) {
        return RA0 * A_STAGE + kGW * NBUF0 * B_BLOCK + kGW * 4 * 32 * ng;
    }
    __host__ __device__ static constexpr int b_off() { return RA0 * A_STAGE; }
    __host__ __device__ static constexpr int s_off() { return RA0 * A_STAGE + kGW * NBUF0 * B_BLOCK; }
};

// Outstanding DMAs allowed at the top of k-step kb (kb % SB = j): those of the batches issued at
// k-steps kb - L + 1 .. kb - 1 (NA each, plus NBC in the k-steps that issue a B block).
template <int L, int SB, int NA, int NBC>
__host__ __device__ constexpr int wait_count(int j) {
    int n = 0;
    for (int d = 1; d <= L - 1; ++d) {
        const int tm = ((j - d) % SB + SB) % SB;
        n += NA + ((tm + 1 + L) % SB == 0 ? NBC : 0);
    }
    return n;
}
template <int L, int SB, int NA, int NBC, int J>
__device__ __forceinline__ void wait_step() {
    vm_wait<wait_count<L, SB, NA, NBC>(J)>();
}

// Both 16-row blocks' fragments of one k-step.
struct BQ {
    half8_t r0q0, r0q1, r1q0, r1q1;
};

// A wave's weight DMA lanes. The wave's 32 rows are rowof(0..31); rows 0..15 form its first 16-row
// block, 16..31 its second. B block b of the wave: 32 rows x BB bytes (row r's bytes [b BB, +BB)),
// stored row-major with 16-byte piece p of row r at piece p ^ (r & (BB / 16 - 1)). DMA u, lane l
// fills LDS slot 1024 u + 16 l (row r = slot / BB, piece p) from the row's piece p ^ (r & ...).
// Scales: four quarters per wave (scales of rows 0..15, of rows 16..31, biases of rows 0..15, of
// rows 16..31), each 16 rows x ng groups x 2 bytes, contiguous in memory and in LDS.
template <int BITS, bool DN>
struct WDma {
    uint32_t coff[GCfg<BITS, DN>::NBC];  // per DMA: the lane's byte offset from the block's base
    const uint16_t *q[4];                // the four quarters' first elements
};
template <int BITS, bool DN, typename RowOf>
__device__ __forceinline__ WDma<BITS, DN> wdma_lanes(const GroupW &W, int ng, int lane, RowOf rowof) {
    using C = GCfg<BITS, DN>;
    WDma<BITS, DN> d;
    const size_t rowbytes = (size_t)ng * 8 * BITS;
#pragma unroll
    for (int u = 0; u < C::NBC; ++u) {
        const int f = 1024 * u + 16 * lane, r = f / C::BB, pc = (f % C::BB) / 16;
        d.coff[u] = (uint32_t)(rowof(r) * rowbytes + (pc ^ (r & (C::BB / 16 - 1))) * 16);
    }
    d.q[0] = W.s + rowof(0) * (size_t)ng;
    d.q[1] = W.s + rowof(16) * (size_t)ng;
    d.q[2] = W.b + rowof(0) * (size_t)ng;
    d.q[3] = W.b + rowof(16) * (size_t)ng;
    return d;
}
// The four scale quarters of the wave (32 ng bytes each; lanes past a quarter's end do not load).
template <int BITS, bool DN>
__device__ __forceinline__ void wdma_scales(const WDma<BITS, DN> &d, int ng, int lane, char *sq) {
    const int qbytes = 32 * ng;  // <= 1024: ng <= 32
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t m0 = lds_addr(sq + k * qbytes);
        if (16 * lane < qbytes) dma16s(16 * lane, d.q[k], m0);
    }
}
template <int BITS, bool DN>
__device__ __forceinline__ void wdma_block(const WDma<BITS, DN> &d, const GroupW &W, int b, char *buf) {
    using C = GCfg<BITS, DN>;
    const uint8_t *base = W.c + (size_t)b * C::BB;
#pragma unroll
    for (int u = 0; u < C::NBC; ++u) dma16s(d.coff[u], base, lds_addr(buf + 1024 * u));
}
// The lane's scale and bias halves (bf16 bits) of one B block's SB k-steps for its two rows:
// quarter k (scales of rows fi, 16 + fi, then biases), k-step j at bits 16 (j & 1) of w[k][j / 2].
// One LDS read per quarter and block (SB halves at once) instead of one per k-step: a quarter's
// 16 rows sit ng halves apart, so these reads conflict on the banks whatever their width.
template <int SB>
struct SBlk {
    uint32_t w[4][(SB + 1) / 2];
};
template <int SB>
__device__ __forceinline__ SBlk<SB> load_sblk(const char *sq, int ng, int kb0, int fi) {
    SBlk<SB> b;
    const int qb = 32 * ng;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const char *a = sq + k * qb + (fi * ng + kb0) * 2;  // kb0 % SB == 0: aligned to 2 SB bytes
        if constexpr (SB == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(a);
            b.w[k][0] = v.x;
            b.w[k][1] = v.y;
        } else if constexpr (SB == 2) {
            b.w[k][0] = *reinterpret_cast<const uint32_t *>(a);
        } else {
            b.w[k][0] = *reinterpret_cast<const uint16_t *>(a);
        }
    }
    return b;
}
template <int SB, int J>
__device__ __forceinline__ uint16_t sblk_half(const SBlk<SB> &b, int k) {
    return static_cast<uint16_t>(b.w[k][J / 2] >> (16 * (J & 1)));
}
// The lane's fragments of k-step kb = J (mod SB) (slice J of the block in buf; f scales s and b).
template <int BITS, bool DN, int J>
__device__ __forceinline__ BQ dequant_step(const char *buf, const SBlk<GCfg<BITS, DN>::SB> &sb, float f, int fi,
                                           int fj) {
    using C = GCfg<BITS, DN>;
    constexpr int m = C::BB / 16 - 1;
    constexpr int s = J;
    const half2_t s0 = f16_splat(sblk_half<C::SB, J>(sb, 0), f);
    const half2_t s1 = f16_splat(sblk_half<C::SB, J>(sb, 1), f);
    const half2_t b0 = f16_splat(sblk_half<C::SB, J>(sb, 2), f);
    const half2_t b1 = f16_splat(sblk_half<C::SB, J>(sb, 3), f);
    const int r0 = fi, r1 = 16 + fi;
    BQ q;
    if constexpr (BITS == 4) {
        const int P = 2 * s + (fj >> 1), o = (fj & 1) * 8;
        const uint2 c0 = *reinterpret_cast<const uint2 *>(buf + r0 * C::BB + ((P ^ (r0 & m)) * 16) + o);
        const uint2 c1 = *reinterpret_cast<const uint2 *>(buf + r1 * C::BB + ((P ^ (r1 & m)) * 16) + o);
        q.r0q0 = dequant_frag<4>(c0.x, 0, s0, b0);
        q.r0q1 = dequant_frag<4>(c0.y, 0, s0, b0);
        q.r1q0 = dequant_frag<4>(c1.x, 0, s1, b1);
        q.r1q1 = dequant_frag<4>(c1.y, 0, s1, b1);
    } else {
        const int P = 4 * s + fj;
        const uint4 c0 = *reinterpret_cast<const uint4 *>(buf + r0 * C::BB + ((P ^ (r0 & m)) * 16));
        const uint4 c1 = *reinterpret_cast<const uint4 *>(buf + r1 * C::BB + ((P ^ (r1 & m)) * 16));
        q.r0q0 = dequant_frag<8>(c0.x, c0.y, s0, b0);
        q.r0q1 = dequant_frag<8>(c0.z, c0.w, s0, b0);
        q.r1q0 = dequant_frag<8>(c1.x, c1.y, s1, b1);
        q.r1q1 = dequant_frag<8>(c1.z, c1.w, s1, b1);
    }
    return q;
}

// f(integral_constant<J>) for J = B .. E - 1, each with J a constant expression.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// The k-loop shared by both GEMMs, unrolled by SB so that every wait count is a constant.
// issue_a(kb): the A DMAs of k-step kb (NA per wave); mfma(stage, bq): the MFMAs of one k-step on
// A stage `stage`; dq(kb, buf, j): the fragments of k-step kb from B buffer `buf`, j = kb % SB as an
// integral constant.
// BAR = false: every wave reads only LDS it filled itself (its own copy of the A rows), so its own
// vmcnt waits suffice and the k-steps need no workgroup barrier.
template <typename C, int NA, bool BAR, typename IssueA, typename IssueB, typename Mfma, typename Dq>
__device__ __forceinline__ void kloop(int nk, IssueA issue_a, IssueB issue_b, Mfma mfma, Dq dq) {
    constexpr int L = C::L, SB = C::SB, NBC = C::NBC;
    // the batches of k-steps -1 - L .. -1 (A only from A(0) on)
#pragma unroll
    for (int t = -1 - L; t <= -1; ++t) {
        if (t + L >= 0) issue_a(t + L);
        if ((t + 1 + L) % SB == 0) issue_b((t + 1 + L) / SB);
    }
    wait_step<L, SB, NA, NBC, 0>();
    BQ bq = dq(0, 0, std::integral_constant<int, 0>{});
    for (int kb0 = 0; kb0 < nk; kb0 += SB) {
        static_for<0, SB>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int kb = kb0 + j;
            wait_step<L, SB, NA, NBC, j>();
            if constexpr (BAR) lds_barrier();
            else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own LDS reads done before the DMAs reuse a stage
            issue_a(kb + L);
            if constexpr ((j + 1 + L) % SB == 0) issue_b((kb + 1 + L) / SB);
            mfma(kb % C::RA, bq);
            bq = dq(kb + 1, ((kb + 1) / SB) % C::NBUF, std::integral_constant<int, (j + 1) % SB>{});
        });
    }
    vm_wait<0>();  // no DMA may still write this workgroup's LDS once it leaves
}

// Items of at most kPrivMT subtiles whose private A stages fit the shared A region take private A
// rows and a barrier-free k-loop, with the lookahead priv_lookahead.
constexpr int kPrivMT = 1;
template <int BITS, bool DN>
constexpr int priv_lookahead(int mt) {
    return GCfg<BITS, DN>::L0;
}
template <int BITS, bool DN>
constexpr bool priv_items(int mt) {
    using C = GCfg<BITS, DN>;
    return mt <= kPrivMT && kGW * (priv_lookahead<BITS, DN>(mt) + 1) * (DN ? 2 : 1) * mt * 16 * 128 <= C::RA0 * C::A_STAGE;
}

// gate|up + SwiGLU. Item: rows P0 .. P0+M-1 of group g against gate rows j0 .. j0+127 and up rows
// inter + j0 .. +127. Wave w: gate rows j0 + 16 w + (0..15) (its first row block) and the up rows
// of the same j (its second), so a lane's accumulators hold gate and up of the same (row, j).
template <int BITS, int MT>
__device__ __forceinline__ void gu_body(const BatchedParams &p, char *lds, int g, int P0, int M, int j0, int tile) {
    // few subtiles: every wave stages its own copy of the A rows (MT 16-row blocks per k-step, RA
    // stages per wave within the shared A region) and the k-loop runs barrier-free
    constexpr bool PRIV = priv_items<BITS, false>(MT);
    using C = GCfg<BITS, false, PRIV ? priv_lookahead<BITS, false>(MT) : 0>;
    constexpr int NA = PRIV ? 2 * MT : (MT + 3) / 4;  // A DMAs per wave and k-step: 8 NA waves x 8 rows >= 16 MT
    const GroupW W = group_w13(p, g);
    const int tid = threadIdx.x, lane = tid % kWave, wave = (int)uniform(tid / kWave), fi = lane % 16, fj = lane / 16;
    const int H = p.H, K = p.K, nk = H / 64, ng = nk;
    uint4(*As)[kBM][8] = reinterpret_cast<uint4(*)[kBM][8]>(lds);
    uint4(*Ap)[16 * MT][8] = reinterpret_cast<uint4(*)[16 * MT][8]>(lds + wave * C::RA * MT * 16 * 128);  // PRIV
    static_assert(!PRIV || kGW * C::RA * MT * 16 * 128 <= C::RA0 * C::A_STAGE, "private A stages");
    char *bbuf = lds + C::b_off() + wave * C::NBUF0 * C::B_BLOCK;
    char *sq = lds + C::s_off() + wave * 4 * 32 * ng;
    // A DMA lanes: DMA u of wave w covers tile rows 8 d .. 8 d + 7, d = w + 8 u (PRIV: d = u); lane
    // l -> row 8 d + l / 8, LDS slot l % 8 = chunk (l % 8) ^ (row & 7). Rows past M read row 0's token.
    uint32_t aoff[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) {
        const int d = PRIV ? u : wave + kGW * u, r = 8 * d + lane / 8, c = (lane % 8) ^ (r & 7);
        const int tok = gp(p.perm)[P0 + (r < M ? r : 0)] / K;
        aoff[u] = (uint32_t)(((size_t)tok * H + c * 8) * 2);
    }
    const WDma<BITS, false> wd = wdma_lanes<BITS, false>(W, ng, lane, [&](int r) {
        return (size_t)(r < 16 ? j0 + 16 * wave + r : W.inter + j0 + 16 * wave + r - 16);
    });
    wdma_scales<BITS, false>(wd, ng, lane, sq);
    const int nblk = nk / C::SB;
    auto issue_a = [&](int kb) __attribute__((always_inline)) {
        const _Float16 *base = p.x16 + (size_t)min(kb, nk - 1) * 64;
#pragma unroll
        for (int u = 0; u < NA; ++u)
            dma16s(aoff[u], base,
                   lds_addr(PRIV ? &Ap[kb % C::RA][8 * u][0] : &As[kb % C::RA][8 * (wave + kGW * u)][0]));
    };
    auto issue_b = [&](int b) __attribute__((always_inline)) {
        wdma_block<BITS, false>(wd, W, min(b, nblk - 1), bbuf + (b % C::NBUF) * C::B_BLOCK);
    };
    float4_t ag[MT], au[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) ag[i] = au[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto mfma = [&](int stage, const BQ &bq) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const half8_t bg = q ? bq.r0q1 : bq.r0q0, bu = q ? bq.r1q1 : bq.r1q0;
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int ra = 16 * i + fi;
                const uint4 av = PRIV ? Ap[stage][ra][chunk_pos(ra, 2 * fj + q)] : As[stage][ra][chunk_pos(ra, 2 * fj + q)];
                const half8_t a = __builtin_bit_cast(half8_t, av);
                ag[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bg, ag[i], 0, 0, 0);
                au[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bu, au[i], 0, 0, 0);
            }
        }
    };
    SBlk<C::SB> sb;
    auto dq = [&](int kb, int buf, auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        if constexpr (J == 0) sb = load_sblk<C::SB>(sq, ng, min(kb, nk - C::SB), fi);
        return dequant_step<BITS, false, J>(bbuf + buf * C::B_BLOCK, sb, 1.0f, fi, fj);
    };
    kloop<C, NA, !PRIV>(nk, issue_a, issue_b, mfma, dq);
    // epilogue: lane l, register r of subtile i -> row 16 i + 4 (l / 16) + r, j = j0 + 16 w + l % 16.
    // The accumulators are scaled back by the token's 2^xe, SwiGLU applied, and h stored as fp16
    // hi + lo halves of h * 2^-e, e = max(0, E - 15) for the largest |h| of the tile in this
    // 64-column group (waves 0..3: j0 .., 4..7: j0 + 64 ..) in [2^(E-1), 2^E), in pair order.
    bool finite = true;
    float hmax = 0.0f;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * fj + r;
            const float sc = m < M ? ldexpf(1.0f, gp(p.xe)[gp(p.perm)[P0 + m] / K]) : 0.0f;
            const float gv = ag[i][r] * sc, uv = au[i][r] * sc;
            const float h = m < M ? gv / (1.0f + expf(-gv)) * uv : 0.0f;
            finite &= m >= M || (__builtin_isfinite(gv) && __builtin_isfinite(uv));  // rows past M: stale
            hmax = fmaxf(hmax, fabsf(h));
            ag[i][r] = h;
        }
    hmax = __int_as_float((int)wave_max_u32(__float_as_uint(hmax)));
    float *tmax = reinterpret_cast<float *>(lds);  // A stage 0, no longer read by any wave
    lds_barrier();
    if (lane == 0) tmax[wave] = hmax;
    lds_barrier();
    const int half = wave / 4;
    hmax = fmaxf(fmaxf(tmax[4 * half], tmax[4 * half + 1]), fmaxf(tmax[4 * half + 2], tmax[4 * half + 3]));
    int e = 0;
    if (hmax > 0.0f && __builtin_isfinite(hmax)) {
        frexpf(hmax, &e);
        e = max(0, e - 15);
    }
    const float hs = ldexpf(1.0f, -e);
    const int Imax = p.Imax;
    const int jj = j0 + 16 * wave + fi;
    const size_t col = (size_t)pair_pos<BITS>(jj);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * fj + r;
            if (m >= M) continue;
            const float h = ag[i][r] * hs;
            const _Float16 hh = (_Float16)h;
            const _Float16 hl = (_Float16)(h - (float)hh);
            const size_t o = (size_t)(P0 + m) * Imax + col;
            p.hh[o] = hh;
            p.hl[o] = hl;
        }
    if (lane == 0 && (wave & 3) == 0) p.hexp[(size_t)tile * (Imax / 64) + j0 / 64 + half] = e;
    if (!finite) flag_unsupported(p.status);
}

template <int BITS>
__global__ void __launch_bounds__(kGT, 1) gu_gemm(BatchedParams p) {
    extern __shared__ __align__(16) char smem[];
    const auto wq = gp(reinterpret_cast<const int *>(p.wgu + blockIdx.x));
    const int g = wq[0], P0 = wq[1], M = wq[2] & 0xFFFF, j0 = wq[2] >> 16, tile = wq[3];
    if (M == 0) return;  // a slot past the list's items
    switch ((M + 15) / 16) {
        case 1: gu_body<BITS, 1>(p, smem, g, P0, M, j0, tile); break;
        case 2: gu_body<BITS, 2>(p, smem, g, P0, M, j0, tile); break;
        case 3: gu_body<BITS, 3>(p, smem, g, P0, M, j0, tile); break;
        case 4: gu_body<BITS, 4>(p, smem, g, P0, M, j0, tile); break;
        case 5: gu_body<BITS, 5>(p, smem, g, P0, M, j0, tile); break;
        case 6: gu_body<BITS, 6>(p, smem, g, P0, M, j0, tile); break;
        case 7: gu_body<BITS, 7>(p, smem, g, P0, M, j0, tile); break;
        default: gu_body<BITS, 8>(p, smem, g, P0, M, j0, tile); break;
    }
}

// down projection x routing weight. Item: rows P0 .. P0+M-1 of group g (h hi and lo halves)
// against output rows n0 .. n0+255, k-steps of 64 over the group's inter. Wave w: output rows
// n0 + 32 w + (0..31) as two 16-row blocks; each k-step runs the MFMAs once on h hi and once on
// h lo. The k-step's weights are dequantised with scale and bias times 2^e, e the exponent of the
// h halves of this tile in this group, so that every product is the unscaled one.
template <int BITS, int MT>
__device__ __forceinline__ void dn_body(const BatchedParams &p, char *lds, int g, int P0, int M, int n0, int tile) {
    constexpr bool PRIV = priv_items<BITS, true>(MT);  // as in gate|up: private A rows (hi and lo), barrier-free k-loop
    using C = GCfg<BITS, true, PRIV ? priv_lookahead<BITS, true>(MT) : 0>;
    constexpr int NA = PRIV ? 2 * MT : (MT + 3) / 4;
    const GroupW W = group_w2(p, g);
    const int tid = threadIdx.x, lane = tid % kWave, wave = (int)uniform(tid / kWave), fi = lane % 16, fj = lane / 16;
    const int H = p.H, Imax = p.Imax, nk = W.inter / 64, ng = nk;
    // A stage s: hi tile at s * A_STAGE, lo tile 16 KiB after it
    uint4(*Ah)[kBM][8] = reinterpret_cast<uint4(*)[kBM][8]>(lds);
    uint4(*Ahp)[2][16 * MT][8] = reinterpret_cast<uint4(*)[2][16 * MT][8]>(lds + wave * C::RA * 2 * MT * 16 * 128);  // PRIV
    static_assert(!PRIV || kGW * C::RA * 2 * MT * 16 * 128 <= C::RA0 * C::A_STAGE, "private A stages");
    char *bbuf = lds + C::b_off() + wave * C::NBUF0 * C::B_BLOCK;
    char *sq = lds + C::s_off() + wave * 4 * 32 * ng;
    const int hexp0 = (int)((size_t)tile * (Imax / 64));
    uint32_t aoff[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) {
        const int d = PRIV ? u : wave + kGW * u, r = 8 * d + lane / 8, c = (lane % 8) ^ (r & 7);
        aoff[u] = (uint32_t)(((size_t)(P0 + (r < M ? r : 0)) * Imax + c * 8) * 2);
    }
    // the epilogue's routing weights of this lane's accumulator rows (rows past M repeat row M - 1):
    // their pair indices load with the h exponents, the weights themselves stay in flight through
    // the k-loop
    int qr[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) qr[i][r] = gp(p.perm)[P0 + min(16 * i + 4 * fj + r, M - 1)];
    // the tile's h exponents of every group, in registers of lanes 0..ng-1 (read with readlane)
    const int hexp_lane = lane < ng ? gp(p.hexp)[hexp0 + lane] : 0;
    asm volatile("" ::"v"(hexp_lane));  // the load completes here, before the first DMA is issued
    float wsc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wsc[i][r] = g < p.E ? gp(p.w)[qr[i][r]] : gp(p.gamma)[qr[i][r] / p.K];
    const WDma<BITS, true> wd =
        wdma_lanes<BITS, true>(W, ng, lane, [&](int r) { return (size_t)(n0 + 32 * wave + r); });
    wdma_scales<BITS, true>(wd, ng, lane, sq);
    const int nblk = nk / C::SB;
    auto issue_a = [&](int kb) __attribute__((always_inline)) {
        const size_t o = (size_t)min(kb, nk - 1) * 64;
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int st = kb % C::RA, row = 8 * (PRIV ? u : wave + kGW * u);
            dma16s(aoff[u], p.hh + o, lds_addr(PRIV ? &Ahp[st][0][row][0] : &Ah[2 * st][row][0]));
            dma16s(aoff[u], p.hl + o, lds_addr(PRIV ? &Ahp[st][1][row][0] : &Ah[2 * st + 1][row][0]));
        }
    };
    auto issue_b = [&](int b) __attribute__((always_inline)) {
        wdma_block<BITS, true>(wd, W, min(b, nblk - 1), bbuf + (b % C::NBUF) * C::B_BLOCK);
    };
    float4_t a0[MT], a1[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) a0[i] = a1[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto mfma = [&](int stage, const BQ &bq) __attribute__((always_inline)) {
        const uint4(*Hh)[8] = PRIV ? Ahp[stage][0] : Ah[2 * stage];
        const uint4(*Hl)[8] = PRIV ? Ahp[stage][1] : Ah[2 * stage + 1];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const half8_t b0 = q ? bq.r0q1 : bq.r0q0, b1 = q ? bq.r1q1 : bq.r1q0;
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int ra = 16 * i + fi;
                const half8_t ah = __builtin_bit_cast(half8_t, Hh[ra][chunk_pos(ra, 2 * fj + q)]);
                a0[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, b0, a0[i], 0, 0, 0);
                a1[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, b1, a1[i], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int ra = 16 * i + fi;
                const half8_t al = __builtin_bit_cast(half8_t, Hl[ra][chunk_pos(ra, 2 * fj + q)]);
                a0[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, b0, a0[i], 0, 0, 0);
                a1[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, b1, a1[i], 0, 0, 0);
            }
        }
    };
    SBlk<C::SB> sb;
    auto dq = [&](int kb, int buf, auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        const int k = min(kb, nk - 1);
        const float f = ldexpf(1.0f, __builtin_amdgcn_readlane(hexp_lane, k));
        if constexpr (J == 0) sb = load_sblk<C::SB>(sq, ng, min(kb, nk - C::SB), fi);
        return dequant_step<BITS, true, J>(bbuf + buf * C::B_BLOCK, sb, f, fi, fj);
    };
    kloop<C, 2 * NA, !PRIV>(nk, issue_a, issue_b, mfma, dq);
    // epilogue: lane l, register r of subtile i, block nb -> row 16 i + 4 (l / 16) + r, output row
    // n0 + 32 w + 16 nb + l % 16; scaled by the routing weight (gamma for the shared group)
    bool finite = true;
    const int n = n0 + 32 * wave + fi;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * fj + r;
            if (m >= M) continue;
            const float sc = wsc[i][r];
            finite &= __builtin_isfinite(a0[i][r]) && __builtin_isfinite(a1[i][r]);
            float *o = p.out + (size_t)(P0 + m) * H + n;
            o[0] = sc * a0[i][r];
            o[16] = sc * a1[i][r];
        }
    if (!finite) flag_unsupported(p.status);
}

template <int BITS>
__global__ void __launch_bounds__(kGT, 1) dn_gemm(BatchedParams p) {
    extern __shared__ __align__(16) char smem[];
    const auto wq = gp(reinterpret_cast<const int *>(p.wdn + blockIdx.x));
    const int g = wq[0], P0 = wq[1], M = wq[2] & 0xFFFF, n0 = wq[2] >> 16, tile = wq[3];
    if (M == 0) return;  // a slot past the list's items
    switch ((M + 15) / 16) {
        case 1: dn_body<BITS, 1>(p, smem, g, P0, M, n0, tile); break;
        case 2: dn_body<BITS, 2>(p, smem, g, P0, M, n0, tile); break;
        case 3: dn_body<BITS, 3>(p, smem, g, P0, M, n0, tile); break;
        case 4: dn_body<BITS, 4>(p, smem, g, P0, M, n0, tile); break;
        case 5: dn_body<BITS, 5>(p, smem, g, P0, M, n0, tile); break;
        case 6: dn_body<BITS, 6>(p, smem, g, P0, M, n0, tile); break;
        case 7: dn_body<BITS, 7>(p, smem, g, P0, M, n0, tile); break;
        default: dn_body<BITS, 8>(p, smem, g, P0, M, n0, tile); break;
    }
}

// ---- 6. fixed-order combine --------------------------------------------------------------------------
__global__ void __launch_bounds__(256) combine_kernel(BatchedParams p) {
    const int H = p.H, K = p.K, T = p.T;
    const int nq = H / 4;
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long long)T * nq) return;
    const int t = (int)(i / nq), c = (int)(i - (long long)t * nq) * 4;
    // every position, then every row, in flight at once (K <= 16); the sum keeps the order k = 0..K-1,
    // then the shared row
    int pk[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) pk[k] = k < K ? p.pos[(size_t)t * K + k] : 0;
    float4 v[17];
#pragma unroll
    for (int k = 0; k < 16; ++k)
        v[k] = k < K ? *reinterpret_cast<const float4 *>(p.out + (size_t)pk[k] * H + c) : make_float4(0, 0, 0, 0);
    v[16] = p.Is ? *reinterpret_cast<const float4 *>(p.out + ((size_t)T * K + t) * H + c) : make_float4(0, 0, 0, 0);
    float4 acc = make_float4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (k < K) {
            acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
        }
    if (p.Is) {
        acc.x += v[16].x; acc.y += v[16].y; acc.z += v[16].z; acc.w += v[16].w;
    }
    *reinterpret_cast<float4 *>(p.y + (size_t)t * H + c) = acc;
}

// ---- launch sequence ---------------------------------------------------------------------------------
hipError_t launch_router_topk(const BatchedParams &p, hipStream_t stream) {
    const int N = p.E + (p.sgate ? 1 : 0);
    hipLaunchKernelGGL(router_gemm, dim3((p.T + kRtT - 1) / kRtT, (N + kRtN - 1) / kRtN, router_ksplit(p.H)),
                       dim3(kGemmThreads), 0,
                       stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t lds = sizeof(float) * (size_t)kTopkTokens * p.E;
    hipLaunchKernelGGL(topk_kernel, dim3((p.T + kTopkTokens - 1) / kTopkTokens), dim3(2 * kTopkTokens * kWave), lds,
                       stream, p);
    return hipGetLastError();
}

size_t bucket_lds_bytes(int E) { return 8 * (size_t)kCountWaves * E; }

hipError_t launch_bucket(const BatchedParams &p, hipStream_t stream) {
    if (p.E > kMaxGroups - 1 || p.K > 16) return hipErrorInvalidValue;
    const int nblk = (p.T + kWave - 1) / kWave;
    if (nblk <= kPlanWaves && p.E <= kSmallBucketE) {
        const size_t lds = bucket_small_lds_bytes(p.E);
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&bucket_small),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(bucket_small, dim3(1), dim3(kPlanThreads), lds, stream, p);
        return hipGetLastError();
    }
    const size_t blds = bucket_lds_bytes(p.E);
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&bucket_count),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)blds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bucket_count, dim3((nblk + kCountWaves - 1) / kCountWaves), dim3(kCountWaves * kWave), blds,
                       stream, p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(bucket_plan, dim3(1), dim3(kPlanThreads), 0, stream, p);
    return hipGetLastError();
}

// A grouped-GEMM launch with `lds` bytes of dynamic LDS (above the default limit: the attribute
// first). The shapes that reach here keep lds within the compute unit's 160 KiB.
hipError_t launch_gemm(void (*kern)(BatchedParams), unsigned grid, int lds, hipStream_t stream, const BatchedParams &p) {
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kGT), (size_t)lds, stream, p);
    return hipGetLastError();
}

hipError_t launch_batched(const BatchedParams &p, const BatchedWs &lay, hipStream_t stream) {
    hipError_t err = launch_router_topk(p, stream);
    if (err != hipSuccess) return err;
    if ((err = launch_bucket(p, stream)) != hipSuccess) return err;
    // grids cover the work lists' capacities (blocks past the list's items find rows = 0 and return)
    const unsigned ggu = (unsigned)lay.max_wgu, gdn = (unsigned)lay.max_wdn;
    const int gu_lds4 = GCfg<4, false>::lds_bytes(p.H / 64), dn_lds4 = GCfg<4, true>::lds_bytes(p.Imax / 64);
    const int gu_lds8 = GCfg<8, false>::lds_bytes(p.H / 64), dn_lds8 = GCfg<8, true>::lds_bytes(p.Imax / 64);
    if (p.bits == 4) {
        if ((err = launch_gemm(gu_gemm<4>, ggu, gu_lds4, stream, p)) != hipSuccess) return err;
        if ((err = launch_gemm(dn_gemm<4>, gdn, dn_lds4, stream, p)) != hipSuccess) return err;
    } else {
        if ((err = launch_gemm(gu_gemm<8>, ggu, gu_lds8, stream, p)) != hipSuccess) return err;
        if ((err = launch_gemm(dn_gemm<8>, gdn, dn_lds8, stream, p)) != hipSuccess) return err;
    }
    const long long n = (long long)p.T * (p.H / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace moe
