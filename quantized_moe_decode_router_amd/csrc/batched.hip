// batched.hip -- one MoE layer for a batch of T tokens (prefill / batched decode) on gfx950.
//
// Seven launches on one stream, no host synchronisation:
//   1. router_split  the fp32 router (and shared gate) as bf16 hi + lo halves, once per call
//      router_gemm   logits[T][E] (+ shared-gate logit) = x . R^T on v_mfma_f32_16x16x32_bf16 over
//                    both halves (x is bf16, exact)
//   2. topk_kernel   one wave per token: top-k by (logit desc, index asc), renormalised weights
//                    (softmax of the kept logits), gamma = sigmoid(gate logit)
//   3. bucket_kernel one workgroup: per-expert histogram of the (token, slot) pairs, exclusive scan,
//                    stable scatter (pairs of one expert stay in pair order), the inverse map and
//                    the list of 64-row tiles of every group (routed experts, then the shared
//                    expert as group E with one row per token)
//   4. gu_gemm       per tile: [64 pairs x H] . [H x (64 gate + 64 up) rows] on
//                    v_mfma_f32_16x16x32_f16, codes dequantised to fp16 in LDS, SwiGLU epilogue;
//                    h is stored as fp16 hi + lo halves (22 significant bits)
//   5. dn_gemm       per tile: [64 pairs x I] . [I x 64 output rows], once with h hi and once with
//                    h lo; epilogue scales by the routing weight (gamma for the shared group)
//   6. combine       y[t] = sum_k out[pos(t, k)] + out[shared row of t], k = 0..K-1 in order
//
// MFMA operands are fp16, products exact in the fp32 accumulators: x scaled by a power of two per
// token (x16_kernel: any bf16 x fits), the dequantised weights s * q + b rounded once, and h as fp16
// hi + lo halves scaled down by a power of two per tile and 64-column group where its magnitude
// needs it (the down GEMM scales that k-step's dequantised weights up by the same power, so each
// product is unchanged). So s, b and s * q + b must lie within fp16's range (+-65504), and so must a
// down weight times that power (|W2| max|h| below ~2^31); a weight beyond it becomes infinite, the
// accumulators it reaches are not finite, and the epilogues then set the status word to
// MOE_ERR_UNSUPPORTED (the outputs are then undefined). Weights and h below 2^-14 in magnitude are
// held as fp16 subnormals.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = kTileRows;   // pair rows per tile
constexpr int kGemmThreads = 256;
constexpr int kRing = 4;         // k-steps of operand loads in flight per thread in the grouped GEMMs
constexpr int kLdsK = 72;        // fp16 per LDS tile row: 64 + 8 padding (16 bytes)

__device__ __forceinline__ _Float16 bf16_to_f16(uint16_t b) { return (_Float16)bf16_to_f32(b); }

// ---- 1. router GEMM ------------------------------------------------------------------------------
// logits = x . R^T on bf16 MFMA: x is bf16 (exact), every fp32 router weight is split into
// bf16 hi = rne(R) and lo = rne(R - hi), so R - hi - lo is below 2^-17 |R|; both products are exact
// in the fp32 accumulators. The split is done once per call by router_split (rows E+1: the router,
// then the shared gate), so that the GEMM only moves bf16 tiles.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr int kSplitThreads = 256;

__global__ void __launch_bounds__(kSplitThreads) router_split(BatchedParams p) {
    const int H = p.H, N = p.E + (p.sgate ? 1 : 0);
    const size_t i = ((size_t)blockIdx.x * kSplitThreads + threadIdx.x) * 8;  // 8 weights per thread
    if (i >= (size_t)N * H) return;
    const size_t row = i / H, col = i - row * H;
    const float *src = (row < (size_t)p.E ? p.router + row * H : p.sgate) + col;
    const float4 a = reinterpret_cast<const float4 *>(src)[0], b = reinterpret_cast<const float4 *>(src)[1];
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint16_t h0 = f32_to_bf16_rne(f[2 * q]), h1 = f32_to_bf16_rne(f[2 * q + 1]);
        const uint16_t l0 = f32_to_bf16_rne(f[2 * q] - bf16_to_f32(h0));
        const uint16_t l1 = f32_to_bf16_rne(f[2 * q + 1] - bf16_to_f32(h1));
        hi[q] = h0 | (uint32_t)h1 << 16;
        lo[q] = l0 | (uint32_t)l1 << 16;
    }
    *reinterpret_cast<uint4 *>(p.rhi + i) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4 *>(p.rlo + i) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// Tile: 32 tokens x 32 router rows x one of ks contiguous ranges of H (blockIdx.z), k-steps of 64;
// wave w: tokens 16 (w & 1) .., rows 16 (w >> 1) ... The range's partial sums go to lpart; the
// top-k kernel adds the ranges in order (the ranges keep the k-loop of a workgroup short, so
// that many workgroups hide each other's load latency).
constexpr int kRtT = 32, kRtN = 32;
__host__ __device__ inline int router_ksplit(int H) { return H / 64 < kRouterSplitK ? H / 64 : kRouterSplitK; }

__global__ void __launch_bounds__(kGemmThreads) router_gemm(BatchedParams p) {
    __shared__ __align__(16) uint16_t xs[kRtT][kLdsK];
    __shared__ __align__(16) uint16_t rh[kRtN][kLdsK];
    __shared__ __align__(16) uint16_t rl[kRtN][kLdsK];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int t0 = blockIdx.x * kRtT, n0 = blockIdx.y * kRtN;
    const int H = p.H, E = p.E, T = p.T;
    const int N = E + (p.sgate ? 1 : 0);
    // loads: row r (8 bf16 at c) of the x tile and of both router tiles
    const int r = tid / 8, c = (tid % 8) * 8;
    const bool xok = t0 + r < T, rok = n0 + r < N;
    const uint16_t *xrow = p.x + (size_t)(xok ? t0 + r : 0) * H;
    const uint16_t *hrow = p.rhi + (size_t)(rok ? n0 + r : 0) * H, *lrow = p.rlo + (size_t)(rok ? n0 + r : 0) * H;
    struct St {
        uint4 x, h, l;
    };
    auto load = [&](int kb) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        St st;
        st.x = xok ? *reinterpret_cast<const uint4 *>(xrow + kb * 64 + c) : z;
        st.h = rok ? *reinterpret_cast<const uint4 *>(hrow + kb * 64 + c) : z;
        st.l = rok ? *reinterpret_cast<const uint4 *>(lrow + kb * 64 + c) : z;
        return st;
    };
    auto store = [&](const St &st) {
        *reinterpret_cast<uint4 *>(&xs[r][c]) = st.x;
        *reinterpret_cast<uint4 *>(&rh[r][c]) = st.h;
        *reinterpret_cast<uint4 *>(&rl[r][c]) = st.l;
    };
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const int th = wave & 1, nh = wave >> 1;
    auto mfma_step = [&]() {
#pragma unroll
        for (int ks = 0; ks < 64; ks += 32) {
            const int kc = ks + 8 * (lane / 16);
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(&xs[16 * th + lane % 16][kc]);
            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&rh[16 * nh + lane % 16][kc]);
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&rl[16 * nh + lane % 16][kc]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc, 0, 0, 0);
        }
    };
    const int nk = H / 64 / router_ksplit(H), k0 = blockIdx.z * nk;  // this range's k-steps
    St S0 = load(k0), S1 = load(k0 + (nk > 1 ? 1 : 0));
    for (int kb = 0; kb < nk; kb += 2) {
        store(S0);
        __syncthreads();
        if (kb + 2 < nk) S0 = load(k0 + kb + 2);
        mfma_step();
        __syncthreads();
        if (kb + 1 < nk) {
            store(S1);
            __syncthreads();
            if (kb + 3 < nk) S1 = load(k0 + kb + 3);
            mfma_step();
            __syncthreads();
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

// ---- 2. top-k per token ------------------------------------------------------------------------
constexpr int kTopkWaves = 4;
__global__ void __launch_bounds__(kTopkWaves * kWave) topk_kernel(BatchedParams p) {
    extern __shared__ __align__(16) char smem[];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int E = p.E, K = p.K;
    const int t = blockIdx.x * kTopkWaves + wave;
    float *lt = reinterpret_cast<float *>(smem) + (size_t)wave * E;
    if (t >= p.T) return;  // whole wave leaves together; no workgroup barrier follows
    // logits: the router GEMM's range partial sums added in range order, then the bias
    const int N = E + (p.sgate ? 1 : 0), ks = router_ksplit(p.H);
    const float *part = p.lpart + (size_t)t * N;
    const size_t zs = (size_t)p.T * N;
    for (int e = lane; e < E; e += kWave) {
        float v = part[e];
        for (int z = 1; z < ks; ++z) v += part[z * zs + e];
        if (p.rbias) v += p.rbias[e];
        lt[e] = v;
        p.logits[(size_t)t * E + e] = v;
    }
    float gate = 0.0f;
    if (p.sgate) {
        gate = part[E];
        for (int z = 1; z < ks; ++z) gate += part[z * zs + E];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    wave_topk(lt, E, K, p.idx + (size_t)t * K, p.w + (size_t)t * K);
    if (lane == 0 && p.gamma) p.gamma[t] = p.sgate ? 1.0f / (1.0f + expf(-gate)) : 0.0f;
}

// ---- 3. histogram, exclusive scan, stable scatter, tile list -------------------------------------
// One workgroup of 512 threads. Tokens are taken in blocks of 64 (one lane each); for a block,
// wave-private LDS holds one 64-bit mask per expert with bit l set when token (block, l) selected
// that expert. popcount(mask) is the block's count for the expert and popcount(mask & lanes below)
// the pair's rank among the block's pairs of the same expert. Per-expert exclusive prefixes over
// blocks plus the expert offsets place every pair: pairs of one expert stay in token order, which
// is pair order (a token selects an expert at most once).
constexpr int kBucketThreads = 512;
constexpr int kBucketWaves = kBucketThreads / kWave;

__global__ void __launch_bounds__(kBucketThreads) bucket_kernel(BatchedParams p) {
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int T = p.T, K = p.K, E = p.E;
    const int ng = E + (p.Is ? 1 : 0);  // groups: experts, then the shared expert
    const int nblk = (T + kWave - 1) / kWave;
    unsigned long long *masks = reinterpret_cast<unsigned long long *>(smem) + (size_t)wave * E;
    int *gcnt = reinterpret_cast<int *>(reinterpret_cast<unsigned long long *>(smem) + (size_t)kBucketWaves * E);
    int *goff = gcnt + (E + 1);
    int *gtoff = goff + (E + 2);
    int *guoff = gtoff + (E + 2);  // first gate|up work item of each group
    int *dnoff = guoff + (E + 2);  // first down work item of each group
    const unsigned long long below = (1ull << lane) - 1ull;

    for (int blk = wave; blk < nblk; blk += kBucketWaves) {
        const int t = blk * kWave + lane;
        const bool valid = t < T;
        for (int e = lane; e < E; e += kWave) masks[e] = 0ull;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (valid)
            for (int k = 0; k < K; ++k) {
                const int e = min((unsigned)p.idx[(size_t)t * K + k], (unsigned)(E - 1));
                atomicOr(&masks[e], 1ull << lane);
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (valid)
            for (int k = 0; k < K; ++k) {
                const int e = min((unsigned)p.idx[(size_t)t * K + k], (unsigned)(E - 1));
                p.rank[(size_t)t * K + k] = __popcll(masks[e] & below);
            }
        for (int e = lane; e < E; e += kWave) p.blkcnt[(size_t)blk * E + e] = __popcll(masks[e]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
    // per expert: exclusive prefix over blocks (in place) and the total; the counts of eight blocks
    // are loaded before any is rewritten, so that a chunk costs one memory round trip
    for (int e = tid; e < E; e += kBucketThreads) {
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
    if (tid == 0 && p.Is) gcnt[E] = T;
    __syncthreads();
    // exclusive scans of the group sizes, their tile counts and their gate|up and down work items
    // (tiles x column blocks), by wave 0: lane l owns a chunk
    const int ndn = p.H / kDnCols;
    auto ngu_of = [&](int g) { return (g < E ? p.I : p.Is) / kGuCols; };
    if (wave == 0) {
        const int chunk = (ng + kWave - 1) / kWave;
        const int g0 = min(ng, lane * chunk), g1 = min(ng, g0 + chunk);
        int s = 0, st = 0, su = 0, sd = 0;
        for (int g = g0; g < g1; ++g) {
            const int nt = (gcnt[g] + kBM - 1) / kBM;
            s += gcnt[g];
            st += nt;
            su += nt * ngu_of(g);
            sd += nt * ndn;
        }
        int is = s, ist = st, isu = su, isd = sd;  // inclusive wave scans
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int a = __shfl_up(is, o, kWave), b = __shfl_up(ist, o, kWave);
            const int c = __shfl_up(isu, o, kWave), d = __shfl_up(isd, o, kWave);
            if (lane >= o) { is += a; ist += b; isu += c; isd += d; }
        }
        int run = is - s, trun = ist - st, urun = isu - su, drun = isd - sd;
        for (int g = g0; g < g1; ++g) {
            const int nt = (gcnt[g] + kBM - 1) / kBM;
            goff[g] = run;
            gtoff[g] = trun;
            guoff[g] = urun;
            dnoff[g] = drun;
            run += gcnt[g];
            trun += nt;
            urun += nt * ngu_of(g);
            drun += nt * ndn;
        }
        if (lane == kWave - 1) {
            goff[ng] = is;
            gtoff[ng] = ist;
            guoff[ng] = isu;
            dnoff[ng] = isd;
        }
    }
    __syncthreads();
    for (int g = tid; g <= ng; g += kBucketThreads) {
        p.goff[g] = goff[g];
        if (g < ng) p.gcnt[g] = gcnt[g];
    }
    if (tid == 0) {
        p.ntiles[0] = gtoff[ng];
        p.ntiles[1] = guoff[ng];
        p.ntiles[2] = dnoff[ng];
    }
    for (int g = tid; g < ng; g += kBucketThreads) {
        const int nt = (gcnt[g] + kBM - 1) / kBM;
        for (int i = 0; i < nt; ++i) p.tiles[gtoff[g] + i] = make_int2(g, i * kBM);
    }
    // work items of the grouped GEMMs, longest first: bucketed by the tile's row count (a counting
    // sort, 128 rows down to 1), so that the workgroups taken in list order fill the compute units
    // greedily and the heavy tiles do not form the tail. Within a bucket the order is arbitrary
    // (each item writes its own block of the output, so it does not change any result).
    if (p.wgu) {
        int *hgu = dnoff + (E + 2), *hdn = hgu + (kBM + 1);  // [kBM + 1] each: counts, then cursors
        for (int i = tid; i <= kBM; i += kBucketThreads) hgu[i] = hdn[i] = 0;
        __syncthreads();
        for (int g = tid; g < ng; g += kBucketThreads) {
            const int nt = (gcnt[g] + kBM - 1) / kBM, ngu = ngu_of(g);
            for (int i = 0; i < nt; ++i) {
                const int rows = min(kBM, gcnt[g] - i * kBM);
                atomicAdd(&hgu[rows], ngu);
                atomicAdd(&hdn[rows], ndn);
            }
        }
        __syncthreads();
        if (tid == 0) {
            int ru = 0, rd = 0;
            for (int r = kBM; r >= 1; --r) {
                const int cu = hgu[r], cd = hdn[r];
                hgu[r] = ru;
                hdn[r] = rd;
                ru += cu;
                rd += cd;
            }
        }
        __syncthreads();
        for (int g = wave; g < ng; g += kBucketWaves) {
            const int nt = (gcnt[g] + kBM - 1) / kBM, ngu = ngu_of(g);
            for (int i = lane; i < nt * max(ngu, ndn); i += kWave) {
                const int mi = i % nt, col = i / nt, m0 = mi * kBM;
                const int rows = min(kBM, gcnt[g] - m0);
                if (col < ngu)
                    p.wgu[atomicAdd(&hgu[rows], 1)] =
                        make_int4(g, goff[g] + m0, rows | (col * kGuCols) << 16, gtoff[g] + mi);
                if (col < ndn)
                    p.wdn[atomicAdd(&hdn[rows], 1)] =
                        make_int4(g, goff[g] + m0, rows | (col * kDnCols) << 16, gtoff[g] + mi);
            }
        }
    }
    // scatter
    for (int q = tid; q < T * K; q += kBucketThreads) {
        const int t = q / K;
        const int e = min((unsigned)p.idx[q], (unsigned)(E - 1));
        const int P = goff[e] + p.blkcnt[(size_t)(t / kWave) * E + e] + p.rank[q];
        p.perm[P] = q;
        p.pos[q] = P;
    }
    if (p.Is)
        for (int t = tid; t < T; t += kBucketThreads) p.perm[(size_t)T * K + t] = t * K;
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

// ---- fp16 tiles in pair order ----------------------------------------------------------------------
// Inside every 8-column block (4-bit) or 4-column block (8-bit) the fp16 tiles hold their columns in
// the order the packed dequantisation produces them: 4-bit (0,4,1,5,2,6,3,7), 8-bit (0,2,1,3).
// Both operands of every MFMA use the same order, so each product and each k-sum is that of the
// natural order; h is stored in this order by gu_gemm for dn_gemm's A operand.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int BITS>
__device__ __forceinline__ int pair_pos(int c) {  // position of column c (within its 64-column step)
    if constexpr (BITS == 4) return (c & ~7) + 2 * (c & 3) + ((c >> 2) & 1);
    else return (c & ~3) + 2 * (c & 1) + ((c >> 1) & 1);
}

// Codes -> fp16 s q + b, two per instruction: a nibble (byte) masked into the mantissa of the fp16
// constant 1024 is exactly 1024 + q; subtracting 1024 is exact; one packed fma rounds s q + b once.
// 4-bit: a dword holds columns 0..7 of a block and gives pairs (p, p+4), p = 0..3.
// 8-bit: a dword holds columns 0..3 of a block and gives pairs (p, p+2), p = 0..1.
template <int BITS>
__device__ __forceinline__ void dequant_dword(uint32_t w, half2_t s2, half2_t b2, half2_t *out) {
    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    constexpr int NP = BITS == 4 ? 4 : 2;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const uint32_t u = BITS == 4 ? (((w >> (4 * p)) & 0x000F000Fu) | 0x64006400u)
                                     : (((w >> (8 * p)) & 0x00FF00FFu) | 0x64006400u);
        const half2_t q = __builtin_bit_cast(half2_t, u) - k1024;
        out[p] = __builtin_elementwise_fma(q, s2, b2);
    }
}
__device__ __forceinline__ half2_t bf16_pair_to_f16(uint16_t a, uint16_t b) {
    return half2_t{(_Float16)bf16_to_f32(a), (_Float16)bf16_to_f32(b)};
}
__device__ __forceinline__ half2_t bf16_splat_f16(uint16_t v) {
    const _Float16 h = (_Float16)bf16_to_f32(v);
    return half2_t{h, h};
}
// 8 bf16 activations (natural order) times 2^sh -> 8 fp16 in pair order (4-bit: one block of 8;
// 8-bit: two blocks of 4).
template <int BITS>
__device__ __forceinline__ void act16_to_pairs8(const uint4 r, int sh, half2_t *out) {
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

// ---- x as fp16 -------------------------------------------------------------------------------------
// x16[t] = x[t] * 2^-xe[t] in fp16, columns in pair order (the order of dequant_dword's output),
// with xe[t] = E - 15 for the token's largest magnitude in [2^(E-1), 2^E): the token's values fill
// fp16's range up to 2^15 whatever their bf16 magnitude (only values more than 2^29 below the
// token's largest become fp16 subnormals); the power-of-two scaling is exact and the gate|up
// epilogue multiplies it back. One workgroup per token.
constexpr int kX16Threads = 256;
template <int BITS>
__global__ void __launch_bounds__(kX16Threads) x16_kernel(BatchedParams p) {
    __shared__ float red[kX16Threads / kWave];
    const int t = blockIdx.x, H = p.H, tid = threadIdx.x;
    const uint16_t *xr = p.x + (size_t)t * H;
    float amax = 0.0f;
    for (int c = tid * 8; c < H; c += kX16Threads * 8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(xr + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(w[i] & 0xFFFF)), fabsf(bf16_to_f32(w[i] >> 16))));
    }
    amax = __int_as_float((int)wave_max_u32(__float_as_uint(amax)));  // non-negative floats order as integers
    if (tid % kWave == 0) red[tid / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (amax > 0.0f) {
        frexpf(amax, &e);
        e -= 15;
    }
    for (int c = tid * 8; c < H; c += kX16Threads * 8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(xr + c);
        half2_t hv[4];
        act16_to_pairs8<BITS>(v, -e, hv);
        *reinterpret_cast<uint4 *>(p.x16 + (size_t)t * H + c) = __builtin_bit_cast(uint4, hv);
    }
    if (tid == 0) p.xe[t] = e;
}

// ---- 4 / 5. grouped GEMMs --------------------------------------------------------------------------
// Both GEMMs run one work item per workgroup of 256 threads (4 waves): a tile of up to 128 pair rows
// of one group against a block of the group's weight rows, k-steps of 64 columns (one quantisation
// group). Operands are fp16 in LDS, each tile row 64 values = eight 16-byte chunks stored at
// chunk ^ (row & 7), so the 16 rows an MFMA fragment read takes at one chunk spread over the banks.
// The LDS tiles are double buffered, with one LDS-only barrier per k-step (a full workgroup barrier
// would also wait for every global load in flight, draining the register prefetch each k-step). Block b runs work item b of a list ordered longest first (see bucket_kernel).
__device__ __forceinline__ int list_item(int n) { return (int)blockIdx.x < n ? (int)blockIdx.x : -1; }
__device__ __forceinline__ int chunk_pos(int row, int c) { return c ^ (row & 7); }

// The fp16 value of a bf16 scale or bias times 2^e (exact for finite in-range results).
__device__ __forceinline__ half2_t bf16_splat_f16_scaled(uint16_t v, float f) {
    const _Float16 h = (_Float16)(bf16_to_f32(v) * f);
    return half2_t{h, h};
}

// One thread's share of a 64-column k-step of 64 weight rows' codes: 32 columns (4-bit: 16 bytes,
// 8-bit: 32 bytes), plus that row's scale and bias.
template <int BITS>
struct BLoad {
    uint4 c0, c1;
    uint16_t s, b;
};
template <int BITS>
__device__ __forceinline__ BLoad<BITS> b_load(const uint8_t *crow, const uint16_t *srow, const uint16_t *brow,
                                               int kb, int half) {
    BLoad<BITS> L;
    const uint8_t *cp = crow + ((size_t)kb * 64 + half * 32) * BITS / 8;
    L.c0 = gload16(cp);
    if constexpr (BITS == 8) L.c1 = gload16(cp + 16);
    else L.c1 = make_uint4(0, 0, 0, 0);
    L.s = gp(srow)[kb];
    L.b = gp(brow)[kb];
    return L;
}
// Dequantise a BLoad (scale and bias times f) into four 16-byte chunks of fp16 in pair order.
template <int BITS>
__device__ __forceinline__ void b_dequant(const BLoad<BITS> &L, float f, uint4 *out) {
    const half2_t s2 = bf16_splat_f16_scaled(L.s, f), b2 = bf16_splat_f16_scaled(L.b, f);
    half2_t bv[16];
    const uint32_t cw[8] = {L.c0.x, L.c0.y, L.c0.z, L.c0.w, L.c1.x, L.c1.y, L.c1.z, L.c1.w};
    if constexpr (BITS == 4) {
#pragma unroll
        for (int d = 0; d < 4; ++d) dequant_dword<4>(cw[d], s2, b2, bv + 4 * d);
    } else {
#pragma unroll
        for (int d = 0; d < 8; ++d) dequant_dword<8>(cw[d], s2, b2, bv + 2 * d);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = __builtin_bit_cast(uint4, half8_t{bv[4 * q][0], bv[4 * q][1], bv[4 * q + 1][0],
                                                                          bv[4 * q + 1][1], bv[4 * q + 2][0],
                                                                          bv[4 * q + 2][1], bv[4 * q + 3][0],
                                                                          bv[4 * q + 3][1]});
}

// gate|up + SwiGLU. Item: rows P0 .. P0+M-1 of group g against gate rows j0 .. j0+63 and up rows
// inter + j0 .. +63 (B tile rows 0..63 gate, 64..127 up). Wave w: rows 64 (w & 1) .. +64, j
// 32 (w >> 1) .. +32 of both gate and up, so a lane holds gate and up of the same (row, j).
template <int BITS>
__global__ void __launch_bounds__(kGemmThreads, 2) gu_gemm(BatchedParams p) {
    __shared__ __align__(16) uint4 As[2][kBM][8];
    __shared__ __align__(16) uint4 Bs[2][128][8];
    __shared__ float tmax[kGemmThreads / kWave];
    const int w = list_item(gp(p.ntiles)[1]);
    if (w < 0) return;
    const auto wq = gp(reinterpret_cast<const int *>(p.wgu + w));
    const int4 wi = make_int4(wq[0], wq[1], wq[2], wq[3]);
    const int g = wi.x, P0 = wi.y, M = wi.z & 0xFFFF, j0 = wi.z >> 16, tile = wi.w;
    const GroupW W = group_w13(p, g);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = p.H, K = p.K, nk = H / 64;
    // A: thread row ar, chunks 4 ah .. 4 ah + 3 (x16 row of the pair's token)
    const int ar = tid >> 1, ah = tid & 1;
    const bool aok = ar < M;
    const _Float16 *xrow = p.x16 + (size_t)(aok ? gp(p.perm)[P0 + ar] / K : 0) * H + ah * 32;
    // B: thread tile row br (0..63 gate, 64..127 up), columns 32 bh .. +31
    const int br = tid >> 1, bh = tid & 1;
    const size_t wrow = br < 64 ? (size_t)(j0 + br) : (size_t)(W.inter + j0 + br - 64);
    const uint8_t *crow = W.c + wrow * ((size_t)H * BITS / 8);
    const uint16_t *srow = W.s + wrow * (H / 64), *brow = W.b + wrow * (H / 64);
    // A: 64 bytes of one x16 row per thread and k-step; rows past the tile read a valid row (of token
    // 0) whose LDS store is skipped, so the loads stay unconditional. B: the codes, scale and bias of
    // one weight row, dequantised into LDS one k-step ahead of the MFMAs.
    struct AReg {
        uint4 a0, a1, a2, a3;
    };
    auto a_load = [&](int kb) __attribute__((always_inline)) {
        const _Float16 *src = xrow + (size_t)kb * 64;
        return AReg{gload16(src), gload16(src + 8), gload16(src + 16), gload16(src + 24)};
    };
    auto a_store = [&](const AReg &v, int buf) __attribute__((always_inline)) {
        if (!aok) return;
        As[buf][ar][chunk_pos(ar, 4 * ah + 0)] = v.a0;
        As[buf][ar][chunk_pos(ar, 4 * ah + 1)] = v.a1;
        As[buf][ar][chunk_pos(ar, 4 * ah + 2)] = v.a2;
        As[buf][ar][chunk_pos(ar, 4 * ah + 3)] = v.a3;
    };
    auto b_store = [&](const BLoad<BITS> &v, int buf) __attribute__((always_inline)) {
        uint4 bq[4];
        b_dequant<BITS>(v, 1.0f, bq);
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[buf][br][chunk_pos(br, 4 * bh + q)] = bq[q];
    };
    auto b_fetch = [&](int kb) __attribute__((always_inline)) {
        return b_load<BITS>(crow, srow, brow, min(kb, nk - 1), bh);
    };
    float4_t ag[4][2], au[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            ag[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            au[i][j] = ag[i][j];
        }
    const int mh = wave & 1, jh = wave >> 1, fi = lane % 16, fk = lane / 16;
    // row tiles of this wave that hold any of the M rows (the others are skipped)
    const int mt = min(4, max(0, (M - 64 * mh + 15) / 16));
    auto mfma_step = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = 4 * q + fk;
            half8_t bg[2], bu[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int rg = 32 * jh + 16 * j + fi, ru = 64 + rg;
                bg[j] = __builtin_bit_cast(half8_t, Bs[buf][rg][chunk_pos(rg, c)]);
                bu[j] = __builtin_bit_cast(half8_t, Bs[buf][ru][chunk_pos(ru, c)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= mt) break;
                const int ra = 64 * mh + 16 * i + fi;
                const half8_t a = __builtin_bit_cast(half8_t, As[buf][ra][chunk_pos(ra, c)]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    ag[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bg[j], ag[i][j], 0, 0, 0);
                    au[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bu[j], au[i][j], 0, 0, 0);
                }
            }
        }
    };
    // k-step kb lives in LDS stage kb & 1 and, kRing k-steps ahead, in register ring slot kb % kRing
    // (kb0 below is a multiple of kRing, so every slot index is static): each k-step consumes the
    // oldest slot into LDS and refills it with the loads of k-step kb + kRing + 1, all issued
    // together, so a wait for the oldest slot leaves the kRing - 1 younger ones in flight.
    AReg ra[kRing];
    BLoad<BITS> rb[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
        ra[j] = a_load(min(j, nk - 1));
        rb[j] = b_fetch(j);
    }
    a_store(ra[0], 0);
    b_store(rb[0], 0);
    ra[0] = a_load(min(kRing, nk - 1));
    rb[0] = b_fetch(kRing);
    lds_barrier();
    for (int kb0 = 0; kb0 < nk; kb0 += kRing) {
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            const int kb = kb0 + j;
            if (kb >= nk) break;
            mfma_step(j & 1);
            if (kb + 1 < nk) {
                const int s1 = (j + 1) % kRing;  // static once the loop is unrolled
                a_store(ra[s1], (j + 1) & 1);
                b_store(rb[s1], (j + 1) & 1);
                ra[s1] = a_load(min(kb + 1 + kRing, nk - 1));
                rb[s1] = b_fetch(kb + 1 + kRing);
            }
            lds_barrier();
        }
    }
    // epilogue: lane l, register r of tile (i, j) -> row 64 mh + 16 i + 4 (l / 16) + r, j = j0 + 32 jh +
    // 16 j + l % 16. The accumulators are scaled back by the token's 2^xe, SwiGLU applied, and h
    // stored as fp16 hi + lo halves of h * 2^-e, e = max(0, E - 15) for the tile's largest |h| in
    // [2^(E-1), 2^E), in its pair-order position (the down GEMM's A operand).
    bool finite = true;
    float hmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * mh + 16 * i + 4 * fk + r;
            const float sc = m < M ? ldexpf(1.0f, gp(p.xe)[gp(p.perm)[P0 + m] / K]) : 0.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float gv = ag[i][j][r] * sc, uv = au[i][j][r] * sc;
                const float h = m < M ? gv / (1.0f + expf(-gv)) * uv : 0.0f;
                finite &= m >= M || (__builtin_isfinite(gv) && __builtin_isfinite(uv));  // rows past M: stale
                hmax = fmaxf(hmax, fabsf(h));
                ag[i][j][r] = h;
            }
        }
    hmax = __int_as_float((int)wave_max_u32(__float_as_uint(hmax)));
    if (lane == 0) tmax[wave] = hmax;
    lds_barrier();
    hmax = fmaxf(fmaxf(tmax[0], tmax[1]), fmaxf(tmax[2], tmax[3]));
    int e = 0;
    if (hmax > 0.0f && __builtin_isfinite(hmax)) {
        frexpf(hmax, &e);
        e = max(0, e - 15);
    }
    const float hs = ldexpf(1.0f, -e);
    const int Imax = p.Imax;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * mh + 16 * i + 4 * fk + r;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int jj = j0 + 32 * jh + 16 * j + fi;
                const float h = ag[i][j][r] * hs;
                const _Float16 hh = (_Float16)h;
                const _Float16 hl = (_Float16)(h - (float)hh);
                const size_t o = (size_t)(P0 + m) * Imax + pair_pos<BITS>(jj & 63) + (jj & ~63);
                p.hh[o] = hh;
                p.hl[o] = hl;
            }
        }
    if (tid == 0) p.hexp[(size_t)tile * (Imax / 64) + j0 / 64] = e;
    if (!finite) flag_unsupported(p.status);
}

// down projection x routing weight. Item: rows P0 .. P0+M-1 of group g (h hi and lo halves)
// against output rows n0 .. n0+127, k-steps of 64 over the group's inter. Wave w: rows 64 (w & 1) ..
// +64, output rows 64 (w >> 1) .. +64; each k-step runs the MFMAs once on h hi and once on h lo. The
// k-step's weights are dequantised with scale and bias times 2^e, e the exponent of the h halves
// of this (tile, k-step), so that every product is the unscaled one.
template <int BITS>
__global__ void __launch_bounds__(kGemmThreads, 1) dn_gemm(BatchedParams p) {
    __shared__ __align__(16) uint4 Ah[2][kBM][8];
    __shared__ __align__(16) uint4 Al[2][kBM][8];
    __shared__ __align__(16) uint4 Bs[2][kDnCols][8];
    const int w = list_item(gp(p.ntiles)[2]);
    if (w < 0) return;
    const auto wq = gp(reinterpret_cast<const int *>(p.wdn + w));
    const int4 wi = make_int4(wq[0], wq[1], wq[2], wq[3]);
    const int g = wi.x, P0 = wi.y, M = wi.z & 0xFFFF, n0 = wi.z >> 16, tile = wi.w;
    const GroupW W = group_w2(p, g);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = p.H, Imax = p.Imax, nk = W.inter / 64;
    const int ar = tid >> 1, ah = tid & 1;
    const bool aok = ar < M;
    const _Float16 *hrow = p.hh + (size_t)(P0 + (aok ? ar : 0)) * Imax + ah * 32;
    const _Float16 *lrow = p.hl + (size_t)(P0 + (aok ? ar : 0)) * Imax + ah * 32;
    const int br = tid >> 1, bh = tid & 1;  // output row n0 + br, columns 32 bh .. +31
    const size_t wrow = (size_t)(n0 + br);
    const uint8_t *crow = W.c + wrow * ((size_t)W.inter * BITS / 8);
    const uint16_t *srow = W.s + wrow * (W.inter / 64), *brow = W.b + wrow * (W.inter / 64);
    const int *hexp = p.hexp + (size_t)tile * (Imax / 64);
    // A: h hi and lo halves (rows past the tile read the tile's first row, store skipped); B: codes,
    // scale and bias of one output row, dequantised with the k-step's h exponent into LDS one k-step
    // ahead of the MFMAs.
    struct AReg {
        uint4 h0, h1, h2, h3, l0, l1, l2, l3;
    };
    auto a_load = [&](int kb) __attribute__((always_inline)) {
        const _Float16 *hs = hrow + (size_t)kb * 64, *ls = lrow + (size_t)kb * 64;
        return AReg{gload16(hs), gload16(hs + 8), gload16(hs + 16), gload16(hs + 24),
                    gload16(ls), gload16(ls + 8), gload16(ls + 16), gload16(ls + 24)};
    };
    auto a_store = [&](const AReg &v, int buf) __attribute__((always_inline)) {
        if (!aok) return;
        Ah[buf][ar][chunk_pos(ar, 4 * ah + 0)] = v.h0;
        Ah[buf][ar][chunk_pos(ar, 4 * ah + 1)] = v.h1;
        Ah[buf][ar][chunk_pos(ar, 4 * ah + 2)] = v.h2;
        Ah[buf][ar][chunk_pos(ar, 4 * ah + 3)] = v.h3;
        Al[buf][ar][chunk_pos(ar, 4 * ah + 0)] = v.l0;
        Al[buf][ar][chunk_pos(ar, 4 * ah + 1)] = v.l1;
        Al[buf][ar][chunk_pos(ar, 4 * ah + 2)] = v.l2;
        Al[buf][ar][chunk_pos(ar, 4 * ah + 3)] = v.l3;
    };
    auto b_store = [&](const BLoad<BITS> &v, int kb, int buf) __attribute__((always_inline)) {
        uint4 bq[4];
        b_dequant<BITS>(v, ldexpf(1.0f, gp(hexp)[kb]), bq);
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[buf][br][chunk_pos(br, 4 * bh + q)] = bq[q];
    };
    auto b_fetch = [&](int kb) __attribute__((always_inline)) {
        return b_load<BITS>(crow, srow, brow, min(kb, nk - 1), bh);
    };
    float4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int mh = wave & 1, nh = wave >> 1, fi = lane % 16, fk = lane / 16;
    const int mt = min(4, max(0, (M - 64 * mh + 15) / 16));
    auto mfma_step = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = 4 * q + fk;
            half8_t b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rb = 64 * nh + 16 * j + fi;
                b[j] = __builtin_bit_cast(half8_t, Bs[buf][rb][chunk_pos(rb, c)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= mt) break;
                const int ra = 64 * mh + 16 * i + fi;
                const half8_t a = __builtin_bit_cast(half8_t, Ah[buf][ra][chunk_pos(ra, c)]);
                const half8_t al = __builtin_bit_cast(half8_t, Al[buf][ra][chunk_pos(ra, c)]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, b[j], acc[i][j], 0, 0, 0);
                }
            }
        }
    };
    // k-step kb lives in LDS stage kb & 1 and, kRing k-steps ahead, in register ring slot kb % kRing
    // (kb0 below is a multiple of kRing, so every slot index is static): each k-step consumes the
    // oldest slot into LDS and refills it with the loads of k-step kb + kRing + 1, all issued
    // together, so a wait for the oldest slot leaves the kRing - 1 younger ones in flight.
    AReg ra[kRing];
    BLoad<BITS> rb[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
        ra[j] = a_load(min(j, nk - 1));
        rb[j] = b_fetch(j);
    }
    a_store(ra[0], 0);
    b_store(rb[0], 0, 0);
    ra[0] = a_load(min(kRing, nk - 1));
    rb[0] = b_fetch(kRing);
    lds_barrier();
    for (int kb0 = 0; kb0 < nk; kb0 += kRing) {
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            const int kb = kb0 + j;
            if (kb >= nk) break;
            mfma_step(j & 1);
            if (kb + 1 < nk) {
                const int s1 = (j + 1) % kRing;  // static once the loop is unrolled
                a_store(ra[s1], (j + 1) & 1);
                b_store(rb[s1], kb + 1, (j + 1) & 1);
                ra[s1] = a_load(min(kb + 1 + kRing, nk - 1));
                rb[s1] = b_fetch(kb + 1 + kRing);
            }
            lds_barrier();
        }
    }
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 64 * mh + 16 * i + 4 * fk + r;
            if (m >= M) continue;
            const int q = gp(p.perm)[P0 + m];
            const float sc = g < p.E ? gp(p.w)[q] : gp(p.gamma)[q / p.K];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + 64 * nh + 16 * j + fi;
                finite &= __builtin_isfinite(acc[i][j][r]);
                p.out[(size_t)(P0 + m) * H + n] = sc * acc[i][j][r];
            }
        }
    if (!finite) flag_unsupported(p.status);
}

// ---- 6. fixed-order combine --------------------------------------------------------------------------
__global__ void __launch_bounds__(256) combine_kernel(BatchedParams p) {
    const int H = p.H, K = p.K, T = p.T;
    const int nq = H / 4;
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long long)T * nq) return;
    const int t = (int)(i / nq), c = (int)(i - (long long)t * nq) * 4;
    float4 acc = make_float4(0, 0, 0, 0);
    for (int k = 0; k < K; ++k) {
        const float4 v = *reinterpret_cast<const float4 *>(p.out + (size_t)p.pos[(size_t)t * K + k] * H + c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (p.Is) {
        const float4 v = *reinterpret_cast<const float4 *>(p.out + ((size_t)T * K + t) * H + c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4 *>(p.y + (size_t)t * H + c) = acc;
}

// ---- launch sequence ---------------------------------------------------------------------------------
hipError_t launch_router_topk(const BatchedParams &p, hipStream_t stream) {
    const int N = p.E + (p.sgate ? 1 : 0);
    const size_t nsplit = ((size_t)N * p.H / 8 + kSplitThreads - 1) / kSplitThreads;
    hipLaunchKernelGGL(router_split, dim3((unsigned)nsplit), dim3(kSplitThreads), 0, stream, p);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(router_gemm, dim3((p.T + kRtT - 1) / kRtT, (N + kRtN - 1) / kRtN, router_ksplit(p.H)),
                       dim3(kGemmThreads), 0,
                       stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t lds = sizeof(float) * (size_t)kTopkWaves * p.E;
    hipLaunchKernelGGL(topk_kernel, dim3((p.T + kTopkWaves - 1) / kTopkWaves), dim3(kTopkWaves * kWave), lds, stream,
                       p);
    return hipGetLastError();
}

size_t bucket_lds_bytes(int E) {
    return 8 * (size_t)kBucketWaves * E + 4 * (size_t)(5 * E + 9 + 2 * (kBM + 1));
}

hipError_t launch_bucket(const BatchedParams &p, hipStream_t stream) {
    const size_t blds = bucket_lds_bytes(p.E);
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&bucket_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)blds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), blds, stream, p);
    return hipGetLastError();
}

hipError_t launch_batched(const BatchedParams &p, const BatchedWs &lay, hipStream_t stream) {
    hipError_t err = launch_router_topk(p, stream);
    if (err != hipSuccess) return err;
    if ((err = launch_bucket(p, stream)) != hipSuccess) return err;
    // grids cover the work lists' upper bounds (blocks past the list's length return at once)
    const unsigned ggu = (unsigned)lay.max_wgu, gdn = (unsigned)lay.max_wdn;
    if (p.bits == 4) {
        hipLaunchKernelGGL(x16_kernel<4>, dim3(p.T), dim3(kX16Threads), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(gu_gemm<4>, dim3(ggu), dim3(kGemmThreads), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(dn_gemm<4>, dim3(gdn), dim3(kGemmThreads), 0, stream, p);
    } else {
        hipLaunchKernelGGL(x16_kernel<8>, dim3(p.T), dim3(kX16Threads), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(gu_gemm<8>, dim3(ggu), dim3(kGemmThreads), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(dn_gemm<8>, dim3(gdn), dim3(kGemmThreads), 0, stream, p);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const long long n = (long long)p.T * (p.H / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace moe
