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
// Dequantised weights are s * q + b rounded once to fp16, bf16 activations are converted to fp16
// (exact in fp16's normal range) and h is held as fp16 hi + lo halves; products are exact in the
// fp32 accumulators of the MFMA. So x, s * q + b and h must lie within fp16's range (+-65504):
// an operand beyond it becomes infinite, the accumulators it reaches are not finite, and the
// epilogues then set the status word to MOE_ERR_UNSUPPORTED (the outputs are then undefined).
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;          // pair rows per tile
constexpr int kGemmThreads = 256;
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
    // exclusive scans of the group sizes and of their tile counts, by wave 0: lane l owns a chunk
    if (wave == 0) {
        const int chunk = (ng + kWave - 1) / kWave;
        const int g0 = min(ng, lane * chunk), g1 = min(ng, g0 + chunk);
        int s = 0, st = 0;
        for (int g = g0; g < g1; ++g) {
            s += gcnt[g];
            st += (gcnt[g] + kBM - 1) / kBM;
        }
        int is = s, ist = st;  // inclusive wave scans
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int a = __shfl_up(is, o, kWave), b = __shfl_up(ist, o, kWave);
            if (lane >= o) { is += a; ist += b; }
        }
        int run = is - s, trun = ist - st;
        for (int g = g0; g < g1; ++g) {
            goff[g] = run;
            gtoff[g] = trun;
            run += gcnt[g];
            trun += (gcnt[g] + kBM - 1) / kBM;
        }
        if (lane == kWave - 1) {
            goff[ng] = is;
            gtoff[ng] = ist;
        }
    }
    __syncthreads();
    for (int g = tid; g <= ng; g += kBucketThreads) {
        p.goff[g] = goff[g];
        if (g < ng) p.gcnt[g] = gcnt[g];
    }
    if (tid == 0) p.ntiles[0] = gtoff[ng];
    for (int g = tid; g < ng; g += kBucketThreads) {
        const int nt = (gcnt[g] + kBM - 1) / kBM;
        for (int i = 0; i < nt; ++i) p.tiles[gtoff[g] + i] = make_int2(g, i * kBM);
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
// 16 bf16 activations (natural order) -> 16 fp16 in pair order (two blocks of 8 or four of 4).
template <int BITS>
__device__ __forceinline__ void act16_to_pairs(const uint4 r0, const uint4 r1, half2_t *out) {
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    uint16_t x[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[2 * i] = w[i] & 0xFFFF;
        x[2 * i + 1] = w[i] >> 16;
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const uint16_t *v = x + 8 * blk;
        if constexpr (BITS == 4) {
#pragma unroll
            for (int p = 0; p < 4; ++p) out[4 * blk + p] = bf16_pair_to_f16(v[p], v[p + 4]);
        } else {
            out[4 * blk + 0] = bf16_pair_to_f16(v[0], v[2]);
            out[4 * blk + 1] = bf16_pair_to_f16(v[1], v[3]);
            out[4 * blk + 2] = bf16_pair_to_f16(v[4], v[6]);
            out[4 * blk + 3] = bf16_pair_to_f16(v[5], v[7]);
        }
    }
}

// ---- 4. grouped gate|up + SwiGLU -----------------------------------------------------------------
// Tile: 64 pair rows x 64 j (128 weight rows: 64 gate then 64 up), k-steps of 64 columns of H (one
// quantisation group). Wave w: rows 32 (w & 1) .. +32, j 32 (w >> 1) .. +32; 2 x 2 MFMA tiles each
// for gate and up, so a lane holds gate and up of the same (row, j) and SwiGLU needs no exchange.
// Global loads run two k-steps ahead of the MFMAs (register stages S0 / S1).
template <int BITS>
struct GuStage {
    uint4 a0, a1;      // 16 bf16 of activation row ar
    uint4 c0, c1;      // 32 codes of weight row br (c1 only at 8-bit)
    uint16_t s, b;     // that row's group scale and bias
};
template <int BITS>
__global__ void __launch_bounds__(kGemmThreads) gu_gemm(BatchedParams p) {
    __shared__ __align__(16) _Float16 As[kBM][kLdsK];
    __shared__ __align__(16) _Float16 Bs[128][kLdsK];
    const int tile = blockIdx.x;
    if (tile >= p.ntiles[0]) return;
    const int2 tg = p.tiles[tile];
    const int g = tg.x, m0 = tg.y;
    const GroupW w = group_w13(p, g);
    const int j0 = blockIdx.y * 64;
    if (j0 >= w.inter) return;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = p.H, K = p.K;
    const int P0 = p.goff[g] + m0;
    const int M = min(kBM, p.gcnt[g] - m0);
    const int ar = tid / 4, ac = (tid % 4) * 16;  // A: row, first of 16 columns
    const bool aok = ar < M;
    const uint16_t *xrow = p.x + (size_t)(aok ? p.perm[P0 + ar] / K : 0) * H;
    const int br = tid / 2, bc = (tid % 2) * 32;  // B: tile row, first of 32 columns
    const size_t wrow = (br < 64) ? (size_t)(j0 + br) : (size_t)(w.inter + j0 + br - 64);
    const uint8_t *crow = w.c + wrow * ((size_t)H * BITS / 8);
    const int gpr = H / 64;
    const int nk = H / 64;

    auto load = [&](int kb) {
        GuStage<BITS> st;
        if (aok) {
            const uint4 *src = reinterpret_cast<const uint4 *>(xrow + kb * 64 + ac);
            st.a0 = src[0];
            st.a1 = src[1];
        } else {
            st.a0 = make_uint4(0, 0, 0, 0);
            st.a1 = st.a0;
        }
        const uint4 *cp = reinterpret_cast<const uint4 *>(crow + ((size_t)kb * 64 + bc) * BITS / 8);
        st.c0 = cp[0];
        st.c1 = BITS == 8 ? cp[1] : make_uint4(0, 0, 0, 0);
        st.s = w.s[wrow * gpr + kb];
        st.b = w.b[wrow * gpr + kb];
        return st;
    };
    auto store = [&](const GuStage<BITS> &st) {
        half2_t av[8];
        act16_to_pairs<BITS>(st.a0, st.a1, av);
        reinterpret_cast<uint4 *>(&As[ar][ac])[0] = __builtin_bit_cast(uint4, half8_t{av[0][0], av[0][1], av[1][0], av[1][1], av[2][0], av[2][1], av[3][0], av[3][1]});
        reinterpret_cast<uint4 *>(&As[ar][ac])[1] = __builtin_bit_cast(uint4, half8_t{av[4][0], av[4][1], av[5][0], av[5][1], av[6][0], av[6][1], av[7][0], av[7][1]});
        const half2_t s2 = bf16_splat_f16(st.s), b2 = bf16_splat_f16(st.b);
        half2_t bv[16];
        const uint32_t cw[8] = {st.c0.x, st.c0.y, st.c0.z, st.c0.w, st.c1.x, st.c1.y, st.c1.z, st.c1.w};
        if constexpr (BITS == 4) {
#pragma unroll
            for (int d = 0; d < 4; ++d) dequant_dword<4>(cw[d], s2, b2, bv + 4 * d);
        } else {
#pragma unroll
            for (int d = 0; d < 8; ++d) dequant_dword<8>(cw[d], s2, b2, bv + 2 * d);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(&Bs[br][bc]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dst[q] = __builtin_bit_cast(uint4, half8_t{bv[4 * q][0], bv[4 * q][1], bv[4 * q + 1][0], bv[4 * q + 1][1],
                                                       bv[4 * q + 2][0], bv[4 * q + 2][1], bv[4 * q + 3][0],
                                                       bv[4 * q + 3][1]});
    };

    float4_t ag[2][2], au[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            ag[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            au[i][j] = ag[i][j];
        }
    const int mh = wave & 1, jh = wave >> 1;
    auto mfma_step = [&]() {
#pragma unroll
        for (int ks = 0; ks < 64; ks += 32) {
            const int kc = ks + 8 * (lane / 16);
            half8_t a[2], bg[2], bu[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const half8_t *>(&As[32 * mh + 16 * i + lane % 16][kc]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bg[j] = *reinterpret_cast<const half8_t *>(&Bs[32 * jh + 16 * j + lane % 16][kc]);
                bu[j] = *reinterpret_cast<const half8_t *>(&Bs[64 + 32 * jh + 16 * j + lane % 16][kc]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    ag[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bg[j], ag[i][j], 0, 0, 0);
                    au[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bu[j], au[i][j], 0, 0, 0);
                }
        }
    };
    GuStage<BITS> S0 = load(0), S1 = load(nk > 1 ? 1 : 0);
    for (int kb = 0; kb < nk; kb += 2) {
        store(S0);
        __syncthreads();
        if (kb + 2 < nk) S0 = load(kb + 2);
        mfma_step();
        __syncthreads();
        if (kb + 1 < nk) {
            store(S1);
            __syncthreads();
            if (kb + 3 < nk) S1 = load(kb + 3);
            mfma_step();
            __syncthreads();
        }
    }
    // epilogue: lane l, register r -> row 32 mh + 16 i + 4 (l / 16) + r, j = j0 + 32 jh + 16 j + l % 16;
    // h goes to its pair-order position (dn_gemm's A operand)
    const int Imax = p.Imax;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 32 * mh + 16 * i + 4 * (lane / 16) + r;
                if (m >= M) continue;
                const int jj = j0 + 32 * jh + 16 * j + lane % 16;
                const float gv = ag[i][j][r], uv = au[i][j][r];
                const float h = gv / (1.0f + expf(-gv)) * uv;
                finite &= __builtin_isfinite(gv) && __builtin_isfinite(uv);
                const _Float16 hh = (_Float16)h;
                const _Float16 hl = (_Float16)(h - (float)hh);
                const size_t o = (size_t)(P0 + m) * Imax + pair_pos<BITS>(jj & 63) + (jj & ~63);
                p.hh[o] = hh;
                p.hl[o] = hl;
            }
    if (!finite) flag_unsupported(p.status);
}

// ---- 5. grouped down projection ------------------------------------------------------------------
// Tile: 64 pair rows x 64 output rows n, k-steps of 64 columns of the group's inter. Wave w: rows
// 32 (w & 1) .., n 32 (w >> 1) ..; each k-step runs the MFMA once on h hi and once on h lo.
template <int BITS>
struct DnStage {
    uint4 h0, h1, l0, l1;  // 16 fp16 of h hi / lo, row ar (pair order)
    uint4 c;               // 16 codes of weight row br (8 bytes used at 4-bit)
    uint16_t s, b;
};
template <int BITS>
__global__ void __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(5, 5))) dn_gemm(BatchedParams p) {
    __shared__ __align__(16) _Float16 Ah[kBM][kLdsK];
    __shared__ __align__(16) _Float16 Al[kBM][kLdsK];
    __shared__ __align__(16) _Float16 Bs[64][kLdsK];
    const int tile = blockIdx.x;
    if (tile >= p.ntiles[0]) return;
    const int2 tg = p.tiles[tile];
    const int g = tg.x, m0 = tg.y;
    const GroupW w = group_w2(p, g);
    const int n0 = blockIdx.y * 64;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = p.H, Imax = p.Imax;
    const int P0 = p.goff[g] + m0;
    const int M = min(kBM, p.gcnt[g] - m0);
    const int ar = tid / 4, ac = (tid % 4) * 16;
    const bool aok = ar < M;
    const _Float16 *hrow = p.hh + (size_t)(P0 + (aok ? ar : 0)) * Imax;
    const _Float16 *lrow = p.hl + (size_t)(P0 + (aok ? ar : 0)) * Imax;
    const int br = tid / 4, bc = (tid % 4) * 16;  // 64 rows x 4 chunks of 16 codes
    const size_t wrow = (size_t)(n0 + br);
    const uint8_t *crow = w.c + wrow * ((size_t)w.inter * BITS / 8);
    const int gpr = w.inter / 64;
    const int nk = w.inter / 64;

    auto load = [&](int kb) {
        DnStage<BITS> st;
        if (aok) {
            const uint4 *hs = reinterpret_cast<const uint4 *>(hrow + kb * 64 + ac);
            const uint4 *ls = reinterpret_cast<const uint4 *>(lrow + kb * 64 + ac);
            st.h0 = hs[0]; st.h1 = hs[1];
            st.l0 = ls[0]; st.l1 = ls[1];
        } else {
            st.h0 = make_uint4(0, 0, 0, 0);
            st.h1 = st.h0; st.l0 = st.h0; st.l1 = st.h0;
        }
        const uint8_t *cp = crow + ((size_t)kb * 64 + bc) * BITS / 8;
        if constexpr (BITS == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(cp);
            st.c = make_uint4(v.x, v.y, 0, 0);
        } else {
            st.c = *reinterpret_cast<const uint4 *>(cp);
        }
        st.s = w.s[wrow * gpr + kb];
        st.b = w.b[wrow * gpr + kb];
        return st;
    };
    auto store = [&](const DnStage<BITS> &st) {
        reinterpret_cast<uint4 *>(&Ah[ar][ac])[0] = st.h0;
        reinterpret_cast<uint4 *>(&Ah[ar][ac])[1] = st.h1;
        reinterpret_cast<uint4 *>(&Al[ar][ac])[0] = st.l0;
        reinterpret_cast<uint4 *>(&Al[ar][ac])[1] = st.l1;
        const half2_t s2 = bf16_splat_f16(st.s), b2 = bf16_splat_f16(st.b);
        half2_t bv[8];
        const uint32_t cw[4] = {st.c.x, st.c.y, st.c.z, st.c.w};
        if constexpr (BITS == 4) {
            dequant_dword<4>(cw[0], s2, b2, bv);
            dequant_dword<4>(cw[1], s2, b2, bv + 4);
        } else {
#pragma unroll
            for (int d = 0; d < 4; ++d) dequant_dword<8>(cw[d], s2, b2, bv + 2 * d);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(&Bs[br][bc]);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            dst[q] = __builtin_bit_cast(uint4, half8_t{bv[4 * q][0], bv[4 * q][1], bv[4 * q + 1][0], bv[4 * q + 1][1],
                                                       bv[4 * q + 2][0], bv[4 * q + 2][1], bv[4 * q + 3][0],
                                                       bv[4 * q + 3][1]});
    };

    float4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int mh = wave & 1, nh = wave >> 1;
    auto mfma_step = [&]() {
#pragma unroll
        for (int ks = 0; ks < 64; ks += 32) {
            const int kc = ks + 8 * (lane / 16);
            half8_t ah[2], al[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                ah[i] = *reinterpret_cast<const half8_t *>(&Ah[32 * mh + 16 * i + lane % 16][kc]);
                al[i] = *reinterpret_cast<const half8_t *>(&Al[32 * mh + 16 * i + lane % 16][kc]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const half8_t *>(&Bs[32 * nh + 16 * j + lane % 16][kc]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], b[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[i], b[j], acc[i][j], 0, 0, 0);
                }
        }
    };
    DnStage<BITS> S0 = load(0), S1 = load(nk > 1 ? 1 : 0);
    for (int kb = 0; kb < nk; kb += 2) {
        store(S0);
        __syncthreads();
        if (kb + 2 < nk) S0 = load(kb + 2);
        mfma_step();
        __syncthreads();
        if (kb + 1 < nk) {
            store(S1);
            __syncthreads();
            if (kb + 3 < nk) S1 = load(kb + 3);
            mfma_step();
            __syncthreads();
        }
    }
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 32 * mh + 16 * i + 4 * (lane / 16) + r;
            if (m >= M) continue;
            const int q = p.perm[P0 + m];
            const float sc = g < p.E ? p.w[q] : p.gamma[q / p.K];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + 32 * nh + 16 * j + lane % 16;
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
    return 8 * (size_t)kBucketWaves * E + 4 * (size_t)(3 * E + 5);
}

hipError_t launch_bucket(const BatchedParams &p, hipStream_t stream) {
    const size_t blds = bucket_lds_bytes(p.E);
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&bucket_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)blds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), blds, stream, p);
    return hipGetLastError();
}

hipError_t launch_batched(const BatchedParams &p, int max_tiles, hipStream_t stream) {
    hipError_t err = launch_router_topk(p, stream);
    if (err != hipSuccess) return err;
    if ((err = launch_bucket(p, stream)) != hipSuccess) return err;
    const dim3 ggu(max_tiles, p.Imax / 64), gdn(max_tiles, p.H / 64);
    if (p.bits == 4) {
        hipLaunchKernelGGL(gu_gemm<4>, ggu, dim3(kGemmThreads), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(dn_gemm<4>, gdn, dim3(kGemmThreads), 0, stream, p);
    } else {
        hipLaunchKernelGGL(gu_gemm<8>, ggu, dim3(kGemmThreads), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(dn_gemm<8>, gdn, dim3(kGemmThreads), 0, stream, p);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const long long n = (long long)p.T * (p.H / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace moe
