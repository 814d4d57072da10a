// batched.hip -- one MoE layer for a batch of T tokens (prefill / batched decode) on gfx950.
//
// Six launches on one stream, no host synchronisation:
//   1. router_gemm   logits[T][E] (+ shared-gate logit) = x . R^T on v_mfma_f32_16x16x4_f32
//                    (fp32 operands: x is bf16, exact in fp32; the router stays fp32)
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
// Dequantised weights are s * q + b rounded to fp16; bf16 activations are exact in fp16 in the
// normal range. Products are exact in the fp32 accumulators of the MFMA.
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
// Workgroup tile: 16 tokens x 64 router rows (row E = shared gate); wave w owns rows 16w..16w+15.
// k-step of 32 columns staged in LDS as fp32 (+1 word padding per row).
constexpr int kRtT = 16, kRtN = 64, kRtK = 32;

__global__ void __launch_bounds__(kGemmThreads) router_gemm(BatchedParams p) {
    __shared__ float xs[kRtT][kRtK + 1];
    __shared__ float rs[kRtN][kRtK + 1];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int t0 = blockIdx.x * kRtT, n0 = blockIdx.y * kRtN;
    const int H = p.H, E = p.E, T = p.T;
    const int N = E + (p.sgate ? 1 : 0);
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < H; k0 += kRtK) {
        // x: 16 rows x 32 bf16 -> 64 threads x 8 values
        if (tid < 64) {
            const int r = tid / 4, c = (tid % 4) * 8, t = t0 + r;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < T) v = *reinterpret_cast<const uint4 *>(p.x + (size_t)t * H + k0 + c);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xs[r][c + 2 * q] = bf16_to_f32(w[q] & 0xFFFF);
                xs[r][c + 2 * q + 1] = bf16_to_f32(w[q] >> 16);
            }
        }
        // router rows: 64 rows x 32 fp32 -> 256 threads x 8 values
        {
            const int r = tid / 4, c = (tid % 4) * 8, n = n0 + r;
            float4 a = make_float4(0, 0, 0, 0), b = a;
            if (n < N) {
                const float *row = n < E ? p.router + (size_t)n * H : p.sgate;
                a = *reinterpret_cast<const float4 *>(row + k0 + c);
                b = *reinterpret_cast<const float4 *>(row + k0 + c + 4);
            }
            rs[r][c + 0] = a.x; rs[r][c + 1] = a.y; rs[r][c + 2] = a.z; rs[r][c + 3] = a.w;
            rs[r][c + 4] = b.x; rs[r][c + 5] = b.y; rs[r][c + 6] = b.z; rs[r][c + 7] = b.w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kRtK; kk += 4) {
            const float a = xs[lane % 16][kk + lane / 16];
            const float b = rs[16 * wave + lane % 16][kk + lane / 16];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // lane l, register r -> token t0 + 4 (l / 16) + r, row n0 + 16 wave + l % 16
    const int n = n0 + 16 * wave + lane % 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * (lane / 16) + r;
        if (t >= T || n >= N) continue;
        if (n < E) p.logits[(size_t)t * E + n] = acc[r] + (p.rbias ? p.rbias[n] : 0.0f);
        else p.gate[t] = acc[r];
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
    for (int e = lane; e < E; e += kWave) lt[e] = p.logits[(size_t)t * E + e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    wave_topk(lt, E, K, p.idx + (size_t)t * K, p.w + (size_t)t * K);
    if (lane == 0 && p.gamma) p.gamma[t] = p.sgate ? 1.0f / (1.0f + expf(-p.gate[t])) : 0.0f;
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
    // per expert: exclusive prefix over blocks (in place) and the total
    for (int e = tid; e < E; e += kBucketThreads) {
        int run = 0;
        for (int blk = 0; blk < nblk; ++blk) {
            const int c = p.blkcnt[(size_t)blk * E + e];
            p.blkcnt[(size_t)blk * E + e] = run;
            run += c;
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
    if (g < p.E) {
        const size_t rows = 2 * (size_t)p.I;
        return {p.w13.c + g * rows * H * p.bits / 8, p.w13.s + g * rows * (H / 64), p.w13.b + g * rows * (H / 64),
                p.I};
    }
    return {p.s13.c, p.s13.s, p.s13.b, p.Is};
}
__device__ __forceinline__ GroupW group_w2(const BatchedParams &p, int g) {
    const size_t H = p.H;
    if (g < p.E) {
        const size_t cols = p.I;
        return {p.w2.c + g * H * cols * p.bits / 8, p.w2.s + g * H * (cols / 64), p.w2.b + g * H * (cols / 64), p.I};
    }
    return {p.s2.c, p.s2.s, p.s2.b, p.Is};
}

// Dequantise 16 consecutive codes of one row (4-bit: 8 bytes, low nibble first; 8-bit: 16 bytes)
// to fp16 s * q + b and store them as two 16-byte LDS writes at dst.
template <int BITS>
__device__ __forceinline__ void dequant16(const uint4 raw, float s, float b, _Float16 *dst) {
    half8_t lo, hi;
    if constexpr (BITS == 4) {
        const uint32_t w[2] = {raw.x, raw.y};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t c = (w[q / 4] >> (8 * (q % 4))) & 0xFFu;
            const float v0 = fmaf(s, (float)(c & 0xF), b), v1 = fmaf(s, (float)(c >> 4), b);
            if (q < 4) { lo[2 * q] = (_Float16)v0; lo[2 * q + 1] = (_Float16)v1; }
            else { hi[2 * q - 8] = (_Float16)v0; hi[2 * q - 7] = (_Float16)v1; }
        }
    } else {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float v = fmaf(s, (float)((w[q / 4] >> (8 * (q % 4))) & 0xFFu), b);
            if (q < 8) lo[q] = (_Float16)v;
            else hi[q - 8] = (_Float16)v;
        }
    }
    reinterpret_cast<half8_t *>(dst)[0] = lo;
    reinterpret_cast<half8_t *>(dst)[1] = hi;
}

// One thread's share of a weight k-step: row r (of the tile), 16 codes at column c16 * 16 of the
// 64-column step `kb`, and that group's scale and bias.
template <int BITS>
struct WFrag {
    uint4 raw;
    uint16_t s, b;
};
template <int BITS>
__device__ __forceinline__ void wfrag_load(WFrag<BITS> &f, const GroupW &w, size_t row, int cols, int kb, int c16,
                                           bool ok) {
    if (!ok) {
        f.raw = make_uint4(0, 0, 0, 0);
        f.s = 0;
        f.b = 0;
        return;
    }
    const uint8_t *cp = w.c + row * ((size_t)cols * BITS / 8) + ((size_t)kb * 64 + c16 * 16) * BITS / 8;
    if constexpr (BITS == 4) {
        const uint2 v = *reinterpret_cast<const uint2 *>(cp);
        f.raw = make_uint4(v.x, v.y, 0, 0);
    } else {
        f.raw = *reinterpret_cast<const uint4 *>(cp);
    }
    f.s = w.s[row * (cols / 64) + kb];
    f.b = w.b[row * (cols / 64) + kb];
}

// ---- 4. grouped gate|up + SwiGLU -----------------------------------------------------------------
// Tile: 64 pair rows x 64 j (128 weight rows: 64 gate then 64 up), k-steps of 64 columns of H.
// Wave w: rows 32 (w & 1) .. +32, j 32 (w >> 1) .. +32; 2 x 2 MFMA tiles each for gate and up, so
// a lane holds gate and up of the same (row, j) and SwiGLU needs no exchange.
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
    // A loads: row ar = tid / 4, 16 columns at (tid % 4) * 16
    const int ar = tid / 4, ac = (tid % 4) * 16;
    const bool aok = ar < M;
    const uint16_t *xrow = p.x + (size_t)(aok ? p.perm[P0 + ar] / K : 0) * H;
    // B loads: tile row br = tid / 2 (0..127), 16 codes at columns (tid % 2) * 16 and +32
    const int br = tid / 2, bc = tid % 2;
    const size_t wrow = (br < 64) ? (size_t)(j0 + br) : (size_t)(w.inter + j0 + br - 64);
    const int nk = H / 64;

    uint4 xa0, xa1;
    WFrag<BITS> f0, f1;
    auto load_step = [&](int kb) {
        if (aok) {
            const uint4 *src = reinterpret_cast<const uint4 *>(xrow + kb * 64 + ac);
            xa0 = src[0];
            xa1 = src[1];
        } else {
            xa0 = make_uint4(0, 0, 0, 0);
            xa1 = xa0;
        }
        wfrag_load<BITS>(f0, w, wrow, H, kb, bc, true);
        wfrag_load<BITS>(f1, w, wrow, H, kb, bc + 2, true);
    };
    auto store_step = [&]() {
        half8_t h0, h1;
        const uint32_t a[8] = {xa0.x, xa0.y, xa0.z, xa0.w, xa1.x, xa1.y, xa1.z, xa1.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h0[2 * q] = bf16_to_f16(a[q] & 0xFFFF);
            h0[2 * q + 1] = bf16_to_f16(a[q] >> 16);
            h1[2 * q] = bf16_to_f16(a[q + 4] & 0xFFFF);
            h1[2 * q + 1] = bf16_to_f16(a[q + 4] >> 16);
        }
        reinterpret_cast<half8_t *>(&As[ar][ac])[0] = h0;
        reinterpret_cast<half8_t *>(&As[ar][ac])[1] = h1;
        dequant16<BITS>(f0.raw, bf16_to_f32(f0.s), bf16_to_f32(f0.b), &Bs[br][bc * 16]);
        dequant16<BITS>(f1.raw, bf16_to_f32(f1.s), bf16_to_f32(f1.b), &Bs[br][bc * 16 + 32]);
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
    load_step(0);
    for (int kb = 0; kb < nk; ++kb) {
        store_step();
        __syncthreads();
        if (kb + 1 < nk) load_step(kb + 1);
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
        __syncthreads();
    }
    // epilogue: lane l, register r -> row 32 mh + 16 i + 4 (l / 16) + r, j = j0 + 32 jh + 16 j + l % 16
    const int Imax = p.Imax;
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
                const _Float16 hh = (_Float16)h;
                const _Float16 hl = (_Float16)(h - (float)hh);
                const size_t o = (size_t)(P0 + m) * Imax + jj;
                p.hh[o] = hh;
                p.hl[o] = hl;
            }
}

// ---- 5. grouped down projection ------------------------------------------------------------------
// Tile: 64 pair rows x 64 output rows n, k-steps of 64 columns of the group's inter. Wave w: rows
// 32 (w & 1) .., n 32 (w >> 1) ..; each k-step runs the MFMA once on h hi and once on h lo.
template <int BITS>
__global__ void __launch_bounds__(kGemmThreads) dn_gemm(BatchedParams p) {
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
    const int br = tid / 4, bc = tid % 4;  // 64 rows x 4 chunks of 16 codes
    const size_t wrow = (size_t)(n0 + br);
    const int nk = w.inter / 64;

    uint4 ha0, ha1, la0, la1;
    WFrag<BITS> f;
    auto load_step = [&](int kb) {
        if (aok) {
            const uint4 *hs = reinterpret_cast<const uint4 *>(hrow + kb * 64 + ac);
            const uint4 *ls = reinterpret_cast<const uint4 *>(lrow + kb * 64 + ac);
            ha0 = hs[0]; ha1 = hs[1];
            la0 = ls[0]; la1 = ls[1];
        } else {
            ha0 = make_uint4(0, 0, 0, 0);
            ha1 = ha0; la0 = ha0; la1 = ha0;
        }
        wfrag_load<BITS>(f, w, wrow, w.inter, kb, bc, true);
    };
    auto store_step = [&]() {
        reinterpret_cast<uint4 *>(&Ah[ar][ac])[0] = ha0;
        reinterpret_cast<uint4 *>(&Ah[ar][ac])[1] = ha1;
        reinterpret_cast<uint4 *>(&Al[ar][ac])[0] = la0;
        reinterpret_cast<uint4 *>(&Al[ar][ac])[1] = la1;
        dequant16<BITS>(f.raw, bf16_to_f32(f.s), bf16_to_f32(f.b), &Bs[br][bc * 16]);
    };

    float4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int mh = wave & 1, nh = wave >> 1;
    load_step(0);
    for (int kb = 0; kb < nk; ++kb) {
        store_step();
        __syncthreads();
        if (kb + 1 < nk) load_step(kb + 1);
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
        __syncthreads();
    }
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
                p.out[(size_t)(P0 + m) * H + n] = sc * acc[i][j][r];
            }
        }
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
    hipLaunchKernelGGL(router_gemm, dim3((p.T + kRtT - 1) / kRtT, (N + kRtN - 1) / kRtN), dim3(kGemmThreads), 0,
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
