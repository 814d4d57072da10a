// moe_device.hpp -- device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---- bf16 ------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }
__device__ __forceinline__ float sigmoid(float v) { return 1.0f / (1.0f + __expf(-v)); }

// ---- workgroup barrier for LDS only -------------------------------------------------------------
// Orders LDS accesses across the workgroup without waiting for outstanding global stores (a full
// __syncthreads() also drains them, which costs a store round trip after every publish). Valid
// wherever threads of a workgroup share data through LDS only.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- division by a runtime constant ----------------------------------------------------------------
// n / d = mulhi(n, m) with m = ceil(2^32 / d), exact for 0 <= n < 2^32 / d (d >= 2); m = 0 stands
// for d = 1. Integer division on the GPU is a long instruction sequence; the reciprocal is
// computed once (on the host, or once per kernel) and every later division is one mulhi.
__host__ __device__ inline uint32_t div_magic(uint32_t d) {
    return d <= 1 ? 0u : static_cast<uint32_t>(0xFFFFFFFFull / d + 1ull);
}
__device__ __forceinline__ int div_by(int n, uint32_t m) {
    return m == 0 ? n : static_cast<int>(__umulhi(static_cast<uint32_t>(n), m));
}

// ---- lane reductions (DPP) ---------------------------------------------------------------------
// Data-parallel-primitive lane moves inside rows of 16 lanes (quad permutations, half-row and
// row mirrors, row rotations) feed the ALU directly, without an LDS round trip; rows are then
// combined with readlane, in a fixed order, so every lane returns the same bits.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each half-row of 8
constexpr int kDppRowMirror = 0x140;  // lane i <-> 15 - i within each row of 16
// Every pattern used reads a lane of the same row, so callers keep whole rows active; the plain
// move form lets the compiler fold it into the consuming ALU instruction (one DPP-modified op).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// Sum over aligned groups of n lanes (n a power of two <= 64, runtime): every lane of a group
// gets the group's sum.
__device__ __forceinline__ float seg_sum(float v, int n) {
    if (n >= 2) v += dpp_f32<kDppQuadXor1>(v);
    if (n >= 4) v += dpp_f32<kDppQuadXor2>(v);
    if (n >= 8) v += dpp_f32<kDppHalfMirror>(v);
    if (n >= 16) v += dpp_f32<kDppRowMirror>(v);
    if (n >= 32) {
        const float a = readlane_f32(v, 0) + readlane_f32(v, 16), b = readlane_f32(v, 32) + readlane_f32(v, 48);
        v = n >= 64 ? a + b : ((threadIdx.x & 32) ? b : a);
    }
    return v;
}
__device__ __forceinline__ float wave_sum(float v) { return seg_sum(v, kWave); }
// Maximum over the wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppQuadXor1>(v));
    v = max(v, dpp_u32<kDppQuadXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppRowMirror>(v));
    // readlane returns int: compare as unsigned
    const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
    const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
    const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
    const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
    return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dpp_u32<kDppQuadXor1>(v));
    v = min(v, dpp_u32<kDppQuadXor2>(v));
    v = min(v, dpp_u32<kDppHalfMirror>(v));
    v = min(v, dpp_u32<kDppRowMirror>(v));
    const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
    const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
    const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
    const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
    return min(min(r0, r1), min(r2, r3));
}

// Maximum / minimum over the wave left in every lane's VGPR, with no scalar round trip: rows of 16
// lanes reduced by DPP, then row pairs and wave halves combined by the gfx950 lane swaps
// (permlane16_swap: odd rows of the first operand <-> even rows of the second; permlane32_swap:
// upper half of the first <-> lower half of the second; with both operands the same value, the
// maximum of the two results combines row r with row r ^ 1, then half h with half h ^ 1).
__device__ __forceinline__ uint32_t wave_max_vgpr(uint32_t v) {
    v = max(v, dpp_u32<kDppQuadXor1>(v));
    v = max(v, dpp_u32<kDppQuadXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppRowMirror>(v));
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(static_cast<uint32_t>(c[0]), static_cast<uint32_t>(c[1]));
}
__device__ __forceinline__ uint32_t wave_min_vgpr(uint32_t v) {
    v = min(v, dpp_u32<kDppQuadXor1>(v));
    v = min(v, dpp_u32<kDppQuadXor2>(v));
    v = min(v, dpp_u32<kDppHalfMirror>(v));
    v = min(v, dpp_u32<kDppRowMirror>(v));
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = min(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return min(static_cast<uint32_t>(c[0]), static_cast<uint32_t>(c[1]));
}

// Partial dot product of an fp32 row with v[0..cols) (cols % 4 == 0).
__device__ __forceinline__ float frow_dot_partial(const float *row, int cols, const float *v, int lane) {
    float acc = 0.0f;
    for (int q = lane; q < cols / 4; q += kWave) {
        const float4 r = reinterpret_cast<const float4 *>(row)[q];
        const float *vc = v + 4 * q;
        acc += r.x * vc[0];
        acc += r.y * vc[1];
        acc += r.z * vc[2];
        acc += r.w * vc[3];
    }
    return acc;
}

// ---- top-k selection ------------------------------------------------------------------------
// Order-preserving key of a finite float: larger value <=> larger key; -0 and +0 share one key so
// that they tie (and the lower expert index wins, like any other tie).
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkMaxE = 1024;

// Top-k of lt[0..E) (LDS) by one whole wave, NJ = ceil(E / 64) keys per lane (expert e = lane +
// 64 j in slot j): the K indices with the largest values, ordered by (value descending, index
// ascending). Exact and deterministic: K rounds of (wave maximum of the remaining keys; the lowest
// expert index holding it wins; that key is removed). Each lane names the lowest index it holds
// at the maximum; when one lane alone holds it (the usual case) a ballot finds that lane and its
// index is read from it, else the wave minimum of the named indices decides. Writes idx[0..K) and
// the renormalised softmax weights w[0..K) (softmax over the kept logits equals
// softmax-then-renormalise), the exponentials summed by a fixed lane reduction.
template <int NJ>
__device__ inline void wave_topk_n(const float *lt, int E, int K, int *idx, float *w) {
    const int lane = threadIdx.x % kWave;
    uint32_t key[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + kWave * j;
        const float v = lt[min(e, E - 1)];  // every read in flight at once; padding masked below
        key[j] = e < E ? order_key(v) : 0u; // 0 sorts below the key of every finite value
    }
    int mine = 0;  // lane r < K ends with the rank-r winner
    for (int r = 0; r < K; ++r) {
        uint32_t m = key[0];
#pragma unroll
        for (int j = 1; j < NJ; ++j) m = max(m, key[j]);
        m = wave_max_vgpr(m);
        // the lowest expert index holding the maximum: per lane its first matching slot
        uint32_t c = 0xFFFFFFFFu;
#pragma unroll
        for (int j = NJ - 1; j >= 0; --j) c = key[j] == m ? static_cast<uint32_t>(lane + kWave * j) : c;
        const unsigned long long holders = __ballot(c != 0xFFFFFFFFu);
        int win;
        if (__popcll(holders) == 1)
            win = __builtin_amdgcn_readlane(static_cast<int>(c), __builtin_amdgcn_readfirstlane(__ffsll(holders) - 1));
        else
            win = static_cast<int>(wave_min_vgpr(c));
        if (lane == r) mine = win;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (lane + kWave * j == win) key[j] = 0u;
    }
    const float v = lt[lane < K ? mine : 0];
    const float vmax = readlane_f32(v, 0);
    const float pe = lane < K ? expf(v - vmax) : 0.0f;
    const float z = wave_sum(pe);  // fixed reduction tree: the same bits every time
    if (lane < K) {
        idx[lane] = mine;
        w[lane] = pe / z;
    }
}

// The same selection with each lane's NJ keys sorted first (key descending; equal keys keep their
// ascending expert order, the network exchanging only adjacent slots and only on a strictly larger
// key), so that a lane competes with its head alone: a round is the wave maximum of the heads, the
// lane holding it (lowest expert index among tied heads, by a wave minimum in that rare case)
// records its head's expert and shifts its list up. Same result as wave_topk_n: the first key of
// the global (value descending, index ascending) order is always some lane's head.
template <int NJ>
__device__ inline void wave_topk_sorted(const float *lt, int E, int K, int *idx, float *w) {
    const int lane = threadIdx.x % kWave;
    uint32_t key[NJ];
    int ex[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + kWave * j;
        const float v = lt[min(e, E - 1)];
        key[j] = e < E ? order_key(v) : 0u;
        ex[j] = e;
    }
#pragma unroll
    for (int a = 1; a < NJ; ++a) {
#pragma unroll
        for (int b = a; b > 0; --b) {
            const bool sw = key[b] > key[b - 1];
            const uint32_t k0 = key[b - 1], k1 = key[b];
            const int e0 = ex[b - 1], e1 = ex[b];
            key[b - 1] = sw ? k1 : k0;
            key[b] = sw ? k0 : k1;
            ex[b - 1] = sw ? e1 : e0;
            ex[b] = sw ? e0 : e1;
        }
    }
    int mine = 0;  // lane r < K ends with the rank-r winner
    for (int r = 0; r < K; ++r) {
        const uint32_t m = wave_max_vgpr(key[0]);
        const unsigned long long holders = __ballot(key[0] == m);
        int wl;  // the winning lane
        if (__popcll(holders) == 1) {
            wl = __builtin_amdgcn_readfirstlane(__ffsll(holders) - 1);
        } else {
            const uint32_t c = key[0] == m ? static_cast<uint32_t>(ex[0]) : 0xFFFFFFFFu;
            wl = static_cast<int>(wave_min_vgpr(c)) & (kWave - 1);
        }
        const int win = __builtin_amdgcn_readlane(ex[0], wl);
        if (lane == r) mine = win;
        if (lane == wl) {
#pragma unroll
            for (int j = 0; j + 1 < NJ; ++j) {
                key[j] = key[j + 1];
                ex[j] = ex[j + 1];
            }
            key[NJ - 1] = 0u;
        }
    }
    const float v = lt[lane < K ? mine : 0];
    const float vmax = readlane_f32(v, 0);
    const float pe = lane < K ? expf(v - vmax) : 0.0f;
    const float z = wave_sum(pe);  // fixed reduction tree: the same bits every time
    if (lane < K) {
        idx[lane] = mine;
        w[lane] = pe / z;
    }
}

__device__ inline void wave_topk(const float *lt, int E, int K, int *idx, float *w) {
    const int nj = (E + kWave - 1) / kWave;
    if (nj <= 1) wave_topk_n<1>(lt, E, K, idx, w);
    else if (nj <= 2) wave_topk_sorted<2>(lt, E, K, idx, w);
    else if (nj <= 4) wave_topk_sorted<4>(lt, E, K, idx, w);
    else if (nj <= 8) wave_topk_sorted<8>(lt, E, K, idx, w);
    else wave_topk_n<16>(lt, E, K, idx, w);
}

}  // namespace moe
