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

// ---- lane reductions -------------------------------------------------------------------------
// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of a group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = N / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<kWave>(v); }

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

// Top-k of lt[0..E) (LDS) by one whole wave, NJ = ceil(E / 64) keys per lane: the K indices with
// the largest values, ordered by (value descending, index ascending). Exact and deterministic:
//   1. theta = the K-th largest key, built bit by bit from the top: a candidate bit stays set when
//      at least K keys are >= the candidate (each lane compare is itself the wave ballot);
//   2. every key > theta is taken, then keys == theta in increasing index order until K;
//   3. the K winners (one per lane < K) are ranked among themselves with readlane broadcasts.
// Writes idx[0..K) and the renormalised softmax weights w[0..K) (softmax over the kept logits
// equals softmax-then-renormalise). `scratch` is LDS for K ints owned by this wave.
template <int NJ>
__device__ inline void wave_topk_n(const float *lt, int E, int K, int *idx, float *w, int *scratch) {
    const int lane = threadIdx.x % kWave;
    uint32_t key[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + kWave * j;
        const float v = lt[min(e, E - 1)];  // every read in flight at once; padding masked below
        key[j] = e < E ? order_key(v) : 0u; // padding keys sort below every value
    }
    uint32_t theta = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = theta | (1u << bit);  // never 0, so padding keys never count
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) cnt += __popcll(__ballot(key[j] >= cand));
        if (cnt >= K) theta = cand;
    }
    int need = K;
#pragma unroll
    for (int j = 0; j < NJ; ++j) need -= __popcll(__ballot(key[j] > theta));
    // take ties (key == theta) in increasing index order: index = lane + 64 j
    const unsigned long long below = (1ull << lane) - 1ull;
    int base = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const unsigned long long eq = __ballot(key[j] == theta);
        const bool sel = key[j] > theta || ((key[j] == theta) && (int)__popcll(eq & below) < need);
        need -= min(need, (int)__popcll(eq));
        const unsigned long long sm = __ballot(sel);
        if (sel) scratch[base + __popcll(sm & below)] = lane + kWave * j;
        base += __popcll(sm);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int e = lane < K ? scratch[lane] : 0;
    const float v = lt[e];
    const uint32_t ke = order_key(v);
    int rank = 0;
    for (int m = 0; m < K; ++m) {
        const uint32_t km = __builtin_amdgcn_readlane(ke, m);
        const int em = __builtin_amdgcn_readlane(e, m);
        rank += (km > ke) || (km == ke && em < e);
    }
    // the maximum logit is the rank-0 winner's; sum the exponentials in winner order
    const unsigned long long top = __ballot(lane < K && rank == 0);
    const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), __ffsll((long long)top) - 1));
    const float pe = expf(v - vmax);
    float z = 0.0f;
    for (int m = 0; m < K; ++m) z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), m));
    if (lane < K) {
        idx[rank] = e;
        w[rank] = pe / z;
    }
}

__device__ inline void wave_topk(const float *lt, int E, int K, int *idx, float *w, int *scratch) {
    const int nj = (E + kWave - 1) / kWave;
    if (nj <= 1) wave_topk_n<1>(lt, E, K, idx, w, scratch);
    else if (nj <= 2) wave_topk_n<2>(lt, E, K, idx, w, scratch);
    else if (nj <= 4) wave_topk_n<4>(lt, E, K, idx, w, scratch);
    else if (nj <= 8) wave_topk_n<8>(lt, E, K, idx, w, scratch);
    else wave_topk_n<16>(lt, E, K, idx, w, scratch);
}

// ---- grid-wide barrier for a cooperative (all workgroups co-resident) launch ------------------
// ctrl[0] = status (0 ok, else a moe_status), ctrl[1] = arrivals, ctrl[2] = generation.
// Bounded: after `spin_limit` polls a waiting workgroup records MOE_ERR_TIMEOUT (5) and every
// workgroup then leaves at its next barrier, so a fault in the protocol cannot hang the GPU.
// Returns false once the status is non-zero.
__device__ __forceinline__ bool grid_barrier(int *ctrl, unsigned nblocks, unsigned spin_limit) {
    __shared__ int s_ok;
    __syncthreads();
    if (threadIdx.x == 0) {
        int ok = 1;
        const int gen = __hip_atomic_load(&ctrl[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned arrived = static_cast<unsigned>(
            __hip_atomic_fetch_add(&ctrl[1], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT));
        if (arrived == nblocks - 1) {
            __hip_atomic_store(&ctrl[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&ctrl[2], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            unsigned n = 0;
            while (__hip_atomic_load(&ctrl[2], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen) {
                if (__hip_atomic_load(&ctrl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
                if (++n > spin_limit) {
                    __hip_atomic_store(&ctrl[0], 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (__hip_atomic_load(&ctrl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) ok = 0;
        s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

}  // namespace moe
