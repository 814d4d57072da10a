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
