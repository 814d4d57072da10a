// route.hip -- router for T tokens: fp32 router GEMV (or given logits), top-k selection under
// (logit descending, index ascending) and renormalised softmax weights. One workgroup per token;
// its first wave selects (wave_topk).
// Each token goes to 8 of 256 experts (35B-A3B) or 10 of 512 (80B-A3B) (xix.ai Swiftlet article,
// paragraph on scheduling); the selection rule and renormalisation are the plainest reading of
// top-k routing, and softmax-then-renormalise over the kept experts equals the softmax of the
// kept logits, so only K exponentials are evaluated.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

constexpr int kRouteThreads = 256;

__global__ void __launch_bounds__(kRouteThreads) route_kernel(RouteParams p) {
    extern __shared__ __align__(16) char smem[];
    const int H = p.H, E = p.E, K = p.K;
    const int t = blockIdx.x;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    float *xs = reinterpret_cast<float *>(smem);
    float *lg = xs + H;
    int *sidx = reinterpret_cast<int *>(lg + E + 1);
    float gate_logit = 0.0f;
    if (!p.logits_in) {
        for (int h = threadIdx.x; h < H; h += blockDim.x) xs[h] = bf16_to_f32(p.x[(size_t)t * H + h]);
        __syncthreads();
        const int nrows = E + (p.has_gate ? 1 : 0);
        for (int e = wave; e < nrows; e += kRouteThreads / kWave) {
            const float *row = e < E ? p.router + (size_t)e * H : p.sgate;
            const float s = wave_sum(frow_dot_partial(row, H, xs, lane));
            if (lane == 0) lg[e] = s + ((e < E && p.rbias) ? p.rbias[e] : 0.0f);
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += blockDim.x) p.logits[(size_t)t * E + e] = lg[e];
        if (p.has_gate) gate_logit = lg[E];
    } else {
        for (int e = threadIdx.x; e < E; e += blockDim.x) lg[e] = p.logits[(size_t)t * E + e];
        __syncthreads();
    }
    if (wave == 0) wave_topk(lg, E, K, sidx + 2 * K, reinterpret_cast<float *>(sidx + 3 * K));
    __syncthreads();
    if (threadIdx.x < K) {
        p.idx[(size_t)t * K + threadIdx.x] = sidx[2 * K + threadIdx.x];
        p.w[(size_t)t * K + threadIdx.x] = reinterpret_cast<float *>(sidx + 3 * K)[threadIdx.x];
    }
    if (threadIdx.x == 0 && p.gamma) p.gamma[t] = 1.0f / (1.0f + expf(-gate_logit));
}

hipError_t launch_route(const RouteParams &p, hipStream_t stream) {
    const size_t lds = sizeof(float) * ((size_t)p.H + p.E + 1) + sizeof(int) * 4 * (size_t)p.K;
    if (lds > 65536) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&route_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(route_kernel, dim3(p.T), dim3(kRouteThreads), lds, stream, p);
    return hipGetLastError();
}

}  // namespace moe
