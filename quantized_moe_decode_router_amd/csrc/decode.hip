// decode.hip -- MoE layer(s) at decode (T <= 8 tokens) as one persistent, grid-synchronised
// kernel on gfx950.
//
// One workgroup per compute unit loops over the layers; each layer has three phases separated
// by grid barriers (the layer is a strict dependency chain: routing needs all logits, the down
// projection needs every h, the next layer needs all of y):
//   R  router GEMV (E rows + the shared-gate row) and the shared expert's gate|up + SwiGLU
//   G  top-k + renormalised weights (every workgroup, redundantly, from the E logits), then the
//      routed experts' packed gate|up dequant-GEMV + SwiGLU into h
//   D  down dequant-GEMV of the K routed experts and the shared expert for the rows of y this
//      workgroup owns, and the fixed-order weighted combine (k = 0..K-1, then shared)
// Between layers every workgroup recomputes the same RMS-normalised bf16 input from y.
//
// Quantised rows are read in 16-byte chunks (32 4-bit or 16 8-bit codes, always inside one
// 64-column quantisation group), one chunk per lane per step, so a wave reads 1 KiB of a row
// per load instruction. Address arithmetic into the weights is 64-bit.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

constexpr int kWaves = kDecodeThreads / kWave;

// Partial (this lane's chunks) dot product of one quantised row with v[0..cols).
template <int BITS>
__device__ __forceinline__ float qrow_dot_partial(const uint8_t *crow, const uint16_t *srow,
                                                  const uint16_t *brow, int cols, const float *v,
                                                  int lane) {
    constexpr int kColsPerChunk = BITS == 4 ? 32 : 16;
    const int nch = cols / kColsPerChunk;
    float acc = 0.0f;
    for (int ch = lane; ch < nch; ch += kWave) {
        const uint4 code = *reinterpret_cast<const uint4 *>(crow + (size_t)ch * 16);
        const int col0 = ch * kColsPerChunk;
        const float s = bf16_to_f32(srow[col0 >> 6]);
        const float b = bf16_to_f32(brow[col0 >> 6]);
        const uint32_t wd[4] = {code.x, code.y, code.z, code.w};
        const float *vc = v + col0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            if constexpr (BITS == 4) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float q = (float)((wd[d] >> (4 * i)) & 15u);
                    acc += fmaf(s, q, b) * vc[8 * d + i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float q = (float)((wd[d] >> (8 * i)) & 255u);
                    acc += fmaf(s, q, b) * vc[4 * d + i];
                }
            }
        }
    }
    return acc;
}

struct LayerPtrs {
    const float *router, *rbias, *sgate;
    QMat w13, w2, s13, s2;
};

__device__ __forceinline__ LayerPtrs layer_ptrs(const DecodeParams &p, int l) {
    LayerPtrs q;
    q.router = p.router + (size_t)l * p.ls_router;
    q.rbias = p.rbias ? p.rbias + (size_t)l * p.ls_rbias : nullptr;
    q.sgate = p.sgate ? p.sgate + (size_t)l * p.ls_sgate : nullptr;
    q.w13 = {p.w13.c + (size_t)l * p.ls_w13c, p.w13.s + (size_t)l * p.ls_w13s, p.w13.b + (size_t)l * p.ls_w13s};
    q.w2 = {p.w2.c + (size_t)l * p.ls_w2c, p.w2.s + (size_t)l * p.ls_w2s, p.w2.b + (size_t)l * p.ls_w2s};
    if (p.Is) {
        q.s13 = {p.s13.c + (size_t)l * p.ls_s13c, p.s13.s + (size_t)l * p.ls_s13s, p.s13.b + (size_t)l * p.ls_s13s};
        q.s2 = {p.s2.c + (size_t)l * p.ls_s2c, p.s2.s + (size_t)l * p.ls_s2s, p.s2.b + (size_t)l * p.ls_s2s};
    } else {
        q.s13 = {nullptr, nullptr, nullptr};
        q.s2 = {nullptr, nullptr, nullptr};
    }
    return q;
}

// Sum over the whole workgroup; identical order in every workgroup, so every workgroup gets
// the same bits. `red` is LDS scratch of kWaves floats.
__device__ __forceinline__ float block_sum(float v, float *red) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) s += red[i];
    return s;
}

// Input of layer l into LDS xs[T][H] (fp32 values of bf16): the given x for l == 0, else the
// RMS glue applied to y of layer l-1.
__device__ void load_layer_input(const DecodeParams &p, int l, float *xs, float *red) {
    const int T = p.T, H = p.H;
    if (l == 0 || !p.glue) {
        const uint16_t *src = p.x_in;
        for (int i = threadIdx.x; i < T * H; i += blockDim.x) xs[i] = bf16_to_f32(src[i]);
        if (p.x_all && blockIdx.x == 0)
            for (int i = threadIdx.x; i < T * H; i += blockDim.x) p.x_all[(size_t)l * T * H + i] = src[i];
    } else {
        for (int t = 0; t < T; ++t) {
            const float *y = p.ybuf + (size_t)t * H;
            float ss = 0.0f;
            for (int h = threadIdx.x; h < H; h += blockDim.x) ss += y[h] * y[h];
            ss = block_sum(ss, red);
            const float inv = 1.0f / sqrtf(ss / (float)H + p.eps);
            for (int h = threadIdx.x; h < H; h += blockDim.x) {
                const uint16_t xb = f32_to_bf16_rne(y[h] * inv);
                xs[t * H + h] = bf16_to_f32(xb);
                if (p.x_all && blockIdx.x == 0) p.x_all[((size_t)l * T + t) * H + h] = xb;
            }
        }
    }
    __syncthreads();
}

// Phase R: router logits, shared-gate logit, shared expert gate|up + SwiGLU.
template <int BITS>
__device__ void phase_router_shared(const DecodeParams &p, const LayerPtrs &L, const float *xs) {
    const int lane = threadIdx.x % kWave;
    const int gw = blockIdx.x * kWaves + threadIdx.x / kWave;
    const int nw = gridDim.x * kWaves;
    const int T = p.T, H = p.H, E = p.E, K = p.K, Is = p.Is;
    const int ntasks = E + 1 + Is;
    const size_t cpr = (size_t)H * BITS / 8;  // code bytes per gate/up row
    const int gpr = H / 64;                   // groups per gate/up row
    for (int task = gw; task < ntasks; task += nw) {
        if (task < E) {
            const float *row = L.router + (size_t)task * H;
            const float bias = L.rbias ? L.rbias[task] : 0.0f;
            for (int t = 0; t < T; ++t) {
                const float s = wave_sum(frow_dot_partial(row, H, xs + t * H, lane));
                if (lane == 0) p.logits[t * (E + 1) + task] = s + bias;
            }
        } else if (task == E) {
            if (Is) {
                for (int t = 0; t < T; ++t) {
                    const float s = wave_sum(frow_dot_partial(L.sgate, H, xs + t * H, lane));
                    if (lane == 0) p.logits[t * (E + 1) + E] = s;
                }
            }
        } else {
            const int j = task - E - 1;
            const uint8_t *cg = L.s13.c + (size_t)j * cpr;
            const uint8_t *cu = L.s13.c + (size_t)(Is + j) * cpr;
            const uint16_t *sg = L.s13.s + (size_t)j * gpr, *bg = L.s13.b + (size_t)j * gpr;
            const uint16_t *su = L.s13.s + (size_t)(Is + j) * gpr, *bu = L.s13.b + (size_t)(Is + j) * gpr;
            for (int t = 0; t < T; ++t) {
                const float g = wave_sum(qrow_dot_partial<BITS>(cg, sg, bg, H, xs + t * H, lane));
                const float u = wave_sum(qrow_dot_partial<BITS>(cu, su, bu, H, xs + t * H, lane));
                if (lane == 0) p.hbuf[((size_t)t * (K + 1) + K) * p.Imax + j] = silu(g) * u;
            }
        }
    }
}

// Top-k on logits (rank of each expert under (logit desc, index asc)), renormalised weights
// and gamma, for all T tokens, into LDS. Every workgroup computes the same result.
__device__ void route_topk(const DecodeParams &p, int l, float *lg, int *sidx, float *sw, float *gam) {
    const int T = p.T, E = p.E, K = p.K;
    for (int i = threadIdx.x; i < T * (E + 1); i += blockDim.x) lg[i] = p.logits[i];
    __syncthreads();
    for (int t = 0; t < T; ++t) {
        const float *lt = lg + t * (E + 1);
        for (int e = threadIdx.x; e < E; e += blockDim.x) {
            const float v = lt[e];
            int rank = 0;
            for (int e2 = 0; e2 < E; ++e2) {
                const float v2 = lt[e2];
                rank += (v2 > v) || (v2 == v && e2 < e);
            }
            if (rank < K) sidx[t * K + rank] = e;
        }
    }
    __syncthreads();
    if (threadIdx.x < T) {
        const int t = threadIdx.x;
        const float *lt = lg + t * (E + 1);
        const float m = lt[sidx[t * K]];
        float z = 0.0f;
        for (int k = 0; k < K; ++k) z += expf(lt[sidx[t * K + k]] - m);
        for (int k = 0; k < K; ++k) sw[t * K + k] = expf(lt[sidx[t * K + k]] - m) / z;
        gam[t] = p.Is ? 1.0f / (1.0f + expf(-lt[E])) : 0.0f;
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        const size_t base = (size_t)l * T;
        if (p.idx_all)
            for (int i = threadIdx.x; i < T * K; i += blockDim.x) p.idx_all[base * K + i] = sidx[i];
        if (p.w_all)
            for (int i = threadIdx.x; i < T * K; i += blockDim.x) p.w_all[base * K + i] = sw[i];
        if (p.logits_all)
            for (int i = threadIdx.x; i < T * E; i += blockDim.x)
                p.logits_all[base * E + i] = lg[(i / E) * (E + 1) + i % E];
    }
}

// Phase G: routed experts' gate|up + SwiGLU for every (token, slot, j).
template <int BITS>
__device__ void phase_routed_gate_up(const DecodeParams &p, const LayerPtrs &L, const float *xs,
                                     const int *sidx) {
    const int lane = threadIdx.x % kWave;
    const int gw = blockIdx.x * kWaves + threadIdx.x / kWave;
    const int nw = gridDim.x * kWaves;
    const int T = p.T, H = p.H, K = p.K, I = p.I;
    const size_t cpr = (size_t)H * BITS / 8;
    const int gpr = H / 64;
    const int ntasks = T * K * I;
    for (int task = gw; task < ntasks; task += nw) {
        const int t = task / (K * I);
        const int rem = task - t * K * I;
        const int k = rem / I;
        const int j = rem - k * I;
        const size_t e = (size_t)sidx[t * K + k];
        const size_t rg = e * 2 * I + j, ru = e * 2 * I + I + j;
        const float g = wave_sum(qrow_dot_partial<BITS>(L.w13.c + rg * cpr, L.w13.s + rg * gpr,
                                                        L.w13.b + rg * gpr, H, xs + t * H, lane));
        const float u = wave_sum(qrow_dot_partial<BITS>(L.w13.c + ru * cpr, L.w13.s + ru * gpr,
                                                        L.w13.b + ru * gpr, H, xs + t * H, lane));
        if (lane == 0) p.hbuf[((size_t)t * (K + 1) + k) * p.Imax + j] = silu(g) * u;
    }
}

// Phase D: down projections for this workgroup's rows of y and the fixed-order combine.
template <int BITS>
__device__ void phase_down_combine(const DecodeParams &p, const LayerPtrs &L, int l, const int *sidx,
                                   const float *sw, const float *gam, float *part) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int T = p.T, H = p.H, K = p.K, I = p.I, Is = p.Is, RB = p.rows_per_wg;
    const int r0 = blockIdx.x * RB;
    const int nr = r0 >= H ? 0 : (H - r0 < RB ? H - r0 : RB);
    const int nslot = K + (Is ? 1 : 0);
    const int ntasks = T * nslot * nr;
    for (int task = wave; task < ntasks; task += kWaves) {
        const int t = task / (nslot * nr);
        const int rem = task - t * nslot * nr;
        const int kk = rem / nr;
        const int rl = rem - kk * nr;
        const size_t r = (size_t)(r0 + rl);
        const float *hv = p.hbuf + ((size_t)t * (K + 1) + kk) * p.Imax;
        float d;
        if (kk < K) {
            const size_t e = (size_t)sidx[t * K + kk];
            const size_t row = e * H + r;
            const size_t cpr = (size_t)I * BITS / 8;
            d = wave_sum(qrow_dot_partial<BITS>(L.w2.c + row * cpr, L.w2.s + row * (I / 64),
                                                L.w2.b + row * (I / 64), I, hv, lane));
        } else {
            const size_t cpr = (size_t)Is * BITS / 8;
            d = wave_sum(qrow_dot_partial<BITS>(L.s2.c + r * cpr, L.s2.s + r * (Is / 64),
                                                L.s2.b + r * (Is / 64), Is, hv, lane));
        }
        if (lane == 0) part[(t * (K + 1) + kk) * RB + rl] = d;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * nr; i += blockDim.x) {
        const int t = i / nr, rl = i - (i / nr) * nr;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) acc += sw[t * K + k] * part[(t * (K + 1) + k) * RB + rl];
        if (Is) acc += gam[t] * part[(t * (K + 1) + K) * RB + rl];
        const size_t o = (size_t)t * H + r0 + rl;
        p.ybuf[o] = acc;
        if (l == p.L - 1) p.y_out[o] = acc;
        if (p.y_all) p.y_all[(size_t)l * T * H + o] = acc;
    }
}

struct Lds {
    float *xs, *lg, *sw, *gam, *part, *red;
    int *sidx;
};

__device__ __forceinline__ Lds carve_lds(const DecodeParams &p, char *smem) {
    const DecodeLds o = decode_lds_layout(p.T, p.H, p.E, p.K, p.rows_per_wg);
    Lds s;
    s.xs = reinterpret_cast<float *>(smem + o.xs);
    s.lg = reinterpret_cast<float *>(smem + o.lg);
    s.sidx = reinterpret_cast<int *>(smem + o.sidx);
    s.sw = reinterpret_cast<float *>(smem + o.sw);
    s.gam = reinterpret_cast<float *>(smem + o.gam);
    s.part = reinterpret_cast<float *>(smem + o.part);
    s.red = reinterpret_cast<float *>(smem + o.red);
    return s;
}

template <int BITS>
__global__ void __launch_bounds__(kDecodeThreads) decode_persistent(DecodeParams p) {
    extern __shared__ __align__(16) char smem[];
    const Lds s = carve_lds(p, smem);
    const unsigned nb = gridDim.x;
    for (int l = 0; l < p.L; ++l) {
        const LayerPtrs L = layer_ptrs(p, l);
        load_layer_input(p, l, s.xs, s.red);
        phase_router_shared<BITS>(p, L, s.xs);
        if (!grid_barrier(p.ctrl, nb, p.spin_limit)) return;
        route_topk(p, l, s.lg, s.sidx, s.sw, s.gam);
        phase_routed_gate_up<BITS>(p, L, s.xs, s.sidx);
        if (!grid_barrier(p.ctrl, nb, p.spin_limit)) return;
        phase_down_combine<BITS>(p, L, l, s.sidx, s.sw, s.gam, s.part);
        if (l + 1 < p.L && !grid_barrier(p.ctrl, nb, p.spin_limit)) return;
    }
}

// One phase of one layer per launch (kernel boundaries instead of grid barriers).
template <int BITS>
__global__ void __launch_bounds__(kDecodeThreads) decode_phase(DecodeParams p, int l, int phase) {
    extern __shared__ __align__(16) char smem[];
    const Lds s = carve_lds(p, smem);
    const LayerPtrs L = layer_ptrs(p, l);
    if (phase == 0) {
        load_layer_input(p, l, s.xs, s.red);
        phase_router_shared<BITS>(p, L, s.xs);
    } else if (phase == 1) {
        load_layer_input(p, l, s.xs, s.red);
        route_topk(p, l, s.lg, s.sidx, s.sw, s.gam);
        phase_routed_gate_up<BITS>(p, L, s.xs, s.sidx);
    } else {
        // the routing outputs were already written by phase 1
        DecodeParams q = p;
        q.idx_all = nullptr;
        q.w_all = nullptr;
        q.logits_all = nullptr;
        route_topk(q, l, s.lg, s.sidx, s.sw, s.gam);
        phase_down_combine<BITS>(p, L, l, s.sidx, s.sw, s.gam, s.part);
    }
}

__global__ void zero_ints(int *p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

template <int BITS>
static hipError_t launch_bits(const DecodeParams &p, int grid, hipStream_t stream, int persistent) {
    const size_t lds = decode_lds_layout(p.T, p.H, p.E, p.K, p.rows_per_wg).total;
    hipLaunchKernelGGL(zero_ints, dim3(1), dim3(64), 0, stream, p.ctrl, 64);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (persistent) {
        const void *fn = reinterpret_cast<const void *>(&decode_persistent<BITS>);
        if (lds > 65536) {
            err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (err != hipSuccess) return err;
        }
        DecodeParams arg = p;
        void *args[] = {&arg};
        return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kDecodeThreads), args, (unsigned)lds, stream);
    }
    const void *fn = reinterpret_cast<const void *>(&decode_phase<BITS>);
    if (lds > 65536) {
        err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    for (int l = 0; l < p.L; ++l)
        for (int ph = 0; ph < 3; ++ph) {
            hipLaunchKernelGGL(decode_phase<BITS>, dim3(grid), dim3(kDecodeThreads), lds, stream, p, l, ph);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
    return hipSuccess;
}

hipError_t launch_decode(const DecodeParams &p, int grid, hipStream_t stream, int persistent) {
    return p.bits == 4 ? launch_bits<4>(p, grid, stream, persistent)
                       : launch_bits<8>(p, grid, stream, persistent);
}

}  // namespace moe
