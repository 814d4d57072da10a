// decode.hip -- MoE layer(s) at decode (T <= 8 tokens) as one persistent kernel on gfx950.
//
// One workgroup of 512 threads per compute unit loops over the layers. A layer is a strict
// dependency chain -- routing needs every logit, the down projection needs every h, the next
// layer needs all of y -- so workgroups exchange those values through 8-byte words in the
// workspace, each carrying a 32-bit value and the 32-bit epoch of the call that wrote it, stored
// and loaded with agent-scope relaxed atomics. A word is its own message: a consumer that sees
// the current epoch in a word has that word's value, so no grid barrier, no cache-maintenance
// fence and no separate flag is needed, and each workgroup waits only for the words it reads.
//
// Per layer and workgroup b:
//   R  (after x is known) router logits of the experts e = b (mod grid) [+ the shared-gate row E]
//      and gate|up + SwiGLU of the shared expert's pairs j = b (mod grid)  -> logits, shared h
//   G  every workgroup reads all E logits, ranks them (logit desc, index asc) and keeps the top-k
//      with renormalised weights; then issues the loads of its share of the routed gate|up rows
//      and of its routed down rows together, computes gate|up + SwiGLU -> routed h; then the
//      shared expert's down projection for its rows of y
//   D  reads the routed h of every (token, slot), computes its rows of every routed down
//      projection from the already-loaded codes and combines them in a fixed order
//      (k = 0..K-1, then the shared expert) -> y
// Between layers each workgroup recomputes the same RMS-normalised bf16 input from all of y.
//
// Quantised rows are split into 32-column slices (16 bytes of 4-bit or 32 bytes of 8-bit codes,
// always inside one 64-column quantisation group); lane l of a wave always takes slice l % SPR of
// its row (SPR = slices per row), so its slice of the activation vector stays in registers as
// bf16 pairs. Codes become the bf16 values 128 + nibble with one v_and_or (exact), feed
// v_dot2_f32_bf16 against the bf16 activations (products exact, fp32 sums), and the 128 * sum(x)
// offset folds into the group bias: s * sum(q x) + b * sum(x) = s * sum((128+q) x) + (b - 128 s) * sum(x).
// The fp32 h of the down projection is split into bf16 hi + lo halves (16 significant bits).
// All address arithmetic into the weights is 64-bit.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

constexpr int kWaves = kDecodeThreads / kWave;  // 8
constexpr int kMaxWL = 4;                       // gate|up wave-loads of codes a wave holds at once
constexpr int kDnWL = 2;                        // down-projection wave-loads a wave holds at once
constexpr int kShWL = 2;                        // shared gate|up wave-loads prefetched per wave
constexpr uint32_t kMagic = 0x43004300u;        // bf16 pair (128, 128)
constexpr int kGatherWords = 8;                 // exchange words one thread waits for at once

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// ---- exchange words ---------------------------------------------------------------------------
__device__ __forceinline__ void ll_put(uint64_t *p, float v, uint32_t ep) {
    const uint64_t w = (static_cast<uint64_t>(ep) << 32) | __float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ll_get(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int status_of(const int *ctrl) {
    return __hip_atomic_load(const_cast<int *>(ctrl), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fail(int *ctrl) {
    __hip_atomic_store(ctrl, 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until words src[0..n) (n <= kGatherWords * 512) carry epoch ep and copy their values to dst (LDS).
// Called by the whole workgroup. All of a thread's loads are in flight together; only the words
// not yet current are polled again. Returns false on timeout or when any workgroup has failed.
__device__ bool ll_gather(const uint64_t *src, int n, uint32_t ep, float *dst, int *ctrl, unsigned spin) {
    constexpr int kMax = kGatherWords;
    const int tid = threadIdx.x;
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < kMax; ++k)
        if (tid + k * kDecodeThreads < n) pending |= 1u << k;
    bool ok = true;
    unsigned it = 0;
    while (pending) {
        uint64_t w[kMax];
#pragma unroll
        for (int k = 0; k < kMax; ++k) {
            const int i = tid + k * kDecodeThreads;
            w[k] = ((pending >> k) & 1u) ? ll_get(src + i) : 0;
        }
#pragma unroll
        for (int k = 0; k < kMax; ++k) {
            if (((pending >> k) & 1u) && static_cast<uint32_t>(w[k] >> 32) == ep) {
                dst[tid + k * kDecodeThreads] = __uint_as_float(static_cast<uint32_t>(w[k]));
                pending &= ~(1u << k);
            }
        }
        if (!pending) break;
        if (++it > spin) { fail(ctrl); ok = false; break; }
        if ((it & 31u) == 0 && status_of(ctrl) != 0) { ok = false; break; }
        __builtin_amdgcn_s_sleep(1);
    }
    // workgroup-wide AND of ok through LDS (slots written, read, then released again)
    __shared__ int vote[kDecodeThreads / kWave];
    const unsigned long long bad = __ballot(!ok);
    if ((threadIdx.x % kWave) == 0) vote[threadIdx.x / kWave] = bad ? 0 : 1;
    lds_barrier();
    int all = 1;
#pragma unroll
    for (int w = 0; w < kDecodeThreads / kWave; ++w) all &= vote[w];
    lds_barrier();
    return all != 0;
}

// ---- slice dot products -------------------------------------------------------------------------
// 4-bit slice: 16 bytes = 32 codes; dword d holds columns 8d..8d+7 (nibble i = column 8d+i).
// xp[4d+p] = bf16 pair (x[8d+p], x[8d+p+4]). Returns acc + sum((128+q) x).
__device__ __forceinline__ float slice_dot4(const uint4 c, const uint32_t *xp, float acc) {
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = wd[d];
        acc = dot2((w & 0x000F000Fu) | kMagic, xp[4 * d + 0], acc);
        acc = dot2(((w >> 4) & 0x000F000Fu) | kMagic, xp[4 * d + 1], acc);
        acc = dot2(((w >> 8) & 0x000F000Fu) | kMagic, xp[4 * d + 2], acc);
        acc = dot2(((w >> 12) & 0x000F000Fu) | kMagic, xp[4 * d + 3], acc);
    }
    return acc;
}
// 8-bit slice: 32 bytes = 32 codes in two uint4; dword d holds columns 4d..4d+3.
// xp[2d+p] = bf16 pair (x[4d+p], x[4d+p+2]). Each byte q = lo + 16 hi is split into nibbles:
// lo += sum((128+lo) x), hi += sum((128+hi) x).
__device__ __forceinline__ void slice_dot8(const uint4 c0, const uint4 c1, const uint32_t *xp, float &lo, float &hi) {
    const uint32_t wd[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        const uint32_t w = wd[d];
        lo = dot2((w & 0x000F000Fu) | kMagic, xp[2 * d + 0], lo);
        lo = dot2(((w >> 8) & 0x000F000Fu) | kMagic, xp[2 * d + 1], lo);
        hi = dot2(((w >> 4) & 0x000F000Fu) | kMagic, xp[2 * d + 0], hi);
        hi = dot2(((w >> 12) & 0x000F000Fu) | kMagic, xp[2 * d + 1], hi);
    }
}

// Column (within a 32-column slice) of the two halves of pair slot q.
template <int BITS>
__device__ __forceinline__ int pair_col_a(int q) {
    return BITS == 4 ? 8 * (q >> 2) + (q & 3) : 4 * (q >> 1) + (q & 1);
}
template <int BITS>
__device__ __forceinline__ int pair_col_b(int q) {
    return pair_col_a<BITS>(q) + (BITS == 4 ? 4 : 2);
}

// Codes of one lane for one row slice (16 bytes at 4-bit, 32 at 8-bit) and its group's scale and
// bias bf16 bit patterns, held exactly as loaded: no arithmetic touches them until the math, so
// the loads of many rows stay in flight together instead of each waiting for its own scale.
template <int BITS>
struct SliceCodes;
template <>
struct SliceCodes<4> {
    uint4 c0;
    uint32_t s16, b16;
};
template <>
struct SliceCodes<8> {
    uint4 c0, c1;
    uint32_t s16, b16;
};
template <int BITS>
__device__ __forceinline__ void load_slice(SliceCodes<BITS> &sc, const uint8_t *crow, const uint16_t *srow,
                                           const uint16_t *brow, int slice) {
    const uint4 *cp = reinterpret_cast<const uint4 *>(crow + (size_t)slice * (BITS == 4 ? 16 : 32));
    sc.c0 = cp[0];
    if constexpr (BITS == 8) sc.c1 = cp[1];
    sc.s16 = srow[slice >> 1];
    sc.b16 = brow[slice >> 1];
}
template <int BITS>
__device__ __forceinline__ float sc_scale(const SliceCodes<BITS> &sc) { return __uint_as_float(sc.s16 << 16); }
template <int BITS>
__device__ __forceinline__ float sc_bias(const SliceCodes<BITS> &sc) { return __uint_as_float(sc.b16 << 16); }

// Per-slice constants of an activation slice v (built once per vector, shared by every row):
//   sum = sum(v);  z0 / z1 = the dot chains of slice_dot4 / slice_dot8 evaluated with every code
//   at the zero point (4-bit: q = 8 -> pairs (136, 136); 8-bit: q = 128 -> lo nibble 0, hi 8), in
//   exactly the same order as for a real row. Then, exactly in algebra,
//     sum((s q + b) v) = s * sum((q - zp) v) + (b + zp s) * sum(v)
//   and sum((q - zp) v) = acc - z0 (4-bit) or (lo - z0) + 16 (hi - z1) (8-bit). A row whose codes
//   all sit at the zero point gives acc == z0 bit for bit, so an all-zero expert yields exactly 0.
struct SliceRef {
    float sum, z0, z1;
};
constexpr uint32_t kZero4 = 0x43084308u;  // bf16 pair (136, 136) = 128 + 8
template <int BITS>
__device__ __forceinline__ SliceRef slice_ref(const uint32_t *vp, int npass, const uint32_t *vp2) {
    // npass = 1: one pair set; npass = 2: chain continues over a second pair set (hi then lo)
    SliceRef r;
    float sum = 0.0f;
    const uint32_t *sets[2] = {vp, vp2};
    for (int ps = 0; ps < npass; ++ps)
        for (int q = 0; q < 16; ++q)
            sum += bf16_to_f32(sets[ps][q] & 0xFFFF) + bf16_to_f32(sets[ps][q] >> 16);
    r.sum = sum;
    if constexpr (BITS == 4) {
        const uint4 zc = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        float acc = 0.0f;
        for (int ps = 0; ps < npass; ++ps) acc = slice_dot4(zc, sets[ps], acc);
        r.z0 = acc;
        r.z1 = 0.0f;
    } else {
        const uint4 zc = make_uint4(0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u);
        float lo = 0.0f, hi = 0.0f;
        for (int ps = 0; ps < npass; ++ps) slice_dot8(zc, zc, sets[ps], lo, hi);
        r.z0 = lo;
        r.z1 = hi;
    }
    return r;
}
// Partial row value of one lane: sum over its slice of (s q + b) v, with vp the slice's bf16
// pairs of v and ref its SliceRef.
template <int BITS>
__device__ __forceinline__ float slice_value(const SliceCodes<BITS> &sc, const uint32_t *vp, const SliceRef &ref) {
    const float sv = sc_scale(sc), bv = sc_bias(sc);
    if constexpr (BITS == 4) {
        const float acc = slice_dot4(sc.c0, vp, 0.0f);
        return sv * (acc - ref.z0) + fmaf(8.0f, sv, bv) * ref.sum;
    } else {
        float lo = 0.0f, hi = 0.0f;
        slice_dot8(sc.c0, sc.c1, vp, lo, hi);
        return sv * ((lo - ref.z0) + 16.0f * (hi - ref.z1)) + fmaf(128.0f, sv, bv) * ref.sum;
    }
}
// Same with v split into bf16 hi and lo pair sets (one chain over hi, then lo).
template <int BITS>
__device__ __forceinline__ float slice_value2(const SliceCodes<BITS> &sc, const uint32_t *vhi, const uint32_t *vlo,
                                              const SliceRef &ref) {
    const float sv = sc_scale(sc), bv = sc_bias(sc);
    if constexpr (BITS == 4) {
        float acc = slice_dot4(sc.c0, vhi, 0.0f);
        acc = slice_dot4(sc.c0, vlo, acc);
        return sv * (acc - ref.z0) + fmaf(8.0f, sv, bv) * ref.sum;
    } else {
        float lo = 0.0f, hi = 0.0f;
        slice_dot8(sc.c0, sc.c1, vhi, lo, hi);
        slice_dot8(sc.c0, sc.c1, vlo, lo, hi);
        return sv * ((lo - ref.z0) + 16.0f * (hi - ref.z1)) + fmaf(128.0f, sv, bv) * ref.sum;
    }
}

// An expert index used as an address: clamped into [0, E) so that the weights are never read out
// of bounds, whatever the selection produced (it always produces valid indices).
__device__ __forceinline__ size_t expert_at(int e, int E) {
    return (size_t)min((unsigned)e, (unsigned)(E - 1));
}

// Sum over aligned groups of n lanes (n a power of two <= 64, runtime).
__device__ __forceinline__ float seg_sum(float v, int n) {
    for (int o = n >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// ---- layer pointers --------------------------------------------------------------------------
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

// ---- LDS layout --------------------------------------------------------------------------------
// Pair tables are stored per 32-column slice with 4 dwords of padding (20 or 36 dwords per slice)
// so that lanes reading consecutive slices with 16-byte loads spread over the banks.
struct Lds {
    uint16_t *xb;   // [T][H] bf16 input of the layer
    uint32_t *xp;   // [T][H/32][20] bf16 pairs of x (16 used)
    SliceRef *xref; // [T][H/32] per-slice constants of x
    float *fbuf;    // gathered words / per-row results: max(H, K*I, T*Is, grid) floats
    uint32_t *hp;   // [max(K,T)][Imax/32][36] bf16 hi pairs (16), lo pairs (16), padding
    SliceRef *href; // [max(K,T)][Imax/32] per-slice constants of h (hi then lo)
    float *lg;      // [T][E+1]
    int *sidx;      // [T][K]
    float *sw;      // [T][K]
    float *gam;     // [T]
    float *rowv;    // [kRowv] row results of one gate|up batch
    float *part;    // [T][K+1][RB] down-projection rows of this workgroup (slot K = shared)
    float *red;     // [T * kMaxRR * kWaves] block-reduction scratch
    int *tks;       // [kWaves][32] top-k scratch, one slice per wave
};
constexpr int kRowv = kWaves * kMaxWL * 8;  // rows per wave-load <= 8 since H >= 256
constexpr int kMaxRR = 3;                   // router rows per workgroup: (E + 1) / grid <= 3
constexpr int kMaxQ = 1;                    // float4 of a router row per thread: H / 4 <= 512

__host__ __device__ inline size_t lds_offsets(int T, int H, int E, int K, int I, int Is, int RB, size_t *o) {
    const int Imax = I > Is ? I : Is;
    const int nh = K > T ? K : T;
    size_t fb = (size_t)H;
    if ((size_t)K * I > fb) fb = (size_t)K * I;
    if ((size_t)T * Is > fb) fb = (size_t)T * Is;
    if ((size_t)T * (K + 1) * RB > fb) fb = (size_t)T * (K + 1) * RB;
    if (fb < kMaxGrid) fb = kMaxGrid;
    size_t off = 0;
    const size_t sz[14] = {2 * (size_t)T * H,
                           4 * (size_t)T * (H / 32) * 20,
                           sizeof(SliceRef) * (size_t)T * (H / 32),
                           4 * fb,
                           4 * (size_t)nh * (Imax / 32) * 36,
                           sizeof(SliceRef) * (size_t)nh * (Imax / 32),
                           4 * (size_t)T * (E + 1),
                           4 * (size_t)T * K,
                           4 * (size_t)T * K,
                           4 * (size_t)T,
                           4 * (size_t)kRowv,
                           4 * (size_t)T * (K + 1) * RB,
                           4 * (size_t)T * kMaxRR * kWaves,
                           4 * (size_t)kWaves * 32};
    for (int i = 0; i < 14; ++i) {
        o[i] = off;
        off = align_up(off + sz[i], 16);
    }
    return off;
}

__device__ __forceinline__ Lds carve(const DecodeParams &p, char *smem) {
    size_t o[14];
    lds_offsets(p.T, p.H, p.E, p.K, p.I, p.Is, p.rows_per_wg, o);
    Lds s;
    s.xb = reinterpret_cast<uint16_t *>(smem + o[0]);
    s.xp = reinterpret_cast<uint32_t *>(smem + o[1]);
    s.xref = reinterpret_cast<SliceRef *>(smem + o[2]);
    s.fbuf = reinterpret_cast<float *>(smem + o[3]);
    s.hp = reinterpret_cast<uint32_t *>(smem + o[4]);
    s.href = reinterpret_cast<SliceRef *>(smem + o[5]);
    s.lg = reinterpret_cast<float *>(smem + o[6]);
    s.sidx = reinterpret_cast<int *>(smem + o[7]);
    s.sw = reinterpret_cast<float *>(smem + o[8]);
    s.gam = reinterpret_cast<float *>(smem + o[9]);
    s.rowv = reinterpret_cast<float *>(smem + o[10]);
    s.part = reinterpret_cast<float *>(smem + o[11]);
    s.red = reinterpret_cast<float *>(smem + o[12]);
    s.tks = reinterpret_cast<int *>(smem + o[13]);
    return s;
}

// Build the bf16 pair table and per-slice sums of x (from s.xb) for all T tokens.
template <int BITS>
__device__ void build_x_pairs(const DecodeParams &p, const Lds &s) {
    const int H = p.H, T = p.T, nsl = H / 32;
    for (int i = threadIdx.x; i < T * nsl * 16; i += blockDim.x) {
        const int t = i / (nsl * 16), r = i - t * nsl * 16, sl = r >> 4, q = r & 15;
        const uint16_t *xr = s.xb + t * H + sl * 32;
        const uint32_t a = xr[pair_col_a<BITS>(q)], c = xr[pair_col_b<BITS>(q)];
        s.xp[(t * nsl + sl) * 20 + q] = a | (c << 16);
    }
    lds_barrier();
    for (int i = threadIdx.x; i < T * nsl; i += blockDim.x) {
        uint32_t v[16];
        for (int q = 0; q < 16; ++q) v[q] = s.xp[i * 20 + q];
        s.xref[i] = slice_ref<BITS>(v, 1, v);
    }
    lds_barrier();
}

// Input of layer l into s.xb: x_in for l == 0 (or unchained), else the RMS glue of y_{l-1}:
// x = bf16_rne(y / sqrt(mean(y^2) + eps)). Every workgroup computes the same bits.
template <int BITS>
__device__ bool layer_input(const DecodeParams &p, int l, uint32_t ep, const Lds &s) {
    const int T = p.T, H = p.H;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (l == 0 || !p.chained) {
        for (int i = threadIdx.x; i < T * H; i += blockDim.x) s.xb[i] = p.x_in[i];
    } else {
        const uint64_t *ysrc = p.ll_y + (size_t)(l - 1) * T * H;
        for (int t = 0; t < T; ++t) {
            if (!ll_gather(ysrc + (size_t)t * H, H, ep, s.fbuf, p.ctrl, p.spin_limit)) return false;
            float ss = 0.0f;
            for (int h = threadIdx.x; h < H; h += blockDim.x) ss += s.fbuf[h] * s.fbuf[h];
            ss = wave_sum(ss);
            if (lane == 0) s.red[wave] = ss;
            lds_barrier();
            ss = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) ss += s.red[w];
            const float inv = 1.0f / sqrtf(ss / (float)H + p.eps);
            for (int h = threadIdx.x; h < H; h += blockDim.x) s.xb[t * H + h] = f32_to_bf16_rne(s.fbuf[h] * inv);
            lds_barrier();
        }
    }
    lds_barrier();
    if (p.x_all && blockIdx.x == 0)
        for (int i = threadIdx.x; i < T * H; i += blockDim.x) p.x_all[(size_t)l * T * H + i] = s.xb[i];
    build_x_pairs<BITS>(p, s);
    return true;
}

// Gate|up + SwiGLU for `npairs` row pairs. Pair i: gate row row_of(i, m) of matrix m, up row
// gate row + inter, token tok_of(i); h = silu(gate) * up goes to the word dst_of(i).
// Row slots 2i (gate) and 2i+1 (up) are processed rpw per wave-load, wave-loads round-robin over
// the waves, in batches of kWaves * kMaxWL wave-loads whose loads are all issued before any math:
// gu_load issues one batch's loads, gu_finish does its math and publishes its h.
struct GuPlan {
    int spr, rpw, nslots, nwl;
};
__device__ __forceinline__ GuPlan gu_plan(int H, int npairs) {
    GuPlan g;
    g.spr = H / 32;
    g.rpw = kWave / g.spr;
    g.nslots = 2 * npairs;
    g.nwl = (g.nslots + g.rpw - 1) / g.rpw;
    return g;
}
// A batch is kWaves * NK wave-loads; wave w takes wave-loads base + w + k * kWaves, k < NK.
template <int BITS, int NK, typename RowOf>
__device__ __forceinline__ void gu_load(const DecodeParams &p, const GuPlan &g, int base, int inter, RowOf row_of,
                                        SliceCodes<BITS> *sc) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int H = p.H, seg = lane / g.spr, sl = lane % g.spr;
    const size_t cpr = (size_t)H * BITS / 8;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const int wl = base + wave + k * kWaves;
        const int slot = wl * g.rpw + seg;
        if (wl < g.nwl && slot < g.nslots) {
            QMat m;
            const size_t row = row_of(slot >> 1, m) + (size_t)(slot & 1) * inter;
            load_slice<BITS>(sc[k], m.c + row * cpr, m.s + row * (H / 64), m.b + row * (H / 64), sl);
        }
    }
}
template <int BITS, int NK, typename TokOf, typename DstOf>
__device__ __forceinline__ void gu_finish(const DecodeParams &p, const Lds &s, const GuPlan &g, int base, int npairs,
                                          const SliceCodes<BITS> *sc, TokOf tok_of, DstOf dst_of, uint32_t ep) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int seg = lane / g.spr, sl = lane % g.spr;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const int wl = base + wave + k * kWaves;
        const int slot = wl * g.rpw + seg;
        if (wl < g.nwl) {
            float v = 0.0f;
            if (slot < g.nslots) {
                const int t = tok_of(slot >> 1);
                v = slice_value<BITS>(sc[k], s.xp + (t * g.spr + sl) * 20, s.xref[t * g.spr + sl]);
            }
            v = seg_sum(v, g.spr);
            if (sl == 0 && slot < g.nslots) s.rowv[slot - base * g.rpw] = v;
        }
    }
    lds_barrier();
    const int lo = base * g.rpw / 2;
    const int hi = min(npairs, (base + kWaves * NK) * g.rpw / 2);
    for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
        const float gv = s.rowv[2 * i - base * g.rpw], uv = s.rowv[2 * i + 1 - base * g.rpw];
        ll_put(dst_of(i), silu(gv) * uv, ep);
    }
    lds_barrier();
}
// Batches from `first` on (the batches before it were handled by the caller).
template <int BITS, typename RowOf, typename TokOf, typename DstOf>
__device__ void gate_up_pairs(const DecodeParams &p, const Lds &s, int npairs, int inter, RowOf row_of,
                              TokOf tok_of, DstOf dst_of, uint32_t ep, int first = 0) {
    const GuPlan g = gu_plan(p.H, npairs);
    for (int base = first; base < g.nwl; base += kWaves * kMaxWL) {
        SliceCodes<BITS> sc[kMaxWL];
        gu_load<BITS, kMaxWL>(p, g, base, inter, row_of, sc);
        gu_finish<BITS, kMaxWL>(p, s, g, base, npairs, sc, tok_of, dst_of, ep);
    }
}

// Gather `nvec` h vectors of length len (vector v from src_of(v)) into the LDS pair table:
// hp[v][slice][0..15] = bf16 hi pairs, [16..31] = bf16 lo pairs; href[v][slice] its constants.
// src_of(v) must be contiguous in v with stride len (one gather covers them all).
template <int BITS>
__device__ bool stage_h(const DecodeParams &p, const Lds &s, const uint64_t *src, int nvec, int len, uint32_t ep) {
    const int nsl = len / 32, n = nvec * len;
    for (int c0 = 0; c0 < n; c0 += kGatherWords * kDecodeThreads)
        if (!ll_gather(src + c0, min(n - c0, kGatherWords * kDecodeThreads), ep, s.fbuf + c0, p.ctrl, p.spin_limit))
            return false;
    for (int i = threadIdx.x; i < nvec * nsl * 16; i += blockDim.x) {
        const int vs = i >> 4, q = i & 15;  // vs = v * nsl + slice
        const float a = s.fbuf[vs * 32 + pair_col_a<BITS>(q)], c = s.fbuf[vs * 32 + pair_col_b<BITS>(q)];
        const uint16_t ah = f32_to_bf16_rne(a), ch = f32_to_bf16_rne(c);
        const uint16_t al = f32_to_bf16_rne(a - bf16_to_f32(ah)), cl = f32_to_bf16_rne(c - bf16_to_f32(ch));
        uint32_t *dst = s.hp + (size_t)vs * 36;
        dst[q] = (uint32_t)ah | ((uint32_t)ch << 16);
        dst[16 + q] = (uint32_t)al | ((uint32_t)cl << 16);
    }
    lds_barrier();
    for (int i = threadIdx.x; i < nvec * nsl; i += blockDim.x) {
        uint32_t hi[16], lo[16];
        for (int q = 0; q < 16; ++q) {
            hi[q] = s.hp[(size_t)i * 36 + q];
            lo[q] = s.hp[(size_t)i * 36 + 16 + q];
        }
        s.href[i] = slice_ref<BITS>(hi, 2, lo);
    }
    lds_barrier();
    return true;
}

// Down projection of `nvec` h vectors (staged in s.hp) for this workgroup's rows r0..r0+nr-1:
// out[v * RB + rl] = W_v[r0 + rl] . h_v. A wave-load puts vectors g*rpw .. g*rpw+rpw-1 (one per
// lane segment) at one row rl; wave-load wl covers g = wl / nr, rl = wl % nr, and wave w takes the
// contiguous wave-loads [w*nwl/8, (w+1)*nwl/8), so a lane's h slice changes rarely.
struct DownPlan {
    int spr, rpw, nwl, wl0, nwl_w;
};
__device__ __forceinline__ DownPlan down_plan(int len, int nvec, int nr) {
    DownPlan d;
    const int wave = threadIdx.x / kWave;
    d.spr = len / 32;
    d.rpw = kWave / d.spr;
    d.nwl = ((nvec + d.rpw - 1) / d.rpw) * nr;
    d.wl0 = (int)((long long)wave * d.nwl / kWaves);
    d.nwl_w = (int)((long long)(wave + 1) * d.nwl / kWaves) - d.wl0;
    return d;
}
template <int BITS, typename MatOf>
__device__ __forceinline__ void down_load(const DownPlan &d, int len, int r0, int nr, int nvec, MatOf mat_of,
                                          SliceCodes<BITS> *sc, int first, int count) {
    const int lane = threadIdx.x % kWave;
    const int seg = lane / d.spr, sl = lane % d.spr;
    const size_t cpr = (size_t)len * BITS / 8;
#pragma unroll
    for (int k = 0; k < kDnWL; ++k) {
        if (k < count) {
            const int wl = d.wl0 + first + k;
            const int g = wl / nr, rl = wl - g * nr;
            const int v = g * d.rpw + seg;
            if (v < nvec) {
                const QMat m = mat_of(v);
                const size_t row = (size_t)(r0 + rl);
                load_slice<BITS>(sc[k], m.c + row * cpr, m.s + row * (len / 64), m.b + row * (len / 64), sl);
            }
        }
    }
}
template <int BITS>
__device__ __forceinline__ void down_compute(const DownPlan &d, const Lds &s, int len, int nr, int nvec,
                                             const SliceCodes<BITS> *sc, int first, int count, float *out, int RB) {
    const int lane = threadIdx.x % kWave;
    const int seg = lane / d.spr, sl = lane % d.spr;
    const int nsl = len / 32;
    int cur = -1;
    uint32_t hv[32];
    SliceRef hr;
#pragma unroll
    for (int k = 0; k < kDnWL; ++k) {
        if (k < count) {
            const int wl = d.wl0 + first + k;
            const int g = wl / nr, rl = wl - g * nr;
            const int v = g * d.rpw + seg;
            float val = 0.0f;
            if (v < nvec) {
                if (v != cur) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(s.hp + ((size_t)v * nsl + sl) * 36);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const uint4 u = src[q];
                        hv[4 * q] = u.x;
                        hv[4 * q + 1] = u.y;
                        hv[4 * q + 2] = u.z;
                        hv[4 * q + 3] = u.w;
                    }
                    hr = s.href[v * nsl + sl];
                    cur = v;
                }
                val = slice_value2<BITS>(sc[k], hv, hv + 16, hr);
            }
            val = seg_sum(val, d.spr);
            if (sl == 0 && v < nvec) out[v * RB + rl] = val;
        }
    }
}

template <int BITS>
__global__ void __launch_bounds__(kDecodeThreads, 1) decode_kernel(DecodeParams p) {
    extern __shared__ __align__(16) char smem[];
    const Lds s = carve(p, smem);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int nb = gridDim.x, b = blockIdx.x;
    const int T = p.T, H = p.H, E = p.E, K = p.K, I = p.I, Is = p.Is, RB = p.rows_per_wg;
    if (p.ctrl[0] != 0) return;  // sticky failure of an earlier call: do nothing
    uint32_t ep = static_cast<uint32_t>(p.ctrl[1]) + 1u;
    if (ep == 0) ep = 1;
    if (tid == 0) ll_put(p.ll_start + b, 0.0f, ep);
    const int r0 = b * RB;
    const int nr = r0 >= H ? 0 : min(RB, H - r0);
    const int nlg = E + (Is ? 1 : 0);  // logit words per token (column E = shared gate)

    for (int l = 0; l < p.L; ++l) {
        const LayerPtrs L = layer_ptrs(p, l);
        uint64_t *ll_lg = p.ll_logits + (size_t)l * T * (E + 1);
        uint64_t *ll_h = p.ll_h + (size_t)l * T * K * I;
        uint64_t *ll_hs = p.ll_hs + (size_t)l * T * (Is > 0 ? Is : 1);
        uint64_t *ll_y = p.ll_y + (size_t)l * T * H;

        // ---- R: the router rows e = b (mod nb) and the shared-gate row E, and the shared expert's
        // gate|up and down rows of this workgroup: none depends on the layer input, so their loads
        // are issued before the input is awaited.
        float4 rv[kMaxRR];
        const int nq = H / 4;
#pragma unroll
        for (int r = 0; r < kMaxRR; ++r) {
            const int e = b + r * nb;
            const float *row = e < E ? L.router + (size_t)e * H : (e == E && Is ? L.sgate : nullptr);
            rv[r] = (row && tid < nq) ? reinterpret_cast<const float4 *>(row)[tid] : make_float4(0, 0, 0, 0);
        }
        const int nps = (Is && b < Is) ? (Is - 1 - b) / nb + 1 : 0;  // shared pairs j = b (mod nb)
        auto sh_row = [&](int i, QMat &m) -> size_t { m = L.s13; return (size_t)(b + (i / T) * nb); };
        const GuPlan sg = gu_plan(H, nps * T);
        SliceCodes<BITS> shsc[kShWL];
        if (nps) gu_load<BITS, kShWL>(p, sg, 0, Is, sh_row, shsc);
        const DownPlan sp = down_plan(Is > 0 ? Is : 64, T, nr);
        SliceCodes<BITS> ssc[kDnWL];
        const int spre = min(kDnWL, sp.nwl_w);
        if (Is && nr > 0) down_load<BITS>(sp, Is, r0, nr, T, [&](int) { return L.s2; }, ssc, 0, spre);

        if (!layer_input<BITS>(p, l, ep, s)) return;
        for (int t = 0; t < T; ++t) {
            float xv[4] = {0, 0, 0, 0};
            if (tid < nq) {
                const uint16_t *xr = s.xb + t * H + 4 * tid;
                xv[0] = bf16_to_f32(xr[0]); xv[1] = bf16_to_f32(xr[1]);
                xv[2] = bf16_to_f32(xr[2]); xv[3] = bf16_to_f32(xr[3]);
            }
#pragma unroll
            for (int r = 0; r < kMaxRR; ++r) {
                float acc = rv[r].x * xv[0] + rv[r].y * xv[1] + rv[r].z * xv[2] + rv[r].w * xv[3];
                acc = wave_sum(acc);
                if (lane == 0) s.red[(t * kMaxRR + r) * kWaves + wave] = acc;
            }
        }
        lds_barrier();
        if (tid < T * kMaxRR) {
            const int t = tid / kMaxRR, r = tid - t * kMaxRR, e = b + r * nb;
            if (e < nlg) {
                float tot = 0.0f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) tot += s.red[tid * kWaves + w];
                if (e < E && L.rbias) tot += L.rbias[e];
                ll_put(ll_lg + (size_t)t * (E + 1) + e, tot, ep);
            }
        }
        // shared expert gate|up for pairs j = b (mod nb), every token
        if (nps) {
            auto sh_tok = [&](int i) { return i % T; };
            auto sh_dst = [&](int i) { return ll_hs + (size_t)(i % T) * Is + (b + (i / T) * nb); };
            gu_finish<BITS, kShWL>(p, s, sg, 0, nps * T, shsc, sh_tok, sh_dst, ep);
            gate_up_pairs<BITS>(p, s, nps * T, Is, sh_row, sh_tok, sh_dst, ep, kWaves * kShWL);
        }

        // ---- G: routing, identical in every workgroup (one wave per token)
        for (int t = 0; t < T; ++t)
            if (!ll_gather(ll_lg + (size_t)t * (E + 1), nlg, ep, s.lg + t * (E + 1), p.ctrl, p.spin_limit)) return;
        if (wave < T) wave_topk(s.lg + wave * (E + 1), E, K, s.sidx + wave * K, s.sw + wave * K, s.tks + wave * 32);
        if (tid < T) s.gam[tid] = Is ? 1.0f / (1.0f + expf(-s.lg[tid * (E + 1) + E])) : 0.0f;
        lds_barrier();
        if (b == 0) {
            const size_t base = (size_t)l * T;
            if (p.idx_all)
                for (int i = tid; i < T * K; i += blockDim.x) p.idx_all[base * K + i] = s.sidx[i];
            if (p.w_all)
                for (int i = tid; i < T * K; i += blockDim.x) p.w_all[base * K + i] = s.sw[i];
            if (p.logits_all)
                for (int i = tid; i < T * E; i += blockDim.x)
                    p.logits_all[base * E + i] = s.lg[(i / E) * (E + 1) + i % E];
        }

        // routed down rows of token 0: their loads go out now, with the gate|up loads below
        auto routed_mat = [&](int t) {
            return [&, t](int k) -> QMat {
                const size_t e = expert_at(s.sidx[t * K + k], E);
                const size_t oc = e * H * ((size_t)I * BITS / 8), os = e * H * (I / 64);
                return QMat{L.w2.c + oc, L.w2.s + os, L.w2.b + os};
            };
        };
        const DownPlan dp = down_plan(I, K, nr);
        SliceCodes<BITS> dsc[kDnWL];
        const int pre = min(kDnWL, dp.nwl_w);
        if (nr > 0) down_load<BITS>(dp, I, r0, nr, K, routed_mat(0), dsc, 0, pre);

        // routed gate|up + SwiGLU: this workgroup's share of the flattened (token, slot, j) pairs
        {
            const long long total = (long long)T * K * I;
            const int p0 = (int)(total * b / nb), p1 = (int)(total * (b + 1) / nb);
            gate_up_pairs<BITS>(
                p, s, p1 - p0, I,
                [&](int i, QMat &m) -> size_t {
                    const int P = p0 + i, tk = P / I, j = P - tk * I;
                    m = L.w13;
                    return expert_at(s.sidx[tk], E) * 2 * I + j;
                },
                [&](int i) { return (p0 + i) / (K * I); },
                [&](int i) { return ll_h + (size_t)(p0 + i); }, ep);
        }

        // shared expert down for this workgroup's rows, every token -> part[t][K][rl]
        if (Is && nr > 0) {
            if (!stage_h<BITS>(p, s, ll_hs, T, Is, ep)) return;
            for (int c0 = 0; c0 < sp.nwl_w; c0 += kDnWL) {
                const int cn = min(kDnWL, sp.nwl_w - c0);
                if (c0 > 0) down_load<BITS>(sp, Is, r0, nr, T, [&](int) { return L.s2; }, ssc, c0, cn);
                down_compute<BITS>(sp, s, Is, nr, T, ssc, c0, cn, s.fbuf, RB);
            }
            lds_barrier();
            for (int i = tid; i < T * nr; i += blockDim.x) {
                const int t = i / nr, rl = i - t * nr;
                s.part[(t * (K + 1) + K) * RB + rl] = s.fbuf[t * RB + rl];
            }
            lds_barrier();
        }

        // ---- D: routed down projections of this workgroup's rows, token by token, and the combine
        for (int t = 0; t < T; ++t) {
            if (!stage_h<BITS>(p, s, ll_h + (size_t)t * K * I, K, I, ep)) return;
            if (nr > 0) {
                for (int c0 = 0; c0 < dp.nwl_w; c0 += kDnWL) {
                    const int cn = min(kDnWL, dp.nwl_w - c0);
                    if (t > 0 || c0 > 0) down_load<BITS>(dp, I, r0, nr, K, routed_mat(t), dsc, c0, cn);
                    down_compute<BITS>(dp, s, I, nr, K, dsc, c0, cn, s.part + t * (K + 1) * RB, RB);
                }
            }
            lds_barrier();
        }
        for (int i = tid; i < T * nr; i += blockDim.x) {
            const int t = i / nr, rl = i - t * nr;
            const float *pt = s.part + t * (K + 1) * RB;
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) acc += s.sw[t * K + k] * pt[k * RB + rl];
            if (Is) acc += s.gam[t] * pt[K * RB + rl];
            const size_t o = (size_t)t * H + r0 + rl;
            if (l + 1 < p.L && p.chained) ll_put(ll_y + o, acc, ep);
            if (l == p.L - 1) p.y_out[o] = acc;
            if (p.y_all) p.y_all[(size_t)l * T * H + o] = acc;
        }
        lds_barrier();
    }
    // the next call may advance the epoch once every workgroup has read it
    if (b == 0) {
        if (!ll_gather(p.ll_start, nb, ep, s.fbuf, p.ctrl, p.spin_limit)) return;
        if (tid == 0) p.ctrl[1] = static_cast<int>(ep);
    }
}

size_t decode_lds_bytes(int T, int H, int E, int K, int I, int Is, int bits, int rows_per_wg) {
    (void)bits;
    size_t o[14];
    return lds_offsets(T, H, E, K, I, Is, rows_per_wg, o);
}

template <int BITS>
static hipError_t launch_bits(const DecodeParams &p, int grid, hipStream_t stream) {
    const size_t lds = decode_lds_bytes(p.T, p.H, p.E, p.K, p.I, p.Is, p.bits, p.rows_per_wg);
    const void *fn = reinterpret_cast<const void *>(&decode_kernel<BITS>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    DecodeParams arg = p;
    void *args[] = {&arg};
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kDecodeThreads), args, (unsigned)lds, stream);
}

hipError_t launch_decode(const DecodeParams &p, int grid, hipStream_t stream) {
    return p.bits == 4 ? launch_bits<4>(p, grid, stream) : launch_bits<8>(p, grid, stream);
}

}  // namespace moe
