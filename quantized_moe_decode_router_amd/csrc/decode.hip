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
// Per layer and workgroup b (grid = number of CUs):
//   input   x of every token: x_in, or the RMS glue of all of y_{l-1} (chained stacks)
//   R       router rows e = b (mod grid) [row E = the shared-expert gate], staged in LDS, against
//           x -> logit words; x turned into int8 limbs
//   G       all logits -> top-k (identical in every workgroup; one wave per token) beside the
//           shared expert's gate|up pairs j = b (mod grid) on the other waves -> this workgroup's
//           share of the flattened (token, slot, j) routed gate|up pairs, DMA'd into LDS -> h words
//   D       per token: all K routed h vectors and the shared h -> the workgroup's H/grid rows of
//           every routed down projection (rows DMA'd into LDS while h is in flight) and of the
//           shared one -> fixed-order combine (k = 0..K-1, then the shared expert) -> y
// Weights reach LDS through the LDS-DMA form of the global load (global_load_lds_dwordx4 /
// _dword), issued while the workgroup waits for an exchange, so they cost neither registers nor
// time on the chain.
//
// Every dot product with quantised rows runs on v_mfma_i32_16x16x64_i8 in exact integer
// arithmetic: the activations (x, or h) of each 64-column quantisation group are held as three
// int8 limbs of a 24-bit fixed-point value, the codes enter as signed bytes relative to the zero
// point (see build_limbs). All address arithmetic into the weights is 64-bit.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

constexpr int kWaves = kDecodeThreads / kWave;  // 8
// Block-strided loops step by kDecodeThreads, the block size of every launch: blockDim.x would be a
// scalar load from the kernel-argument segment inside the layer loop.
constexpr int kMaxGather = 16;                  // exchange words one thread waits for at once

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Global-memory view of a pointer. The parameter block is re-read word by word inside the layer
// loop (see fresh_params), which hides from the compiler that its pointers are global; accesses
// through G() stay global loads and stores instead of flat ones (a flat access counts against the
// LDS wait counter too, which would couple every LDS wait to outstanding global loads).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *G(T *p) {
    return (__attribute__((address_space(1))) T *)p;
}

// ---- phase timer (compile-time option MOE_PHASE_TIMER) -------------------------------------------
// Wave 0 of every workgroup stamps the 100 MHz real-time counter at each of kPhaseMarks marks of a
// layer into the workspace (p.phase[l][block][mark]); bench.py --phases reads and summarises them.
// In the default build the marks compile to nothing.
enum PhaseMark {
    kMarkLayer = 0,      // top of the layer
    kMarkInput,          // x of every token in LDS (y of the previous layer gathered, RMS glue)
    kMarkRouterRows,     // this layer's router and shared rows landed
    kMarkLogitsPut,      // this workgroup's logits published
    kMarkXLimbs,         // x as limbs
    kMarkLogitsGot,      // every logit gathered
    kMarkTopk,           // expert selection done (wave 0: token 0)
    kMarkSharedGu,       // shared gate|up done, routing published to the workgroup
    kMarkRoutedIssued,   // first chunk of routed gate|up rows issued
    kMarkRoutedLanded,   // first chunk landed
    kMarkGuUnits,        // last chunk: wave 0's gate|up units done
    kMarkGuBarrier,      // last chunk: every wave's units done
    kMarkGuPut,          // last chunk: SwiGLU of the pairs and their h words stored
    kMarkRoutedDone,     // every routed gate|up pair computed, h published
    kMarkDownIssued,     // routed down rows (and next shared gate|up rows) issued
    kMarkHPolled,        // every h word of token 0 current (before its limbs)
    kMarkHGot,           // every h of token 0 gathered, down rows landed
    kMarkDownUnits,      // token T-1: wave 0's down tiles done
    kMarkDownDone,       // down projections of every token done
    kMarkYPut,           // y published
    kMarkLayerEnd        // next layer's shared down rows issued
};
#ifdef MOE_PHASE_TIMER
__device__ __forceinline__ void phase_mark(uint64_t *ph, int l, int m) {
    if (threadIdx.x == 0 && ph) {
        const uint64_t t = __builtin_amdgcn_s_memrealtime();
        ((__attribute__((address_space(1))) uint64_t *)ph)[((size_t)l * gridDim.x + blockIdx.x) * kPhaseMarks + m] = t;
    }
}
#else
__device__ __forceinline__ void phase_mark(uint64_t *, int, int) {}
#endif

// ---- exchange words ---------------------------------------------------------------------------
__device__ __forceinline__ void ll_put(uint64_t *p, float v, uint32_t ep) {
    const uint64_t w = (static_cast<uint64_t>(ep) << 32) | __float_as_uint(v);
    __hip_atomic_store(G(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ll_get(const uint64_t *p) {
    return __hip_atomic_load(G(const_cast<uint64_t *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int status_of(const int *ctrl) {
    return __hip_atomic_load(G(const_cast<int *>(ctrl)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fail(int *ctrl) {
    __hip_atomic_store(G(ctrl), 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until words src[0..n) carry epoch ep and copy their values into LDS (word i to dst[i]).
// Called by the whole workgroup; n may be any size (passes of kMaxGather words per thread). Thread
// tid holds words tid + k * kDecodeThreads (slot k) of a pass in registers; a wave re-reads all its slots
// (every load of a poll in flight together) until one poll finds all of them current -- a current
// word stays current, so re-reading words that were already there is harmless. The poll loop is
// instantiated for the number of slots the wave has (rounded up to 1, 4, 12 or 16), so it stays short
// and its period -- the delay between a word's arrival and its detection -- with it. The values
// go to LDS once at the end. Returns false on timeout or when any workgroup has failed.
template <int NW>
__device__ __forceinline__ bool poll_slots(const uint64_t *src, int m, uint32_t ep, uint64_t (&w)[NW], int *ctrl,
                                           unsigned spin) {
    const int tid = threadIdx.x;
    for (unsigned it = 0;; ++it) {
        // lanes past m read word m - 1 (it becomes current like any other), which keeps the loads
        // unpredicated
#pragma unroll
        for (int k = 0; k < NW; ++k) w[k] = ll_get(src + min(tid + k * kDecodeThreads, m - 1));
        bool done = true;
#pragma unroll
        for (int k = 0; k < NW; ++k) done &= static_cast<uint32_t>(w[k] >> 32) == ep;
        if (__ballot(!done) == 0ull) break;
        if (it >= spin) { fail(ctrl); return false; }
        if ((it & 31u) == 31u && status_of(ctrl) != 0) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}
template <int NW>
__device__ __forceinline__ bool gather_slots(const uint64_t *src, int m, uint32_t ep, float *dst, int *ctrl,
                                             unsigned spin) {
    const int tid = threadIdx.x;
    uint64_t w[NW];
    if (!poll_slots<NW>(src, m, ep, w, ctrl, spin)) return false;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        const int i = tid + k * kDecodeThreads;
        if (i < m) dst[i] = __uint_as_float(static_cast<uint32_t>(w[k]));
    }
    return true;
}
// Workgroup-wide AND of every thread's ok through LDS (slots written, read, then released again).
__device__ __forceinline__ bool all_ok(bool ok) {
    __shared__ int vote[kWaves];
    const unsigned long long bad = __ballot(!ok);
    if ((threadIdx.x % kWave) == 0) vote[threadIdx.x / kWave] = bad ? 0 : 1;
    lds_barrier();
    int all = 1;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) all &= vote[w];
    lds_barrier();
    return all != 0;
}
__device__ bool ll_gather(const uint64_t *src, int n, uint32_t ep, float *dst, int *ctrl, unsigned spin) {
    constexpr int kPass = kMaxGather * kDecodeThreads;
    const int wbase = __builtin_amdgcn_readfirstlane(threadIdx.x & ~(kWave - 1));
    bool ok = true;
    for (int base = 0; base < n && ok; base += kPass) {
        const int m = min(n - base, kPass);
        // slots of this wave: k < kw (the wave's first word of slot k is below m); wave-uniform
        const int kw = m > wbase ? (m - wbase + kDecodeThreads - 1) / kDecodeThreads : 0;
        if (kw == 0) continue;
        if (kw <= 1) ok = gather_slots<1>(src + base, m, ep, dst + base, ctrl, spin);
        else if (kw <= 4) ok = gather_slots<4>(src + base, m, ep, dst + base, ctrl, spin);
        else if (kw <= 12) ok = gather_slots<12>(src + base, m, ep, dst + base, ctrl, spin);
        else ok = gather_slots<kMaxGather>(src + base, m, ep, dst + base, ctrl, spin);
    }
    return all_ok(ok);
}

// ---- LDS DMA ------------------------------------------------------------------------------------
// The LDS-DMA form of the global load writes lane l's 16 (or 4) bytes to LDS address
// M0 + 16 l (4 l), M0 wave-uniform. It is issued from inline assembly so that the compiler does
// not treat it as an LDS store it must wait for at every barrier; every consumer therefore waits
// explicitly (dma_wait: all of this wave's vector-memory loads, then a workgroup barrier). The
// issue itself carries no memory clobber, so that the LDS reads computing later DMAs' addresses
// can be issued ahead of earlier DMAs; the waits (with a memory clobber) and the barriers keep
// every read of the destination after its DMA lands and every earlier read of it before the DMA.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    // a generic pointer into LDS converted to its 32-bit LDS address (address space 3)
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)p));
}
__device__ __forceinline__ void dma16(const void *g, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "m0");
}
__device__ __forceinline__ void dma4(const void *g, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "m0");
}
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most n of this wave's vector-memory loads are outstanding (n wave-uniform). Loads
// complete in issue order, so this waits for everything issued before the last n loads; values
// of n above 15 wait for more than needed (still correct).
__device__ __forceinline__ void dma_wait_but(int n) {
    switch (n < 0 ? 0 : (n > 15 ? 15 : n)) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
        case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    }
}

// Waves [first, first + n) of the workgroup that issue a DMA.
struct DmaWaves {
    int first, n;
};
constexpr DmaWaves kAllWaves = {0, kWaves};
// Block permutation of staged rows: LDS chunk c (16 bytes) of row r receives source chunk
// c ^ ((r & mask) << shift), i.e. the 2^shift-chunk blocks of a row are XOR-permuted by the row
// index, so a column block read across consecutive rows spreads over the LDS banks.
struct Swz {
    int mask, shift;
};
constexpr Swz kNoSwz = {0, 0};
// Copy n rows of `bytes` bytes each (a power of two, a multiple of U = 16 or 4; src_of(r) aligned
// to U) into LDS at dst + r * bytes. Unit u = r * (bytes / U) + c is lane u % 64 of instruction
// u / 64; wave dw.first + w issues instructions w, w + dw.n, ... (swz only with U = 16).
template <int U, typename SrcOf>
__device__ __forceinline__ void dma_rows(int n, int bytes, SrcOf src_of, char *dst, Swz swz = kNoSwz,
                                         DmaWaves dw = kAllWaves) {
    const int sh = __builtin_ctz(static_cast<unsigned>(bytes / U)), total = n << sh;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave - dw.first;
    if (wave < 0 || wave >= dw.n) return;
    for (int i = wave; i * kWave < total; i += dw.n) {
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(dst + (size_t)i * kWave * U));
        const int u = i * kWave + lane;
        if (u < total) {
            const int r = u >> sh, c = (u & ((1 << sh) - 1)) ^ ((r & swz.mask) << swz.shift);
            const char *g = src_of(r) + (size_t)c * U;
            if constexpr (U == 16) dma16(g, m0);
            else dma4(g, m0);
        }
    }
}

// DMA instructions this wave issues in dma_rows for `total` units (instruction i goes to wave i % 8).
__device__ __forceinline__ int dma_count(int total) {
    const int wave = threadIdx.x / kWave, n = (total + kWave - 1) / kWave;
    return n > wave ? (n - wave + kWaves - 1) / kWaves : 0;
}

// Rows of a quantised matrix staged in LDS: codes [n][cb], scales [n][sb], biases [n][sb].
struct Rows {
    char *c, *s, *b;
    int cb, sb;
};
__device__ __forceinline__ Rows rows_at(char *base, int n, int cols, int bits) {
    const int cb = cols * bits / 8, sb = cols / 32;
    return Rows{base, base + (size_t)n * cb, base + (size_t)n * (cb + sb), cb, sb};
}
// DMA instructions this wave issues in dma_qrows for n rows of `cols` columns.
__device__ __forceinline__ int dma_qrows_count(int n, int cols, int bits) {
    return dma_count(n * (cols * bits / 8) / 16) + 2 * dma_count(n * (cols / 32) / 4);
}
// Stage n rows; row r of the matrix family q is matrix row row_of(r) (64-bit), cols columns; swz
// permutes the code blocks as in dma_rows (scales and biases are never permuted).
template <typename RowOf>
__device__ __forceinline__ void dma_qrows(const QMat &q, int cols, int bits, int n, RowOf row_of, const Rows &dst,
                                          Swz swz = kNoSwz) {
    const size_t cb = (size_t)cols * bits / 8, gpr = cols / 64;
    dma_rows<16>(n, dst.cb, [&](int r) { return reinterpret_cast<const char *>(q.c + row_of(r) * cb); }, dst.c, swz);
    dma_rows<4>(n, dst.sb, [&](int r) { return reinterpret_cast<const char *>(q.s + row_of(r) * gpr); }, dst.s);
    dma_rows<4>(n, dst.sb, [&](int r) { return reinterpret_cast<const char *>(q.b + row_of(r) * gpr); }, dst.b);
}

// Expert-table form of dma_qrows: row r is row x.row of the matrix piece whose codes start at
// address x.base (row_of(r) -> XRow); its scales and biases start off_s and off_b bytes further.
struct XRow {
    uint64_t base;
    uint32_t row;
};
template <typename RowOf>
__device__ __forceinline__ void dma_xrows(int cols, int bits, int n, RowOf row_of, uint32_t off_s, uint32_t off_b,
                                          const Rows &dst, Swz swz) {
    const uint32_t cb = (uint32_t)cols * bits / 8, sb = (uint32_t)cols / 32;
    dma_rows<16>(n, dst.cb, [&](int r) {
        const XRow x = row_of(r);
        return reinterpret_cast<const char *>(x.base + (uint64_t)x.row * cb);
    }, dst.c, swz);
    dma_rows<4>(n, dst.sb, [&](int r) {
        const XRow x = row_of(r);
        return reinterpret_cast<const char *>(x.base + off_s + (uint64_t)x.row * sb);
    }, dst.s);
    dma_rows<4>(n, dst.sb, [&](int r) {
        const XRow x = row_of(r);
        return reinterpret_cast<const char *>(x.base + off_b + (uint64_t)x.row * sb);
    }, dst.b);
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
// Inverse: pair slot and half (0 = low 16 bits) holding column c of a slice.
template <int BITS>
__device__ __forceinline__ void col_pair(int c, int &q, int &half) {
    if constexpr (BITS == 4) {
        q = 4 * (c >> 3) + (c & 3);
        half = (c >> 2) & 1;
    } else {
        q = 2 * (c >> 2) + (c & 1);
        half = (c >> 1) & 1;
    }
}

__device__ __forceinline__ size_t expert_at(int e, int E) {
    return (size_t)min((unsigned)e, (unsigned)(E - 1));
}

// ---- layer pointers --------------------------------------------------------------------------
struct LayerPtrs {
    const float *router, *rbias, *sgate;
    QMat w13, w2, s13, s2;
};

// Layer l's arrays: per-layer strides follow from the shape ([L]-stacked arrays, each layer one
// contiguous block).
__device__ __forceinline__ LayerPtrs layer_ptrs(const DecodeParams &p, int l) {
    const size_t H = p.H, E = p.E, I = p.I, Is = p.Is, bits = p.bits, L = l;
    LayerPtrs q;
    q.router = p.router + L * E * H;
    q.rbias = p.rbias ? p.rbias + L * E : nullptr;
    q.sgate = p.sgate ? p.sgate + L * H : nullptr;
    const size_t w13c = E * 2 * I * H * bits / 8, w13s = E * 2 * I * H / 64;
    const size_t w2c = E * H * I * bits / 8, w2s = E * H * I / 64;
    q.w13 = {p.w13.c + L * w13c, p.w13.s + L * w13s, p.w13.b + L * w13s};
    q.w2 = {p.w2.c + L * w2c, p.w2.s + L * w2s, p.w2.b + L * w2s};
    if (Is) {
        const size_t s13c = 2 * Is * H * bits / 8, s13s = 2 * Is * H / 64, s2c = H * Is * bits / 8, s2s = H * Is / 64;
        q.s13 = {p.s13.c + L * s13c, p.s13.s + L * s13s, p.s13.b + L * s13s};
        q.s2 = {p.s2.c + L * s2c, p.s2.s + L * s2s, p.s2.b + L * s2s};
    } else {
        q.s13 = {nullptr, nullptr, nullptr};
        q.s2 = {nullptr, nullptr, nullptr};
    }
    return q;
}

// The kernel's parameter block: copied once into LDS at kernel start (params_to_lds) and re-read
// from there at the top of every layer (fresh_params) through a pointer the compiler cannot prove
// invariant -- without it every field would be hoisted out of the layer loop and held in scalar
// registers for the whole kernel. Re-reading the kernel-argument segment itself inside the loop
// (a scalar load per field group) measured 1 us per layer slower on the 40-layer stack.
constexpr int kParamWords = sizeof(DecodeParams) / 4;
static_assert(sizeof(DecodeParams) % 4 == 0, "parameter block is copied in 32-bit words");
// the static LDS (this copy and the barrier votes) stays inside the 1 KiB the host keeps out of
// the dynamic LDS plan
static_assert(sizeof(DecodeParams) + 64 <= 1024, "static LDS");
__device__ __forceinline__ void params_to_lds(uint32_t *dst) {
    typedef const __attribute__((address_space(4))) uint32_t *KP;
    const KP src = reinterpret_cast<KP>(reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr()));
    for (int i = threadIdx.x; i < kParamWords; i += kDecodeThreads) dst[i] = src[i];
}
__device__ __forceinline__ DecodeParams fresh_params(const uint32_t *words) {
    uint32_t a = lds_addr(words);
    asm volatile("" : "+v"(a));
    const __attribute__((address_space(3))) uint32_t *src =
        reinterpret_cast<const __attribute__((address_space(3))) uint32_t *>(static_cast<uintptr_t>(a));
    DecodeParams out;
    uint32_t *dst = reinterpret_cast<uint32_t *>(&out);
    typedef const __attribute__((address_space(3))) u32x4_t *Q4;
    const Q4 src4 = reinterpret_cast<Q4>(src);
    u32x4_t q[(kParamWords + 3) / 4];
#pragma unroll
    for (int i = 0; i < (kParamWords + 3) / 4; ++i) q[i] = src4[i];  // every read in flight at once
#pragma unroll
    for (int i = 0; i < kParamWords; ++i) dst[i] = __builtin_amdgcn_readfirstlane(q[i / 4][i % 4]);
    return out;
}

// ---- LDS ---------------------------------------------------------------------------------------
// Pair tables are stored per 32-column slice with 4 dwords of padding (20 or 36 dwords per slice)
// so that lanes reading consecutive slices with 16-byte loads spread over the banks.
struct Lds {
    uint32_t *xp;    // [T][H/32][20] bf16 pairs of x (16 used)
    float *lg;       // [T][E+1] logits (column E = shared-gate logit)
    int *sidx;       // [T][K]
    float *sw;       // [T][K]
    float *gam;      // [T]
    float *rt;       // [nrr][H] router rows, chunk-transposed (see stage_router)
    char *sg;        // shared gate|up rows (pairs of this workgroup), staged
    char *sd;        // shared down rows of this workgroup, staged
    char *rd;        // routed down rows of this workgroup for one token, staged
    char *rg;        // routed gate|up rows of one chunk of this workgroup's pairs, staged
    uint32_t *hp;    // gathered h of one token (fp32); also the y gather buffer and gate|up partials
    float *part;     // [T][K+1][RB] down-projection rows of this workgroup (slot K = shared)
    float *red;      // [64] reduction scratch
    // activations as three int8 limbs per 64-column group (see build_limbs)
    int8_t *xq;      // [T][H/64][3][64]
    float2 *xsx;     // [T][H/64] (sum of the limb values, group scale)
    int8_t *hq;      // [(K*I + Is)/64][3][64] h of one token (routed vectors, then the shared one)
    float2 *hsx;     // [(K*I + Is)/64]
    uint64_t *xt;    // [2][E] expert-table mode: the table rows of layers l (buffer l & 1) and l + 1
};
__device__ __forceinline__ Lds carve(const DecodeParams &p, char *smem) {
    const DecodeLds &o = p.lds;
    Lds s;
    s.xp = reinterpret_cast<uint32_t *>(smem + o.xp);
    s.lg = reinterpret_cast<float *>(smem + o.lg);
    s.sidx = reinterpret_cast<int *>(smem + o.sidx);
    s.sw = reinterpret_cast<float *>(smem + o.sw);
    s.gam = reinterpret_cast<float *>(smem + o.gam);
    s.rt = reinterpret_cast<float *>(smem + o.rt);
    s.sg = smem + o.sg;
    s.sd = smem + o.sd;
    s.rd = smem + o.rd;
    s.rg = smem + o.rg;
    s.hp = reinterpret_cast<uint32_t *>(smem + o.hp);
    s.part = reinterpret_cast<float *>(smem + o.part);
    s.red = reinterpret_cast<float *>(smem + o.red);
    s.xq = reinterpret_cast<int8_t *>(smem + o.xq);
    s.xsx = reinterpret_cast<float2 *>(smem + o.xsx);
    s.hq = reinterpret_cast<int8_t *>(smem + o.hq);
    s.hsx = reinterpret_cast<float2 *>(smem + o.hsx);
    s.xt = reinterpret_cast<uint64_t *>(smem + o.xt);
    return s;
}

// What this workgroup b owns, computed once per call (integer divisions by the grid included):
//   rows r0 .. r0 + nr - 1 of y (nrm = div_magic(nr)); nrr router rows e = b + r * grid <= E (row E
//   only with a shared expert); nps shared pairs j = b + r * grid < Is; routed gate|up pairs
//   [q0, q1) of the T*K*I flattened (token, slot, j) pairs.
struct WgShare {
    int r0, nr, nrr, nps, q0, q1;
    uint32_t nrm;
};
__device__ __forceinline__ WgShare wg_share(const DecodeParams &p) {
    WgShare w;
    const int b = blockIdx.x, g = gridDim.x;
    w.r0 = b * p.rows_per_wg;
    w.nr = w.r0 >= p.H ? 0 : min(p.rows_per_wg, p.H - w.r0);
    w.nrm = div_magic(static_cast<uint32_t>(w.nr));
    const int n = p.E + (p.Is ? 1 : 0);
    w.nrr = b < n ? min(p.nrr, (n - 1 - b) / g + 1) : 0;
    w.nps = (p.Is && b < p.Is) ? min(p.nps, (p.Is - 1 - b) / g + 1) : 0;
    const unsigned long long total = (unsigned long long)p.T * p.K * p.I;
    w.q0 = (int)(total * b / g);
    w.q1 = (int)(total * (b + 1) / g);
    return w;
}

// ---- staging of the weights that do not depend on routing ----------------------------------------
// Router rows are stored chunk-transposed: 16-byte chunk k (k < 8) of 32-column slice sl of a row
// goes to chunk position k * (H/32) + sl, so that lane sl reading its k-th chunk is one
// conflict-free 16-byte LDS read per wave.
__device__ __forceinline__ void stage_router(const DecodeParams &p, int l, const Lds &s, const WgShare &w,
                                             DmaWaves dw = kAllWaves) {
    const LayerPtrs L = layer_ptrs(p, l);
    const int nr = w.nrr, H = p.H, nsl = H / 32, b = blockIdx.x, g = gridDim.x;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave - dw.first;
    if (wave < 0 || wave >= dw.n) return;
    const int cs = __builtin_ctz(static_cast<unsigned>(H / 4)), ss = __builtin_ctz(static_cast<unsigned>(nsl));
    const int total = nr << cs;  // 16-byte chunks
    for (int i = wave; i * kWave < total; i += dw.n) {
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(s.rt + (size_t)i * kWave * 4));
        const int u = i * kWave + lane;
        if (u < total) {
            const int r = u >> cs, pos = u & ((1 << cs) - 1);
            const int k = pos >> ss, sl = pos & (nsl - 1);
            const int e = b + r * g;
            const float *row = e < p.E ? L.router + (size_t)e * H : L.sgate;
            dma16(row + sl * 32 + k * 4, m0);
        }
    }
}
__device__ __forceinline__ Rows sg_rows(const DecodeParams &p, const Lds &s) {
    return rows_at(s.sg, 2 * p.nps, p.H, p.bits);
}
__device__ __forceinline__ Rows sd_rows(const DecodeParams &p, const Lds &s) {
    return rows_at(s.sd, p.rows_per_wg, p.Is, p.bits);
}
__device__ __forceinline__ Rows rd_rows(const DecodeParams &p, const Lds &s) {
    return rows_at(s.rd, p.K * p.rows_per_wg, p.I, p.bits);
}
// Block permutation of staged rows (see dma_rows): the MFMA dot products read one 64-column group
// (32 bytes of 4-bit, 64 of 8-bit codes) of 16 consecutive staged rows at a time.
__device__ __forceinline__ Swz mfma_swz(int bits, int cols) { return Swz{min(cols / 64, 8) - 1, bits == 4 ? 1 : 2}; }
// Shared gate|up rows of this workgroup's pairs: staged row 2r = gate row j, 2r+1 = up row Is + j,
// j = b + r * grid.
__device__ __forceinline__ void stage_shared_gu(const DecodeParams &p, int l, const Lds &s, const WgShare &w) {
    const int np = w.nps, b = blockIdx.x, g = gridDim.x, Is = p.Is;
    if (np == 0) return;
    const LayerPtrs L = layer_ptrs(p, l);
    dma_qrows(L.s13, p.H, p.bits, 2 * np,
              [&](int r) -> size_t { return (size_t)((r & 1) * Is + b + (r >> 1) * g); }, sg_rows(p, s),
              mfma_swz(p.bits, p.H));
}
__device__ __forceinline__ void stage_shared_down(const DecodeParams &p, int l, const Lds &s, int r0, int nr) {
    if (!p.Is || nr <= 0) return;
    const LayerPtrs L = layer_ptrs(p, l);
    dma_qrows(L.s2, p.Is, p.bits, nr, [&](int r) -> size_t { return (size_t)(r0 + r); }, sd_rows(p, s),
              mfma_swz(p.bits, p.Is));
}
// Routed down rows r0..r0+nr-1 of token t's K experts: staged row k * nr + rl.
template <bool XT>
__device__ __forceinline__ void stage_routed_down(const DecodeParams &p, int l, const Lds &s, int t, int r0,
                                                  int nr, uint32_t nrm) {
    if (nr <= 0) return;
    const int K = p.K, E = p.E;
    if constexpr (XT) {
        dma_xrows(p.I, p.bits, K * nr,
                  [&](int r) -> XRow {
                      const int k = div_by(r, nrm), rl = r - k * nr;
                      return XRow{(s.xt[(l & 1) * E + expert_at(s.sidx[t * K + k], E)] & ~1ull) + p.xo2c,
                                  (uint32_t)(r0 + rl)};
                  },
                  p.xo2s - p.xo2c, p.xo2b - p.xo2c, rd_rows(p, s), mfma_swz(p.bits, p.I));
        return;
    }
    const LayerPtrs L = layer_ptrs(p, l);
    const size_t H = p.H;
    dma_qrows(L.w2, p.I, p.bits, K * nr,
              [&](int r) -> size_t {
                  const int k = div_by(r, nrm), rl = r - k * nr;
                  return expert_at(s.sidx[t * K + k], E) * H + (size_t)(r0 + rl);
              },
              rd_rows(p, s), mfma_swz(p.bits, p.I));
}

// Expert-table mode with a landing buffer: rows staged in LDS from a block marked as outside HBM
// are stored to the landing block of their (layer, token, slot), un-permuting the code chunks
// (LDS chunk c of row r holds source chunk c ^ ((r & mask) << shift)); dst_of(r) is the row's
// destination or null. The host then admits such an expert from device memory.
template <typename DstOf>
__device__ __forceinline__ void wb_rows16(int n, int bytes, const char *lds, Swz swz, DstOf dst_of) {
    const int sh = __builtin_ctz(static_cast<unsigned>(bytes / 16)), total = n << sh;
    for (int u = threadIdx.x; u < total; u += kDecodeThreads) {
        const int r = u >> sh, g = u & ((1 << sh) - 1);
        char *d = dst_of(r);
        if (!d) continue;
        const int c = g ^ ((r & swz.mask) << swz.shift);
        *reinterpret_cast<uint4 *>(d + (size_t)g * 16) =
            *reinterpret_cast<const uint4 *>(lds + (size_t)r * bytes + (size_t)c * 16);
    }
}
template <typename DstOf>
__device__ __forceinline__ void wb_rows4(int n, int bytes, const char *lds, DstOf dst_of) {
    const int sh = __builtin_ctz(static_cast<unsigned>(bytes / 4)), total = n << sh;
    for (int u = threadIdx.x; u < total; u += kDecodeThreads) {
        const int r = u >> sh, g = u & ((1 << sh) - 1);
        char *d = dst_of(r);
        if (!d) continue;
        *reinterpret_cast<uint32_t *>(d + (size_t)g * 4) =
            *reinterpret_cast<const uint32_t *>(lds + (size_t)r * bytes + (size_t)g * 4);
    }
}
template <typename DstOf>
__device__ __forceinline__ void wb_qrows(int n, const Rows &src, Swz swz, uint32_t off_s, uint32_t off_b,
                                         DstOf row_dst) {
    wb_rows16(n, src.cb, src.c, swz, [&](int r) { return row_dst(r, 0u, src.cb); });
    wb_rows4(n, src.sb, src.s, [&](int r) { return row_dst(r, off_s, src.sb); });
    wb_rows4(n, src.sb, src.b, [&](int r) { return row_dst(r, off_b, src.sb); });
}

// Expert-table mode: layer l's row of the table (E block addresses) into LDS buffer l & 1.
__device__ __forceinline__ void stage_xtab(const DecodeParams &p, int l, const Lds &s, DmaWaves dw) {
    const int E = p.E;
    const uint64_t *src = p.xtab + (size_t)l * E;
    char *dst = reinterpret_cast<char *>(s.xt + (l & 1) * E);
    if ((E & 1) == 0)
        dma_rows<16>(E / 2, 16, [&](int r) { return reinterpret_cast<const char *>(src + 2 * r); }, dst, kNoSwz, dw);
    else
        dma_rows<4>(2 * E, 4, [&](int r) { return reinterpret_cast<const char *>(src) + 4 * r; }, dst, kNoSwz, dw);
}

// ---- activations as int8 limbs -------------------------------------------------------------------
// Dot products with quantised rows run on v_mfma_i32_16x16x64_i8 in exact integer arithmetic. A
// 64-column group of activations v is held as the integers X = rint(v / 2^e), e taken from the
// group's largest magnitude so that |X| <= 2^22, each split into three signed 8-bit limbs
// X = L0 2^16 + L1 2^8 + L2 (L1, L2 balanced in [-128, 127], |L0| <= 65). The codes enter as the
// signed bytes u (q - zp) relative to the zero point (4-bit: zp 8, u 16, the nibble at the top of
// its byte; 8-bit: zp 128, u 1), so C_j = sum u (q - zp) L_j is an exact integer (|C_j| <= 2^20) and
//   sum((s q + b) v) = (2^e / u) (s comb3(C_0, C_1, C_2) + (b + zp s) u comb3(sum L_0, sum L_1, sum L_2));
// the group entry keeps (u comb3 of the limb sums, 2^e / u). Codes all at the zero point with
// b = -zp s give exactly 0 (every C_j is 0 and b + zp s rounds to 0).
// Position p of a 64-byte limb row holds column limb_col(p): lane kb of an MFMA takes columns
// 16 kb .. 16 kb + 15 of the group, in the order code_bytes produces them -- 4-bit: nibbles of two
// code dwords, (0,2,4,6, 1,3,5,7, 8,10,12,14, 9,11,13,15) + 16 kb; 8-bit: natural order.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int BITS>
struct CodeFmt;
template <>
struct CodeFmt<4> {
    static constexpr int zp = 8, unit = 16, group_bytes = 32;
    typedef uint2 lane_t;  // one lane's codes of one group (16 columns)
};
template <>
struct CodeFmt<8> {
    static constexpr int zp = 128, unit = 1, group_bytes = 64;
    typedef uint4 lane_t;
};

template <int BITS>
__device__ __forceinline__ int limb_col(int p) {
    if constexpr (BITS == 8) return p;
    const int e = p & 15;
    return 16 * (p >> 4) + ((e >> 3) << 3) + 2 * (e & 3) + ((e >> 2) & 1);
}
// 4-bit: q ^ 8 is the 4-bit two's complement of q - 8, moved to the top of its byte (16 (q - 8)).
// 8-bit: q ^ 0x80 is the signed byte q - 128.
__device__ __forceinline__ i32x4_t code_bytes(uint2 q) {
    const uint32_t w0 = q.x ^ 0x88888888u, w1 = q.y ^ 0x88888888u;
    return i32x4_t{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u), (int)((w1 << 4) & 0xF0F0F0F0u),
                   (int)(w1 & 0xF0F0F0F0u)};
}
__device__ __forceinline__ i32x4_t code_bytes(uint4 q) {
    return i32x4_t{(int)(q.x ^ 0x80808080u), (int)(q.y ^ 0x80808080u), (int)(q.z ^ 0x80808080u),
                   (int)(q.w ^ 0x80808080u)};
}
__device__ __forceinline__ float comb3(int a0, int a1, int a2) {
    return fmaf((float)(a0 * 256 + a1), 256.0f, (float)a2);  // |a0| <= 2^20: a0 * 256 + a1 fits
}
__device__ __forceinline__ int row16_sum(int v) {
    v += (int)dpp_u32<kDppQuadXor1>((uint32_t)v);
    v += (int)dpp_u32<kDppQuadXor2>((uint32_t)v);
    v += (int)dpp_u32<kDppHalfMirror>((uint32_t)v);
    v += (int)dpp_u32<kDppRowMirror>((uint32_t)v);
    return v;
}
// Called by the 16 lanes of one DPP row for one group: lane m holds the values of positions
// 4m .. 4m+3 and writes limb dword m of rows 0..2 at dst; lane 0 writes the group entry.
template <int BITS>
__device__ __forceinline__ void build_limbs(const float (&v)[4], int8_t *dst, float2 *entry) {
    const int m = threadIdx.x & 15;
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = fmaxf(amax, dpp_f32<kDppQuadXor1>(amax));
    amax = fmaxf(amax, dpp_f32<kDppQuadXor2>(amax));
    amax = fmaxf(amax, dpp_f32<kDppHalfMirror>(amax));
    amax = fmaxf(amax, dpp_f32<kDppRowMirror>(amax));
    int ex = 0;
    if (amax > 0.0f) {
        frexpf(amax, &ex);  // amax < 2^ex
        ex -= 22;
    }
    uint32_t w0 = 0, w1 = 0, w2 = 0;
    int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int X = (int)rintf(ldexpf(v[e], -ex));
        const int l2 = ((X + 128) & 255) - 128, x1 = (X - l2) >> 8;
        const int l1 = ((x1 + 128) & 255) - 128, l0 = (x1 - l1) >> 8;
        w0 |= (uint32_t)(l0 & 255) << (8 * e);
        w1 |= (uint32_t)(l1 & 255) << (8 * e);
        w2 |= (uint32_t)(l2 & 255) << (8 * e);
        s0 += l0;
        s1 += l1;
        s2 += l2;
    }
    s0 = row16_sum(s0);
    s1 = row16_sum(s1);
    s2 = row16_sum(s2);
    reinterpret_cast<uint32_t *>(dst)[m] = w0;
    reinterpret_cast<uint32_t *>(dst + 64)[m] = w1;
    reinterpret_cast<uint32_t *>(dst + 128)[m] = w2;
    constexpr int u = CodeFmt<BITS>::unit;
    if (m == 0) *entry = make_float2((float)u * comb3(s0, s1, s2), ldexpf(1.0f, ex) / (float)u);
}

// ---- layer input ---------------------------------------------------------------------------------
// RMS glue of y_{l-1} for tokens t0 .. t0 + n - 1 (n <= TT) of H = 512 S columns, straight from
// registers: their words are polled at once (slot u S + j of thread tid: y[t0 + u][tid + 512 j]);
// per token the sum of squares adds the thread's words in column order, then the wave sum, then
// the waves in order -- the order of a thread-strided loop over the row -- and x = bf16_rne(y /
// sqrt(mean(y^2) + eps)) goes from the register holding y to its half of the pair table. One wait
// for the exchange and one barrier per group of tokens.
template <int BITS, int S, int TT>
__device__ bool chained_group(const DecodeParams &p, const uint64_t *ysrc, int t0, int n, uint32_t ep,
                              const Lds &s, unsigned spin) {
    constexpr int NW = S * TT;
    constexpr int H = 512 * S, nsl = H / 32;
    static_assert(kDecodeThreads == 512 && NW <= kMaxGather, "slot layout");
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    uint64_t w[NW];
    if (!all_ok(poll_slots<NW>(ysrc + (size_t)t0 * H, n * H, ep, w, p.ctrl, spin))) return false;
#pragma unroll
    for (int u = 0; u < TT; ++u) {
        if (u < n) {
            float ss = 0.0f;
#pragma unroll
            for (int j = 0; j < S; ++j) {
                const float v = __uint_as_float(static_cast<uint32_t>(w[u * S + j]));
                ss += v * v;
            }
            ss = wave_sum(ss);
            if (lane == 0) s.red[u * kWaves + wave] = ss;  // TT * kWaves <= 64 slots
        }
    }
    lds_barrier();
    uint16_t *xp16 = reinterpret_cast<uint16_t *>(s.xp);
#pragma unroll
    for (int u = 0; u < TT; ++u) {
        if (u < n) {
            float ss = 0.0f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) ss += s.red[u * kWaves + v];
            const float inv = 1.0f / sqrtf(ss / (float)H + p.eps);
#pragma unroll
            for (int j = 0; j < S; ++j) {
                const int h = tid + 512 * j, sl = h >> 5;
                int q, half;
                col_pair<BITS>(h & 31, q, half);
                const float v = __uint_as_float(static_cast<uint32_t>(w[u * S + j]));
                xp16[(((t0 + u) * nsl + sl) * 20 + q) * 2 + half] = static_cast<uint16_t>(f32_to_bf16_rne(v * inv));
            }
        }
    }
    lds_barrier();  // s.red is reused by the next group
    return true;
}
// All T tokens in groups of TT (words per thread <= kMaxGather).
template <int BITS, int S>
__device__ bool chained_input(const DecodeParams &p, const uint64_t *ysrc, uint32_t ep, const Lds &s,
                              unsigned spin) {
    constexpr int TT = kMaxGather / S < 8 ? kMaxGather / S : 8;
    const int T = p.T;
    if (T == 1) return chained_group<BITS, S, 1>(p, ysrc, 0, 1, ep, s, spin);
    for (int t0 = 0; t0 < T; t0 += TT)
        if (!chained_group<BITS, S, TT>(p, ysrc, t0, min(TT, T - t0), ep, s, spin)) return false;
    return true;
}

// x of every token into the pair table s.xp (and its slice constants): x_in for l == 0 (or
// unchained), else the RMS glue of y_{l-1}: x = bf16_rne(y / sqrt(mean(y^2) + eps)); every
// workgroup computes the same bits.
template <int BITS>
__device__ bool layer_input(const DecodeParams &p, int l, uint32_t ep, const Lds &s, unsigned spin) {
    const int T = p.T, H = p.H, nsl = H / 32;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (l == 0 || !p.chained) {
        for (int i = threadIdx.x; i < T * nsl * 16; i += kDecodeThreads) {
            const int sh = __builtin_ctz(static_cast<unsigned>(nsl * 16));
            const int t = i >> sh, r = i & ((nsl * 16) - 1), sl = r >> 4, q = r & 15;
            const auto xr = G(p.x_in + (size_t)t * H + sl * 32);
            const uint32_t a = xr[pair_col_a<BITS>(q)], c = xr[pair_col_b<BITS>(q)];
            s.xp[(t * nsl + sl) * 20 + q] = a | (c << 16);
        }
    } else if (H >= 512) {
        const uint64_t *ysrc = p.ll_y + (size_t)(l - 1) * T * H;
        bool ok;
        if (H == 512) ok = chained_input<BITS, 1>(p, ysrc, ep, s, spin);
        else if (H == 1024) ok = chained_input<BITS, 2>(p, ysrc, ep, s, spin);
        else ok = chained_input<BITS, 4>(p, ysrc, ep, s, spin);  // H == 2048
        if (!ok) return false;
    } else {
        // H = 256: token by token through LDS
        const uint64_t *ysrc = p.ll_y + (size_t)(l - 1) * T * H;
        float *yb = reinterpret_cast<float *>(s.hp);
        for (int t = 0; t < T; ++t) {
            if (!ll_gather(ysrc + (size_t)t * H, H, ep, yb, p.ctrl, spin)) return false;
            float ss = 0.0f;
            for (int h = threadIdx.x; h < H; h += kDecodeThreads) ss += yb[h] * yb[h];
            ss = wave_sum(ss);
            if (lane == 0) s.red[wave] = ss;
            lds_barrier();
            ss = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) ss += s.red[w];
            const float inv = 1.0f / sqrtf(ss / (float)H + p.eps);
            for (int i = threadIdx.x; i < nsl * 16; i += kDecodeThreads) {
                const int sl = i >> 4, q = i & 15;
                const float *yr = yb + sl * 32;
                const uint32_t a = f32_to_bf16_rne(yr[pair_col_a<BITS>(q)] * inv);
                const uint32_t c = f32_to_bf16_rne(yr[pair_col_b<BITS>(q)] * inv);
                s.xp[(t * nsl + sl) * 20 + q] = a | (c << 16);
            }
            lds_barrier();
        }
    }
    lds_barrier();
    if (p.x_all && blockIdx.x == 0)
        for (int i = threadIdx.x; i < T * H; i += kDecodeThreads) {
            const int t = i >> __builtin_ctz(static_cast<unsigned>(H)), h = i & (H - 1), sl = h >> 5;
            int q, half;
            col_pair<BITS>(h & 31, q, half);
            G(p.x_all)[(size_t)l * T * H + i] = static_cast<uint16_t>(s.xp[(t * nsl + sl) * 20 + q] >> (16 * half));
        }
    lds_barrier();
    return true;
}

// ---- x as limbs --------------------------------------------------------------------------------------
// The limb table overwrites the bf16 pairs of x (same LDS region), so every thread first reads its
// items into registers, then all write after a barrier; called once the router has read x.
template <int BITS>
__device__ void build_x_limbs(const DecodeParams &p, const Lds &s) {
    const int T = p.T, nsl = p.H / 32, ng = p.H / 64, lng = __builtin_ctz(static_cast<unsigned>(ng));
    const int n = T * ng * 16;  // 16 lanes per group; n and the block size are multiples of 16
    constexpr int kItems = 8;   // n <= 8 * 512 (T <= 8, H <= 2048)
    float v[kItems][4];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const int it = threadIdx.x + k * kDecodeThreads;
        if (it < n) {
            const int tg = it >> 4, m = it & 15, t = tg >> lng, g = tg & (ng - 1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = 64 * g + limb_col<BITS>(4 * m + e);
                int q, half;
                col_pair<BITS>(col & 31, q, half);
                v[k][e] = bf16_to_f32((s.xp[(t * nsl + (col >> 5)) * 20 + q] >> (16 * half)) & 0xFFFFu);
            }
        }
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const int it = threadIdx.x + k * kDecodeThreads;
        if (it < n) build_limbs<BITS>(v[k], s.xq + (size_t)(it >> 4) * 192, s.xsx + (it >> 4));
    }
    lds_barrier();
}

// ---- router --------------------------------------------------------------------------------------
// (row r, token t) combinations round-robin over the waves; lane sl takes 32-column slice sl.
template <int BITS>
__device__ void router_logits(const DecodeParams &p, int l, const Lds &s, const WgShare &w, uint64_t *ll_lg,
                              uint32_t ep) {
    const float *rbias = p.rbias ? p.rbias + (size_t)l * p.E : nullptr;
    const int T = p.T, H = p.H, E = p.E, nsl = H / 32, b = blockIdx.x, g = gridDim.x;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int nr = w.nrr;
    for (int c = wave; c < nr * T; c += kWaves) {
        const int r = div_by(c, p.tdiv), t = c - r * T;
        const float4 *row = reinterpret_cast<const float4 *>(s.rt + (size_t)r * H);
        float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int sl = lane; sl < nsl; sl += kWave) {
            const uint32_t *xw = s.xp + (t * nsl + sl) * 20;
            float rv[32];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float4 f = row[k * nsl + sl];
                rv[4 * k] = f.x; rv[4 * k + 1] = f.y; rv[4 * k + 2] = f.z; rv[4 * k + 3] = f.w;
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const uint32_t w = xw[q];
                a4[q & 3] = fmaf(rv[pair_col_a<BITS>(q)], bf16_to_f32(w & 0xFFFF), a4[q & 3]);
                a4[q & 3] = fmaf(rv[pair_col_b<BITS>(q)], bf16_to_f32(w >> 16), a4[q & 3]);
            }
        }
        float acc = wave_sum((a4[0] + a4[1]) + (a4[2] + a4[3]));
        if (lane == 0) {
            const int e = b + r * g;
            if (e < E && rbias) acc += G(rbias)[e];
            ll_put(ll_lg + (size_t)t * (E + 1) + e, acc, ep);
        }
    }
}

// ---- h of one token as limbs -------------------------------------------------------------------------
template <int BITS>
__device__ bool stage_hq(const DecodeParams &p, const Lds &s, const uint64_t *src, uint32_t ep, unsigned spin,
                         int mark_l = -1) {
    const int n = p.K * p.I + p.Is;
    const float *hf = reinterpret_cast<const float *>(s.hp);
    if (!ll_gather(src, n, ep, reinterpret_cast<float *>(s.hp), p.ctrl, spin)) return false;
    if (mark_l >= 0) phase_mark(p.phase, mark_l, kMarkHPolled);
    // 16 lanes per group; n / 4 and the block size are multiples of 16, so DPP rows stay whole
    for (int it = threadIdx.x; it < n / 4; it += kDecodeThreads) {
        const int gi = it >> 4, m = it & 15;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = hf[gi * 64 + limb_col<BITS>(4 * m + e)];
        build_limbs<BITS>(v, s.hq + (size_t)gi * 192, s.hsx + gi);
    }
    lds_barrier();
    return true;
}

// ---- down projection on MFMA ------------------------------------------------------------------------
// Jobs (v, rl) of nv vectors x nr rows are numbered job = v * nr + rl (the staged row); a tile is
// th = min(16, 3 nr + 1) consecutive jobs, which touch at most 4 vectors. A row 4u + j = limb j of
// the tile's u-th vector (row 4u + 3 repeats limb 2); B column i = the codes of weight row i of the
// tile. Operand layouts (lane l, i = l % 16, kb = l / 16): A[i][16 kb + e], B[16 kb + e][i],
// C[4 kb + r][i], so lane (i, kb) ends with weight row i against the three limbs of tile vector
// kb: it owns row i when that is the row's vector. Groups of h: gbase + v * len / 64 + g.
template <int BITS>
__device__ void down_tile_mfma(const Lds &s, const Rows &R, int nv, int len, int nr, uint32_t nrm, int th, int tau,
                               int gbase, float *out, int RB) {
    typedef CodeFmt<BITS> F;
    typedef typename F::lane_t qv_t;
    const int lane = threadIdx.x % kWave, i = lane % 16, kb = lane / 16;
    const int njobs = nv * nr, j0 = tau * th, jn = min(j0 + th, njobs);
    const int ngv = len / 64, gm = min(ngv, 8) - 1;
    const int vfirst = div_by(j0, nrm), nsp = div_by(jn - 1, nrm) - vfirst + 1;
    // B column i: weight row j0 + i (columns past the tile repeat its first row, unused)
    const bool wok = i < th && j0 + i < jn;
    const int wrow = wok ? j0 + i : j0, vi = div_by(wrow, nrm);
    const bool own = wok && vi - vfirst == kb;
    const char *qbase = R.c + (size_t)wrow * R.cb + kb * (F::group_bytes / 4);
    const int qswz = wrow & gm;
    const uint16_t *sp = reinterpret_cast<const uint16_t *>(R.s + (size_t)wrow * R.sb);
    const uint16_t *bp = reinterpret_cast<const uint16_t *>(R.b + (size_t)wrow * R.sb);
    // A row i: limb min(i % 4, 2) of tile vector min(i / 4, nsp - 1)
    const int va = vfirst + min(i >> 2, nsp - 1), ja = min(i & 3, 2);
    const int8_t *abase = s.hq + ((size_t)(gbase + va * ngv) * 3 + ja) * 64 + 16 * kb;
    // group entries of this lane's vector (tile vector kb)
    const float2 *gsx = s.hsx + gbase + (vfirst + min(kb, nsp - 1)) * ngv;
    // operands of the group pair (g, g + 1), g even; the next pair's loads are issued before the
    // current pair's math (scheduling barriers keep the compiler from sinking them)
    struct Pair {
        i32x4_t a0, a1;
        qv_t q0, q1;
        uint32_t sv, bv;  // bf16 scale / bias of groups g (low half) and g + 1 (high half)
        float4 gx;        // entries of groups g and g + 1
    };
    auto load = [&](int g) -> Pair {
        Pair d;
        d.a0 = *reinterpret_cast<const i32x4_t *>(abase + (size_t)g * 192);
        d.a1 = *reinterpret_cast<const i32x4_t *>(abase + (size_t)g * 192 + 192);
        d.q0 = *reinterpret_cast<const qv_t *>(qbase + ((g ^ qswz) * F::group_bytes));
        d.q1 = *reinterpret_cast<const qv_t *>(qbase + (((g + 1) ^ qswz) * F::group_bytes));
        d.sv = *reinterpret_cast<const uint32_t *>(sp + g);
        d.bv = *reinterpret_cast<const uint32_t *>(bp + g);
        d.gx = *reinterpret_cast<const float4 *>(gsx + g);
        return d;
    };
    float acc = 0.0f;
    auto step = [&](const Pair &d) {
        const i32x4_t zero = {0, 0, 0, 0};
        const i32x4_t c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(d.a0, code_bytes(d.q0), zero, 0, 0, 0);
        const i32x4_t c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(d.a1, code_bytes(d.q1), zero, 0, 0, 0);
        const float s0 = __uint_as_float(d.sv << 16), b0 = __uint_as_float(d.bv << 16);
        const float s1 = __uint_as_float(d.sv & 0xFFFF0000u), b1 = __uint_as_float(d.bv & 0xFFFF0000u);
        constexpr float zp = F::zp;
        acc = fmaf(d.gx.y, fmaf(s0, comb3(c0[0], c0[1], c0[2]), fmaf(zp, s0, b0) * d.gx.x), acc);
        acc = fmaf(d.gx.w, fmaf(s1, comb3(c1[0], c1[1], c1[2]), fmaf(zp, s1, b1) * d.gx.z), acc);
    };
    const int glast = ngv - 2;
    Pair pa = load(0);
    for (int g = 0; g < ngv; g += 4) {
        const Pair pb = load(min(g + 2, glast));
        __builtin_amdgcn_sched_barrier(0);
        step(pa);
        if (g + 2 >= ngv) break;
        pa = load(min(g + 4, glast));
        __builtin_amdgcn_sched_barrier(0);
        step(pb);
    }
    if (own) out[vi * RB + (wrow - vi * nr)] = acc;
}

// Every routed vector (rows from rd) and the shared vector (rows from sd) of one token; tiles are
// dealt round-robin over the waves.
template <int BITS>
__device__ void down_all_mfma(const Lds &s, const Rows &rd, const Rows &sd, int K, int I, int Is, int nr,
                              uint32_t nrm, float *out, int RB) {
    const int wave = threadIdx.x / kWave;
    const int th = min(16, 3 * nr + 1);
    const int nrt = (K * nr + th - 1) / th, nst = Is ? (nr + th - 1) / th : 0;
    for (int u = wave; u < nrt + nst; u += kWaves) {
        if (u < nrt) down_tile_mfma<BITS>(s, rd, K, I, nr, nrm, th, u, 0, out, RB);
        else down_tile_mfma<BITS>(s, sd, 1, Is, nr, nrm, th, u - nrt, K * I / 64, out + K * RB, RB);
    }
}

// ---- gate|up + SwiGLU on MFMA -----------------------------------------------------------------------
// The same engine with A row 4t' + j = limb j of token 4 tb + t' (token blocks tb of 4; rows past
// T repeat token T - 1) and B column i = staged row i of a 16-row tile (rows 2m / 2m + 1 = gate /
// up of pair m); lane (i, kb) ends with row i against token 4 tb + kb. The H columns are split into
// ks contiguous ranges of whole groups so that tiles x ranges fill the 8 waves; each range's sum
// goes to an LDS partial (the h staging area is idle during gate|up), and after a barrier the
// partials are added in range order, SwiGLU applied and the result exchanged.
//   ALL = true: every pair serves every token (the shared expert); else pair m serves tok_of(m).
//   dst_of(m, t): the exchange word of pair m for token t.
//   busy: waves 0 .. busy-1 arrive late (they are selecting experts), so the units go to the other
//   waves first; max_units bounds ranges x tiles (it alone fixes the ranges, so results do not
//   depend on busy).
template <int BITS, bool ALL, typename TokOf, typename DstOf>
__device__ void gate_up_mfma(const DecodeParams &p, const Lds &s, const Rows &R, int np, TokOf tok_of,
                             DstOf dst_of, uint32_t ep, int busy = 0, int max_units = kWaves, int mark_l = -1) {
    typedef CodeFmt<BITS> F;
    typedef typename F::lane_t qv_t;
    const int lane = threadIdx.x % kWave, i = lane % 16, kb = lane / 16;
    const int wave = (threadIdx.x / kWave + kWaves - busy) % kWaves;  // busy waves come last
    const int T = p.T, ng = p.H / 64, gm = min(ng, 8) - 1;
    const int nrows = 2 * np, ntile = (nrows + 15) / 16, nslot = ALL ? T : 1;
    const bool two = T > 4;  // a second token block (T <= 8)
    int lks = 0;  // log2 of the number of column ranges: ranges x tiles <= max_units, >= 2 groups per range
    while ((2 << lks) * ntile <= max_units && (4 << lks) <= ng) ++lks;
    const int ks = 1 << lks, gpr = ng >> lks;
    float *part = reinterpret_cast<float *>(s.hp);  // [ks][nslot][nrows]
    const int ja = min(i & 3, 2);
    const int ta0 = min(i >> 2, T - 1), ta1 = min(4 + (i >> 2), T - 1);
    const int tl0 = min(kb, T - 1), tl1 = min(4 + kb, T - 1);  // this lane's tokens in blocks 0 and 1
    for (int unit = wave; unit < (ntile << lks); unit += kWaves) {
        const int tau = unit >> lks, kq = unit & (ks - 1), g0 = kq * gpr;
        const int row = 16 * tau + i;
        const bool wok = row < nrows;
        const int wrow = wok ? row : 16 * tau;
        const int tk = ALL ? 0 : tok_of(wrow >> 1);
        const char *qbase = R.c + (size_t)wrow * R.cb + kb * (F::group_bytes / 4);
        const int qswz = wrow & gm;
        const uint16_t *sp = reinterpret_cast<const uint16_t *>(R.s + (size_t)wrow * R.sb);
        const uint16_t *bp = reinterpret_cast<const uint16_t *>(R.b + (size_t)wrow * R.sb);
        const int8_t *a0p = s.xq + ((size_t)ta0 * ng * 3 + ja) * 64 + 16 * kb;
        const int8_t *a1p = s.xq + ((size_t)ta1 * ng * 3 + ja) * 64 + 16 * kb;
        const float2 *x0p = s.xsx + tl0 * ng, *x1p = s.xsx + tl1 * ng;
        // operands of the group pair (g, g + 1), g even (token blocks 0 and 1)
        struct Pair {
            i32x4_t a00, a01, a10, a11;
            qv_t q0, q1;
            uint32_t sv, bv;
            float4 x0, x1;
        };
        auto load = [&](int g) -> Pair {
            Pair d;
            d.a00 = *reinterpret_cast<const i32x4_t *>(a0p + (size_t)g * 192);
            d.a01 = *reinterpret_cast<const i32x4_t *>(a0p + (size_t)g * 192 + 192);
            d.q0 = *reinterpret_cast<const qv_t *>(qbase + ((g ^ qswz) * F::group_bytes));
            d.q1 = *reinterpret_cast<const qv_t *>(qbase + (((g + 1) ^ qswz) * F::group_bytes));
            d.sv = *reinterpret_cast<const uint32_t *>(sp + g);
            d.bv = *reinterpret_cast<const uint32_t *>(bp + g);
            d.x0 = *reinterpret_cast<const float4 *>(x0p + g);
            if (two) {
                d.a10 = *reinterpret_cast<const i32x4_t *>(a1p + (size_t)g * 192);
                d.a11 = *reinterpret_cast<const i32x4_t *>(a1p + (size_t)g * 192 + 192);
                d.x1 = *reinterpret_cast<const float4 *>(x1p + g);
            }
            return d;
        };
        float acc0 = 0.0f, acc1 = 0.0f;
        auto step = [&](const Pair &d) {
            const i32x4_t zero = {0, 0, 0, 0}, b0 = code_bytes(d.q0), b1 = code_bytes(d.q1);
            constexpr float zp = F::zp;
            const float s0 = __uint_as_float(d.sv << 16), z0 = fmaf(zp, s0, __uint_as_float(d.bv << 16));
            const float s1 = __uint_as_float(d.sv & 0xFFFF0000u);
            const float z1 = fmaf(zp, s1, __uint_as_float(d.bv & 0xFFFF0000u));
            i32x4_t c = __builtin_amdgcn_mfma_i32_16x16x64_i8(d.a00, b0, zero, 0, 0, 0);
            acc0 = fmaf(d.x0.y, fmaf(s0, comb3(c[0], c[1], c[2]), z0 * d.x0.x), acc0);
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(d.a01, b1, zero, 0, 0, 0);
            acc0 = fmaf(d.x0.w, fmaf(s1, comb3(c[0], c[1], c[2]), z1 * d.x0.z), acc0);
            if (two) {
                c = __builtin_amdgcn_mfma_i32_16x16x64_i8(d.a10, b0, zero, 0, 0, 0);
                acc1 = fmaf(d.x1.y, fmaf(s0, comb3(c[0], c[1], c[2]), z0 * d.x1.x), acc1);
                c = __builtin_amdgcn_mfma_i32_16x16x64_i8(d.a11, b1, zero, 0, 0, 0);
                acc1 = fmaf(d.x1.w, fmaf(s1, comb3(c[0], c[1], c[2]), z1 * d.x1.z), acc1);
            }
        };
        const int glast = g0 + gpr - 2;
        Pair pa = load(g0);
        for (int g = g0; g < g0 + gpr; g += 4) {
            const Pair pb = load(min(g + 2, glast));
            __builtin_amdgcn_sched_barrier(0);
            step(pa);
            if (g + 2 >= g0 + gpr) break;
            pa = load(min(g + 4, glast));
            __builtin_amdgcn_sched_barrier(0);
            step(pb);
        }
        if (wok) {
            if constexpr (ALL) {
                if (kb < T) part[(kq * T + kb) * nrows + row] = acc0;
                if (two && 4 + kb < T) part[(kq * T + 4 + kb) * nrows + row] = acc1;
            } else {
                if ((tk & 3) == kb) part[kq * nrows + row] = tk < 4 ? acc0 : acc1;
            }
        }
    }
    if (mark_l >= 0) phase_mark(p.phase, mark_l, kMarkGuUnits);
    lds_barrier();
    if (mark_l >= 0) phase_mark(p.phase, mark_l, kMarkGuBarrier);
    for (int e = threadIdx.x; e < np * nslot; e += kDecodeThreads) {
        const int m = ALL ? div_by(e, p.tdiv) : e, t = ALL ? e - m * T : 0;
        float gsum = 0.0f, usum = 0.0f;
        for (int k = 0; k < ks; ++k) {
            gsum += part[(k * nslot + t) * nrows + 2 * m];
            usum += part[(k * nslot + t) * nrows + 2 * m + 1];
        }
        ll_put(dst_of(m, t), silu(gsum) * usum, ep);
    }
    if (mark_l >= 0) phase_mark(p.phase, mark_l, kMarkGuPut);
}

// ---- routing of every token (identical in every workgroup) ---------------------------------------
// Wave t selects token t's experts (wave_topk); gamma from the shared-gate logit (column E).
// Wave t < T selects token t's experts; the caller publishes the results with a barrier.
__device__ void route_tokens(const DecodeParams &p, const Lds &s) {
    const int T = p.T, E = p.E, K = p.K, wave = threadIdx.x / kWave;
    if (wave < T) {
        // the selection is one wave's dependent chain on the critical path; the wave sharing its
        // SIMD runs the shared gate|up meanwhile, so the selecting wave issues first
        __builtin_amdgcn_s_setprio(3);
        wave_topk(s.lg + wave * (E + 1), E, K, s.sidx + wave * K, s.sw + wave * K);
        __builtin_amdgcn_s_setprio(0);
    }
    // gamma by the last wave, so that wave 0 goes from its selection straight to the barrier
    for (int t = threadIdx.x - (kWaves - 1) * kWave; t >= 0 && t < T; t += kDecodeThreads)
        s.gam[t] = p.Is ? 1.0f / (1.0f + expf(-s.lg[t * (E + 1) + E])) : 0.0f;
}

template <int BITS, bool XT, bool T1>
__global__ void __launch_bounds__(kDecodeThreads, 1) decode_kernel(DecodeParams p0) {
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x;
    const int nb = gridDim.x, b = blockIdx.x;
    if (p0.ctrl[0] != 0) return;  // sticky failure of an earlier call: do nothing
    __shared__ __align__(16) uint32_t pwords[(kParamWords + 3) / 4 * 4];
    params_to_lds(pwords);
    lds_barrier();
    // bound on every wait: the workspace's control word 2 when the caller set one, else the default
    const unsigned spin = p0.ctrl[2] > 0 ? static_cast<unsigned>(p0.ctrl[2]) : p0.spin_limit;
    uint32_t ep = static_cast<uint32_t>(p0.ctrl[1]) + 1u;
    if (ep == 0) ep = 1;
    if (tid == 0) ll_put(p0.ll_start + b, 0.0f, ep);
    const WgShare w = wg_share(p0);
    {
        const Lds s = carve(p0, smem);
        stage_router(p0, 0, s, w);
        if constexpr (XT) stage_xtab(p0, 0, s, kAllWaves);
        stage_shared_gu(p0, 0, s, w);
        stage_shared_down(p0, 0, s, w.r0, w.nr);
    }
    const int nlayers = p0.L;
    for (int l = 0; l < nlayers; ++l) {
        DecodeParams p = fresh_params(pwords);
        if constexpr (T1) {  // one token per call: every token count and division by it is a constant
            p.T = 1;
            p.tdiv = 0;
        }
        const Lds s = carve(p, smem);
        const int T = p.T, H = p.H, E = p.E, K = p.K, I = p.I, Is = p.Is, RB = p.rows_per_wg;
        const int KI = K * I, HW = KI + Is;  // h words per token
        const int r0 = w.r0, nr = w.nr;
        const bool has_next = l + 1 < nlayers;
        uint64_t *ll_lg = p.ll_logits + (size_t)l * T * (E + 1);
        uint64_t *ll_h = p.ll_h + (size_t)l * T * HW;
        uint64_t *ll_y = p.ll_y + (size_t)l * T * H;

        phase_mark(p.phase, l, kMarkLayer);
        if (!layer_input<BITS>(p, l, ep, s, spin)) { dma_wait(); return; }
        phase_mark(p.phase, l, kMarkInput);
        dma_wait();  // this layer's router and shared rows (staged during the previous layer)
        lds_barrier();
        phase_mark(p.phase, l, kMarkRouterRows);

        // ---- R: router logits from LDS, then x as limbs (its barriers also end this phase)
        router_logits<BITS>(p, l, s, w, ll_lg, ep);
        if (!Is && b == 0 && tid < T) ll_put(ll_lg + (size_t)tid * (E + 1) + E, 0.0f, ep);  // unused column
        phase_mark(p.phase, l, kMarkLogitsPut);
        build_x_limbs<BITS>(p, s);
        phase_mark(p.phase, l, kMarkXLimbs);

        // ---- G: routing (identical in every workgroup), then routed gate|up + SwiGLU
        if (!ll_gather(ll_lg, T * (E + 1), ep, s.lg, p.ctrl, spin)) { dma_wait(); return; }
        phase_mark(p.phase, l, kMarkLogitsGot);
        route_tokens(p, s);
        phase_mark(p.phase, l, kMarkTopk);
        // layer l+1's router rows (the LDS copy was last read before the logits exchange) stream in
        // during the expert selection, issued by waves with nothing else to do then
        if (has_next) {
            const int first = min(T + kWaves / 2, kWaves - 1);
            stage_router(p, l + 1, s, w, DmaWaves{first, kWaves - first});
            if constexpr (XT) stage_xtab(p, l + 1, s, DmaWaves{first, kWaves - first});
        }
        if (Is) {
            // the shared expert's gate|up runs on the waves not selecting experts; its barrier also
            // publishes the routing
            gate_up_mfma<BITS, true>(
                p, s, sg_rows(p, s), w.nps, [](int) { return 0; },
                [&](int m, int t) { return ll_h + (size_t)t * HW + KI + (b + m * nb); }, ep, T, kWaves / 2);
        } else {
            lds_barrier();
        }
        phase_mark(p.phase, l, kMarkSharedGu);
        if (b == 0) {
            const size_t base = (size_t)l * T;
            if (p.idx_all)
                for (int i = tid; i < T * K; i += kDecodeThreads) G(p.idx_all)[base * K + i] = s.sidx[i];
            if (p.w_all)
                for (int i = tid; i < T * K; i += kDecodeThreads) G(p.w_all)[base * K + i] = s.sw[i];
            if (p.logits_all)
                for (int i = tid; i < T * E; i += kDecodeThreads)
                    G(p.logits_all)[base * E + i] = s.lg[(i / E) * (E + 1) + i % E];
        }
        // routed gate|up: this workgroup's pairs [q0, q1) of the flattened (token, slot, j) pairs,
        // staged into LDS chunk by chunk (one chunk at T = 1): LDS row 2i = gate row, 2i+1 = up row
        {
            const int np = w.q1 - w.q0, lgI = p.log2I, cp = p.cp;
            const uint32_t kdiv = p.kdiv;
            const QMat w13 = layer_ptrs(p, l).w13;
            const Rows rg = rows_at(s.rg, 2 * cp, H, BITS);
            for (int c0 = 0; c0 < np; c0 += cp) {
                const int nc = min(cp, np - c0), pb = w.q0 + c0;
                if constexpr (XT) {
                    dma_xrows(H, BITS, 2 * nc,
                              [&](int r) -> XRow {
                                  const int P = pb + (r >> 1), tk = P >> lgI, j = P & (I - 1);
                                  return XRow{s.xt[(l & 1) * E + expert_at(s.sidx[tk], E)] & ~1ull,
                                              (uint32_t)((r & 1) * I + j)};
                              },
                              p.xo13s, p.xo13b, rg, mfma_swz(BITS, H));
                } else {
                    dma_qrows(w13, H, BITS, 2 * nc,
                              [&](int r) -> size_t {
                                  const int P = pb + (r >> 1), tk = P >> lgI, j = P & (I - 1);
                                  return expert_at(s.sidx[tk], E) * 2 * I + (size_t)(r & 1) * I + j;
                              },
                              rg, mfma_swz(BITS, H));
                }
                if (c0 == 0) phase_mark(p.phase, l, kMarkRoutedIssued);
                dma_wait();
                lds_barrier();
                if (c0 == 0) phase_mark(p.phase, l, kMarkRoutedLanded);
                gate_up_mfma<BITS, false>(
                    p, s, rg, nc, [&](int i) { return div_by((pb + i) >> lgI, kdiv); },
                    [&](int i, int) {
                        const int P = pb + i, t = div_by(P >> lgI, kdiv);
                        return ll_h + (size_t)t * HW + (P - t * KI);
                    },
                    ep, 0, kWaves, c0 + cp >= np ? l : -1);
                if constexpr (XT) {
                    // the chunk's pairs belong to (token, slot)s tk_lo .. tk_hi; write through only
                    // if one of them is marked (wave-uniform test on LDS broadcasts)
                    bool marked = false;
                    if (p.landing)
                        for (int tk = pb >> lgI; tk <= (pb + nc - 1) >> lgI; ++tk)
                            marked |= (s.xt[(l & 1) * E + expert_at(s.sidx[tk], E)] & 1) != 0;
                    if (marked) {
                        wb_qrows(2 * nc, rg, mfma_swz(BITS, H), p.xo13s, p.xo13b,
                                 [&](int r, uint32_t piece, int rowbytes) -> char * {
                                     const int P = pb + (r >> 1), tk = P >> lgI, j = P & (I - 1);
                                     if (!(s.xt[(l & 1) * E + expert_at(s.sidx[tk], E)] & 1)) return nullptr;
                                     return p.landing + ((size_t)l * T * K + tk) * p.xstride + piece +
                                            (size_t)((r & 1) * I + j) * rowbytes;
                                 });
                    }
                }
                lds_barrier();
            }
        }

        // ---- D: per token, all h -> this workgroup's rows of every down projection -> combine
        // Token 0's routed down rows, then layer l+1's shared gate|up rows (the shared gate|up of this
        // layer is done), stream in during the h exchange; the down projection waits for the routed
        // down rows only.
        phase_mark(p.phase, l, kMarkRoutedDone);
        stage_routed_down<XT>(p, l, s, 0, r0, nr, w.nrm);
        int later = 0;  // DMA instructions this wave issued after the routed down rows
        if (has_next) {
            stage_shared_gu(p, l + 1, s, w);
            later = w.nps ? dma_qrows_count(2 * w.nps, H, BITS) : 0;
        }
        phase_mark(p.phase, l, kMarkDownIssued);
        for (int t = 0; t < T; ++t) {
            if (!stage_hq<BITS>(p, s, ll_h + (size_t)t * HW, ep, spin, t == 0 ? l : -1)) { dma_wait(); return; }
            if (t == 0) dma_wait_but(later);
            else dma_wait();
            lds_barrier();
            if (t == 0) phase_mark(p.phase, l, kMarkHGot);
            if (nr > 0) {
                float *pt = s.part + (size_t)t * (K + 1) * RB;
                down_all_mfma<BITS>(s, rd_rows(p, s), sd_rows(p, s), K, I, Is, nr, w.nrm, pt, RB);
                if (t + 1 == T) phase_mark(p.phase, l, kMarkDownUnits);
                if constexpr (XT) {
                    bool marked = false;
                    if (p.landing)
                        for (int k = 0; k < K; ++k)
                            marked |= (s.xt[(l & 1) * E + expert_at(s.sidx[t * K + k], E)] & 1) != 0;
                    if (marked) {
                        wb_qrows(K * nr, rd_rows(p, s), mfma_swz(BITS, I), p.xo2s - p.xo2c, p.xo2b - p.xo2c,
                                 [&](int r, uint32_t piece, int rowbytes) -> char * {
                                     const int k = div_by(r, w.nrm), rl = r - k * nr;
                                     if (!(s.xt[(l & 1) * E + expert_at(s.sidx[t * K + k], E)] & 1)) return nullptr;
                                     return p.landing + ((size_t)l * T * K + t * K + k) * p.xstride + p.xo2c +
                                            piece + (size_t)(r0 + rl) * rowbytes;
                                 });
                    }
                }
            }
            lds_barrier();
            if (t + 1 < T) stage_routed_down<XT>(p, l, s, t + 1, r0, nr, w.nrm);
        }
        phase_mark(p.phase, l, kMarkDownDone);
        for (int i = tid; i < T * nr; i += kDecodeThreads) {
            const int t = div_by(i, w.nrm), rl = i - t * nr;
            const float *pt = s.part + t * (K + 1) * RB;
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) acc += s.sw[t * K + k] * pt[k * RB + rl];
            if (Is) acc += s.gam[t] * pt[K * RB + rl];
            const size_t o = (size_t)t * H + r0 + rl;
            if (has_next && p.chained) ll_put(ll_y + o, acc, ep);
            if (!has_next) G(p.y_out)[o] = acc;
            if (p.y_all) G(p.y_all)[(size_t)l * T * H + o] = acc;
        }
        phase_mark(p.phase, l, kMarkYPut);
        lds_barrier();
        if (has_next) stage_shared_down(p, l + 1, s, r0, nr);  // streams in during the y exchange
        phase_mark(p.phase, l, kMarkLayerEnd);
    }
    dma_wait();
    // the next call may advance the epoch once every workgroup has read it
    if (b == 0) {
        if (!ll_gather(p0.ll_start, nb, ep, reinterpret_cast<float *>(smem + p0.lds.hp), p0.ctrl, spin))
            return;
        if (tid == 0) p0.ctrl[1] = static_cast<int>(ep);
    }
}

// Calls with one token run an instance compiled for T = 1 (the token loops, the second token block
// and every division by T fold away: a quarter fewer instructions, 4 % less time per layer).
template <int BITS, bool XT>
static hipError_t launch_bits(const DecodeParams &p, int grid, hipStream_t stream) {
    const void *fn = p.T == 1 ? reinterpret_cast<const void *>(&decode_kernel<BITS, XT, true>)
                              : reinterpret_cast<const void *>(&decode_kernel<BITS, XT, false>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds.total);
    if (err != hipSuccess) return err;
    DecodeParams arg = p;
    void *args[] = {&arg};
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kDecodeThreads), args, (unsigned)p.lds.total, stream);
}

hipError_t launch_decode(const DecodeParams &p, int grid, hipStream_t stream) {
    if (p.xtab) return p.bits == 4 ? launch_bits<4, true>(p, grid, stream) : launch_bits<8, true>(p, grid, stream);
    return p.bits == 4 ? launch_bits<4, false>(p, grid, stream) : launch_bits<8, false>(p, grid, stream);
}

}  // namespace moe
