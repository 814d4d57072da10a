/*
 * moe.h -- C ABI of the quantised sparse Mixture-of-Experts FFN layer (MI355X / gfx950).
 *
 * The layer (per token, x a bf16 row of H values):
 *   logits  l[e] = x . R[e] (+ bias[e])                      router, fp32 weights [E][H]
 *   select  S    = the top_k experts by logit, ties to the lower index, ordered by
 *                  (logit descending, index ascending)
 *   weights w_k  = softmax(l)[S_k] / sum_{j in S} softmax(l)[j]   (renormalised top-k softmax)
 *   expert  d_e  = W2_e ( silu(Wg_e x) * (Wu_e x) ),  gate|up packed as one matrix W13_e
 *   shared  gamma = sigmoid(x . g_s),  d_s = the shared expert's MLP, same form
 *   output  y    = sum_k w_k d_{S_k} + gamma d_s   (fp32)
 * Sources on the pages: each token goes to 8 of 256 experts (35B-A3B) or 10 of 512
 * (80B-A3B), beside an always-on shared expert (xix.ai Swiftlet article, paragraph on
 * scheduling; Runnel README, "Target"); experts are MLX-style int4/int8 group-quantised with
 * byte-addressable kernels and 64-bit offsets (xix.ai Swiftlet article, paragraph on lineage);
 * routed gate and up are packed into one projection (Runnel README, intro and "Streaming CLI").
 * The pages print no routing, SwiGLU or gate formula; the forms above are the plainest reading.
 *
 * Quantised matrices (moe_qweight), each [n_exp][rows][cols], row-major, expert-major with a
 * fixed stride per expert (expert e at base + e * stride, 64-bit arithmetic):
 *   codes  : uint8 [n_exp][rows][cols*bits/8]; 4-bit: input column 2j is the LOW nibble of
 *            byte j; 8-bit: one code per byte
 *   scales : bf16 bit patterns [n_exp][rows][cols/group_size]
 *   biases : bf16 bit patterns, same shape; weight = scale * code + bias
 *   W13 (routed gate|up): rows 2*inter (0..inter-1 gate, inter..2*inter-1 up), cols hidden
 *   W2  (routed down)   : rows hidden, cols inter
 *   S13 / S2 (shared)   : as W13 / W2 with n_exp = 1 and shared_inter in place of inter
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller (an expert container may also
 *     be pinned host memory the device reads); the library allocates nothing, keeps no state
 *     between calls and never synchronises the stream -- except the expert cache (moe_cache_*),
 *     which holds host state and pinned staging from create to destroy and synchronises its
 *     stream where its declarations say so.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is enqueued
 *     asynchronously; results are valid once the stream reaches that point.
 *   - Arguments are checked on the host before anything is enqueued; on a failed check the
 *     call returns the error and writes nothing.
 *   - Every pointer must be 16-byte aligned (4-byte for the small fp32 vectors router_bias,
 *     shared_gate and all optional outputs).
 *   - Supported: bits in {4, 8}; group_size 64; hidden, inter, shared_inter powers of two with
 *     256 <= hidden <= 4096 and 64 <= inter, shared_inter <= 4096; 1 <= top_k <= 16,
 *     top_k <= num_experts <= 1024. Other shapes return MOE_ERR_UNSUPPORTED.
 *   - A workspace is device memory of at least moe_workspace_bytes() for the same arguments,
 *     zero-filled before its first use; calls leave it ready for the next call. Its first 4
 *     bytes are a sticky device status word: 0 after successful runs, or a moe_status a kernel
 *     set (MOE_ERR_TIMEOUT from a decode wait, MOE_ERR_UNSUPPORTED from the batched path, see
 *     below). A decode kernel that finds it non-zero does nothing and writes no output; zero-fill
 *     the workspace again to recover. moe_read_status() reads it.
 *   - The decode kernels' grid-wide waits are bounded: int32 word 2 of a decode, stack or forward
 *     workspace (bytes 8..11) is the bound in polls of one wait, 0 (as zero-filled) meaning the
 *     default 2^20 polls (well over 0.1 s). A wait that exceeds it sets MOE_ERR_TIMEOUT and every
 *     workgroup of the launch then ends; the outputs are undefined.
 *   - The batched path computes with fp16 MFMA operands: x scaled by a power of two per token (any
 *     bf16 x fits), the dequantised weights s * q + b rounded once to fp16, and the SwiGLU output h
 *     as fp16 high and low parts, scaled down by a power of two per 128-row tile and 64-column group
 *     where its magnitude needs it (folded into that group's down weights, so products are
 *     unchanged). So s, b and s * q + b must lie within fp16's range (|v| <= 65504), and |W2| times
 *     the largest |h| of a tile must stay below about 2^31; weights and h below 2^-14 in magnitude
 *     are held as fp16 subnormals (absolute precision 2^-24). A weight beyond the range makes a
 *     gate|up or down accumulator non-finite, and the call then sets the status word to
 *     MOE_ERR_UNSUPPORTED (for moe_layer_forward: the forward workspace's first word); its
 *     outputs are undefined. The decode path has no such limit (its dot products are exact
 *     integer sums on activation limbs, scaled in fp32).
 *   - Two calls that share a workspace must not run concurrently.
 *   - The decode calls additionally need hidden, inter, shared_inter <= 2048, inter and a
 *     non-zero shared_inter >= 128, and an LDS footprint within 160 KiB (it grows with T); other
 *     shapes return MOE_ERR_UNSUPPORTED.
 *   - The batched calls additionally need hidden, inter, shared_inter <= 2048 and inter and a
 *     non-zero shared_inter >= 128; other shapes return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* NULL required pointer, misaligned pointer, bad count or shape   */
    MOE_ERR_UNSUPPORTED = 2, /* valid layer that this build has no kernel for (see above)     */
    MOE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than moe_workspace_bytes()          */
    MOE_ERR_HIP = 4,         /* the HIP runtime refused a launch (hipGetLastError)            */
    MOE_ERR_TIMEOUT = 5      /* device status only: a grid-wide wait exceeded its spin bound;
                                outputs are undefined (never seen on a healthy device)        */
} moe_status;

typedef struct {
    int32_t hidden;       /* H */
    int32_t num_experts;  /* E */
    int32_t top_k;        /* K */
    int32_t inter;        /* I, routed expert intermediate size */
    int32_t shared_inter; /* Is, shared expert intermediate size; 0 = no shared expert */
    int32_t bits;         /* 4 or 8 */
    int32_t group_size;   /* 64 */
} moe_shape;

typedef struct {
    const uint8_t *codes;
    const uint16_t *scales;
    const uint16_t *biases;
} moe_qweight;

/* One layer. For moe_stack_decode the same struct describes a stack of L layers: every
 * pointer is the base of an [L][...] array whose per-layer stride is the size above. */
typedef struct {
    const float *router;      /* [E][H] fp32                                             */
    const float *router_bias; /* [E] fp32 added to the logits, or NULL                   */
    const float *shared_gate; /* [H] fp32 (gamma = sigmoid(x . shared_gate)); required iff
                                 shared_inter > 0                                          */
    moe_qweight w13;          /* routed gate|up  */
    moe_qweight w2;           /* routed down     */
    moe_qweight s13;          /* shared gate|up  (ignored when shared_inter == 0) */
    moe_qweight s2;           /* shared down     */
} moe_layer;

/* moe_route flags */
#define MOE_ROUTE_LOGITS_IN 1u /* `logits` is an input [T][E]; the router GEMV is skipped and
                                  layer->router may be NULL. Used to decide routing from given
                                  logits (ties, +-0, duplicates) exactly as the layer does.    */

/* Which call a workspace is sized for */
#define MOE_WS_DECODE 0
#define MOE_WS_BATCHED 1
#define MOE_WS_STACK 2
#define MOE_WS_FORWARD 3 /* moe_layer_forward: a decode part (status word first), then a batched part */

/* The two evaluations of a layer, as moe_layer_path names them */
#define MOE_PATH_DECODE 0
#define MOE_PATH_BATCHED 1
/* Largest token count moe_layer_forward sends to the decode path when given crossover <= 0.
 * Measured on MI355X for one 35B-shaped 4-bit layer (H 2048, E 256, top-8, I = Is = 512): the
 * single-layer decode call is the faster one at T = 1 (40 vs 46 us) and the batched one
 * from T = 2 on (46 vs 49 us; T = 8: 77 vs 110 us). A stack of layers in one
 * moe_stack_decode call pays the decode kernel's launch and first staging once, so there the decode
 * path stays ahead. */
#define MOE_DEFAULT_CROSSOVER 1

/*
 * Router: logits, top-k selection and renormalised weights for T tokens (1 <= T <= 65536).
 * Pages: every layer routes each token to 8 of 256 experts (35B) or 10 of 512 (80B), the routers
 * being among the resident dense weights (xix.ai Swiftlet article, paragraph on scheduling;
 * AgentLens Swiftlet page, "How it works"); 256 routed experts, top-8, one shared expert (Runnel
 * README, "Target"). The softmax / top-k / renormalise form and the tie rule are the plainest
 * reading (the pages print no routing formula).
 *   x       : bf16 [T][H] (unused with MOE_ROUTE_LOGITS_IN, may be NULL)
 *   logits  : fp32 [T][E]; output, or input with MOE_ROUTE_LOGITS_IN; required
 *   topk_idx: int32 [T][K] out; topk_w: fp32 [T][K] out; gamma: fp32 [T] out or NULL
 *             (needs shared_inter > 0 and no MOE_ROUTE_LOGITS_IN)
 * Needs no workspace.
 */
moe_status moe_route(const moe_shape *shape, const moe_layer *layer, const uint16_t *x, int32_t T,
                     float *logits, int32_t *topk_idx, float *topk_w, float *gamma, uint32_t flags,
                     void *stream);

/*
 * Pages: batch-1 decode of the MoE layer (Runnel README, "Target"); MLX-style int4/int8 group
 * quantised experts read through 64-bit offsets (xix.ai Swiftlet article, paragraph on lineage);
 * the routed gate and up projections packed into one matrix (Runnel README, intro and "Streaming
 * CLI"); the shared expert always on (xix.ai article, paragraph on scheduling).
 * One layer at decode for 1 <= T <= 8 tokens: router, top-k, packed gate|up dequant-GEMV with
 * SwiGLU, down dequant-GEMV and the fixed-order combine (k = 0..K-1, then the shared expert),
 * as one persistent kernel (one workgroup per compute unit; workgroups exchange logits, h and y
 * through epoch-tagged words in the workspace, with no grid-wide barrier).
 *   x : bf16 [T][H]   y : fp32 [T][H]
 *   topk_idx_opt [T][K], topk_w_opt [T][K], logits_opt [T][E]: routing outputs or NULL
 */
moe_status moe_layer_decode(const moe_shape *shape, const moe_layer *layer, const uint16_t *x,
                            int32_t T, float *y, int32_t *topk_idx_opt, float *topk_w_opt,
                            float *logits_opt, void *workspace, size_t workspace_bytes,
                            void *stream);

/* moe_stack_decode flags */
#define MOE_STACK_INDEPENDENT 1u /* every layer takes x (no chaining); used to check every layer of
                                    a stack against a reference on identical inputs             */

/*
 * L layers at decode (1 <= T <= 8, 1 <= L <= 4096) in one persistent launch. Layer 0 takes x;
 * unless MOE_STACK_INDEPENDENT, layer l+1 takes
 *   x_{l+1} = bf16_rne( y_l / sqrt(mean(y_l^2) + 1e-6) )   per token
 * (a weightless RMS normalisation standing in for the norm and mixer between the MoE layers of
 * a model; it is not part of the MoE method). `stack` holds [L]-stacked arrays (see moe_layer).
 *   y            : fp32 [T][H], output of the last layer
 *   x_all_opt    : bf16 [L][T][H] inputs of every layer (x_all[0] = x), or NULL
 *   y_all_opt    : fp32 [L][T][H], or NULL
 *   topk_idx_all_opt [L][T][K], topk_w_all_opt [L][T][K], logits_all_opt [L][T][E], or NULL
 */
moe_status moe_stack_decode(const moe_shape *shape, const moe_layer *stack, int32_t n_layers,
                            uint32_t flags, const uint16_t *x, int32_t T, float *y,
                            uint16_t *x_all_opt, float *y_all_opt, int32_t *topk_idx_all_opt,
                            float *topk_w_all_opt, float *logits_all_opt, void *workspace,
                            size_t workspace_bytes, void *stream);

/* moe_stack_decode_static flag: clear the fixed scratch (and with it a sticky status) first */
#define MOE_STATIC_RESET 2u

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. moe_stack_decode (same arguments, same results bit for
 * bit) with no workspace argument: the call's exchange words and status live in a fixed scratch
 * array of 32 MiB per device that the library holds from its first use on that device until the
 * process ends (the stack's moe_workspace_bytes(..., MOE_WS_STACK) must fit: MOE_ERR_WORKSPACE
 * otherwise). The call allocates nothing and calls no allocating routine. The scratch is cleared
 * on the stream by a fill kernel at the first call on each device, and again when flags holds
 * MOE_STATIC_RESET; otherwise it keeps the previous call's contents, as a workspace does (a sticky
 * MOE_ERR_TIMEOUT stays until a call with MOE_STATIC_RESET). Every call on one device shares the
 * same scratch: calls that overlap on one device (different streams or threads) race and give
 * undefined results. flags: MOE_STACK_INDEPENDENT and/or MOE_STATIC_RESET.
 */
moe_status moe_stack_decode_static(const moe_shape *shape, const moe_layer *stack, int32_t n_layers,
                                   uint32_t flags, const uint16_t *x, int32_t T, float *y,
                                   uint16_t *x_all_opt, float *y_all_opt, int32_t *topk_idx_all_opt,
                                   float *topk_w_all_opt, float *logits_all_opt, void *stream);

/*
 * Pages: the same layer as moe_layer_decode (same citations), evaluated for many tokens per call;
 * the pages pick a quantised-matmul route by batch size and sweep its boundary (Smelt README, "Lab
 * workflow"). The grouping by expert and the grouped GEMMs are this library's design.
 * One layer for a batch of 1 <= T <= 65536 tokens (prefill or batched decode): router, then a
 * histogram / exclusive-scan / stable scatter that groups (token, slot) pairs by expert, an
 * MFMA grouped GEMM for gate|up with SwiGLU, one for down scaled by the routing weight, the
 * shared expert as one dense group, and a fixed-order un-permute combine.
 * Arguments as moe_layer_decode.
 */
moe_status moe_layer_batched(const moe_shape *shape, const moe_layer *layer, const uint16_t *x,
                             int32_t T, float *y, int32_t *topk_idx_opt, float *topk_w_opt,
                             float *logits_opt, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * The grouping step of moe_layer_batched on its own: histogram, exclusive scan and stable
 * scatter of the T*K (token, slot) pairs of a top-k selection by expert (the "scatter" that turns
 * per-token routing into per-expert row lists in the grouped evaluation of the layer).
 *   topk_idx : int32 [T][K] in, every value in [0, E) (values outside are clamped into it, so
 *              nothing is accessed out of bounds, but the result is then meaningless)
 *   counts   : int32 [E] out, pairs per expert
 *   offsets  : int32 [E+1] out, exclusive prefix sums of counts (offsets[E] = T*K)
 *   perm     : int32 [T*K] out, perm[offsets[e] + r] = the r-th pair q = t*K + k, in increasing
 *              q, whose expert is e
 *   pos      : int32 [T*K] out, pos[q] = row of pair q in perm (perm[pos[q]] == q)
 * Workspace: moe_workspace_bytes(shape, T, 0, MOE_WS_BATCHED) bytes.
 */
moe_status moe_group_pairs(const moe_shape *shape, const int32_t *topk_idx, int32_t T, int32_t *counts,
                           int32_t *offsets, int32_t *perm, int32_t *pos, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * The decode / batched route boundary (the per-batch-size route selection of a quantised matrix
 * kernel that the Smelt README's "Lab workflow" section sweeps and then benchmarks on both sides of
 * the selected boundary): the path moe_layer_forward takes for T tokens.
 * MOE_PATH_DECODE when T <= crossover (crossover <= 0: MOE_DEFAULT_CROSSOVER), T <= 8 and the shape
 * is one the decode call takes (the header's decode limits; its LDS plan is checked for the current
 * device's compute-unit count, or 256 when no device is visible); MOE_PATH_BATCHED otherwise; -1
 * for an invalid shape or T outside 1..65536. Host-only: touches no device memory.
 */
int32_t moe_layer_path(const moe_shape *shape, int32_t T, int32_t crossover);

/*
 * One layer for 1 <= T <= 65536 tokens through the path moe_layer_path(shape, T, crossover)
 * names: exactly moe_layer_decode or moe_layer_batched (same outputs, bit for bit). Arguments as
 * moe_layer_decode; workspace: moe_workspace_bytes(shape, T, 0, MOE_WS_FORWARD) bytes, zero-filled
 * before first use: a decode workspace for 8 tokens (status word first), then a batched one for T.
 * Calls with different T may share a workspace sized for the largest.
 */
moe_status moe_layer_forward(const moe_shape *shape, const moe_layer *layer, const uint16_t *x,
                             int32_t T, int32_t crossover, float *y, int32_t *topk_idx_opt,
                             float *topk_w_opt, float *logits_opt, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * ---- Expert residency (fixed-stride expert container + bounded HBM slot pool) ----
 * Swiftlet's memory scheme as the AgentLens project page ("How it works"), the xix.ai article
 * (scheduling and lineage paragraphs) and the Chinese summary describe it: routed experts repacked
 * into fixed-stride blocks so that fetching one expert is one contiguous read, and a bounded pool
 * of popular experts with LFU + recency eviction in front of the slow tier. Here the slow tier is
 * the container itself (host memory the GPU reads directly, or device memory), the pool lives in
 * HBM, and the decode kernel reads every routed expert through a table of block addresses.
 */

/* Bytes of one routed expert's block in the container: its gate|up codes, scales, biases, then
 * its down codes, scales, biases, each piece at a 256-byte aligned offset, the total rounded up
 * to 4096. 0 for an invalid shape. */
size_t moe_expert_stride(const moe_shape *shape);

/* Copies the routed experts (w13, w2) of an [L]-stacked layer description into the container:
 * expert (l, e) is the block at container + (l * E + e) * moe_expert_stride(shape). `container`
 * (4096-byte aligned, at least n_layers * E * stride bytes) may be device memory or host memory
 * allocated with hipHostMalloc; the copies are queued on `stream` (the caller synchronises). */
moe_status moe_pack_experts(const moe_shape *shape, const moe_layer *stack, int32_t n_layers,
                            void *container, size_t container_bytes, void *stream);

/*
 * moe_stack_decode with the routed experts read through expert_table instead of stack->w13 and
 * stack->w2 (which may then be NULL; every other field of `stack` is used as in moe_stack_decode).
 *   expert_table : uint64 [L][E], device memory, 16-byte aligned: the address of expert (l, e)'s
 *                  block (layout as moe_expert_stride) plus a mark in bit 0 (blocks are 4096-byte
 *                  aligned); each address must stay readable by the device, and its bytes
 *                  unchanged, until the call completes
 *   landing_opt  : NULL, or device memory (4096-byte aligned, landing_bytes >= L * T * K * stride)
 *                  for [L][T][K] blocks: every row the call reads from a marked block is also
 *                  stored to the landing block of its (layer, token, slot), so that all pieces of
 *                  a marked selected expert land there (the padding between pieces is not written)
 * Results are bit for bit those of moe_stack_decode on the same weights, wherever the blocks are.
 */
moe_status moe_stack_decode_table(const moe_shape *shape, const moe_layer *stack, int32_t n_layers,
                                  const uint64_t *expert_table, void *landing_opt,
                                  size_t landing_bytes, uint32_t flags, const uint16_t *x,
                                  int32_t T, float *y, uint16_t *x_all_opt, float *y_all_opt,
                                  int32_t *topk_idx_all_opt, float *topk_w_all_opt,
                                  float *logits_all_opt, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * moe_layer_batched with the routed experts read through one layer's row of an expert table
 * (uint64 [E], device memory, 8-byte aligned, entries as for moe_stack_decode_table, bit 0
 * ignored) instead of layer->w13 and layer->w2 (which may then be NULL). For prefill or batched
 * decode of a stack that lives in a container: blocks outside HBM are read over the bus as the
 * grouped GEMMs load them. Results are bit for bit those of moe_layer_batched.
 */
moe_status moe_layer_batched_table(const moe_shape *shape, const moe_layer *layer,
                                   const uint64_t *expert_table, const uint16_t *x, int32_t T,
                                   float *y, int32_t *topk_idx_opt, float *topk_w_opt,
                                   float *logits_opt, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* An expert cache: host-side policy state plus pinned staging copies of the table. Opaque; not
 * thread-safe (one caller at a time per cache). */
typedef struct moe_cache moe_cache;

/*
 * Creates a cache over a packed container of n_layers * E experts, with `slots` (0 <= slots <=
 * n_layers * E) pool slots of one stride each at `pool` (device memory, 4096-byte aligned, at
 * least slots * stride bytes; may be NULL when slots is 0), and writes the initial table (every
 * expert at its container block) to `table` (device, 16-byte aligned, uint64 [L][E]),
 * synchronously on `stream`. The container must be device memory or pinned host memory that the
 * device sees at the same address (checked: MOE_ERR_INVALID_ARG otherwise).
 * The caller owns container, pool and table and keeps them alive until moe_cache_destroy.
 * landing_opt: NULL, or the landing buffer the decode calls are given (landing_bytes for up to
 * landing_bytes / (n_layers * K * stride) tokens per call). With it every expert outside the pool
 * is marked in the table, and an expert admitted after a call is copied from its landing block
 * (device to device) instead of from the container.
 */
moe_status moe_cache_create(const moe_shape *shape, int32_t n_layers, const void *container,
                            size_t container_bytes, void *pool, size_t pool_bytes, int32_t slots,
                            uint64_t *table, size_t table_bytes, void *landing_opt,
                            size_t landing_bytes, void *stream, moe_cache **out);

/*
 * Feeds one decode call's routing (host int32 [L][T][top_k], every value in [0, E)) through the
 * policy in order (layer, token, slot), then queues on `stream` the copy of every newly admitted
 * expert's block into its slot and the rewrite of the table. Synchronises `stream` first (the
 * routing must come from a call on it that has completed). hits_opt / misses_opt: this call's
 * counts. Policy: a resident expert has a use count (1 on admission, +1 per hit) and a last-use
 * time; a miss takes the lowest free slot, else evicts the smallest count, oldest last use first.
 * The table is rewritten in two steps around the copies, so that it never names a slot being
 * overwritten; if a copy cannot be queued the table stays valid (no admitted expert in it), the
 * call returns MOE_ERR_HIP and so does every later update of this cache (destroy and recreate it).
 */
moe_status moe_cache_update(moe_cache *cache, const int32_t *topk_idx_all, int32_t T, int32_t top_k,
                            void *stream, int32_t *hits_opt, int32_t *misses_opt);

/*
 * Feeds n keys (host int32, each l * E + e) through the policy as accesses, then queues on
 * `stream` the admitted blocks' copies from the container and the table rewrite, as
 * moe_cache_update does (and synchronises `stream` first). For bringing in what a call is about
 * to read, e.g. the experts a prefill layer's routing selects before moe_layer_batched_table.
 */
moe_status moe_cache_admit(moe_cache *cache, const int32_t *keys, int64_t n, void *stream,
                           int32_t *hits_opt, int32_t *misses_opt);

/* Totals since creation: accesses that hit, that missed, and bytes copied into the pool. */
moe_status moe_cache_stats(const moe_cache *cache, uint64_t *hits, uint64_t *misses,
                           uint64_t *bytes_copied);

/* owner[slot] = l * E + e of the expert in each slot (after the copies queued so far), or -1. */
moe_status moe_cache_owners(const moe_cache *cache, int32_t *owner);

/* Frees the cache's host state (not the caller's container, pool or table). NULL is ignored. */
void moe_cache_destroy(moe_cache *cache);

/* The cache's policy on its own, host only: n accesses of keys in [0, n_keys) against `slots`
 * slots; per access hit (0/1), the slot the key then occupies (-1 when slots is 0) and the key it
 * evicted (-1 if none). */
moe_status moe_cache_policy_run(int32_t slots, int32_t n_keys, const int32_t *keys, int64_t n,
                                int32_t *hit, int32_t *slot, int32_t *evicted);

/* Workspace bytes for `kind` (MOE_WS_DECODE, MOE_WS_BATCHED, MOE_WS_STACK or MOE_WS_FORWARD), T
 * tokens and, for MOE_WS_STACK, n_layers layers (ignored otherwise); 0 if the arguments are
 * invalid. */
size_t moe_workspace_bytes(const moe_shape *shape, int32_t T, int32_t n_layers, int32_t kind);

/* Synchronises `stream`, then copies the workspace's device status word into *status. */
moe_status moe_read_status(const void *workspace, void *stream, int32_t *status);

/* Static, human-readable name of a status code. */
const char *moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
