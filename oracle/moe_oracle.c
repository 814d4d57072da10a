/*
 * moe_oracle.c -- plain, slow, fp64 CPU reference of the sparse MoE FFN layer at decode.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load this library. It shares no code, header, table or helper with the HIP library:
 * it has its own structs, its own bf16 decoding and its own nibble unpacking.
 *
 * What the layer computes (per token t; every step is written out with no blocking, fusion
 * or reordering beyond the definition):
 *   1. x = the bf16 input row, read exactly into doubles.
 *   2. Router logits l[e] = sum_h x[h] * R[e][h] (+ bias[e]), fp32 router weights.
 *      Each token is routed to 8 of 256 experts (35B-A3B) or 10 of 512 (80B-A3B)
 *      (xix.ai Swiftlet article, paragraph on scheduling; Runnel README, "Target").
 *   3. p = softmax(l) over all E experts; S = the K indices with the largest logits, ordered
 *      by (logit descending, index ascending); w_k = p[S_k] / sum_{j in S} p[j].
 *      The pages name top-k routing but print no formula: this is the plainest reading,
 *      softmax then top-k then renormalise, with selection on logits (softmax is monotone).
 *   4. For each selected expert: dequantise its packed gate|up matrix W13 ([2I x H], rows
 *      0..I-1 gate, I..2I-1 up; Runnel README, intro and "Streaming CLI") and its down
 *      matrix W2 ([H x I]) with the MLX-style affine group rule w = scale * q + bias, one bf16
 *      scale and bias per row and group of 64 input columns (xix.ai Swiftlet article,
 *      paragraph on lineage). 4-bit: input column 2j is the low nibble of byte j.
 *      g = W13[0:I] x, u = W13[I:2I] x, h = silu(g) * u, d = W2 h.
 *   5. The always-on shared expert (xix.ai article, paragraphs on scheduling and lineage;
 *      Runnel README, "Target") runs the same way with its own intermediate size and is
 *      scaled by gamma = sigmoid(x . g_s), a scalar gate per token.
 *   6. y = sum_k w_k d_{S_k} + gamma * d_shared, summed in the order k = 0..K-1, then shared.
 * All accumulation is in double. Parallel loops (OpenMP) only split independent output rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t hidden, num_experts, top_k, inter, shared_inter, bits, group;
} orc_shape;

typedef struct {
    const float *router;      /* [E][H] */
    const float *router_bias; /* [E] or NULL */
    const float *shared_gate; /* [H] or NULL */
    const uint8_t *w13_codes; const uint16_t *w13_scales, *w13_biases; /* [E][2I][H*bits/8], [E][2I][H/G] */
    const uint8_t *w2_codes;  const uint16_t *w2_scales,  *w2_biases;  /* [E][H][I*bits/8],  [E][H][I/G]  */
    const uint8_t *s13_codes; const uint16_t *s13_scales, *s13_biases; /* shared expert, Is in place of I */
    const uint8_t *s2_codes;  const uint16_t *s2_scales,  *s2_biases;
} orc_layer;

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* bf16 is the top half of an IEEE binary32: widen by appending 16 zero bits. */
double orc_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16, ties to even (8 significant bits, binary32 exponent range). */
uint16_t orc_double_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    double r;
    if (v == 0.0) {
        r = v;
    } else if (fabs(v) < ldexp(1.0, -126)) {
        r = rint(v * ldexp(1.0, 133)) * ldexp(1.0, -133); /* subnormal spacing 2^-133 */
    } else {
        int e;
        double m = frexp(v, &e);          /* v = m * 2^e, 0.5 <= |m| < 1 */
        r = ldexp(rint(m * 256.0), e - 8); /* 8 significant bits, rint = ties-to-even */
    }
    float f = (float)r; /* exact unless it overflows to inf, which is the right answer */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Code of input column c of one packed row. */
static int orc_code(const uint8_t *row, int c, int bits) {
    if (bits == 8) return row[c];
    uint8_t byte = row[c / 2];
    return (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* Dequantise row r of a [rows x cols] group-quantised matrix: w[c] = scale[c/G] * q[c] + bias[c/G]. */
void orc_dequant_row(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                     int cols, int bits, int group, int r, double *out) {
    const uint8_t *crow = codes + (size_t)r * (size_t)(cols * bits / 8);
    const uint16_t *srow = scales + (size_t)r * (size_t)(cols / group);
    const uint16_t *brow = biases + (size_t)r * (size_t)(cols / group);
    for (int c = 0; c < cols; ++c) {
        double s = orc_bf16_to_double(srow[c / group]);
        double b = orc_bf16_to_double(brow[c / group]);
        out[c] = s * (double)orc_code(crow, c, bits) + b;
    }
}

/* out[r] = sum_c W[r][c] * v[c] for a group-quantised [rows x cols] matrix. */
void orc_qmatvec(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                 int rows, int cols, int bits, int group, const double *v, double *out) {
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)cols);
#pragma omp for schedule(static)
        for (int r = 0; r < rows; ++r) {
            orc_dequant_row(codes, scales, biases, cols, bits, group, r, w);
            double acc = 0.0;
            for (int c = 0; c < cols; ++c) acc += w[c] * v[c];
            out[r] = acc;
        }
        free(w);
    }
}

/* l[e] = sum_h x[h] R[e][h] (+ bias[e]). */
void orc_router_logits(const double *x, const float *R, const float *bias, int E, int H, double *l) {
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h) acc += x[h] * (double)R[(size_t)e * H + h];
        l[e] = acc + (bias ? (double)bias[e] : 0.0);
    }
}

/* "a ranks before b": larger logit first, equal logits by lower index (+0 and -0 compare equal). */
static int orc_before(const double *l, int a, int b) {
    return (l[a] > l[b]) || (l[a] == l[b] && a < b);
}

/* The K experts with the largest logits, in order (logit descending, index ascending):
 * K passes of a plain linear scan, each taking the best expert not yet taken. */
void orc_topk(const double *l, int E, int K, int32_t *idx) {
    char *taken = (char *)calloc((size_t)E, 1);
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || orc_before(l, e, best))) best = e;
        taken[best] = 1;
        idx[k] = best;
    }
    free(taken);
}

/* p = softmax(l) over all E experts (maximum subtracted), then w_k = p[S_k] / sum_{j in S} p[j]. */
void orc_route_weights(const double *l, int E, const int32_t *idx, int K, double *w) {
    double m = l[0];
    for (int e = 1; e < E; ++e) if (l[e] > m) m = l[e];
    double z = 0.0;
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    for (int e = 0; e < E; ++e) { p[e] = exp(l[e] - m); z += p[e]; }
    for (int e = 0; e < E; ++e) p[e] /= z;
    double s = 0.0;
    for (int k = 0; k < K; ++k) s += p[idx[k]];
    for (int k = 0; k < K; ++k) w[k] = p[idx[k]] / s;
    free(p);
}

double orc_sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* g = W13[0:I] x and u = W13[I:2I] x for one expert (packed gate|up matrix of 2I rows). */
void orc_gate_up(const uint8_t *c13, const uint16_t *s13, const uint16_t *b13,
                 int H, int I, int bits, int group, const double *x, double *g, double *u) {
    double *gu = (double *)malloc(sizeof(double) * 2 * (size_t)I);
    orc_qmatvec(c13, s13, b13, 2 * I, H, bits, group, x, gu);
    memcpy(g, gu, sizeof(double) * (size_t)I);
    memcpy(u, gu + I, sizeof(double) * (size_t)I);
    free(gu);
}

/* SwiGLU: h = silu(g) * u with silu(v) = v * sigmoid(v). */
void orc_swiglu(const double *g, const double *u, int I, double *h) {
    for (int j = 0; j < I; ++j) h[j] = g[j] * orc_sigmoid(g[j]) * u[j];
}

/* One expert MLP: d = W2 (silu(W_gate x) * (W_up x)); h_out (may be NULL) receives h. */
void orc_expert(const uint8_t *c13, const uint16_t *s13, const uint16_t *b13,
                const uint8_t *c2, const uint16_t *s2, const uint16_t *b2,
                int H, int I, int bits, int group, const double *x, double *h_out, double *d) {
    double *g = (double *)malloc(sizeof(double) * (size_t)I);
    double *u = (double *)malloc(sizeof(double) * (size_t)I);
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    orc_gate_up(c13, s13, b13, H, I, bits, group, x, g, u);
    orc_swiglu(g, u, I, h);
    orc_qmatvec(c2, s2, b2, H, I, bits, group, h, d);
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
    free(g); free(u); free(h);
}

/*
 * The whole layer for T tokens.
 *   logits_in : NULL -> select on the oracle's own fp64 logits;
 *               else [T][E] fp32 logits to select on (read exactly as doubles), so that a test can
 *               make both sides take the selection from identical logits.
 *   outputs   : logits_out [T][E], idx_out [T][K], w_out [T][K], gamma_out [T], y_out [T][H];
 *               any may be NULL except y_out.
 * Returns 0, or -1 on an argument the oracle does not handle.
 */
int orc_layer_forward(const orc_shape *sh, const orc_layer *L, const uint16_t *x_bf16, int T,
              const float *logits_in, double *logits_out, int32_t *idx_out, double *w_out,
              double *gamma_out, double *y_out) {
    const int H = sh->hidden, E = sh->num_experts, K = sh->top_k, I = sh->inter;
    const int Is = sh->shared_inter, bits = sh->bits, G = sh->group;
    if (K < 1 || K > E || (bits != 4 && bits != 8) || G <= 0 || H % G || I % G || (Is && Is % G))
        return -1;
    const size_t cpr13 = (size_t)H * bits / 8, cpr2 = (size_t)I * bits / 8;
    double *x = (double *)malloc(sizeof(double) * (size_t)H);
    double *l = (double *)malloc(sizeof(double) * (size_t)E);
    double *w = (double *)malloc(sizeof(double) * (size_t)K);
    double *d = (double *)malloc(sizeof(double) * (size_t)H);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) x[h] = orc_bf16_to_double(x_bf16[(size_t)t * H + h]);
        if (logits_in) {
            for (int e = 0; e < E; ++e) l[e] = (double)logits_in[(size_t)t * E + e];
        } else {
            orc_router_logits(x, L->router, L->router_bias, E, H, l);
        }
        orc_topk(l, E, K, idx);
        orc_route_weights(l, E, idx, K, w);
        double *y = y_out + (size_t)t * H;
        for (int h = 0; h < H; ++h) y[h] = 0.0;
        for (int k = 0; k < K; ++k) {
            const size_t e = (size_t)idx[k];
            orc_expert(L->w13_codes + e * 2 * I * cpr13, L->w13_scales + e * 2 * I * (H / G),
                       L->w13_biases + e * 2 * I * (H / G),
                       L->w2_codes + e * H * cpr2, L->w2_scales + e * H * (I / G),
                       L->w2_biases + e * H * (I / G), H, I, bits, G, x, NULL, d);
            for (int h = 0; h < H; ++h) y[h] += w[k] * d[h];
        }
        double gamma = 0.0;
        if (Is) {
            double dot = 0.0;
            for (int h = 0; h < H; ++h) dot += x[h] * (double)L->shared_gate[h];
            gamma = orc_sigmoid(dot);
            orc_expert(L->s13_codes, L->s13_scales, L->s13_biases, L->s2_codes, L->s2_scales,
                       L->s2_biases, H, Is, bits, G, x, NULL, d);
            for (int h = 0; h < H; ++h) y[h] += gamma * d[h];
        }
        if (logits_out) memcpy(logits_out + (size_t)t * E, l, sizeof(double) * (size_t)E);
        if (idx_out) memcpy(idx_out + (size_t)t * K, idx, sizeof(int32_t) * (size_t)K);
        if (w_out) memcpy(w_out + (size_t)t * K, w, sizeof(double) * (size_t)K);
        if (gamma_out) gamma_out[t] = gamma;
    }
    free(x); free(l); free(w); free(d); free(idx);
    return 0;
}

/*
 * Inter-layer glue used to chain a stack of MoE layers at decode (not part of the MoE method:
 * it stands in for the norm and mixer that sit between MoE layers in the models):
 *   x_next = bf16_round_to_nearest_even( y / sqrt(mean(y^2) + eps) )
 */
void orc_rms_glue(const double *y, int H, double eps, uint16_t *x_next) {
    double ss = 0.0;
    for (int h = 0; h < H; ++h) ss += y[h] * y[h];
    double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int h = 0; h < H; ++h) x_next[h] = orc_double_to_bf16(y[h] * inv);
}
