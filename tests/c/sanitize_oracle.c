/*
 * Driver of the C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitize_cpu.py (compiled without OpenMP: one thread, the same arithmetic). It takes
 * the oracle's source whole and calls its entry points on small seeded layers whose every array is
 * heap-allocated to its exact size, so that a read or write past any of them is reported; the
 * results are checked for the invariants the definitions fix (distinct in-range selections,
 * weights summing to one, finite outputs).
 */
#include "../../oracle/moe_oracle.c"

#include <stdio.h>

static uint64_t rs = 0x2545F4914F6CDD1Dull;
static uint32_t rnd(void) {  /* xorshift64* */
    rs ^= rs >> 12; rs ^= rs << 25; rs ^= rs >> 27;
    return (uint32_t)((rs * 0x2545F4914F6CDD1Dull) >> 32);
}
static double unif(void) { return (rnd() + 0.5) / 4294967296.0; }       /* (0, 1) */
static uint16_t bf16_of(double v) { return orc_double_to_bf16(v); }

static void *fill_codes(size_t n) { uint8_t *p = malloc(n); for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)rnd(); return p; }
static uint16_t *fill_bf16(size_t n, double lo, double hi) {
    uint16_t *p = malloc(sizeof(uint16_t) * n);
    for (size_t i = 0; i < n; ++i) p[i] = bf16_of(lo + (hi - lo) * unif());
    return p;
}
static float *fill_f32(size_t n, double amp) {
    float *p = malloc(sizeof(float) * n);
    for (size_t i = 0; i < n; ++i) p[i] = (float)(amp * (2.0 * unif() - 1.0));
    return p;
}

static int one_case(int H, int E, int K, int I, int Is, int bits, int T, int with_bias) {
    const int G = 64;
    orc_shape sh = {H, E, K, I, Is, bits, G};
    orc_layer L;
    const size_t cpr13 = (size_t)H * bits / 8, cpr2 = (size_t)I * bits / 8, cprs2 = (size_t)Is * bits / 8;
    L.router = fill_f32((size_t)E * H, 0.05);
    L.router_bias = with_bias ? fill_f32((size_t)E, 0.5) : NULL;
    L.shared_gate = Is ? fill_f32((size_t)H, 0.05) : NULL;
    L.w13_codes = fill_codes((size_t)E * 2 * I * cpr13);
    L.w13_scales = fill_bf16((size_t)E * 2 * I * (H / G), 1e-3, 2e-2);
    L.w13_biases = fill_bf16((size_t)E * 2 * I * (H / G), -0.1, 0.1);
    L.w2_codes = fill_codes((size_t)E * H * cpr2);
    L.w2_scales = fill_bf16((size_t)E * H * (I / G), 1e-3, 2e-2);
    L.w2_biases = fill_bf16((size_t)E * H * (I / G), -0.1, 0.1);
    L.s13_codes = Is ? fill_codes((size_t)2 * Is * cpr13) : NULL;
    L.s13_scales = Is ? fill_bf16((size_t)2 * Is * (H / G), 1e-3, 2e-2) : NULL;
    L.s13_biases = Is ? fill_bf16((size_t)2 * Is * (H / G), -0.1, 0.1) : NULL;
    L.s2_codes = Is ? fill_codes((size_t)H * cprs2) : NULL;
    L.s2_scales = Is ? fill_bf16((size_t)H * (Is / G), 1e-3, 2e-2) : NULL;
    L.s2_biases = Is ? fill_bf16((size_t)H * (Is / G), -0.1, 0.1) : NULL;
    uint16_t *x = fill_bf16((size_t)T * H, -2.0, 2.0);
    double *lg = malloc(sizeof(double) * (size_t)T * E), *w = malloc(sizeof(double) * (size_t)T * K);
    double *gam = malloc(sizeof(double) * (size_t)T), *y = malloc(sizeof(double) * (size_t)T * H);
    double *y2 = malloc(sizeof(double) * (size_t)T * H);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)T * K), *idx2 = malloc(sizeof(int32_t) * (size_t)T * K);
    float *lf = malloc(sizeof(float) * (size_t)T * E);
    uint16_t *xn = malloc(sizeof(uint16_t) * (size_t)H);
    int bad = orc_layer_forward(&sh, &L, x, T, NULL, lg, idx, w, gam, y) != 0;
    for (int t = 0; t < T && !bad; ++t) {
        double ws = 0.0;
        for (int k = 0; k < K; ++k) {
            const int e = idx[t * K + k];
            bad |= e < 0 || e >= E;
            for (int j = 0; j < k; ++j) bad |= idx[t * K + j] == e;
            if (k) bad |= lg[(size_t)t * E + e] > lg[(size_t)t * E + idx[t * K + k - 1]];
            ws += w[t * K + k];
        }
        bad |= fabs(ws - 1.0) > 1e-12;
        for (int h = 0; h < H; ++h) bad |= !isfinite(y[(size_t)t * H + h]);
        if (bad) printf("invariant broken: H=%d E=%d K=%d bits=%d token %d\n", H, E, K, bits, t);
    }
    /* given logits (the fp32 image of the oracle's own) and the outputs left NULL */
    for (size_t i = 0; i < (size_t)T * E; ++i) lf[i] = (float)lg[i];
    bad |= orc_layer_forward(&sh, &L, x, T, lf, NULL, idx2, NULL, NULL, y2) != 0;
    orc_rms_glue(y, H, 1e-6, xn);
    int32_t *all = malloc(sizeof(int32_t) * (size_t)E);
    orc_topk(lg, E, E, all);  /* K = E: a full ordering */
    for (int e = 1; e < E; ++e) bad |= lg[all[e]] > lg[all[e - 1]];
    free(all);
    double *row = malloc(sizeof(double) * (size_t)H);
    orc_dequant_row(L.w13_codes, L.w13_scales, L.w13_biases, H, bits, G, 2 * I - 1, row);  /* last row */
    free(row);
    /* an argument the oracle does not handle is refused, not read */
    orc_shape odd = sh;
    odd.bits = 3;
    bad |= orc_layer_forward(&odd, &L, x, T, NULL, NULL, NULL, NULL, NULL, y2) != -1;
    free((void *)L.router); free((void *)L.router_bias); free((void *)L.shared_gate);
    free((void *)L.w13_codes); free((void *)L.w13_scales); free((void *)L.w13_biases);
    free((void *)L.w2_codes); free((void *)L.w2_scales); free((void *)L.w2_biases);
    free((void *)L.s13_codes); free((void *)L.s13_scales); free((void *)L.s13_biases);
    free((void *)L.s2_codes); free((void *)L.s2_scales); free((void *)L.s2_biases);
    free(x); free(lg); free(w); free(gam); free(y); free(y2); free(idx); free(idx2); free(lf); free(xn);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= one_case(128, 8, 3, 64, 64, 4, 3, 1);
    bad |= one_case(128, 8, 3, 64, 64, 8, 2, 0);
    bad |= one_case(256, 16, 16, 128, 0, 4, 2, 1);  /* K = E, no shared expert */
    bad |= one_case(64, 4, 1, 64, 128, 8, 1, 0);    /* K = 1, shared wider than routed */
    bad |= one_case(192, 5, 2, 192, 64, 4, 4, 1);   /* sizes that are not powers of two */
    if (bad) return 1;
    printf("oracle sanitizer checks passed\n");
    return 0;
}
