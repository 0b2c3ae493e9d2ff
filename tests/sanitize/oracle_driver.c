/* Driver of the CPU oracle (oracle/moe_oracle.c) built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by tests/test_sanitizers.py: every entry
 * point on exactly-sized heap buffers (so any read or write past them is
 * caught), in every weight format, with and without the optional inputs,
 * plus the rejection paths.  Values are only checked for sanity here; the
 * oracle's results are pinned by the tests/test_oracle_*.py suites. */
#include "moe_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int failures = 0;
#define EXPECT(c)                                                              \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c);   \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

static uint64_t st = 20261203u;
static uint32_t rnd(void) {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(st >> 33);
}
static float frand(void) { return (float)(rnd() % 20001) / 10000.0f - 1.0f; }

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

/* Codes and scales of one [O][I] matrix in format fmt (exactly sized). */
static void make_matrix(int fmt, int O, int I, uint8_t **q, void **s) {
    const int packed = fmt == ORC_FMT_NVFP4 || fmt == ORC_FMT_INT4_ROW || fmt == ORC_FMT_INT4_G64;
    const size_t qb = (size_t)O * (packed ? I / 2 : I);
    *q = (uint8_t *)xmalloc(qb);
    for (size_t i = 0; i < qb; i++) {
        uint8_t c = (uint8_t)rnd();
        if ((fmt == ORC_FMT_FP8_B128 || fmt == ORC_FMT_FP8_B128_BF16S) && (c & 0x7F) == 0x7F) c ^= 1; /* no NaN */
        (*q)[i] = c;
    }
    if (fmt == ORC_FMT_FP8_B128) {
        const size_t n = (size_t)(O / 128) * (I / 128);
        float *f = (float *)xmalloc(n * 4);
        for (size_t i = 0; i < n; i++) f[i] = 1e-3f * (1 + rnd() % 7);
        *s = f;
    } else if (fmt == ORC_FMT_FP8_B128_BF16S) {
        const size_t n = (size_t)(O / 128) * (I / 128);
        uint16_t *b = (uint16_t *)xmalloc(n * 2);
        for (size_t i = 0; i < n; i++) b[i] = orc_f32_to_bf16_rne(1e-3f * (1 + rnd() % 7));
        *s = b;
    } else if (fmt == ORC_FMT_NVFP4) {
        const size_t n = (size_t)O * (I / 16);
        uint8_t *b = (uint8_t *)xmalloc(n);
        for (size_t i = 0; i < n; i++) b[i] = (uint8_t)(0x30 + rnd() % 0x20);   /* e4m3 around 1 */
        *s = b;
    } else {
        const int G = fmt == ORC_FMT_INT4_G64 ? 64 : I;
        const size_t n = (size_t)O * (I / G);
        float *f = (float *)xmalloc(n * 4);
        for (size_t i = 0; i < n; i++) f[i] = 1e-3f * (1 + rnd() % 5);
        *s = f;
    }
}

static void layer_case(int fmt, int with_bias, int with_gate, int Is) {
    const int H = 256, E = 16, k = 2, I = 128, R = 3;
    orc_expert *ex = (orc_expert *)xmalloc(sizeof(orc_expert) * E);
    for (int e = 0; e < E; e++) {
        void *gs, *ds;
        make_matrix(fmt, 2 * I, H, (uint8_t **)&ex[e].gu_q, &gs);
        make_matrix(fmt, H, I, (uint8_t **)&ex[e].dn_q, &ds);
        ex[e].gu_s = gs;
        ex[e].dn_s = ds;
        ex[e].gu_g = ex[e].dn_g = 1.0f / 64;
    }
    orc_expert sh;
    void *gs2, *ds2;
    if (Is) {
        make_matrix(fmt, 2 * Is, H, (uint8_t **)&sh.gu_q, &gs2);
        make_matrix(fmt, H, Is, (uint8_t **)&sh.dn_q, &ds2);
        sh.gu_s = gs2;
        sh.dn_s = ds2;
        sh.gu_g = sh.dn_g = 1.0f / 64;
    }
    uint16_t *wr = (uint16_t *)xmalloc((size_t)E * H * 2), *wsg = (uint16_t *)xmalloc((size_t)H * 2);
    float *bias = (float *)xmalloc((size_t)E * 4);
    for (int i = 0; i < E * H; i++) wr[i] = orc_f32_to_bf16_rne(0.05f * frand());
    for (int i = 0; i < H; i++) wsg[i] = orc_f32_to_bf16_rne(0.05f * frand());
    for (int e = 0; e < E; e++) bias[e] = 1e-3f * e;
    orc_layer L = {H, E, k, I, Is, fmt, wr, with_bias ? bias : NULL, with_gate ? wsg : NULL, ex, Is ? &sh : NULL};
    uint16_t *x = (uint16_t *)xmalloc((size_t)R * H * 2), *res = (uint16_t *)xmalloc((size_t)R * H * 2);
    for (int i = 0; i < R * H; i++) {
        x[i] = orc_f32_to_bf16_rne(frand());
        res[i] = orc_f32_to_bf16_rne(frand());
    }
    float *logits = (float *)xmalloc((size_t)R * E * 4), *s = (float *)xmalloc((size_t)R * 4);
    int32_t *ids = (int32_t *)xmalloc((size_t)R * k * 4);
    float *w = (float *)xmalloc((size_t)R * k * 4), *y = (float *)xmalloc((size_t)R * H * 4);
    uint16_t *out = (uint16_t *)xmalloc((size_t)R * H * 2);
    EXPECT(orc_router_logits(&L, x, R, logits) == 0);
    EXPECT(orc_shared_gate(&L, x, R, s) == 0);
    for (int logits_given = 0; logits_given < 2; logits_given++) {
        EXPECT(orc_layer_forward(&L, x, R, logits_given ? logits : NULL, res, ids, w, s, y, out) == 0);
        for (int r = 0; r < R; r++) {
            double sw = 0;
            for (int j = 0; j < k; j++) {
                EXPECT(ids[r * k + j] >= 0 && ids[r * k + j] < E);
                sw += w[r * k + j];
            }
            EXPECT(fabs(sw - 1.0) < 1e-5);
        }
        for (int i = 0; i < R * H; i++) EXPECT(isfinite(y[i]));
        EXPECT(orc_layer_forward(&L, x, R, NULL, NULL, NULL, NULL, NULL, y, NULL) == 0);   /* optional outputs */
    }
    double *d = (double *)xmalloc((size_t)H * 8);
    EXPECT(orc_expert_apply(&L, &ex[3], I, x, d) == 0);
    for (int i = 0; i < H; i++) EXPECT(isfinite(d[i]));
    int32_t *cnt = (int32_t *)xmalloc((size_t)E * 4), *off = (int32_t *)xmalloc((size_t)(E + 1) * 4);
    int32_t *perm = (int32_t *)xmalloc((size_t)R * k * 4);
    EXPECT(orc_group(ids, R, k, E, cnt, off, perm) == 0);
    EXPECT(off[E] == R * k);
    free(d); free(cnt); free(off); free(perm);
    free(logits); free(s); free(ids); free(w); free(y); free(out); free(x); free(res);
    free(wr); free(wsg); free(bias);
    for (int e = 0; e < E; e++) {
        free((void *)ex[e].gu_q); free((void *)ex[e].gu_s); free((void *)ex[e].dn_q); free((void *)ex[e].dn_s);
    }
    free(ex);
    if (Is) { free((void *)sh.gu_q); free((void *)sh.gu_s); free((void *)sh.dn_q); free((void *)sh.dn_s); }
}

int main(void) {
    for (int c = 0; c < 256; c++) { float v = orc_e4m3_to_f32((uint8_t)c); (void)v; }
    for (int c = 0; c < 16; c++) {
        EXPECT(isfinite(orc_e2m1_to_f32((uint8_t)c)));
        EXPECT(isfinite(orc_int4_to_f32((uint8_t)c)));
    }
    for (int c = 0; c < 256; c++) EXPECT(isfinite(orc_int8_to_f32((uint8_t)c)));
    for (uint32_t b = 0; b < 65536; b += 7) { float f = orc_bf16_to_f32((uint16_t)b); (void)orc_f32_to_bf16_rne(f); }
    for (int fmt = 0; fmt <= 5; fmt++)
        for (int variant = 0; variant < 3; variant++)
            layer_case(fmt, variant != 1, variant != 2, variant == 2 ? 0 : 256);
    /* top-k with ties and k = E, on exactly-sized rows */
    {
        const int R = 4, E = 12;
        float *l = (float *)xmalloc((size_t)R * E * 4);
        for (int i = 0; i < R * E; i++) l[i] = (float)(rnd() % 3);
        int32_t *ids = (int32_t *)xmalloc((size_t)R * E * 4);
        float *w = (float *)xmalloc((size_t)R * E * 4);
        EXPECT(orc_topk_softmax(l, R, E, E, ids, w) == 0);
        EXPECT(orc_topk_softmax(l, R, E, 1, ids, w) == 0 && w[0] == 1.0f);
        EXPECT(orc_topk_softmax(l, R, E, E + 1, ids, w) != 0);
        EXPECT(orc_topk_softmax(NULL, R, E, 2, ids, w) != 0);
        free(l); free(ids); free(w);
    }
    /* RMSNorm and the dense projection */
    {
        const int R = 3, H = 256, N = 256, K = 384;
        uint16_t *x = (uint16_t *)xmalloc((size_t)R * K * 2), *g = (uint16_t *)xmalloc((size_t)K * 2);
        uint16_t *o = (uint16_t *)xmalloc((size_t)R * K * 2);
        for (int i = 0; i < R * K; i++) x[i] = orc_f32_to_bf16_rne(frand());
        for (int i = 0; i < K; i++) g[i] = orc_f32_to_bf16_rne(1.0f + 0.1f * frand());
        EXPECT(orc_rms_norm(x, R, H, g, 1e-6, o) == 0);
        uint8_t *q;
        void *sc;
        make_matrix(ORC_FMT_FP8_B128, N, K, &q, &sc);
        double *y = (double *)xmalloc((size_t)R * N * 8);
        EXPECT(orc_dense_fp8(q, (const float *)sc, N, K, x, R, y) == 0);
        for (int i = 0; i < R * N; i++) EXPECT(isfinite(y[i]));
        EXPECT(orc_dense_fp8(q, (const float *)sc, N, 100, x, R, y) != 0);
        float *W = (float *)xmalloc((size_t)N * K * 4);
        EXPECT(orc_dequant_fp8(q, (const float *)sc, N, K, W) == 0);
        free(q); free(sc); free(y); free(W); free(x); free(g); free(o);
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle OK\n");
    return 0;
}
