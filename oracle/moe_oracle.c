/*
 * moe_oracle.c -- plain, slow, obviously correct CPU definition of the
 * decode-step MoE FFN (see moe_oracle.h for the formula and the formats).
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code
 * with the HIP library.  Floating point is carried in double; the weight
 * decoders are written from the bit layouts of the formats, not from tables.
 *
 * Sources for what is computed:
 *  - GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels" table: a bf16 dense
 *    GEMV (the router), moe_topk_softmax (f32 weights, i32 ids: "Precision",
 *    node outputs f32,i32), gate/up of routed and shared experts in one
 *    kernel, silu+down of routed and shared experts, a weighted-sum blend.
 *  - same page, "Precision": fp8/block128x128 weights read bf16 activations
 *    (gate/up) and f32 activations (down, i.e. the f32 silu*mul product).
 *  - colibri pull request 1992, "What it is": the MoE output of a layer joins
 *    the residual; the shared expert has its own gate.
 *  - Qwen3-8B architecture card, "Exported PyTorch": the SwiGLU FFN with
 *    gate_proj, up_proj and down_proj.
 *  - "Inspecting Qwen3.5-397B-A17B-NVFP4", "The Architectural Revelations":
 *    512 experts, 10 per token, weights stored as NVFP4.
 * Readings where the pages are silent are listed in the repository's design
 * notes; each is restated beside the code it governs.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

void orc_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int orc_get_threads(void) { return g_threads; }

/* ---------------------------------------------------------------- formats */

/* bf16 is the upper half of an IEEE-754 binary32: widening is exact. */
float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to the nearest bf16, ties to even; NaN stays NaN. */
uint16_t orc_f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* OCP 8-bit E4M3 ("FN" variant): sign, 4 exponent bits with bias 7, 3
 * mantissa bits.  Exponent field 0 encodes subnormals m/8 * 2^-6; the all-ones
 * pattern S.1111.111 is NaN; there is no infinity, so 0x7E = 448 is the top. */
float orc_e4m3_to_f32(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return (float)NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* 4-bit E2M1: sign, 2 exponent bits with bias 1, 1 mantissa bit.  Exponent
 * field 0 is the subnormal m/2, so the magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6. */
float orc_e2m1_to_f32(uint8_t nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (float)(s ? -v : v);
}

/* Two's-complement 8-bit integer: bytes 0..127 are 0..127, 128..255 are
 * -128..-1. */
float orc_int8_to_f32(uint8_t c)
{
    int v = c;
    return (float)(v >= 128 ? v - 256 : v);
}

/* Two's-complement 4-bit integer: nibbles 0..7 are 0..7, 8..15 are -8..-1. */
float orc_int4_to_f32(uint8_t nib)
{
    int v = nib & 15;
    return (float)(v >= 8 ? v - 16 : v);
}

/* ---------------------------------------------------------------- weights */

/* fp8 block-128x128: scale array is [O/128][I/128], one f32 per block;
 * the dequantised weight is code * scale, held as f32 (GB10 blueprint,
 * "Precision": fp8/block128x128; reading: the scale multiplies). */
static float w_fp8(const uint8_t *q, const float *scale, int I, int o, int i)
{
    double code = orc_e4m3_to_f32(q[(size_t)o * I + i]);
    double sc = scale[(size_t)(o / 128) * (size_t)(I / 128) + (size_t)(i / 128)];
    return (float)(code * sc);
}

/* fp8 block-128x128 with bf16 scales (colibri PR: a fixture of fp8 experts
 * with BF16 128x128 block scales): the scale is a bf16, widened exactly. */
static float w_fp8_bf16s(const uint8_t *q, const uint16_t *scale, int I, int o, int i)
{
    double code = orc_e4m3_to_f32(q[(size_t)o * I + i]);
    double sc = orc_bf16_to_f32(scale[(size_t)(o / 128) * (size_t)(I / 128) + (size_t)(i / 128)]);
    return (float)(code * sc);
}

/* NVFP4 ("Inspecting Qwen3.5-397B-A17B-NVFP4": NVIDIA's 4-bit float).  The
 * layout is a reading: two codes per byte, the even column in the low nibble;
 * one e4m3 scale per 16 consecutive columns of a row; one f32 global scale
 * per matrix; all three multiply. */
static float w_nvfp4(const uint8_t *q, const uint8_t *scale, float g, int I, int o, int i)
{
    uint8_t byte = q[(size_t)o * (size_t)(I / 2) + (size_t)(i / 2)];
    uint8_t nib = (i & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    double code = orc_e2m1_to_f32(nib);
    double sc = orc_e4m3_to_f32(scale[(size_t)o * (size_t)(I / 16) + (size_t)(i / 16)]);
    return (float)(code * sc * (double)g);
}

/* Integer experts (colibri PR: a per-row int4 checkpoint of Qwen3.6, an
 * int4-g64 expert sidecar, int8 rows in its decode GEMV).  The layout is a
 * reading: symmetric two's-complement codes; int4 two per byte with the even
 * column in the low nibble; one f32 scale per G consecutive input columns of
 * a row (G = the row length for the per-row formats, 64 for g64), scale
 * array [O][I/G]; the scale multiplies. */
static int int_group(int fmt, int I) { return fmt == ORC_FMT_INT4_G64 ? 64 : I; }

static float w_int(int fmt, const uint8_t *q, const float *scale, int I, int o, int i)
{
    double code;
    if (fmt == ORC_FMT_INT8_ROW) {
        code = orc_int8_to_f32(q[(size_t)o * (size_t)I + (size_t)i]);
    } else {
        uint8_t byte = q[(size_t)o * (size_t)(I / 2) + (size_t)(i / 2)];
        code = orc_int4_to_f32((i & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15));
    }
    const int G = int_group(fmt, I);
    double sc = scale[(size_t)o * (size_t)(I / G) + (size_t)(i / G)];
    return (float)(code * sc);
}

static int known_format(int fmt) { return fmt >= ORC_FMT_FP8_B128 && fmt <= ORC_FMT_FP8_B128_BF16S; }

static float weight(int fmt, const uint8_t *q, const void *s, float g, int I, int o, int i)
{
    if (fmt == ORC_FMT_NVFP4)
        return w_nvfp4(q, (const uint8_t *)s, g, I, o, i);
    if (fmt == ORC_FMT_FP8_B128)
        return w_fp8(q, (const float *)s, I, o, i);
    if (fmt == ORC_FMT_FP8_B128_BF16S)
        return w_fp8_bf16s(q, (const uint16_t *)s, I, o, i);
    return w_int(fmt, q, (const float *)s, I, o, i);
}

int orc_dequant_fp8(const uint8_t *q, const float *scale, int O, int I, float *W)
{
    if (!q || !scale || !W || O <= 0 || I <= 0 || O % 128 || I % 128)
        return -1;
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = w_fp8(q, scale, I, o, i);
    return 0;
}

int orc_dequant_nvfp4(const uint8_t *q, const uint8_t *scale, float g, int O, int I, float *W)
{
    if (!q || !scale || !W || O <= 0 || I <= 0 || I % 16)
        return -1;
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = w_nvfp4(q, scale, g, I, o, i);
    return 0;
}

int orc_dequant_fp8_bf16s(const uint8_t *q, const uint16_t *scale, int O, int I, float *W)
{
    if (!q || !scale || !W || O <= 0 || I <= 0 || O % 128 || I % 128)
        return -1;
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = w_fp8_bf16s(q, scale, I, o, i);
    return 0;
}

int orc_dequant_int(int fmt, const uint8_t *q, const float *scale, int O, int I, float *W)
{
    if (!q || !scale || !W || O <= 0 || I <= 0)
        return -1;
    if (fmt != ORC_FMT_INT8_ROW && fmt != ORC_FMT_INT4_ROW && fmt != ORC_FMT_INT4_G64)
        return -1;
    if ((fmt != ORC_FMT_INT8_ROW && I % 2) || (fmt == ORC_FMT_INT4_G64 && I % 64))
        return -1;
    for (int o = 0; o < O; o++)
        for (int i = 0; i < I; i++)
            W[(size_t)o * I + i] = w_int(fmt, q, scale, I, o, i);
    return 0;
}

/* ---------------------------------------------------------------- routing */

/* Router GEMV over bf16 weights and activations (GB10 blueprint, "Kernels":
 * gemv::dense_gemv_bf16; "Precision": bf16 weight, bf16 activation).  The sum
 * is exact-ish in double, rounded once to f32, then the optional f32 bias is
 * added in f32. */
int orc_router_logits(const orc_layer *L, const uint16_t *x, int R, float *logits)
{
    if (!L || !x || !logits || !L->router_w || R < 0)
        return -1;
    const int H = L->hidden, E = L->n_experts;
    for (int r = 0; r < R; r++)
        for (int e = 0; e < E; e++) {
            double acc = 0.0;
            for (int h = 0; h < H; h++)
                acc += (double)orc_bf16_to_f32(x[(size_t)r * H + h]) *
                       (double)orc_bf16_to_f32(L->router_w[(size_t)e * H + h]);
            float l = (float)acc;
            if (L->router_bias)
                l = l + L->router_bias[e];
            logits[(size_t)r * E + e] = l;
        }
    return 0;
}

/* The shared expert's gate: a logistic sigmoid of one dot product per row
 * (colibri pull request 1992, "What it is": the shared expert and its gate). */
int orc_shared_gate(const orc_layer *L, const uint16_t *x, int R, float *s)
{
    if (!L || !x || !s || R < 0)
        return -1;
    const int H = L->hidden;
    for (int r = 0; r < R; r++) {
        if (!L->shared_gate_w) {
            s[r] = 1.0f;
            continue;
        }
        double acc = 0.0;
        for (int h = 0; h < H; h++)
            acc += (double)orc_bf16_to_f32(x[(size_t)r * H + h]) *
                   (double)orc_bf16_to_f32(L->shared_gate_w[h]);
        s[r] = (float)(1.0 / (1.0 + exp(-acc)));
    }
    return 0;
}

typedef struct {
    double p;
    int e;
} prob_idx;

/* Total order used for top-k: larger probability first, lower expert index
 * first among equal probabilities. */
static int cmp_prob_desc(const void *a, const void *b)
{
    const prob_idx *x = (const prob_idx *)a, *y = (const prob_idx *)b;
    if (x->p > y->p) return -1;
    if (x->p < y->p) return 1;
    return (x->e > y->e) - (x->e < y->e);
}

/* Softmax over every expert, then the k largest by a full sort, then the
 * chosen probabilities divided by their own sum (GB10 blueprint, "Kernels":
 * moe_topk_softmax, node output f32,i32). */
int orc_topk_softmax(const float *logits, int R, int E, int k, int32_t *ids, float *w)
{
    if (!logits || !ids || !w || R < 0 || E <= 0 || k <= 0 || k > E)
        return -1;
    prob_idx *pi = (prob_idx *)malloc(sizeof(prob_idx) * (size_t)E);
    if (!pi)
        return -2;
    for (int r = 0; r < R; r++) {
        const float *l = logits + (size_t)r * E;
        double m = l[0];
        for (int e = 1; e < E; e++)
            if (l[e] > m) m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; e++) {
            pi[e].p = exp((double)l[e] - m);
            pi[e].e = e;
            z += pi[e].p;
        }
        for (int e = 0; e < E; e++)
            pi[e].p /= z;
        qsort(pi, (size_t)E, sizeof(prob_idx), cmp_prob_desc);
        double sk = 0.0;
        for (int j = 0; j < k; j++)
            sk += pi[j].p;
        for (int j = 0; j < k; j++) {
            ids[(size_t)r * k + j] = pi[j].e;
            w[(size_t)r * k + j] = (float)(pi[j].p / sk);
        }
    }
    free(pi);
    return 0;
}

/* Grouping by expert for a multi-row step: a double loop, experts ascending,
 * rows ascending.  An expert appears at most once in a row's top-k. */
int orc_group(const int32_t *ids, int R, int k, int E,
              int32_t *counts, int32_t *offsets, int32_t *perm)
{
    if (!ids || !counts || !offsets || !perm || R < 0 || k <= 0 || E <= 0)
        return -1;
    int n = 0;
    for (int e = 0; e < E; e++) {
        offsets[e] = n;
        int c = 0;
        for (int r = 0; r < R; r++)
            for (int j = 0; j < k; j++)
                if (ids[(size_t)r * k + j] == e) {
                    perm[n++] = r * k + j;
                    c++;
                }
        counts[e] = c;
    }
    offsets[E] = n;
    return n == R * k ? 0 : -3;
}

/* ---------------------------------------------------------------- experts */

static double silu(double t) { return t / (1.0 + exp(-t)); }

/* One SwiGLU expert on one row (Qwen3-8B card: gate_proj, up_proj,
 * down_proj).  Reading: gate and up are one fused [2I][H] matrix with the
 * gate rows first; h = silu(g)*u is kept as f32 (the GB10 blueprint's down
 * nodes read f32 activations). */
int orc_expert_apply(const orc_layer *L, const orc_expert *X, int inter,
                     const uint16_t *x_row, double *d)
{
    if (!L || !X || !x_row || !d || !X->gu_q || !X->gu_s || !X->dn_q || !X->dn_s || inter <= 0 ||
        !known_format(L->fmt))
        return -1;
    const int H = L->hidden, fmt = L->fmt;
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    float *h = (float *)malloc(sizeof(float) * (size_t)inter);
    if (!xf || !h) {
        free(xf);
        free(h);
        return -2;
    }
    for (int c = 0; c < H; c++)
        xf[c] = orc_bf16_to_f32(x_row[c]);

#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int i = 0; i < inter; i++) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; c++) {
            g += (double)weight(fmt, X->gu_q, X->gu_s, X->gu_g, H, i, c) * (double)xf[c];
            u += (double)weight(fmt, X->gu_q, X->gu_s, X->gu_g, H, inter + i, c) * (double)xf[c];
        }
        h[i] = (float)(silu(g) * u);
    }

#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int o = 0; o < H; o++) {
        double acc = 0.0;
        for (int i = 0; i < inter; i++)
            acc += (double)weight(fmt, X->dn_q, X->dn_s, X->dn_g, inter, o, i) * (double)h[i];
        d[o] = acc;
    }
    free(xf);
    free(h);
    return 0;
}

/* ------------------------------------------------------------------ layer */

int orc_layer_forward(const orc_layer *L, const uint16_t *x, int R,
                      const float *logits_in, const uint16_t *residual,
                      int32_t *ids_out, float *w_out, float *s_out, float *y_out,
                      uint16_t *out)
{
    if (!L || !x || R < 0 || L->hidden <= 0 || L->n_experts <= 0 || L->top_k <= 0 ||
        L->top_k > L->n_experts || L->inter <= 0 || !L->experts)
        return -1;
    if (!logits_in && !L->router_w)
        return -1;
    if (L->shared_inter > 0 && !L->shared)
        return -1;
    const int H = L->hidden, E = L->n_experts, k = L->top_k;
    int rc = 0;
    float *logits = (float *)malloc(sizeof(float) * (size_t)R * E + 1);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)R * k + 1);
    float *w = (float *)malloc(sizeof(float) * (size_t)R * k + 1);
    float *s = (float *)malloc(sizeof(float) * (size_t)R + 1);
    double *d = (double *)malloc(sizeof(double) * (size_t)H);
    double *y = (double *)malloc(sizeof(double) * (size_t)H);
    if (!logits || !ids || !w || !s || !d || !y) {
        rc = -2;
        goto done;
    }
    if (logits_in)
        memcpy(logits, logits_in, sizeof(float) * (size_t)R * E);
    else if ((rc = orc_router_logits(L, x, R, logits)) != 0)
        goto done;
    if ((rc = orc_topk_softmax(logits, R, E, k, ids, w)) != 0)
        goto done;
    if ((rc = orc_shared_gate(L, x, R, s)) != 0)
        goto done;

    for (int r = 0; r < R; r++) {
        const uint16_t *xr = x + (size_t)r * H;
        for (int o = 0; o < H; o++)
            y[o] = 0.0;
        /* Weighted sum of the routed experts in slot order (GB10 blueprint,
         * "Kernels": moe_weighted_sum_blend), with the stored f32 weights. */
        for (int j = 0; j < k; j++) {
            const orc_expert *X = &L->experts[ids[(size_t)r * k + j]];
            if ((rc = orc_expert_apply(L, X, L->inter, xr, d)) != 0)
                goto done;
            double wj = (double)w[(size_t)r * k + j];
            for (int o = 0; o < H; o++)
                y[o] += wj * d[o];
        }
        if (L->shared_inter > 0) {
            if ((rc = orc_expert_apply(L, L->shared, L->shared_inter, xr, d)) != 0)
                goto done;
            double sr = (double)s[r];
            for (int o = 0; o < H; o++)
                y[o] += sr * d[o];
        }
        for (int o = 0; o < H; o++) {
            float yf = (float)y[o];
            if (y_out)
                y_out[(size_t)r * H + o] = yf;
            if (out) {
                /* One rounding to bf16 at the end, after the residual add
                 * (colibri pull request 1992, "What it is": the MoE output
                 * joins the residual). */
                double t = y[o];
                if (residual)
                    t += (double)orc_bf16_to_f32(residual[(size_t)r * H + o]);
                out[(size_t)r * H + o] = orc_f32_to_bf16_rne((float)t);
            }
        }
    }
    if (ids_out)
        memcpy(ids_out, ids, sizeof(int32_t) * (size_t)R * k);
    if (w_out)
        memcpy(w_out, w, sizeof(float) * (size_t)R * k);
    if (s_out)
        memcpy(s_out, s, sizeof(float) * (size_t)R);
done:
    free(logits);
    free(ids);
    free(w);
    free(s);
    free(d);
    free(y);
    return rc;
}

/* ------------------------------------------------------------------ norm */

int orc_rms_norm(const uint16_t *x, int R, int H, const uint16_t *gamma, double eps, uint16_t *out)
{
    if (!x || !gamma || !out || R < 0 || H <= 0 || !(eps >= 0.0))
        return -1;
    for (int r = 0; r < R; r++) {
        const uint16_t *xr = x + (size_t)r * H;
        double ss = 0.0;
        for (int o = 0; o < H; o++) {
            double v = (double)orc_bf16_to_f32(xr[o]);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)H + eps);
        for (int o = 0; o < H; o++) {
            double v = (double)orc_bf16_to_f32(xr[o]) * inv * (double)orc_bf16_to_f32(gamma[o]);
            out[(size_t)r * H + o] = orc_f32_to_bf16_rne((float)v);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ dense */

int orc_dense_fp8(const uint8_t *q, const float *scale, int N, int K, const uint16_t *x, int R, double *y)
{
    if (!q || !scale || !x || !y || N <= 0 || K <= 0 || R < 0 || N % 128 || K % 128)
        return -1;
    float *W = (float *)malloc(sizeof(float) * (size_t)N * K);
    if (!W)
        return -2;
    int rc = orc_dequant_fp8(q, scale, N, K, W);
    if (rc == 0) {
#pragma omp parallel for num_threads(g_threads) schedule(static)
        for (int n = 0; n < N; n++) {
            const float *wn = W + (size_t)n * K;
            for (int r = 0; r < R; r++) {
                const uint16_t *xr = x + (size_t)r * K;
                double acc = 0.0;
                for (int k = 0; k < K; k++)
                    acc += (double)orc_bf16_to_f32(xr[k]) * (double)wn[k];
                y[(size_t)r * N + n] = acc;
            }
        }
    }
    free(W);
    return rc;
}
