/*
 * moe_oracle.h -- plain CPU definition of the decode-step MoE FFN.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load this library.
 * It shares no code, header, table or constant with the HIP library.
 *
 * The layer it defines (colibri pull request 1992, "What it is": the router
 * logits, the host routes, the routed experts plus the shared expert and its
 * gate, the MoE output joining the residual; GB10 blueprint for
 * Qwen3.6-35B-A3B-FP8, "Kernels" table: dense_gemv_bf16 router,
 * moe_topk_softmax, moe_expert_gate_up_shared_fp8,
 * moe_expert_silu_down_shared_fp8, moe_weighted_sum_blend):
 *
 *   logits[r,e] = sum_h x[r,h] * Wr[e,h]  (+ bias[e])
 *   p = softmax(logits[r,:]) over all experts; ids = top-k of p (ties: lower
 *       index first); w_j = p[id_j] / sum_{j<k} p[id_j]
 *   for every routed slot j and for the shared expert:
 *       [g ; u] = W_gu . x      (gate rows first, then up rows)
 *       h = silu(g) * u         (stored as f32)
 *       d = W_dn . h
 *   s = sigmoid(w_sg . x)       (shared-expert gate, a scalar per row)
 *   y = sum_j w_j d_j + s d_shared
 *   out = bf16_rne(residual + y)   (or bf16_rne(y) without a residual)
 *
 * Weight formats:
 *   ORC_FMT_FP8_B128 : OCP e4m3 codes, row-major [O][I], one f32 scale per
 *                      128x128 block, scale array [O/128][I/128]; w = code*scale.
 *   ORC_FMT_NVFP4    : e2m1 codes, two per byte (low nibble = even column),
 *                      row-major [O][I/2] bytes; one e4m3 scale per 16
 *                      consecutive input columns, array [O][I/16]; one f32
 *                      global scale per matrix; w = code*scale*global.
 *   ORC_FMT_INT8_ROW : two's-complement int8 codes, row-major [O][I]; one f32
 *                      scale per row, array [O]; w = code*scale.
 *   ORC_FMT_INT4_ROW : two's-complement int4 codes, two per byte (low nibble =
 *                      even column), [O][I/2] bytes; one f32 scale per row.
 *   ORC_FMT_INT4_G64 : int4 codes as above; one f32 scale per 64 consecutive
 *                      input columns of a row, array [O][I/64].
 *   ORC_FMT_FP8_B128_BF16S : as ORC_FMT_FP8_B128 with bf16 block scales.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FMT_FP8_B128 = 0, ORC_FMT_NVFP4 = 1, ORC_FMT_INT8_ROW = 2, ORC_FMT_INT4_ROW = 3, ORC_FMT_INT4_G64 = 4,
       ORC_FMT_FP8_B128_BF16S = 5 };

typedef struct orc_expert {
    const uint8_t *gu_q;   /* gate|up codes, [2I][H] (fp8) or [2I][H/2] (nvfp4) */
    const void    *gu_s;   /* f32 [2I/128][H/128] (fp8) or e4m3 [2I][H/16] (nvfp4) */
    float          gu_g;   /* nvfp4 global scale of gate|up (ignored for fp8) */
    const uint8_t *dn_q;   /* down codes, [H][I] (fp8) or [H][I/2] (nvfp4) */
    const void    *dn_s;   /* f32 [H/128][I/128] (fp8) or e4m3 [H][I/16] (nvfp4) */
    float          dn_g;   /* nvfp4 global scale of down */
} orc_expert;

typedef struct orc_layer {
    int hidden;            /* H */
    int n_experts;         /* E */
    int top_k;             /* k */
    int inter;             /* I of a routed expert */
    int shared_inter;      /* I of the shared expert, 0 = none */
    int fmt;               /* ORC_FMT_* */
    const uint16_t *router_w;      /* bf16 [E][H], may be NULL when logits are given */
    const float    *router_bias;   /* f32 [E] or NULL */
    const uint16_t *shared_gate_w; /* bf16 [H]; NULL = ungated shared expert (s = 1) */
    const orc_expert *experts;     /* [E]; untouched experts may hold NULL pointers */
    const orc_expert *shared;      /* NULL when shared_inter == 0 */
} orc_layer;

float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16_rne(float f);
float    orc_e4m3_to_f32(uint8_t code);
float    orc_e2m1_to_f32(uint8_t nibble);
float    orc_int8_to_f32(uint8_t code);
float    orc_int4_to_f32(uint8_t nibble);

void orc_set_threads(int n);
int  orc_get_threads(void);

/* Dequantised f32 weight matrices (O x I), for tests of the format decoders. */
int orc_dequant_fp8(const uint8_t *q, const float *scale, int O, int I, float *W);
int orc_dequant_nvfp4(const uint8_t *q, const uint8_t *scale, float g, int O, int I, float *W);
/* The integer formats (fmt = ORC_FMT_INT8_ROW, _INT4_ROW or _INT4_G64); scale
 * is f32 [O][I/G] with G = I for the per-row formats and 64 for g64. */
int orc_dequant_int(int fmt, const uint8_t *q, const float *scale, int O, int I, float *W);
/* fp8 codes with bf16 block scales [O/128][I/128]. */
int orc_dequant_fp8_bf16s(const uint8_t *q, const uint16_t *scale, int O, int I, float *W);

/* Router logits f32 [R][E]. */
int orc_router_logits(const orc_layer *L, const uint16_t *x, int R, float *logits);
/* Shared-expert gate s[r] in (0,1), f32 [R]. */
int orc_shared_gate(const orc_layer *L, const uint16_t *x, int R, float *s);
/* Softmax over all E, top-k (value descending, lower index on ties),
 * renormalised weights.  ids i32 [R][k], w f32 [R][k]. */
int orc_topk_softmax(const float *logits, int R, int E, int k, int32_t *ids, float *w);
/* Token-by-expert grouping: counts [E], offsets [E+1], perm [R*k] where
 * perm[offsets[e] + n] = r*k + j of the n-th row (ascending r) routed to e. */
int orc_group(const int32_t *ids, int R, int k, int E,
              int32_t *counts, int32_t *offsets, int32_t *perm);
/* One expert on one activation row: d[H] = W_dn (silu(W_g x) * W_u x). */
int orc_expert_apply(const orc_layer *L, const orc_expert *X, int inter,
                     const uint16_t *x_row, double *d);
/* The whole layer for R rows.  logits_in (f32 [R][E]) replaces the router
 * GEMV when given.  Outputs (any may be NULL): ids, w, s (f32 [R]),
 * y (f32 [R][H], the MoE output before the residual), out (bf16 [R][H]). */
int orc_layer_forward(const orc_layer *L, const uint16_t *x, int R,
                      const float *logits_in, const uint16_t *residual,
                      int32_t *ids, float *w, float *s, float *y, uint16_t *out);

/* RMSNorm of R bf16 rows of H values (GB10 blueprint, "Kernels":
 * residual_add_rms_norm, the norm that follows the MoE output joining the
 * residual; Qwen3-8B card, "Structure": RMSNorm over the hidden size):
 *   out[r,o] = bf16_rne( x[r,o] / sqrt(mean_o x[r,o]^2 + eps) * gamma[o] ),
 * in double, one rounding at the end. */
int orc_rms_norm(const uint16_t *x, int R, int H, const uint16_t *gamma, double eps, uint16_t *out);

/* Dense fp8 block-128 projection (GB10 blueprint, "Kernels":
 * w8a16_gemm_pipelined_m32; "Precision": fp8/block128x128 weights read bf16
 * activations): y[r][n] = sum_k x[r][k] * dequant(W)[n][k] in double, W the
 * e4m3 codes [N][K] with f32 scales [N/128][K/128]. */
int orc_dense_fp8(const uint8_t *q, const float *scale, int N, int K, const uint16_t *x, int R, double *y);

#ifdef __cplusplus
}
#endif
#endif
