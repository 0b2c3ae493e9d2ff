/*
 * moe.h -- C ABI of the MI355X (gfx950) decode-step mixture-of-experts FFN.
 *
 * The layer (colibri pull request 1992, "What it is": router logits, the
 * routing, the routed experts plus the shared expert and its gate, the MoE
 * output joining the residual; GB10 blueprint for Qwen3.6-35B-A3B-FP8,
 * "Kernels" table: dense_gemv_bf16 router, moe_topk_softmax,
 * moe_expert_gate_up_shared_fp8, moe_expert_silu_down_shared_fp8,
 * moe_weighted_sum_blend) computes, for each activation row r:
 *
 *   logits[r,e] = x[r,:] . Wr[e,:] (+ bias[e])            bf16 x bf16 -> f32
 *   p = softmax over all E; ids = the k largest (ties: lower index first),
 *       in descending order; w_j = p[id_j] / sum_j p[id_j]          f32, i32
 *   s[r] = sigmoid(x[r,:] . w_sg)                      shared-expert gate
 *   for each routed slot j and the shared expert:
 *       [g ; u] = W_gu x    (gate rows 0..I-1, then up rows I..2I-1)
 *       h = silu(g) * u     (f32)
 *       d = W_dn h
 *   y = sum_j w_j d_j + s d_shared
 *   out = bf16_rne(residual + y), or bf16_rne(y) without a residual.
 *
 * Conventions
 *  - Every pointer argument marked "device" is a device address on the ctx's
 *    GPU; "host" pointers are read during the call only.  The caller owns
 *    every buffer.  The library allocates no device memory: a call uses the
 *    caller's workspace, and a ctx's synchronisation words (10 KB) are a slot
 *    of a fixed pool in the library's static device memory (64 ctxs per
 *    device at once).
 *  - Calls are asynchronous: success (MOE_OK) means the work is enqueued on
 *    `stream` (an opaque hipStream_t; NULL = the device's null stream).  No
 *    call synchronises with the host.
 *  - Every argument is validated before anything is enqueued: a call that
 *    returns an error other than MOE_ERR_HIP / MOE_ERR_DEVICE_LOST has
 *    enqueued nothing and written nothing.
 *  - 0 is success and errors are negative (HIP style).  A HIP launch error
 *    marks the ctx lost (sticky, as a CUDA error marks the device lost in the
 *    colibri chain, "What it is"); every later call on it returns
 *    MOE_ERR_DEVICE_LOST without launching until the ctx is destroyed.
 *  - One ctx may be used from one thread, with its calls stream-ordered: the
 *    ctx's synchronisation words are shared by its launches.  Distinct ctxs
 *    are independent.  No exception crosses the ABI.
 *
 * Shape limits (MOE_ERR_UNSUPPORTED_SHAPE otherwise): hidden and every
 * intermediate size a multiple of 128, hidden <= 8192, inter <= 4096;
 * 1 <= top_k <= 16, top_k <= n_experts <= 1024; 0 <= rows <= 1024; grouping
 * for rows >= 2 also needs n_experts * ceil(rows/32) <= 8192.
 * Alignment (MOE_ERR_MISALIGNED otherwise): weight codes (and their byte
 * strides), the router matrix, the gate vector and x 16-byte aligned, ldx a
 * multiple of 8 elements; fp8 scales 4-byte and nvfp4 scales 2-byte aligned;
 * routing arrays and logits 4-byte, outputs 2-byte aligned.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))
#define MOE_ABI_VERSION 5

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,       /* NULL where required, negative size, bad enum */
    MOE_ERR_UNSUPPORTED_SHAPE = -2, /* outside the shape limits above */
    MOE_ERR_MISALIGNED = -3,        /* pointer or leading dimension misaligned */
    MOE_ERR_WORKSPACE_TOO_SMALL = -4,
    MOE_ERR_HIP = -5,               /* a HIP call failed; the ctx is now lost */
    MOE_ERR_DEVICE_LOST = -6,       /* sticky: an earlier HIP error or injected fault */
    MOE_ERR_TOO_MANY_CTX = -7,      /* every ctx slot of the device is in use */
};

enum moe_weight_format {
    /* OCP e4m3 codes, row-major [out][in], one f32 scale per 128x128 block,
     * scale array [out/128][in/128]; w = code * scale (GB10 blueprint,
     * "Precision": fp8/block128x128). */
    MOE_WFMT_FP8_E4M3_B128 = 0,
    /* e2m1 codes two per byte (even column in the low nibble), row-major
     * [out][in/2] bytes; one e4m3 scale byte per 16 consecutive input columns,
     * array [out][in/16]; one f32 global scale per matrix; w = code * scale *
     * global ("Inspecting Qwen3.5-397B-A17B-NVFP4", "The Architectural
     * Revelations": NVFP4 weights). */
    MOE_WFMT_NVFP4 = 1,
    /* Integer experts (colibri PR: int8 rows in its decode GEMV, a per-row
     * int4 checkpoint, an int4-g64 expert sidecar); the layouts are readings
     * of those names: two's-complement codes, one f32 scale per group of G
     * consecutive input columns of a row, array [out][in/G]; w = code * scale.
     * Served by the GEMV arm (multi-row steps of any size) and the
     * three-launch one-row path. */
    MOE_WFMT_INT8_ROW = 2,      /* int8 codes [out][in] bytes; G = in (one scale per row) */
    MOE_WFMT_INT4_ROW = 3,      /* int4 codes two per byte (even column in the low nibble),
                                 * [out][in/2] bytes; G = in */
    MOE_WFMT_INT4_G64 = 4,      /* int4 codes as above; G = 64 */
    /* As MOE_WFMT_FP8_E4M3_B128 with bf16 block scales [out/128][in/128]
     * (colibri PR: fp8 experts with BF16 128x128 block scales).  GEMV arm and
     * the three-launch one-row path. */
    MOE_WFMT_FP8_E4M3_B128_BF16S = 5,
};

typedef struct moe_ctx moe_ctx;

/* One family of experts (the routed ones, or the single shared expert) stored
 * as per-expert slabs at a fixed byte stride.  Device pointers. */
typedef struct moe_expert_weights {
    const void *gate_up;        /* [2I][H] codes (fp8, int8: 1 B each; nvfp4, int4: H/2 B per row) */
    const void *gate_up_scale;  /* fp8: f32 (or bf16) [2I/128][H/128]; nvfp4: e4m3 [2I][H/16];
                                 * integer formats: f32 [2I][H/G] */
    const float *gate_up_global;/* nvfp4: f32 per expert (stride 1 float); others: NULL */
    const void *down;           /* [H][I] codes (fp8, int8) or [H][I/2] bytes (nvfp4, int4) */
    const void *down_scale;     /* fp8: f32 (or bf16) [H/128][I/128]; nvfp4: e4m3 [H][I/16];
                                 * integer formats: f32 [H][I/G] */
    const float *down_global;   /* nvfp4: f32 per expert; others: NULL */
    int64_t gate_up_stride;     /* bytes from one expert's gate_up to the next */
    int64_t gate_up_scale_stride;
    int64_t down_stride;
    int64_t down_scale_stride;
} moe_expert_weights;

typedef struct moe_layer_weights {
    size_t struct_size;         /* sizeof(moe_layer_weights), for versioning */
    int hidden;                 /* H */
    int n_experts;              /* E */
    int top_k;                  /* k */
    int inter;                  /* I of a routed expert */
    int shared_inter;           /* I of the shared expert; 0 = no shared expert */
    int weight_format;          /* enum moe_weight_format */
    const void *router_w;       /* device bf16 [E][H]; may be NULL if logits are always given */
    const float *router_bias;   /* device f32 [E] or NULL */
    const void *shared_gate_w;  /* device bf16 [H]; NULL = ungated shared expert (s = 1) */
    moe_expert_weights routed;  /* E slabs */
    moe_expert_weights shared;  /* one slab (strides unused) */
} moe_layer_weights;

/* Routing results: caller-owned device arrays. */
typedef struct moe_routing {
    size_t struct_size;         /* sizeof(moe_routing) */
    int32_t *topk_ids;          /* [R][k], descending weight */
    float *topk_w;              /* [R][k], renormalised, sums to 1 per row */
    float *shared_gate;         /* [R], s = sigmoid(x . w_sg) (1 when ungated) */
    int32_t *expert_count;      /* [E]   rows routed to each expert (R >= 2; may be NULL at R == 1) */
    int32_t *expert_offset;     /* [E+1] exclusive scan of expert_count */
    int32_t *perm;              /* [R*k] perm[offset[e] + n] = r*k + j, rows ascending per expert */
    float *logits;              /* [R][E] router logits out; may be NULL */
} moe_routing;

/* Kernel kinds, for moe_ctx_kernel_stats. */
enum moe_kernel_id {
    MOE_K_ROUTER = 0,   /* router GEMV (+ shared gate, + top-k for small R) */
    MOE_K_TOPK = 1,     /* top-k softmax from logits (+ shared gate) */
    MOE_K_GROUP = 2,    /* histogram, scan, ranks, permutation */
    MOE_K_GATE_UP = 3,  /* gate/up + silu*mul (routed and shared; R >= 2: GEMV and matrix-core arms) */
    MOE_K_DOWN = 4,     /* down (R == 1: fused with the blend; R >= 2: both arms) */
    MOE_K_BLEND = 5,    /* weighted blend + residual (R >= 2) */
    MOE_K_MFMA_GATE_UP = 6, /* reserved: the matrix-core arm runs inside MOE_K_GATE_UP */
    MOE_K_MFMA_DOWN = 7,    /* reserved: the matrix-core arm runs inside MOE_K_DOWN */
    MOE_K_LAYER = 8,    /* a whole one-row layer in one launch */
    MOE_K_NORM = 9,     /* RMSNorm epilogue on its own (one-row layers outside the single launch) */
    MOE_K_DENSE = 10,   /* dense fp8 block-128 projection (moe_dense_fp8) */
    MOE_K_COUNT = 11
};

MOE_API int moe_abi_version(void);
MOE_API const char *moe_strerror(int status);

/* Create a ctx on HIP device `device`.  Takes a free slot of synchronisation
 * words from the library's static pool on that device and zeroes it
 * (synchronously; MOE_ERR_TOO_MANY_CTX when all 64 are in use); allocates no
 * device memory.  moe_ctx_destroy waits for the device to finish before it
 * returns the slot.  Reads MOE_FAULT_AT (see
 * moe_ctx_set_fault_at), MOE_FORCE_ARM ("gemv" or "mfma") and
 * MOE_MFMA_MIN_ROWS from the environment. */
MOE_API int moe_ctx_create(int device, moe_ctx **out);
MOE_API int moe_ctx_destroy(moe_ctx *ctx);
/* The ctx's sticky status: MOE_OK, or the error that marked it lost. */
MOE_API int moe_ctx_status(const moe_ctx *ctx);
/* Fault injection: the n-th kernel launch from now on (n >= 1) is not made;
 * the ctx becomes lost and the call returns MOE_ERR_DEVICE_LOST.  n <= 0
 * disables it. */
MOE_API int moe_ctx_set_fault_at(moe_ctx *ctx, int64_t n);
/* Rows per expert at and above which (in a grouped step of at least 9 rows)
 * an expert of an fp8 layer takes the MFMA grouped-GEMM arm (default 4); 0
 * restores the default.  The shared expert takes it when the step has that
 * many rows.  NVFP4 layers always use the GEMV arm. */
MOE_API int moe_ctx_set_mfma_min_rows(moe_ctx *ctx, int rows);
/* Force the arm: 0 = automatic, 1 = GEMV arm only, 2 = MFMA arm for every
 * expert with at least one row (steps of >= 2 rows). */
MOE_API int moe_ctx_set_force_arm(moe_ctx *ctx, int arm);
/* One-row layers: 0 = one launch per layer (router, top-k, routed and shared
 * experts and the blend in one kernel; built for the 16- and 256-expert fp8
 * layer shapes and taken only when all its workgroups fit on the device at
 * once; other layers use the three launches), 1 = three launches (router and
 * shared expert; routed gate/up; down and blend).
 * Also MOE_ONE_ROW_PATH=split in the environment.  Both give the same bits. */
MOE_API int moe_ctx_set_one_row_path(moe_ctx *ctx, int path);
/* Steps of 2 to `rows` rows (at the default arm choice) run without grouping:
 * routing, then one GEMV per (row, slot) with the one-row kernels (the shared
 * expert's gate/up once for all rows), down fused with the blend per row.
 * Each row's result has the bits of a one-row call.  0 turns it off; -1 (the
 * default; env MOE_FEW_ROWS) chooses E / (2 top_k) rows, at least 8 and at
 * most 32 (grouping pays once rows share experts: 16 rows on the 35B-A3B
 * shape, 25 on the 397B-A17B shape).  MOE_ERR_INVALID_ARG for rows < -1. */
MOE_API int moe_ctx_set_few_rows(moe_ctx *ctx, int rows);
/* Device-side error word: kernels that meet an expert id outside [0, E)
 * skip it and set bit 0; a wait of the one-launch layer that reached the
 * ctx's wait limit sets bit 1 (the layer's output is then invalid, and the
 * ctx's synchronisation words may be left inconsistent, so later one-launch
 * layers on it are invalid too until the word is cleared).  Synchronises the
 * ctx's device and reads the word into *flags; with `clear` non-zero it
 * zeroes the word and, when bit 1 was set, the synchronisation words. */
MOE_API int moe_ctx_device_errors(moe_ctx *ctx, uint32_t *flags, int clear);
/* Wait limit of the one-launch layer: a workgroup waiting for another one
 * gives up after `us` microseconds of the device's constant clock (measured
 * from its first poll; 0 = a single poll) and sets bit 1 of the device error
 * word.  us < 0 restores the default, 10000 (10 ms); values above 60 s are
 * taken as 60 s.  Normal waits last a few microseconds. */
MOE_API int moe_ctx_set_wait_limit(moe_ctx *ctx, int64_t us);
/* Per-kernel timing with HIP events on the launch stream (diagnostics;
 * adds an event pair around every launch while enabled).  enable != 0
 * starts (and resets) it; stats synchronise on the recorded events. */
MOE_API int moe_ctx_set_timing(moe_ctx *ctx, int enable);
MOE_API int moe_ctx_kernel_stats(moe_ctx *ctx, int kernel_id, double *total_ms,
                                 int64_t *launches);

/* Workspace bytes a call with `rows` rows needs (moe_layer_forward with a
 * NULL routing argument included).  0 on invalid arguments. */
MOE_API size_t moe_workspace_bytes(const moe_layer_weights *w, int rows);

/* Routing (GB10 blueprint, "Kernels": dense_gemv_bf16 as the router,
 * moe_topk_softmax; "Plan arms": multi-row decode steps).
 *   x         device bf16 [rows][ldx] activations
 *   logits_in device f32 [rows][E] or NULL; when given it replaces the router
 *             GEMV (the router matrix is then not read)
 *   out       routing arrays to fill; expert_count/offset/perm are filled when
 *             rows >= 2 (and must then be non-NULL)
 *   ws        device workspace of at least moe_workspace_bytes(w, rows) */
MOE_API int moe_route(moe_ctx *ctx, const moe_layer_weights *w, const void *x, int rows,
                      int64_t ldx, const float *logits_in, const moe_routing *out,
                      void *ws, size_t ws_bytes, void *stream);

/* Experts and blend for already-routed rows (GB10 blueprint, "Kernels":
 * moe_expert_gate_up_shared_fp8, moe_expert_silu_down_shared_fp8,
 * moe_weighted_sum_blend).
 *   in        routing of these rows (as moe_route fills it; the grouping
 *             arrays are read when rows >= 2); ids outside [0, E) are skipped
 *             and flagged in the ctx's device error word
 *   y         device bf16 [rows][ldy] or NULL: receives bf16_rne(y)
 *   residual  device bf16 [rows][ldy] or NULL, in-out: residual <- bf16_rne(residual + y)
 *   At least one of y and residual must be given. */
MOE_API int moe_expert_ffn(moe_ctx *ctx, const moe_layer_weights *w, const void *x, int rows,
                           int64_t ldx, const moe_routing *in, void *y, void *residual,
                           int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/* The whole layer: moe_route then moe_expert_ffn.  `routing` may be NULL,
 * in which case the routing arrays live in the workspace; its grouping arrays
 * (expert_count, expert_offset, perm) may be NULL too (all three or none), and
 * are written only when given. */
MOE_API int moe_layer_forward(moe_ctx *ctx, const moe_layer_weights *w, const void *x, int rows,
                              int64_t ldx, const float *logits_in, const moe_routing *routing,
                              void *y, void *residual, int64_t ldy, void *ws, size_t ws_bytes,
                              void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_layer_forward with its workspace taken from the library's static
 * device scratch instead of a caller's buffer.  The scratch is a fixed
 * 16 MiB array per device (MOE_STATIC_SCRATCH_BYTES), held until the process
 * ends and shared by every call on that device: calls that overlap on one
 * GPU (other streams, other ctxs, other threads) race on it and must be
 * serialised by the caller.  It keeps the last call's contents; no kernel
 * relies on it starting at zero.  Allocates nothing (no hipMalloc, hipFree
 * or allocating library call).  Arguments and errors as moe_layer_forward,
 * plus MOE_ERR_WORKSPACE_TOO_SMALL when the call's workspace
 * (moe_workspace_bytes) exceeds the scratch: at the 35B-A3B shape up to about
 * 170 rows. */
#define MOE_STATIC_SCRATCH_BYTES (16u << 20)
MOE_API int moe_layer_forward_static(moe_ctx *ctx, const moe_layer_weights *w, const void *x, int rows,
                                     int64_t ldx, const float *logits_in, const moe_routing *routing,
                                     void *y, void *residual, int64_t ldy, void *stream);

/* Epilogue of moe_layer_forward_norm: RMSNorm of every output row for the
 * next layer (GB10 blueprint, "Kernels": residual_add_rms_norm, the norm that
 * follows the MoE output joining the residual; Qwen3-8B card, "Structure":
 * RMSNorm over the hidden size):
 *   out[r,o] = bf16_rne( v[r,o] / sqrt(mean_o v[r,o]^2 + eps) * weight[o] )
 * with v the row as written (the residual after the add, or y when the call
 * has no residual), in f32.  A zero-centred weight w is weight = 1 + w. */
typedef struct moe_norm {
    size_t struct_size;         /* sizeof(moe_norm) */
    const void *weight;         /* device bf16 [H] */
    float eps;                  /* finite, >= 0 */
    void *out;                  /* device bf16 [rows][ldo] */
    int64_t ldo;                /* >= H */
} moe_norm;

/* moe_layer_forward with the RMSNorm epilogue (`norm` non-NULL; NULL is
 * moe_layer_forward).  One-row layers on the single launch normalise in its
 * last down workgroup, multi-row steps in the blend; the three-launch
 * one-row path adds one launch (MOE_K_NORM).  Errors as moe_layer_forward,
 * plus MOE_ERR_INVALID_ARG for a bad `norm`. */
MOE_API int moe_layer_forward_norm(moe_ctx *ctx, const moe_layer_weights *w, const void *x, int rows,
                                   int64_t ldx, const float *logits_in, const moe_routing *routing,
                                   void *y, void *residual, int64_t ldy, const moe_norm *norm, void *ws,
                                   size_t ws_bytes, void *stream);

/* Dense fp8 block-128 weights for moe_dense_fp8 (GB10 blueprint, "Kernels":
 * w8a16_gemm_pipelined_m32; "Precision": fp8 weights in 128x128 blocks read
 * bf16 activations).  The dequantised matrix is
 *   W[n][k] = e4m3(codes[n*ldw + k]) * scales[(n/128)*(k/128 count) + k/128]. */
typedef struct moe_dense_weights {
    size_t struct_size;         /* sizeof(moe_dense_weights) */
    const void *codes;          /* device e4m3 [n][ldw], 16-byte aligned */
    int64_t ldw;                /* bytes between rows: >= k, a multiple of 16 */
    const float *scales;        /* device f32 [n/128][k/128] */
    int32_t n;                  /* output columns: a positive multiple of 128 */
    int32_t k;                  /* input columns: a positive multiple of 128, <= 8192 */
} moe_dense_weights;

/* Dense projection of bf16 rows (one MOE_K_DENSE launch; the caller keeps
 * every buffer):
 *   y[r][n] = bf16_rne( sum_k x[r][k] * W[n][k] ), f32 accumulation.
 *   x     device bf16 [rows][ldx], 16-byte aligned, ldx >= k and a multiple of 8
 *   y     device bf16 [rows][ldy], ldy >= n; must not overlap x
 *   rows  0 .. 1048576 (0 enqueues nothing).  Below 8 rows a GEMV, from 8
 *         rows 16-row matrix-core tiles; within an arm a row's result does not
 *         depend on the other rows of the call (rows 1 to 7 give one-row bits).
 * Errors: MOE_ERR_INVALID_ARG for a NULL or malformed argument or a shape
 * outside the limits, MOE_ERR_MISALIGNED for a misaligned pointer or stride,
 * MOE_ERR_DEVICE_LOST on a lost ctx; nothing is enqueued on an error. */
MOE_API int moe_dense_fp8(moe_ctx *ctx, const moe_dense_weights *w, const void *x, int rows, int64_t ldx,
                          void *y, int64_t ldy, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
