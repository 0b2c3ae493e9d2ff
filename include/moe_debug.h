/*
 * moe_debug.h -- diagnostic entry points of the MI355X MoE FFN library.
 * Not on the layer's path; used by tests to check the kernels' own number
 * format converters on the device.
 */
#ifndef MOE_DEBUG_H
#define MOE_DEBUG_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Decode `n` code bytes (n a multiple of 4) at device address `codes` with
 * the converters the expert kernels use, into device f32 `out`:
 *   fmt 0 (OCP e4m3): out[2i] = code i through the bf16 path (the gate/up
 *         GEMV), out[2i+1] = code i through the f32 path (the down GEMV);
 *         2n floats.
 *   fmt 1 (e2m1, two codes per byte, low nibble first): for byte b,
 *         out[4b], out[4b+1] = low and high nibble through the bf16 path,
 *         out[4b+2], out[4b+3] = the same through the f32 path; 4n floats.
 * Asynchronous on `stream`; MOE_ERR_INVALID_ARG / MOE_ERR_MISALIGNED on bad
 * arguments (nothing enqueued). */
MOE_API int moe_debug_decode(moe_ctx *ctx, int fmt, const void *codes, float *out, int n, void *stream);

#ifdef __cplusplus
}
#endif
#endif
