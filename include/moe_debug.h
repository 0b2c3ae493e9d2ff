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

/* Phase stamps of the one-launch layer (diagnostics): while `stamps` is set
 * (device, n_words 64-bit words; NULL or n_words 0 turns it off), every
 * one-launch layer on this ctx writes, per workgroup b, 16 words at
 * stamps[16 b]: word 0 the workgroup's role (0 router, 1 shared gate/up,
 * 2 routed gate/up, 3 down) | slot << 8 | (a last arrival) << 16, and words
 * 1..10 the device's constant clock (s_memrealtime) at its phase boundaries:
 * 1 start; router: 2 row dot done, 3 arrival counted, 4 done word published
 * (last of its sub-counter); gate/up: 2 routing ready seen, 3 top-k done,
 * 4 h stored, 5 arrival counted; down: 2 routing ready seen, 3 top-k done,
 * 4 down-row loads issued, 5 gate/up done words seen, 6 h staged, 7 blend
 * stored, 8 group arrival returned, 9 group line cleared (last of its
 * group); waiters: 10 the logits they select from arrived.  Words a role
 * does not reach read all ones (0xffffffffffffffff).  The stamps are kept in
 * the workgroup's LDS and written out as it ends, so no barrier waits for
 * them.  A launch whose grid needs more than
 * n_words fails (MOE_ERR_HIP, ctx lost).  *clock_khz (host, may be NULL)
 * receives the constant clock's rate in kHz. */
MOE_API int moe_debug_set_phase_stamps(moe_ctx *ctx, uint64_t *stamps, int64_t n_words, int64_t *clock_khz);

#ifdef __cplusplus
}
#endif
#endif
