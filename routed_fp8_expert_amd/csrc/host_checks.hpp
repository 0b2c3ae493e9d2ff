// host_checks.hpp -- the C ABI's host-side argument checks and workspace
// layout: plain C++ over the structs of include/moe.h, no device calls, so
// that a host-only build (the sanitizer test) compiles exactly this code.
//
// Conventions follow colibri pull request 1992, "What it is": ops declined on
// bad arguments; every argument is checked before anything is enqueued.
#pragma once

#include "moe.h"
#include "kernels.hpp"

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>

namespace moe_host {

// Shape limits of include/moe.h.
constexpr int kMaxRows = 1024;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMaxHidden = 8192;
constexpr int kMaxInter = 4096;
constexpr size_t kMaxGroupWords = 8192;   // grouping bitmap and its prefix counts: 64 KB of LDS

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline size_t group_words(int E, int R) { return (size_t)E * (size_t)((R + 31) / 32); }

inline int validate_family(const moe_expert_weights &f, int fmt, bool many) {
    if (!f.gate_up || !f.gate_up_scale || !f.down || !f.down_scale) return MOE_ERR_INVALID_ARG;
    if (fmt == MOE_WFMT_NVFP4 && (!f.gate_up_global || !f.down_global)) return MOE_ERR_INVALID_ARG;
    if (!aligned(f.gate_up, 16) || !aligned(f.down, 16)) return MOE_ERR_MISALIGNED;
    // e4m3 byte pairs (nvfp4), bf16 (fp8 with bf16 scales), else f32
    const size_t salign = fmt == MOE_WFMT_NVFP4 || fmt == MOE_WFMT_FP8_E4M3_B128_BF16S ? 2 : 4;
    if (!aligned(f.gate_up_scale, salign) || !aligned(f.down_scale, salign)) return MOE_ERR_MISALIGNED;
    if (fmt == MOE_WFMT_NVFP4 && (!aligned(f.gate_up_global, 4) || !aligned(f.down_global, 4)))
        return MOE_ERR_MISALIGNED;
    if (many) {
        if (f.gate_up_stride < 0 || f.gate_up_scale_stride < 0 || f.down_stride < 0 || f.down_scale_stride < 0)
            return MOE_ERR_INVALID_ARG;
        if (f.gate_up_stride % 16 || f.down_stride % 16) return MOE_ERR_MISALIGNED;
        if (f.gate_up_scale_stride % (int64_t)salign || f.down_scale_stride % (int64_t)salign)
            return MOE_ERR_MISALIGNED;
    }
    return MOE_OK;
}

// Down-projection lane shape (must match the kernels' launcher): lanes per
// row from the routed intermediate size, chunks per lane for the longer of
// routed and shared; at most 4 chunks per lane.
inline bool down_shape_ok(const moe_layer_weights *w) {
    const int fmt = w->weight_format;
    const int nch = moe::fmt_row_bytes(fmt, w->inter) / 16;
    const int ie = std::max(w->inter, w->shared_inter);
    const int nchmax = moe::fmt_row_bytes(fmt, ie) / 16;
    const int lpr = nch >= 64 ? 64 : nch >= 32 ? 32 : nch >= 16 ? 16 : 8;
    return (nchmax + lpr - 1) / lpr <= 4;
}

inline int validate_weights(const moe_layer_weights *w) {
    if (!w) return MOE_ERR_INVALID_ARG;
    if (w->struct_size != sizeof(moe_layer_weights)) return MOE_ERR_INVALID_ARG;
    if (w->weight_format < MOE_WFMT_FP8_E4M3_B128 || w->weight_format > MOE_WFMT_FP8_E4M3_B128_BF16S)
        return MOE_ERR_INVALID_ARG;
    const int H = w->hidden, E = w->n_experts, k = w->top_k, I = w->inter, Is = w->shared_inter;
    if (H <= 0 || E <= 0 || k <= 0 || I <= 0 || Is < 0) return MOE_ERR_INVALID_ARG;
    if (H % 128 || H > kMaxHidden || I % 128 || I > kMaxInter || Is % 128 || Is > kMaxInter)
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if (k > kMaxTopK || k > E || E > kMaxExperts) return MOE_ERR_UNSUPPORTED_SHAPE;
    if (!down_shape_ok(w)) return MOE_ERR_UNSUPPORTED_SHAPE;
    if (w->router_w && !aligned(w->router_w, 16)) return MOE_ERR_MISALIGNED;
    if (w->router_bias && !aligned(w->router_bias, 4)) return MOE_ERR_MISALIGNED;
    if (w->shared_gate_w && !aligned(w->shared_gate_w, 16)) return MOE_ERR_MISALIGNED;
    int rc = validate_family(w->routed, w->weight_format, true);
    if (rc) return rc;
    if (Is > 0) {
        rc = validate_family(w->shared, w->weight_format, false);
        if (rc) return rc;
    }
    return MOE_OK;
}

inline int validate_rows(const moe_layer_weights *w, int R) {
    if (R < 0) return MOE_ERR_INVALID_ARG;
    if (R > kMaxRows) return MOE_ERR_UNSUPPORTED_SHAPE;
    if (R >= 2 && group_words(w->n_experts, R) > kMaxGroupWords) return MOE_ERR_UNSUPPORTED_SHAPE;
    return MOE_OK;
}

struct Layout {
    size_t logits, ids, w, s, counts, offsets, perm, meta, gemv, mfma, tiles, h, dbuf, lrep, hrep, total;
};

inline Layout make_layout(const moe_layer_weights *w, int R) {
    Layout L{};
    const size_t E = w->n_experts, k = w->top_k, H = w->hidden;
    const size_t ne = (size_t)R * k + (w->shared_inter > 0 ? (size_t)R : 0);
    const size_t hs = (size_t)std::max(w->inter, w->shared_inter);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes, 256);
        return at;
    };
    L.logits = take((size_t)R * E * 4);
    L.ids = take((size_t)R * k * 4);
    L.w = take((size_t)R * k * 4);
    L.s = take((size_t)R * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.perm = take((size_t)R * k * 4);
    L.meta = take(moe::kMetaWords * 4);
    L.gemv = take(E * 4);
    L.mfma = take(E * 4);
    L.tiles = take(2 * (E + 1) * 4);   // two row-tile prefixes (down, gate/up tiles)
    L.h = take(ne * hs * 4);
    L.dbuf = take(R >= 2 ? ne * H * 4 : 0);
    // replicas for the single-launch one-row layer
    L.lrep = take(R == 1 ? (size_t)moe::kReplicas * E * 4 : 0);
    L.hrep = take(R == 1 ? (size_t)moe::kReplicas * ne * hs * 4 : 0);
    L.total = off;
    return L;
}

inline int check_routing(const moe_routing *r, int R, bool need_group) {
    if (!r || r->struct_size != sizeof(moe_routing)) return MOE_ERR_INVALID_ARG;
    if (R == 0) return MOE_OK;
    if (!r->topk_ids || !r->topk_w || !r->shared_gate) return MOE_ERR_INVALID_ARG;
    const int ngroup = (r->expert_count != nullptr) + (r->expert_offset != nullptr) + (r->perm != nullptr);
    if (need_group && R >= 2 && ngroup != 3) return MOE_ERR_INVALID_ARG;
    if (ngroup != 0 && ngroup != 3) return MOE_ERR_INVALID_ARG;   // all three grouping arrays or none
    const void *ps[] = {r->topk_ids, r->topk_w, r->shared_gate, r->expert_count, r->expert_offset, r->perm, r->logits};
    for (const void *p : ps)
        if (p && !aligned(p, 4)) return MOE_ERR_MISALIGNED;
    return MOE_OK;
}

inline int check_x(const moe_layer_weights *w, const void *x, int R, int64_t ldx) {
    if (R == 0) return MOE_OK;
    if (!x) return MOE_ERR_INVALID_ARG;
    if (ldx < w->hidden) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || ldx % 8) return MOE_ERR_MISALIGNED;
    return MOE_OK;
}

inline int check_out(const moe_layer_weights *w, const void *y, const void *res, int R, int64_t ldy) {
    if (R == 0) return MOE_OK;
    if (!y && !res) return MOE_ERR_INVALID_ARG;
    if (ldy < w->hidden) return MOE_ERR_INVALID_ARG;
    if ((y && !aligned(y, 2)) || (res && !aligned(res, 2))) return MOE_ERR_MISALIGNED;
    return MOE_OK;
}

inline int check_norm(const moe_layer_weights *w, const moe_norm *n, const void *y, const void *res) {
    if (!n) return MOE_OK;
    if (n->struct_size < sizeof(moe_norm) || !n->weight || !n->out || n->ldo < w->hidden ||
        !(n->eps >= 0.0f) || !std::isfinite(n->eps) || (!y && !res))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(n->weight, 2) || !aligned(n->out, 2)) return MOE_ERR_MISALIGNED;
    return MOE_OK;
}

inline int check_ws(const moe_layer_weights *w, int R, const void *ws, size_t ws_bytes) {
    if (R == 0) return MOE_OK;
    if (!ws) return MOE_ERR_INVALID_ARG;
    if (!aligned(ws, 16)) return MOE_ERR_MISALIGNED;
    if (ws_bytes < make_layout(w, R).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return MOE_OK;
}

}  // namespace moe_host
