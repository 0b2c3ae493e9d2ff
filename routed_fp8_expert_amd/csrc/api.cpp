// api.cpp -- the C ABI (include/moe.h): argument validation before any
// enqueue, the ctx (sticky lost state, fault injection, arm options, event
// timing), the workspace layout and the launch sequence of a layer.
//
// Conventions follow colibri pull request 1992, "What it is": ops declined on
// bad arguments, a HIP error marks the device lost to the ctx, one stream per
// call; 0 is success here (HIP style) rather than the page's 0 = declined.
#include "moe.h"
#include "moe_debug.h"
#include "kernels.hpp"
#include "host_checks.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>
#include <cmath>
#include <vector>

namespace {

using namespace moe_host;

// ctx words (kernels.hpp): tickets, the error word, the warming sink and the
// single-launch layer's synchronisation lines, from the ctx pool.
using moe::kCtxWords;
using moe::kLayerSyncWords;
using moe::kWordError;
using moe::kWordGroupTicket;
using moe::kWordLayerSync;
using moe::kWordRouterTicket;
using moe::kWordSink;
constexpr int64_t kDefaultWaitUs = 10000;   // a one-launch layer's wait gives up after 10 ms
constexpr int kDenseMaxK = 8192;         // a wave's 64 lanes hold one scale per 128-wide block
constexpr int kDenseMaxRows = 1 << 20;   // matrix-core grid rows stay far below 65535
// Steps of 2 .. E / (2k) rows (at least 8, at most 32) run as few rows: one
// GEMV per row and slot, no grouping.  Grouping pays once rows share experts;
// with R k <= E / 2 they rarely do.  Measured against the grouped path:
// 35B-A3B (E / 2k = 16) at 10 / 12 / 16 / 24 / 32 rows 51.9 / 58.7 / 74.8 /
// 103.0 / 132.7 against 58.0 / 64.0 / 75.6 / 94.7 / 110.3 us; 397B-A17B
// (E / 2k = 25) at 2 / 8 / 12 / 16 / 24 rows 46.9 / 128.1 / 183.8 / 236.3 /
// 346.0 against 56.6 / 155.5 / 220.0 / 276.8 / 382.3 us.
constexpr int kFewRowsMin = 8, kFewRowsMax = 32;
constexpr int kFewRowsAuto = -1;         // ctx default: the rule above
// Few-rows steps up to this many rows select in the gate/up blocks (every
// block reruns its row's top-k) instead of in a top-k launch: 8 rows up to
// 256 experts (35B-A3B 6 / 8 rows 36.7 / 45.2 -> 35.0 / 44.8 us against 4
// rows; no gain at 12 and 16), 4 above (397B-A17B at 8 rows: 128 against
// 141 us with the selection of 512 experts in every block).
inline int fused_topk_rows(int E) { return E <= 256 ? 8 : 4; }
constexpr int kDefaultMfmaMinRows = 4;   // rows per expert from which the MFMA arm pays (measured)
// Step rows from which the MFMA arm runs in grouped steps (grouped steps
// start past the few-rows path by default; with the few-rows path set lower,
// the grouped path below 9 rows keeps GEMV-only bits).
// Measured against 32: 12 rows 84.1 -> 67.2 us, 16 rows 102.0 -> 78.5, 24
// rows 135.7 -> 98.2 (the shared expert's rows leave one long GEMV task); at
// 4 rows it was slower.
constexpr int kMfmaStepRows = 9;
static_assert(moe_host::kMaxTopK == moe::kMaxTopK, "top-k limit");
constexpr size_t kMaxTimingRecords = 1 << 16;

struct TimingRecord {
    hipEvent_t a, b;
    int kind;
};

}  // namespace

struct moe_ctx {
    int device = 0;
    int status = MOE_OK;
    int64_t fault_countdown = 0;
    int mfma_min_rows = kDefaultMfmaMinRows;
    int few_rows = kFewRowsAuto;
    int force_arm = 0;
    int one_row_path = 0;        // 0 = single launch where built, 1 = three launches
    uint32_t *words = nullptr;   // device: kCtxWords words of the ctx pool
    int slot = -1;               // the pool slot holding them
    int64_t clock_khz = 100000;  // the device's constant clock (s_memrealtime)
    int64_t wait_us = kDefaultWaitUs;
    uint64_t *stamps = nullptr;  // diagnostics: phase stamps of the one-launch layer
    int64_t stamp_words = 0;
    bool timing = false;
    std::vector<TimingRecord> recs;
    std::vector<hipEvent_t> spare;
};

namespace {

// Makes the ctx's device current for the call and restores the caller's.
class DeviceGuard {
  public:
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev_) != hipSuccess) {
            ok_ = false;
            return;
        }
        if (prev_ != dev) {
            ok_ = hipSetDevice(dev) == hipSuccess;
            changed_ = ok_;
        }
    }
    ~DeviceGuard() {
        if (changed_) (void)hipSetDevice(prev_);
    }
    bool ok() const { return ok_; }

  private:
    int prev_ = -1;
    bool ok_ = true;
    bool changed_ = false;
};

template <class T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

int fail(moe_ctx *c, int status) {
    c->status = status;
    return status;
}

hipEvent_t take_event(moe_ctx *c) {
    if (!c->spare.empty()) {
        hipEvent_t e = c->spare.back();
        c->spare.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// One kernel launch under the ctx's rules: the injected fault, optional
// event timing, and the sticky lost state on a launch error.
template <class F>
int launch(moe_ctx *c, int kind, hipStream_t st, F &&f) {
    if (c->fault_countdown > 0 && --c->fault_countdown == 0) return fail(c, MOE_ERR_DEVICE_LOST);
    hipEvent_t a = nullptr, b = nullptr;
    if (kind >= 0 && c->timing && c->recs.size() < kMaxTimingRecords) {
        a = take_event(c);
        b = take_event(c);
        if (a && b) (void)hipEventRecord(a, st);
    }
    const hipError_t e = f();
    if (a && b) {
        (void)hipEventRecord(b, st);
        c->recs.push_back({a, b, kind});
    }
    if (e != hipSuccess) return fail(c, MOE_ERR_HIP);
    return MOE_OK;
}

struct RoutingPtrs {
    int32_t *ids;
    float *w, *s;
    int32_t *counts, *offsets, *perm;
    float *logits;
};

// The MFMA arm serves fp8 layers in steps of at least kMfmaStepRows rows (any
// multi-row step when forced), for experts with at least the threshold's rows.
bool mfma_enabled(const moe_ctx *c, const moe_layer_weights *w, int R) {
    if (w->weight_format != MOE_WFMT_FP8_E4M3_B128 || c->force_arm == 1) return false;
    if (c->force_arm == 2) return R >= 2;
    return R >= kMfmaStepRows && c->mfma_min_rows > 0;
}
int mfma_threshold(const moe_ctx *c, const moe_layer_weights *w, int R) {
    if (!mfma_enabled(c, w, R)) return 0;
    return c->force_arm == 2 ? 1 : c->mfma_min_rows;
}

moe::RouteArgs route_args(moe_ctx *c, const moe_layer_weights *w, const void *x, int R, int64_t ldx,
                          const float *logits_in, const RoutingPtrs &rp, void *ws, const Layout &L) {
    moe::RouteArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    a.R = R;
    a.wr = static_cast<const uint16_t *>(w->router_w);
    a.bias = w->router_bias;
    a.wsg = static_cast<const uint16_t *>(w->shared_gate_w);
    a.H = w->hidden;
    a.E = w->n_experts;
    a.k = w->top_k;
    a.logits_in = logits_in;
    a.logits = rp.logits ? rp.logits : at<float>(ws, L.logits);
    a.ids = rp.ids;
    a.w = rp.w;
    a.s = rp.s;
    a.counts = rp.counts;
    a.offsets = rp.offsets;
    a.perm = rp.perm;
    a.meta = at<int32_t>(ws, L.meta);
    a.gemv_list = at<int32_t>(ws, L.gemv);
    a.mfma_list = at<int32_t>(ws, L.mfma);
    a.mfma_tiles = at<int32_t>(ws, L.tiles);
    a.mfma_min_rows = mfma_threshold(c, w, R);
    a.err = c->words + kWordError;
    a.ticket = c->words + kWordRouterTicket;
    a.group_ticket = c->words + kWordGroupTicket;
    return a;
}

int do_route(moe_ctx *c, const moe::RouteArgs &a, bool plan, hipStream_t st) {
    int rc;
    if (!a.logits_in) {
        rc = launch(c, MOE_K_ROUTER, st, [&] { return moe::launch_router(a, st); });
        if (rc) return rc;
    }
    const bool compute_s = a.logits_in != nullptr;   // else the router launch made it
    // a multi-row step's top-k and grouping share one launch
    if (a.R >= 2) return launch(c, MOE_K_TOPK, st, [&] { return moe::launch_topk_group(a, compute_s, plan, st); });
    return launch(c, MOE_K_TOPK, st, [&] { return moe::launch_topk(a, compute_s, st); });
}

moe::ExpertSet expert_set(const moe_expert_weights &f, int inter) {
    moe::ExpertSet s{};
    s.gu = static_cast<const uint8_t *>(f.gate_up);
    s.gu_s = static_cast<const uint8_t *>(f.gate_up_scale);
    s.dn = static_cast<const uint8_t *>(f.down);
    s.dn_s = static_cast<const uint8_t *>(f.down_scale);
    s.gu_g = f.gate_up_global;
    s.dn_g = f.down_global;
    s.gu_stride = f.gate_up_stride;
    s.gu_s_stride = f.gate_up_scale_stride;
    s.dn_stride = f.down_stride;
    s.dn_s_stride = f.down_scale_stride;
    s.inter = inter;
    return s;
}

moe::FfnArgs ffn_args(moe_ctx *c, const moe_layer_weights *w, const void *x, int R, int64_t ldx,
                      const RoutingPtrs &rp, void *y, void *res, int64_t ldy, void *ws, const Layout &L) {
    moe::FfnArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    a.R = R;
    a.H = w->hidden;
    a.E = w->n_experts;
    a.k = w->top_k;
    a.fmt = w->weight_format;
    a.routed = expert_set(w->routed, w->inter);
    if (w->shared_inter > 0) a.shared = expert_set(w->shared, w->shared_inter);
    a.ids = rp.ids;
    a.w = rp.w;
    a.s = rp.s;
    a.counts = rp.counts;
    a.offsets = rp.offsets;
    a.perm = rp.perm;
    a.meta = at<int32_t>(ws, L.meta);
    a.gemv_list = at<int32_t>(ws, L.gemv);
    a.mfma_list = at<int32_t>(ws, L.mfma);
    a.mfma_tiles = at<int32_t>(ws, L.tiles);
    a.h = at<float>(ws, L.h);
    a.hstride = std::max(w->inter, w->shared_inter);
    a.dbuf = at<float>(ws, L.dbuf);
    a.y = static_cast<uint16_t *>(y);
    a.res = static_cast<uint16_t *>(res);
    a.ldy = ldy;
    a.err = c->words + kWordError;
    a.sink = c->words + kWordSink;
    a.logits_rep = at<float>(ws, L.lrep);
    a.h_rep = at<float>(ws, L.hrep);
    a.max_routed_tasks = std::min(w->n_experts, R * w->top_k);
    const int thr = R >= 2 ? mfma_threshold(c, w, R) : 0;
    a.shared_mfma = thr > 0 && w->shared_inter > 0 && R >= thr;
    a.mfma_max_tiles = 0;
    a.mfma_gu_max_tiles = 0;
    if (thr > 0) {
        // sum over MFMA experts of ceil(rows/T) <= R*k/T + (number of such experts)
        const int rk = R * w->top_k;
        auto bound = [&](int T) {
            return (rk + T - 1) / T + std::min(w->n_experts, rk / thr) + (a.shared_mfma ? (R + T - 1) / T : 0);
        };
        a.mfma_max_tiles = bound(moe::kMfmaTileRows);
        a.mfma_gu_max_tiles = bound(moe::kMfmaGuTileRows);
    }
    return a;
}

// Experts and blend for routed rows (generic kernels); the matrix-core
// units run inside the gate/up and down launches.
int do_ffn(moe_ctx *c, const moe::FfnArgs &a, hipStream_t st) {
    int rc = launch(c, MOE_K_GATE_UP, st, [&] { return moe::launch_gate_up(a, st); });
    if (rc) return rc;
    if (a.R == 1) {
        rc = launch(c, MOE_K_DOWN, st, [&] { return moe::launch_down_blend_r1(a, st); });
        if (rc || !a.norm_w) return rc;
        return launch(c, MOE_K_NORM, st, [&] { return moe::launch_rmsnorm(a, st); });
    }
    rc = launch(c, MOE_K_DOWN, st, [&] { return moe::launch_down_grouped(a, st); });
    if (rc) return rc;
    return launch(c, MOE_K_BLEND, st, [&] { return moe::launch_blend(a, st); });
}

// The whole one-row layer in three launches: router rows with the shared
// expert's gate/up; the top-k inside the routed gate/up; down with the blend.
// Steps of a few rows (2 .. few_rows, the default arm choice): no grouping;
// the one-row gate/up and down+blend kernels over every (row, slot), the
// shared expert's gate/up once for all rows.
// The automatic choice: E / (2k) rows, at least kFewRowsMin, at most
// kFewRowsMax (see kFewRowsMin).
bool few_rows_path(const moe_ctx *c, const moe_layer_weights *w, int R) {
    if (R < 2 || c->force_arm != 0) return false;
    int lim = c->few_rows;
    if (lim == kFewRowsAuto)
        lim = std::min(kFewRowsMax, std::max(kFewRowsMin, w->n_experts / (2 * std::max(1, w->top_k))));
    return R <= lim;
}

int do_ffn_few(moe_ctx *c, const moe::FfnArgs &a, hipStream_t st) {
    int rc = launch(c, MOE_K_GATE_UP, st, [&] { return moe::launch_gate_up_r1(a, st); });
    if (rc) return rc;
    rc = launch(c, MOE_K_DOWN, st, [&] { return moe::launch_down_blend_r1(a, st); });
    if (rc || !a.norm_w) return rc;
    return launch(c, MOE_K_NORM, st, [&] { return moe::launch_rmsnorm(a, st); });
}

// A wait's deadline in ticks of the device's constant clock.
uint64_t wait_ticks(const moe_ctx *c) { return (uint64_t)c->wait_us * (uint64_t)c->clock_khz / 1000u; }

int do_layer_r1(moe_ctx *c, const moe::RouteArgs &r, moe::FfnArgs a, hipStream_t st) {
    if (c->one_row_path == 0 && moe::layer_r1_supported(r, a))
        return launch(c, MOE_K_LAYER, st, [&] {
            return moe::launch_layer_r1(r, a, c->words + kWordLayerSync, wait_ticks(c), c->stamps, c->stamp_words, st);
        });
    int rc = launch(c, MOE_K_ROUTER, st, [&] { return moe::launch_lead_r1(r, a, st); });
    if (rc) return rc;
    rc = launch(c, MOE_K_GATE_UP, st, [&] { return moe::launch_gate_up_r1(a, st); });
    if (rc) return rc;
    rc = launch(c, MOE_K_DOWN, st, [&] { return moe::launch_down_blend_r1(a, st); });
    if (rc || !a.norm_w) return rc;
    return launch(c, MOE_K_NORM, st, [&] { return moe::launch_rmsnorm(a, st); });
}

RoutingPtrs routing_ptrs(const moe_routing *r, void *ws, const Layout &L) {
    RoutingPtrs p{};
    if (r) {
        p = {r->topk_ids, r->topk_w, r->shared_gate, r->expert_count, r->expert_offset, r->perm, r->logits};
        if (!p.counts || !p.offsets || !p.perm) {   // grouping arrays not asked for: the workspace's
            p.counts = at<int32_t>(ws, L.counts);
            p.offsets = at<int32_t>(ws, L.offsets);
            p.perm = at<int32_t>(ws, L.perm);
        }
    } else {
        p = {at<int32_t>(ws, L.ids), at<float>(ws, L.w),      at<float>(ws, L.s),      at<int32_t>(ws, L.counts),
             at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.perm), nullptr};
    }
    return p;
}

}  // namespace

// ======================================================================= ABI

extern "C" {

MOE_API int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_API const char *moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case MOE_ERR_MISALIGNED: return "misaligned pointer or leading dimension";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOE_ERR_HIP: return "HIP error (ctx lost)";
        case MOE_ERR_DEVICE_LOST: return "device lost (sticky)";
        case MOE_ERR_TOO_MANY_CTX: return "too many ctxs on the device";
        default: return "unknown status";
    }
}

MOE_API int moe_ctx_create(int device, moe_ctx **out) {
    if (!out) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess) return MOE_ERR_HIP;
    if (device < 0 || device >= n) return MOE_ERR_INVALID_ARG;
    moe_ctx *c = new (std::nothrow) moe_ctx();
    if (!c) return MOE_ERR_INVALID_ARG;
    c->device = device;
    DeviceGuard g(device);
    int khz = 0;
    const hipError_t e = g.ok() ? moe::ctx_slot_acquire(device, &c->slot, &c->words) : hipErrorInvalidDevice;
    if (e != hipSuccess) {
        delete c;
        return e == hipErrorOutOfMemory ? MOE_ERR_TOO_MANY_CTX : MOE_ERR_HIP;
    }
    // the static workspace's address on this device, for moe_layer_forward_static
    if (moe::static_scratch_init(device) != hipSuccess) {
        moe::ctx_slot_release(device, c->slot);
        delete c;
        return MOE_ERR_HIP;
    }
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) == hipSuccess && khz > 0)
        c->clock_khz = khz;
    if (const char *v = getenv("MOE_FAULT_AT")) c->fault_countdown = std::max<long long>(0, atoll(v));
    if (const char *v = getenv("MOE_MFMA_MIN_ROWS")) c->mfma_min_rows = std::max(0, atoi(v));
    if (const char *v = getenv("MOE_FEW_ROWS")) c->few_rows = std::max(kFewRowsAuto, atoi(v));
    if (const char *v = getenv("MOE_ONE_ROW_PATH")) c->one_row_path = !strcmp(v, "split") ? 1 : 0;
    if (const char *v = getenv("MOE_FORCE_ARM")) {
        if (!strcmp(v, "gemv")) c->force_arm = 1;
        if (!strcmp(v, "mfma")) c->force_arm = 2;
    }
    *out = c;
    return MOE_OK;
}

MOE_API int moe_ctx_destroy(moe_ctx *c) {
    if (!c) return MOE_ERR_INVALID_ARG;
    DeviceGuard g(c->device);
    for (auto &r : c->recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (auto e : c->spare) (void)hipEventDestroy(e);
    // the slot may be reused by the next ctx: let this ctx's work finish first
    (void)hipDeviceSynchronize();
    if (c->slot >= 0) moe::ctx_slot_release(c->device, c->slot);
    delete c;
    return MOE_OK;
}

MOE_API int moe_ctx_status(const moe_ctx *c) { return c ? c->status : MOE_ERR_INVALID_ARG; }

MOE_API int moe_ctx_set_fault_at(moe_ctx *c, int64_t n) {
    if (!c) return MOE_ERR_INVALID_ARG;
    c->fault_countdown = n > 0 ? n : 0;
    return MOE_OK;
}

MOE_API int moe_ctx_set_mfma_min_rows(moe_ctx *c, int rows) {
    if (!c || rows < 0) return MOE_ERR_INVALID_ARG;
    c->mfma_min_rows = rows == 0 ? kDefaultMfmaMinRows : rows;
    return MOE_OK;
}

MOE_API int moe_ctx_set_force_arm(moe_ctx *c, int arm) {
    if (!c || arm < 0 || arm > 2) return MOE_ERR_INVALID_ARG;
    c->force_arm = arm;
    return MOE_OK;
}

MOE_API int moe_ctx_set_few_rows(moe_ctx *c, int rows) {
    if (!c || rows < kFewRowsAuto) return MOE_ERR_INVALID_ARG;
    c->few_rows = rows;
    return MOE_OK;
}

MOE_API int moe_ctx_set_one_row_path(moe_ctx *c, int path) {
    if (!c || path < 0 || path > 1) return MOE_ERR_INVALID_ARG;
    c->one_row_path = path;
    return MOE_OK;
}

MOE_API int moe_ctx_device_errors(moe_ctx *c, uint32_t *flags, int clear) {
    if (!c || !flags) return MOE_ERR_INVALID_ARG;
    if (c->status) return MOE_ERR_DEVICE_LOST;
    DeviceGuard g(c->device);
    if (hipDeviceSynchronize() != hipSuccess) return fail(c, MOE_ERR_HIP);
    if (hipMemcpy(flags, c->words + kWordError, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return fail(c, MOE_ERR_HIP);
    if (clear) {
        if (hipMemset(c->words + kWordError, 0, sizeof(uint32_t)) != hipSuccess) return fail(c, MOE_ERR_HIP);
        // a wait that gave up may have left the one-launch layer's
        // synchronisation words inconsistent: nothing runs now, so zero them
        if ((*flags & moe::kErrWaitTimeout) && moe::ctx_layer_words_reset(c->words) != hipSuccess)
            return fail(c, MOE_ERR_HIP);
        if (hipDeviceSynchronize() != hipSuccess) return fail(c, MOE_ERR_HIP);
    }
    return MOE_OK;
}

MOE_API int moe_ctx_set_wait_limit(moe_ctx *c, int64_t us) {
    if (!c) return MOE_ERR_INVALID_ARG;
    c->wait_us = us < 0 ? kDefaultWaitUs : std::min<int64_t>(us, 60 * 1000 * 1000);
    return MOE_OK;
}

MOE_API int moe_ctx_set_timing(moe_ctx *c, int enable) {
    if (!c) return MOE_ERR_INVALID_ARG;
    DeviceGuard g(c->device);
    for (auto &r : c->recs) {
        c->spare.push_back(r.a);
        c->spare.push_back(r.b);
    }
    c->recs.clear();
    c->timing = enable != 0;
    return MOE_OK;
}

MOE_API int moe_ctx_kernel_stats(moe_ctx *c, int kind, double *total_ms, int64_t *launches) {
    if (!c || !total_ms || !launches || kind < 0 || kind >= MOE_K_COUNT) return MOE_ERR_INVALID_ARG;
    DeviceGuard g(c->device);
    double t = 0.0;
    int64_t n = 0;
    for (auto &r : c->recs) {
        if (r.kind != kind) continue;
        if (hipEventSynchronize(r.b) != hipSuccess) return fail(c, MOE_ERR_HIP);
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(c, MOE_ERR_HIP);
        t += ms;
        ++n;
    }
    *total_ms = t;
    *launches = n;
    return MOE_OK;
}

MOE_API size_t moe_workspace_bytes(const moe_layer_weights *w, int rows) {
    if (validate_weights(w) || validate_rows(w, rows)) return 0;
    return make_layout(w, rows).total;
}

MOE_API int moe_route(moe_ctx *c, const moe_layer_weights *w, const void *x, int R, int64_t ldx,
                      const float *logits_in, const moe_routing *out, void *ws, size_t ws_bytes, void *stream) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->status) return MOE_ERR_DEVICE_LOST;
    int rc;
    if ((rc = validate_weights(w)) || (rc = validate_rows(w, R)) || (rc = check_x(w, x, R, ldx)) ||
        (rc = check_routing(out, R, true)) || (rc = check_ws(w, R, ws, ws_bytes)))
        return rc;
    if (!logits_in && !w->router_w) return MOE_ERR_INVALID_ARG;
    if (logits_in && !aligned(logits_in, 4)) return MOE_ERR_MISALIGNED;
    if (R == 0) return MOE_OK;
    DeviceGuard g(c->device);
    if (!g.ok()) return fail(c, MOE_ERR_HIP);
    const Layout L = make_layout(w, R);
    const RoutingPtrs rp = routing_ptrs(out, ws, L);
    return do_route(c, route_args(c, w, x, R, ldx, logits_in, rp, ws, L), false, (hipStream_t)stream);
}

MOE_API int moe_expert_ffn(moe_ctx *c, const moe_layer_weights *w, const void *x, int R, int64_t ldx,
                           const moe_routing *in, void *y, void *res, int64_t ldy, void *ws, size_t ws_bytes,
                           void *stream) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->status) return MOE_ERR_DEVICE_LOST;
    int rc;
    if ((rc = validate_weights(w)) || (rc = validate_rows(w, R)) || (rc = check_x(w, x, R, ldx)) ||
        (rc = check_routing(in, R, true)) || (rc = check_out(w, y, res, R, ldy)) ||
        (rc = check_ws(w, R, ws, ws_bytes)))
        return rc;
    if (R == 0) return MOE_OK;
    DeviceGuard g(c->device);
    if (!g.ok()) return fail(c, MOE_ERR_HIP);
    const hipStream_t st = (hipStream_t)stream;
    const Layout L = make_layout(w, R);
    const RoutingPtrs rp = routing_ptrs(in, ws, L);
    if (few_rows_path(c, w, R)) return do_ffn_few(c, ffn_args(c, w, x, R, ldx, rp, y, res, ldy, ws, L), st);
    if (R >= 2) {
        const moe::RouteArgs a = route_args(c, w, x, R, ldx, nullptr, rp, ws, L);
        rc = launch(c, MOE_K_GROUP, st, [&] { return moe::launch_plan(a, st); });
        if (rc) return rc;
    }
    return do_ffn(c, ffn_args(c, w, x, R, ldx, rp, y, res, ldy, ws, L), st);
}

MOE_API int moe_layer_forward_norm(moe_ctx *c, const moe_layer_weights *w, const void *x, int R, int64_t ldx,
                                   const float *logits_in, const moe_routing *routing, void *y, void *res,
                                   int64_t ldy, const moe_norm *norm, void *ws, size_t ws_bytes, void *stream) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->status) return MOE_ERR_DEVICE_LOST;
    int rc;
    if ((rc = validate_weights(w)) || (rc = validate_rows(w, R)) || (rc = check_x(w, x, R, ldx)) ||
        (routing && (rc = check_routing(routing, R, false))) || (rc = check_out(w, y, res, R, ldy)) ||
        (rc = check_ws(w, R, ws, ws_bytes)) || (rc = check_norm(w, norm, y, res)))
        return rc;
    if (!logits_in && !w->router_w) return MOE_ERR_INVALID_ARG;
    if (logits_in && !aligned(logits_in, 4)) return MOE_ERR_MISALIGNED;
    if (R == 0) return MOE_OK;
    DeviceGuard g(c->device);
    if (!g.ok()) return fail(c, MOE_ERR_HIP);
    const hipStream_t st = (hipStream_t)stream;
    const Layout L = make_layout(w, R);
    const RoutingPtrs rp = routing_ptrs(routing, ws, L);
    const moe::RouteArgs ra = route_args(c, w, x, R, ldx, logits_in, rp, ws, L);
    moe::FfnArgs fa = ffn_args(c, w, x, R, ldx, rp, y, res, ldy, ws, L);
    if (norm) {
        fa.norm_w = static_cast<const uint16_t *>(norm->weight);
        fa.norm_eps = norm->eps;
        fa.norm_out = static_cast<uint16_t *>(norm->out);
        fa.ldn = norm->ldo;
    }
    if (R == 1) return do_layer_r1(c, ra, fa, st);
    if (few_rows_path(c, w, R)) {
        // the router GEMV (unless logits are given); the gate/up blocks take
        // their rows' top-k and publish the routing; the grouping arrays are
        // written only when the caller asked for them
        if (R <= fused_topk_rows(w->n_experts)) {
            if (!logits_in) {
                rc = launch(c, MOE_K_ROUTER, st, [&] { return moe::launch_router(ra, st); });
                if (rc) return rc;
            }
            fa.topk_src = logits_in ? logits_in : ra.logits;
            fa.wsg = static_cast<const uint16_t *>(w->shared_gate_w);
            fa.s_mode = !w->shared_gate_w ? 2 : logits_in ? 1 : 0;
        } else {
            // beyond it every gate/up block redoing the selection costs more
            // than the top-k launch it saves
            if (!logits_in) {
                rc = launch(c, MOE_K_ROUTER, st, [&] { return moe::launch_router(ra, st); });
                if (rc) return rc;
            }
            rc = launch(c, MOE_K_TOPK, st, [&] { return moe::launch_topk(ra, logits_in != nullptr, st); });
            if (rc) return rc;
        }
        rc = do_ffn_few(c, fa, st);
        if (rc) return rc;
        const bool group = routing && routing->expert_count && routing->expert_offset && routing->perm;
        if (!group) return MOE_OK;
        return launch(c, MOE_K_GROUP, st, [&] { return moe::launch_group(ra, false, st); });
    }
    rc = do_route(c, ra, true, st);
    if (rc) return rc;
    return do_ffn(c, fa, st);
}

MOE_API int moe_layer_forward(moe_ctx *c, const moe_layer_weights *w, const void *x, int R, int64_t ldx,
                              const float *logits_in, const moe_routing *routing, void *y, void *res, int64_t ldy,
                              void *ws, size_t ws_bytes, void *stream) {
    return moe_layer_forward_norm(c, w, x, R, ldx, logits_in, routing, y, res, ldy, nullptr, ws, ws_bytes, stream);
}

MOE_API int moe_layer_forward_static(moe_ctx *c, const moe_layer_weights *w, const void *x, int R, int64_t ldx,
                                     const float *logits_in, const moe_routing *routing, void *y, void *res,
                                     int64_t ldy, void *stream) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->status) return MOE_ERR_DEVICE_LOST;
    int rc;
    if ((rc = validate_weights(w)) || (rc = validate_rows(w, R))) return rc;
    if (make_layout(w, R).total > moe::kStaticScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    void *ws = moe::static_scratch_ptr(c->device);
    if (!ws) return MOE_ERR_HIP;
    return moe_layer_forward_norm(c, w, x, R, ldx, logits_in, routing, y, res, ldy, nullptr, ws,
                                  moe::kStaticScratchBytes, stream);
}

MOE_API int moe_dense_fp8(moe_ctx *c, const moe_dense_weights *w, const void *x, int R, int64_t ldx, void *y,
                          int64_t ldy, void *stream) {
    if (!c || !w || w->struct_size < sizeof(moe_dense_weights)) return MOE_ERR_INVALID_ARG;
    if (c->status) return MOE_ERR_DEVICE_LOST;
    const int N = w->n, K = w->k;
    if (N <= 0 || K <= 0 || N % 128 || K % 128 || K > kDenseMaxK || R < 0 || R > kDenseMaxRows)
        return MOE_ERR_INVALID_ARG;
    if (!w->codes || !w->scales || w->ldw < K) return MOE_ERR_INVALID_ARG;
    if (!aligned(w->codes, 16) || w->ldw % 16 || !aligned(w->scales, 4)) return MOE_ERR_MISALIGNED;
    if (R == 0) return MOE_OK;
    if (!x || !y || ldx < K || ldy < N) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || ldx % 8 || !aligned(y, 2)) return MOE_ERR_MISALIGNED;
    DeviceGuard g(c->device);
    if (!g.ok()) return fail(c, MOE_ERR_HIP);
    moe::DenseArgs a{};
    a.w = static_cast<const uint8_t *>(w->codes);
    a.w_stride = w->ldw;
    a.s = w->scales;
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    a.y = static_cast<uint16_t *>(y);
    a.ldy = ldy;
    a.N = N;
    a.K = K;
    a.R = R;
    const hipStream_t st = (hipStream_t)stream;
    return launch(c, MOE_K_DENSE, st, [&] { return moe::launch_dense(a, st); });
}

MOE_API int moe_debug_set_phase_stamps(moe_ctx *c, uint64_t *stamps, int64_t n_words, int64_t *clock_khz) {
    if (!c || n_words < 0 || (stamps && !aligned(stamps, 8))) return MOE_ERR_INVALID_ARG;
    c->stamps = n_words > 0 ? stamps : nullptr;
    c->stamp_words = c->stamps ? n_words : 0;
    if (clock_khz) *clock_khz = c->clock_khz;
    return MOE_OK;
}

MOE_API int moe_debug_decode(moe_ctx *c, int fmt, const void *codes, float *out, int n, void *stream) {
    if (!c || !codes || !out || n < 0 || n % 4 || (fmt != 0 && fmt != 1)) return MOE_ERR_INVALID_ARG;
    if (!aligned(codes, 4) || !aligned(out, 4)) return MOE_ERR_MISALIGNED;
    if (c->status) return MOE_ERR_DEVICE_LOST;
    if (n == 0) return MOE_OK;
    DeviceGuard g(c->device);
    const hipStream_t st = (hipStream_t)stream;
    return launch(c, -1, st, [&] {
        return moe::launch_decode_probe(fmt, static_cast<const uint8_t *>(codes), out, n, st);
    });
}

}  // extern "C"
