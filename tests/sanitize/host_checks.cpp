// Host-only driver of the C ABI's argument checks and workspace layout
// (routed_fp8_expert_amd/csrc/host_checks.hpp), built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  Every
// rejection path the CPU ABI tests exercise through the library is taken
// here on the same code, plus a seeded sweep of shapes and row counts.
#include "host_checks.hpp"

#include <cstdio>
#include <cstdlib>
#include <vector>

using namespace moe_host;

static int failures = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static const uintptr_t kFake = 1u << 20;   // an aligned stand-in address (never dereferenced)

static moe_layer_weights weights(int H = 2048, int E = 256, int k = 8, int I = 512, int Is = 512, int fmt = 0) {
    moe_layer_weights w{};
    w.struct_size = sizeof(moe_layer_weights);
    w.hidden = H;
    w.n_experts = E;
    w.top_k = k;
    w.inter = I;
    w.shared_inter = Is;
    w.weight_format = fmt;
    for (moe_expert_weights *f : {&w.routed, &w.shared}) {
        f->gate_up = f->down = f->gate_up_scale = f->down_scale = reinterpret_cast<const void *>(kFake);
        f->gate_up_global = f->down_global = reinterpret_cast<const float *>(kFake);
    }
    w.routed.gate_up_stride = 2LL * I * H;
    w.routed.down_stride = (int64_t)I * H;
    w.routed.gate_up_scale_stride = 64;
    w.routed.down_scale_stride = 64;
    w.router_w = reinterpret_cast<const void *>(kFake);
    return w;
}

static size_t ws(const moe_layer_weights &w, int R) {
    if (validate_weights(&w) || validate_rows(&w, R)) return 0;
    return make_layout(&w, R).total;
}

int main() {
    // the workspace of the 35B-A3B shape at 1 row: h and its replicas, logits replicas
    {
        const moe_layer_weights w = weights();
        const size_t one = ws(w, 1), h = 9 * 512 * 4;
        EXPECT(9 * h + 8 * 256 * 4 <= one && one <= 9 * h + 8 * 256 * 4 + 64 * 1024);
        EXPECT(ws(w, 64) >= (size_t)64 * 9 * 2048 * 4);
        EXPECT(ws(w, 0) > 0 && ws(w, 1024) > 0);
    }
    // shapes and row counts outside the limits
    EXPECT(ws(weights(200), 1) == 0);
    EXPECT(ws(weights(2048, 256, 8, 100), 1) == 0);
    EXPECT(ws(weights(2048, 256, 0), 1) == 0);
    EXPECT(ws(weights(2048, 256, 17), 1) == 0);
    EXPECT(ws(weights(2048, 4, 8), 1) == 0);
    EXPECT(ws(weights(2048, 2048), 1) == 0);
    EXPECT(ws(weights(2048, 256, 8, 512, 512, 7), 1) == 0);
    EXPECT(ws(weights(16384), 1) == 0);
    EXPECT(ws(weights(), -1) == 0);
    EXPECT(ws(weights(), 1025) == 0);
    EXPECT(ws(weights(2048, 1024), 1024) == 0);
    EXPECT(ws(weights(4096, 512, 10, 1024, 1024, 1), 1024) == 0);
    EXPECT(ws(weights(2048, 256, 8, 128, 4096), 1) == 0);   // down lane shape: too many chunks a lane
    EXPECT(ws(weights(2048, 256, 8, 4096, 128), 1) > 0);
    // null and misaligned pointers, bad struct size, missing nvfp4 globals
    {
        moe_layer_weights w = weights();
        w.routed.gate_up = reinterpret_cast<const void *>(kFake + 8);
        EXPECT(validate_weights(&w) == MOE_ERR_MISALIGNED);
        w = weights();
        w.routed.down = nullptr;
        EXPECT(validate_weights(&w) == MOE_ERR_INVALID_ARG);
        w = weights();
        w.struct_size = 8;
        EXPECT(validate_weights(&w) == MOE_ERR_INVALID_ARG);
        w = weights(4096, 512, 10, 1024, 1024, 1);
        w.routed.gate_up_global = nullptr;
        EXPECT(validate_weights(&w) == MOE_ERR_INVALID_ARG);
        w = weights();
        w.routed.gate_up_stride = -16;
        EXPECT(validate_weights(&w) == MOE_ERR_INVALID_ARG);
        w = weights();
        w.routed.down_stride = 24;
        EXPECT(validate_weights(&w) == MOE_ERR_MISALIGNED);
        w = weights(2048, 256, 8, 512, 512, 5);
        w.routed.gate_up_scale = reinterpret_cast<const void *>(kFake + 1);
        EXPECT(validate_weights(&w) == MOE_ERR_MISALIGNED);
        EXPECT(validate_weights(nullptr) == MOE_ERR_INVALID_ARG);
    }
    // the per-call checks
    {
        const moe_layer_weights w = weights();
        std::vector<int32_t> ids(64), cnt(256), off(257), perm(512);
        std::vector<float> tw(64), s(8), lg(8 * 256);
        moe_routing r{sizeof(moe_routing), ids.data(), tw.data(), s.data(), cnt.data(), off.data(), perm.data(), lg.data()};
        EXPECT(check_routing(&r, 8, true) == MOE_OK);
        moe_routing bad = r;
        bad.perm = nullptr;
        EXPECT(check_routing(&bad, 8, true) == MOE_ERR_INVALID_ARG);
        EXPECT(check_routing(&bad, 1, true) == MOE_ERR_INVALID_ARG);   // all three grouping arrays or none
        bad = r;
        bad.expert_count = bad.expert_offset = bad.perm = nullptr;
        EXPECT(check_routing(&bad, 8, false) == MOE_OK);
        EXPECT(check_routing(&bad, 8, true) == MOE_ERR_INVALID_ARG);
        bad = r;
        bad.topk_w = reinterpret_cast<float *>(reinterpret_cast<char *>(tw.data()) + 2);
        EXPECT(check_routing(&bad, 8, true) == MOE_ERR_MISALIGNED);
        bad = r;
        bad.struct_size = 4;
        EXPECT(check_routing(&bad, 8, true) == MOE_ERR_INVALID_ARG);
        EXPECT(check_routing(nullptr, 8, true) == MOE_ERR_INVALID_ARG);
        const void *x = reinterpret_cast<const void *>(kFake);
        EXPECT(check_x(&w, x, 4, 2048) == MOE_OK);
        EXPECT(check_x(&w, x, 4, 2040) == MOE_ERR_INVALID_ARG);
        EXPECT(check_x(&w, x, 4, 2052) == MOE_ERR_MISALIGNED);
        EXPECT(check_x(&w, reinterpret_cast<const void *>(kFake + 2), 4, 2048) == MOE_ERR_MISALIGNED);
        EXPECT(check_x(&w, nullptr, 4, 2048) == MOE_ERR_INVALID_ARG);
        EXPECT(check_x(&w, nullptr, 0, 0) == MOE_OK);
        EXPECT(check_out(&w, nullptr, nullptr, 1, 2048) == MOE_ERR_INVALID_ARG);
        EXPECT(check_out(&w, x, nullptr, 1, 100) == MOE_ERR_INVALID_ARG);
        EXPECT(check_out(&w, reinterpret_cast<const void *>(kFake + 1), nullptr, 1, 2048) == MOE_ERR_MISALIGNED);
        moe_norm n{sizeof(moe_norm), x, 1e-6f, reinterpret_cast<void *>(kFake), 2048};
        EXPECT(check_norm(&w, &n, x, nullptr) == MOE_OK);
        n.eps = -1.0f;
        EXPECT(check_norm(&w, &n, x, nullptr) == MOE_ERR_INVALID_ARG);
        n.eps = NAN;
        EXPECT(check_norm(&w, &n, x, nullptr) == MOE_ERR_INVALID_ARG);
        n.eps = 1e-6f;
        n.ldo = 10;
        EXPECT(check_norm(&w, &n, x, nullptr) == MOE_ERR_INVALID_ARG);
        const size_t need = make_layout(&w, 8).total;
        EXPECT(check_ws(&w, 8, x, need) == MOE_OK);
        EXPECT(check_ws(&w, 8, x, need - 1) == MOE_ERR_WORKSPACE_TOO_SMALL);
        EXPECT(check_ws(&w, 8, nullptr, need) == MOE_ERR_INVALID_ARG);
        EXPECT(check_ws(&w, 8, reinterpret_cast<const void *>(kFake + 4), need) == MOE_ERR_MISALIGNED);
    }
    // a seeded sweep of shapes and rows: layouts are 256-byte aligned, ordered
    // and cover what the kernels index
    uint64_t st = 20261203;
    auto rnd = [&](int n) { st = st * 6364136223846793005ull + 1442695040888963407ull; return (int)((st >> 33) % (uint64_t)n); };
    int taken = 0;
    for (int t = 0; t < 20000; ++t) {
        const int H = 128 * (1 + rnd(64)), E = 1 + rnd(1024), k = 1 + rnd(16), I = 128 * (1 + rnd(32));
        const int Is = rnd(2) ? 128 * (1 + rnd(32)) : 0, fmt = rnd(6), R = rnd(1100) - 30;
        const moe_layer_weights w = weights(H, E, k, I, Is, fmt);
        if (validate_weights(&w) || validate_rows(&w, R)) continue;
        ++taken;
        const Layout L = make_layout(&w, R);
        const size_t offs[] = {L.logits, L.ids, L.w, L.s, L.counts, L.offsets, L.perm, L.meta, L.gemv,
                               L.mfma, L.tiles, L.h, L.dbuf, L.lrep, L.hrep, L.total};
        for (size_t i = 0; i < sizeof(offs) / sizeof(offs[0]); ++i) {
            EXPECT(offs[i] % 256 == 0);
            if (i) EXPECT(offs[i] >= offs[i - 1]);
        }
        const size_t ne = (size_t)R * k + (Is > 0 ? (size_t)R : 0);
        EXPECT(L.dbuf - L.h >= ne * (size_t)std::max(I, Is) * 4);
        if (R >= 2) EXPECT(L.lrep - L.dbuf >= ne * (size_t)H * 4);
    }
    EXPECT(taken > 1000);
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("host checks OK (%d sweep shapes)\n", taken);
    return 0;
}
