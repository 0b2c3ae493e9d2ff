// layer.hip -- a whole one-row MoE layer in one launch (gfx950).
//
// The layer's steps (colibri pull request 1992, "What it is": router logits,
// routing, the routed experts and the gated shared expert, the sum joining the
// residual; GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels": router GEMV,
// moe_topk_softmax, gate/up + silu, down, weighted blend) depend on each other
// only through small published values, so one launch carries them with
// workgroups in four roles, laid out in index order:
//
//   [router | shared gate/up | routed gate/up | down]
//
//   router          one wave per router row (and the shared-gate row); the
//                   last router workgroup to finish raises a ready flag
//   shared gate/up  the shared expert's h (needs no routing)
//   routed gate/up  wait for the ready flag, take the top-k of the logits,
//                   then a slice of a routed expert's h; count themselves
//                   done per slot
//   down            wait for the ready flag, take the top-k, load row o of
//                   every slot's down matrix at once, wait for the slot
//                   counters, then blend (the first one publishes the routing)
//
// A workgroup only ever waits on lower-indexed workgroups, and workgroups are
// dispatched in index order, so every wait ends without needing all
// workgroups resident.  Every wait is also bounded: past the spin limit the
// workgroup sets the ctx error word and goes on.  Values crossing workgroups
// are written and read at agent scope (write-through stores, coherent loads);
// counters are agent-scope atomics; no cache writeback or invalidate is used.
// The last down workgroup resets the synchronisation words for the next call.
#include "gemv.hpp"

#include <mutex>
#include <vector>

namespace moe {

constexpr int P1 = kPairsPerWave;
constexpr int kSpinLimit = 1 << 16;

// Synchronisation words, each on its own 256-byte line so pollers and
// arrivals on different words do not share a memory channel; the ready flag
// has kReadyCopies copies, polled by block index.
constexpr int kLine = 64;            // words per line
constexpr int kReadyCopies = kReplicas;
enum : int {
    kSyncTicket = 0,
    kSyncReady = 1 * kLine,                                // kReadyCopies lines
    kSyncDownDone = (1 + kReadyCopies) * kLine,
    kSyncSlot0 = (2 + kReadyCopies) * kLine,               // kMaxSlots lines
    kSyncSlotsDone = (2 + kReadyCopies + kMaxSlots) * kLine,
    kSyncHReady = (3 + kReadyCopies + kMaxSlots) * kLine,  // kReadyCopies lines
    kSyncWordsTotal = (3 + 2 * kReadyCopies + kMaxSlots) * kLine
};

// True once *p >= target; false after the spin limit.
__device__ __forceinline__ bool poll_geq(const unsigned *p, unsigned target) {
    for (int i = 0; i < kSpinLimit; ++i) {
        if (ld_agent(p) >= target) return true;
        __builtin_amdgcn_s_sleep(4);
    }
    return false;
}

// Every thread of the block calls this; thread 0 polls, the block waits at
// the barrier.  A timeout sets the error word.
__device__ __forceinline__ void block_wait(const unsigned *p, unsigned target, uint32_t *err) {
    if (threadIdx.x == 0 && !poll_geq(p, target)) flag_error(err, kErrWaitTimeout);
    __syncthreads();
}

// Count this block done on `ctr` once all its waves' stores have completed.
__device__ __forceinline__ unsigned block_arrive(unsigned *ctr, unsigned *ticket_s) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        *ticket_s = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return *ticket_s;
}

// A gate/up block is done with its slot: the last block of the slot counts
// the slot done, and the last slot raises the h-ready flag (all copies).
// Nobody polls the counters themselves, only the flag copies.
__device__ __forceinline__ void slot_done(unsigned *sync, int slot, int blocks_per_slot, int nslots,
                                          unsigned *ticket_s) {
    if (block_arrive(sync + kSyncSlot0 + slot * kLine, ticket_s) != (unsigned)(blocks_per_slot - 1)) return;
    if (threadIdx.x == 0)
        *ticket_s = __hip_atomic_fetch_add(sync + kSyncSlotsDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*ticket_s == (unsigned)(nslots - 1) && threadIdx.x < kReadyCopies)
        __hip_atomic_store(sync + kSyncHReady + threadIdx.x * kLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct LayerGrid {
    int nrb, nsb, ngb, ndb;   // router, shared gate/up, routed gate/up per slot, down blocks
    unsigned *sync;           // kSyncWordsTotal words
};

// h of every slot into LDS, read coherently (8-byte agent-scope loads, all
// of them issued before any is used) from one replica, and stored in
// chunk-quad order per slot (see DownRow::dot_perm): element i of slot j
// goes to float j*HS + ((f/4) * (HS/CPC) + i/CPC) * 4 + f%4, f = i % CPC.
// HS is the h stride, equal to every slot's intermediate size here.
template <int CPC, int HS, int KS>
__device__ __forceinline__ void stage_h(const float *h, int nslots, float *hl) {
    constexpr int PER = (KS * HS / 2 + 255) / 256;   // 8-byte loads per thread
    const uint64_t *src = reinterpret_cast<const uint64_t *>(h);
    const int n2 = nslots * HS / 2;
    uint64_t t[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i2 = u * 256 + threadIdx.x;
        t[u] = i2 < n2 ? __hip_atomic_load(const_cast<uint64_t *>(src + i2), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)
                       : 0;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i2 = u * 256 + threadIdx.x;
        if (i2 < n2) {
            const int i = 2 * i2, j = i / HS, e = i % HS, c = e / CPC, f = e % CPC;
            *reinterpret_cast<uint64_t *>(hl + j * HS + ((f >> 2) * (HS / CPC) + c) * 4 + (f & 3)) = t[u];
        }
    }
}

// Wave 0 takes the top-k of the published logits; the block reads it from
// LDS.  Every waiting workgroup computes the same result from the same
// logits, which saves publishing it (a store and a load round trip).
template <int NV>
__device__ __forceinline__ void block_topk(const RouteArgs &r, const float *lrep, int *ids_s, float *w_s) {
    if ((threadIdx.x >> 6) == 0) {
        const int lane = threadIdx.x & (kWave - 1);
        int e;
        float w;
        topk_wave<NV>(r.logits_in ? r.logits_in : lrep, r.E, r.k, r.logits_in == nullptr, e, w);
        if (lane < r.k) {
            ids_s[lane] = e;
            w_s[lane] = w;
        }
    }
    __syncthreads();
}

template <int FMT, int NCH, int NV, int LPR, int DCH, int KS, int HS>
__global__ __launch_bounds__(256) void k_layer_r1(RouteArgs r, FfnArgs a, LayerGrid g) {
    // gate/up chunks per lane follow from the router's: H/1024 (fp8), H/2048 (nvfp4)
    constexpr int CH = byte_codes(FMT) ? (NCH + 1) / 2 : (NCH + 3) / 4;
    extern __shared__ f32x4 hlds4[];
    __shared__ unsigned ticket_s;
    __shared__ int ids_s[kMaxSlots];
    __shared__ float w_s[kMaxSlots];
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    int b = blockIdx.x;
    unsigned *sync = g.sync;
    const int k = a.k;
    const bool has_shared = a.shared.inter > 0;
    const int rep_id = blockIdx.x % kReplicas;
    const unsigned *ready = sync + kSyncReady + rep_id * kLine;
    const float *lrep = a.logits_rep + (size_t)rep_id * r.E;
    const size_t hrep_stride = (size_t)(k + (has_shared ? 1 : 0)) * a.hstride;

    // ---------------------------------------------------------------- router
    if (b < g.nrb) {
        const int n_router = r.logits_in ? 0 : r.E;
        const int n_rows = n_router + (r.wsg ? 1 : 0);
        if (!r.wsg && b == 0 && threadIdx.x == 0) st_agent(r.s, 1.0f);
        const int row = b * 4 + wid;
        if (row < n_rows) {
            const bool gate_row = row >= n_router;
            u32x4 wv[NCH];
            load_bf16_row<NCH>(gate_row ? r.wsg : r.wr + (size_t)row * r.H, r.H, wv);
            const float acc = dot_bf16_row<NCH>(wv, r.x, r.H);
            if (gate_row) {
                if (lane == 0) st_agent(r.s, sigmoid(acc));
            } else {
                const float l = acc + (r.bias ? r.bias[row] : 0.0f);
                if (lane < kReplicas) st_agent(a.logits_rep + (size_t)lane * r.E + row, l);
                if (lane == kReplicas) r.logits[row] = l;
            }
        }
        // every router block's stores are complete before its ticket, so the
        // last one can raise the ready flag at once
        if (block_arrive(sync + kSyncTicket, &ticket_s) == (unsigned)(g.nrb - 1) && wid == 0) {
            if (lane == 0) __hip_atomic_store(sync + kSyncTicket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane < kReadyCopies)
                __hip_atomic_store(sync + kSyncReady + lane * kLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    b -= g.nrb;

    // ---------------------------------------------------------------- shared gate/up
    if (b < g.nsb) {
        const ExpertSet &X = a.shared;
        const int i0 = (b * 4 + wid) * P1;
        if (i0 < X.inter) {
            GateUpRows<FMT, CH, P1> rows;
            rows.load(X, 0, i0, a.H);
            rows.template apply<true>(a.x, a.H, X.inter, i0, a.h_rep + (size_t)k * a.hstride, hrep_stride,
                                      kReplicas);
        }
        slot_done(sync, k, g.nsb, k + 1, &ticket_s);
        return;
    }
    b -= g.nsb;

    // ---------------------------------------------------------------- routed gate/up
    if (b < k * g.ngb) {
        const int slot = b % k, slice = b / k;
        block_wait(ready, 1u, a.err);
        block_topk<NV>(r, lrep, ids_s, w_s);
        const int e = ids_s[slot];
        const ExpertSet &X = a.routed;
        const int i0 = (slice * 4 + wid) * P1;
        if (i0 < X.inter) {
            GateUpRows<FMT, CH, P1> rows;
            rows.load(X, e, i0, a.H);
            rows.template apply<true>(a.x, a.H, X.inter, i0, a.h_rep + (size_t)slot * a.hstride, hrep_stride,
                                      kReplicas);
        }
        slot_done(sync, slot, g.ngb, k + (has_shared ? 1 : 0), &ticket_s);
        return;
    }
    b -= k * g.ngb;

    // ---------------------------------------------------------------- down + blend
    constexpr int RPW = kWave / LPR;
    const int sub = lane % LPR;
    const int o = (b * 4 + wid) * RPW + lane / LPR;
    const bool live = o < a.H;
    const int nslots = k + (has_shared ? 1 : 0);
    block_wait(ready, 1u, a.err);
    block_topk<NV>(r, lrep, ids_s, w_s);
    if (b == 0 && wid == 0 && lane < k) {
        r.ids[lane] = ids_s[lane];
        r.w[lane] = w_s[lane];
    }
    DownRow<FMT, LPR, DCH> rows[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        if (j < nslots) {
            const bool sh = j == k;
            rows[j].load(sh ? a.shared : a.routed, sh ? 0 : ids_s[j], o, sub, live);
        }
    }
    const float s_gate = has_shared ? ld_agent(a.s) : 0.0f;
    const float res_in = a.res ? bf16_to_f32(a.res[live ? o : 0]) : 0.0f;   // unconditional load (clamped)
    // every slot's h is complete once the h-ready flag is up
    block_wait(sync + kSyncHReady + rep_id * kLine, 1u, a.err);
    stage_h<cols_per_chunk<FMT>(), HS, KS>(a.h_rep + (size_t)rep_id * hrep_stride, nslots,
                                           reinterpret_cast<float *>(hlds4));
    __syncthreads();
    const float *hbase = reinterpret_cast<const float *>(hlds4);
    float y = 0.0f;
    if (has_shared && k == KS - 1) {
        // every slot present (the instantiated shape): no per-slot branches,
        // so the slots' LDS reads and lane reductions overlap; the same dots
        // and the same blend order as below
        float d[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const ExpertSet &X = j == KS - 1 ? a.shared : a.routed;
            d[j] = rows[j].dot_perm(hbase + (size_t)j * HS, X.inter, sub);
            d[j] *= global_scale<FMT>(X.dn_g, j == KS - 1 ? 0 : ids_s[j]);
        }
#pragma unroll
        for (int j = 0; j < KS; ++j) y = fmaf(j == KS - 1 ? s_gate : w_s[j], d[j], y);
    } else {
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            if (j < nslots) {
                const bool sh = j == k;
                const ExpertSet &X = sh ? a.shared : a.routed;
                float d = rows[j].dot_perm(hbase + (size_t)j * HS, X.inter, sub);
                d *= global_scale<FMT>(X.dn_g, sh ? 0 : ids_s[j]);
                y = fmaf(sh ? s_gate : w_s[j], d, y);
            }
        }
    }
    if (live && sub == 0) {
        const uint16_t yb = f32_to_bf16(y), rb = f32_to_bf16(res_in + y);
        if (a.norm_w) {
            // written through: the last down workgroup reads the whole row back
            if (a.y) __hip_atomic_store(a.y + o, yb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (a.res) __hip_atomic_store(a.res + o, rb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (a.y) a.y[o] = yb;
            if (a.res) a.res[o] = rb;
        }
    }
    const bool last = block_arrive(sync + kSyncDownDone, &ticket_s) == (unsigned)(g.ndb - 1);
    if (last && a.norm_w) {
        // RMSNorm epilogue of the row (the residual after the add, else y):
        // every down workgroup's stores completed before its arrival
        float *vrow = reinterpret_cast<float *>(hlds4);
        stage_row<true>(a.res ? a.res : a.y, a.H, vrow);
        block_rms_norm(vrow, a.H, a.norm_w, a.norm_eps, a.norm_out);
    }
    if (last && threadIdx.x == 0) {
        for (int c = 0; c < kReadyCopies; ++c) {
            __hip_atomic_store(sync + kSyncReady + c * kLine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + kSyncHReady + c * kLine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __hip_atomic_store(sync + kSyncSlotsDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int j = 0; j < kMaxSlots; ++j)
            __hip_atomic_store(sync + kSyncSlot0 + j * kLine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sync + kSyncDownDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------------------ launcher

constexpr size_t kLayerMaxHLds = 64 * 1024;

// The compile-time shape of a layer: router chunks per lane (NCH), logits per
// lane (NV), down lanes per row (LPR) and chunks per lane (DCH).
struct LayerShape {
    int fmt, nch, nv, lpr, dch;
};

static LayerShape layer_shape(const RouteArgs &r, const FfnArgs &a) {
    LayerShape s;
    s.fmt = a.fmt;
    s.nch = ((r.H >> 3) + kWave - 1) / kWave;
    s.nch = s.nch <= 1 ? 1 : s.nch <= 2 ? 2 : s.nch <= 4 ? 4 : s.nch <= 8 ? 8 : 16;
    s.nv = topk_nv(r.E);
    down_lane_shape(a.fmt, a.routed.inter, a.shared.inter, s.lpr, s.dch);
    s.dch = s.dch <= 1 ? 1 : s.dch <= 2 ? 2 : 4;
    return s;
}

static LayerGrid layer_grid(const RouteArgs &r, const FfnArgs &a, int lpr, unsigned *sync) {
    LayerGrid g;
    const int n_rows = (r.logits_in ? 0 : r.E) + (r.wsg ? 1 : 0);
    g.nrb = n_rows > 0 ? (n_rows + 3) / 4 : 1;
    g.nsb = a.shared.inter > 0 ? (a.shared.inter + 4 * P1 - 1) / (4 * P1) : 0;
    g.ngb = (a.routed.inter + 4 * P1 - 1) / (4 * P1);
    const int rows_per_block = 4 * (kWave / lpr);
    g.ndb = (a.H + rows_per_block - 1) / rows_per_block;
    g.sync = sync;
    return g;
}
static int layer_blocks(const LayerGrid &g, const FfnArgs &a) { return g.nrb + g.nsb + a.k * g.ngb + g.ndb; }
static size_t layer_lds(const FfnArgs &a) {
    const size_t h = (size_t)(a.k + (a.shared.inter > 0 ? 1 : 0)) * a.hstride * 4;
    const size_t row = a.norm_w ? (size_t)a.H * 8 : 0;   // the epilogue's row and weight
    return h > row ? h : row;
}

template <int FMT, int NCH, int NV, int LPR, int DCH, int KS, int HS>
static hipError_t layer_launch(const RouteArgs &r, const FfnArgs &a, unsigned *sync, hipStream_t st) {
    const LayerGrid g = layer_grid(r, a, LPR, sync);
    hipLaunchKernelGGL((k_layer_r1<FMT, NCH, NV, LPR, DCH, KS, HS>), dim3(layer_blocks(g, a)), dim3(256),
                       layer_lds(a), st, r, a, g);
    return hipGetLastError();
}

// Whether every workgroup of the launch can be resident at once on the
// current device: the workgroups that wait are then running while the ones
// they wait on run, and the phases overlap.  (The waits are correct either
// way: a workgroup only waits on lower-indexed ones.)
template <int FMT, int NCH, int NV, int LPR, int DCH, int KS, int HS>
static bool layer_resident(const RouteArgs &r, const FfnArgs &a) {
    struct Entry { int device; size_t lds; int per_cu; };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    const size_t lds = layer_lds(a);
    int per_cu = -1;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry &e : cache)
            if (e.device == dev && e.lds == lds) per_cu = e.per_cu;
        if (per_cu < 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &per_cu, reinterpret_cast<const void *>(&k_layer_r1<FMT, NCH, NV, LPR, DCH, KS, HS>), 256,
                    lds) != hipSuccess)
                return false;
            cache.push_back({dev, lds, per_cu});
        }
    }
    return layer_blocks(layer_grid(r, a, LPR, nullptr), a) <= per_cu * cus;
}

// The shapes the single launch is built for: the tiny layer (H 256, E 16,
// I 128) and the 35B-A3B layer (H 2048, E 256, I 512) in fp8 and in the
// other expert formats (int8 and int4 per row, int4-g64, fp8 with bf16
// scales; int4 rows of 512 codes take 16 lanes a row in down).  KS: the most
// slots (routed + shared) an instantiation holds; HS: the intermediate size
// of every slot (routed and shared alike).  Other shapes, and any launch
// whose workgroups do not all fit on the device at once (the 397B-A17B
// shape, for one: 2049 workgroups against about 768 resident, measured
// slower than the three launches), take the three-launch path.
#define MOE_LAYER_SHAPES(X)             \
    X(kFp8, 1, 1, 8, 1, 17, 128)        \
    X(kFp8, 4, 4, 32, 1, 9, 512)        \
    X(kFp8Bf16s, 4, 4, 32, 1, 9, 512)   \
    X(kInt8Row, 4, 4, 32, 1, 9, 512)    \
    X(kInt4Row, 4, 4, 16, 1, 9, 512)    \
    X(kInt4G64, 4, 4, 16, 1, 9, 512)

bool layer_r1_supported(const RouteArgs &r, const FfnArgs &a) {
    const int nslots = a.k + (a.shared.inter > 0 ? 1 : 0);
    if (layer_lds(a) > kLayerMaxHLds || (a.hstride & 1)) return false;
    const LayerShape s = layer_shape(r, a);
#define MOE_MATCH(F, N, V, L, D, K, HSV)                                                               \
    if (s.fmt == F && s.nch == N && s.nv == V && s.lpr == L && s.dch == D && nslots <= K &&              \
        a.routed.inter == HSV && (a.shared.inter == 0 || a.shared.inter == HSV))                          \
        return layer_resident<F, N, V, L, D, K, HSV>(r, a);
    MOE_LAYER_SHAPES(MOE_MATCH)
#undef MOE_MATCH
    return false;
}

hipError_t launch_layer_r1(const RouteArgs &r, const FfnArgs &a, unsigned *sync, hipStream_t st) {
    const LayerShape s = layer_shape(r, a);
    const int nslots = a.k + (a.shared.inter > 0 ? 1 : 0);
#define MOE_GO(F, N, V, L, D, K, HSV)                                                                  \
    if (s.fmt == F && s.nch == N && s.nv == V && s.lpr == L && s.dch == D && nslots <= K &&              \
        a.routed.inter == HSV && (a.shared.inter == 0 || a.shared.inter == HSV))                          \
        return layer_launch<F, N, V, L, D, K, HSV>(r, a, sync, st);
    MOE_LAYER_SHAPES(MOE_GO)
#undef MOE_GO
    return hipErrorInvalidValue;
}

}  // namespace moe
