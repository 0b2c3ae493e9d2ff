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
// Every role works a wave at a time on LW-wave workgroups (LW a template
// parameter: 8 for the 35B-A3B shapes, where halving the workgroup count
// against 4 waves shortened the layer by 0.6 us: fewer workgroups to
// dispatch, to poll the routing, to rerun the top-k and to count; 12 and 16
// waves measured slower, one workgroup a CU leaving the roles on fewer CUs).
//
//   router          one wave per router row (and the shared-gate row); each
//                   workgroup stores a done word once its logits are stored
//   shared gate/up  the shared expert's h (needs no routing)
//   routed gate/up  wait for every router done word, take the top-k of the
//                   logits, then a slice of a routed expert's h; store a
//                   done word
//   down            wait for the router done words, take the top-k, load row
//                   o of every slot's down matrix at once, wait for every
//                   gate/up done word, then blend (the first one publishes
//                   the routing)
//
// Forward progress: the launcher takes this kernel only when every workgroup
// of the grid can be resident at once (an occupancy query), so all of them
// run concurrently and every wait is on a running workgroup.  Independently
// of that, a workgroup only ever waits on lower-indexed workgroups, so with
// workgroups dispatched in index order (on each XCD) every wait would end
// even without co-residency.  Every wait is also bounded in time: past the
// deadline (the ctx's wait limit, 10 ms by default, measured on the device's
// constant clock) the workgroup sets the ctx error word and goes on, so a
// starved launch costs at most about two deadlines (the down workgroups' two
// waits), never a hang.
//
// Ordering: values crossing workgroups are written and read only with
// agent-scope atomic operations (relaxed; on gfx950 these are the
// device-coherent stores and loads, which bypass the non-coherent caches), so
// no cache writeback or invalidate is needed.  A producer waits for its own
// stores to complete (s_waitcnt 0, every wave, then a barrier) before its
// done-word stores, so the stores are visible device-wide before the word
// that announces them; a consumer issues its data loads only after its poll
// load has returned the word (in-order issue within a wave, a barrier for
// the other waves).  This is the release/acquire pattern restricted to data
// that is itself accessed atomically.
// The last down workgroup of each replica group clears that group's done
// words for the next call;
// after a timed-out wait they may be left inconsistent, and the host clears
// them with the error word.
#include "gemv.hpp"

#include <mutex>
#include <vector>

namespace moe {

constexpr int P1 = kPairsPerWave;

// Synchronisation words (kLayerSyncWords of the ctx, zero between launches).
//
// Every router and gate/up workgroup announces itself with a done word of
// its own, stored once its stores have completed, in each of the kGroups
// replica lines: no arrival counters on the way (an atomic's round trip per
// hand-off, and arrivals at one address are serialised by the memory side).
// A waiting workgroup polls the lines of its replica group (block index %
// kGroups, its XCD) with one wave-wide load per 64 words and a ballot over
// the words it needs.  The down workgroups count on a per-group counter once
// they have read every done word they read; the last of group c clears
// replica line c.  (Polling the logits themselves instead of a done word,
// with an unset pattern restored after each launch, measured slower: 768
// waves re-reading 1 KB each load the memory side enough to delay the
// routing by 1.4 us.)
//
//   kSyncDone     kGroups replica lines of kDoneWords words:
//                   [0, kMaxRouterBlocks)        router workgroup b done
//                   [kDoneGu, kDoneWords)        gate/up workgroup (slot, slice) done:
//                                                word kDoneGu + slot * ngb + slice
//                                                (the shared expert is slot k)
//   kSyncDown     kGroups down counters (one per replica group)
//   kSyncNorm     the norm epilogue's counter of finished groups
constexpr int kGroups = kReplicas;
constexpr int kCtrWords = 16;        // 64 bytes between counters
constexpr int kDoneWords = 512;      // one replica line set (2 KB)
constexpr int kMaxRouterBlocks = 64;
constexpr int kDoneGu = kMaxRouterBlocks;
static_assert(kDoneGu == kWave, "the router done words fill the first 64-word line");
enum : int {
    kSyncDone = 0,
    kSyncDown = kSyncDone + kGroups * kDoneWords,
    kSyncNorm = kSyncDown + kGroups * kCtrWords,
    kSyncWordsTotal = kSyncNorm + kCtrWords
};
static_assert(kSyncWordsTotal <= kLayerSyncWords, "layer synchronisation words exceed the ctx layout");

// Arrivals at the down counter of replica group `sub` when `total` down
// workgroups are spread over the groups round-robin.
__host__ __device__ constexpr unsigned group_count(int total, int sub) {
    return total > sub ? (unsigned)((total - sub + kGroups - 1) / kGroups) : 0u;
}

// Gate/up done words of the lines (64 words) a down workgroup polls.
__host__ __device__ constexpr int gu_lines(int ks, int ngb) { return (ks * ngb + kWave - 1) / kWave; }

// Wave-wide poll of NC lines of 64 done words at p: true once every word
// c * 64 + lane with need[c] set in that lane is non-zero; false once
// `ticks` ticks of the constant clock have passed since the first poll (at
// least one poll is made).  Every lane of the wave calls it.  The next poll
// follows the last one's return with no sleep between (one wave per waiting
// workgroup polls; a sleep of 128 cycles measured 0.07 us a layer slower).
template <int NC>
__device__ __forceinline__ bool poll_words(const unsigned *p, const bool (&need)[NC], uint64_t ticks) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        unsigned v[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) v[c] = ld_agent(p + c * kWave + lane);
        bool missing = false;
#pragma unroll
        for (int c = 0; c < NC; ++c) missing |= need[c] && v[c] == 0u;
        if (__builtin_amdgcn_ballot_w64(missing) == 0) return true;
        if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) return false;
    }
}

// Every thread of the block calls this; wave 0 polls, the block waits at the
// barrier.  A timeout sets the error word.  The barrier is a bare s_barrier:
// the other waves only need to issue their loads after wave 0's poll has
// returned, and __syncthreads would first wait for every load the waves
// have in flight (the down workgroups' weight rows, issued long before and
// not needed until the blend).  The memory clobber keeps the compiler from
// moving loads across it.
template <int NC>
__device__ __forceinline__ void block_wait_words(const unsigned *p, const bool (&need)[NC], uint32_t *err,
                                                 uint64_t ticks) {
    if ((threadIdx.x >> 6) == 0 && !poll_words<NC>(p, need, ticks) && threadIdx.x == 0)
        flag_error(err, kErrWaitTimeout);
    asm volatile("s_barrier" ::: "memory");
}

// Count this block on `ctr` (of `n` arrivals) once all its waves' stores
// have completed; the last arrival resets the counter (nobody else touches
// it in this launch) and returns true in every thread.
__device__ __forceinline__ bool block_arrive_last(unsigned *ctr, unsigned n, unsigned *ticket_s) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned t = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t == n - 1) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *ticket_s = t;
    }
    __syncthreads();
    return *ticket_s == n - 1;
}

// Once all this block's waves' stores have completed, done word `word` of
// every replica line (threads 0 .. kGroups-1).
__device__ __forceinline__ void block_publish_done(unsigned *sync, int word) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x < kGroups)
        __hip_atomic_store(sync + kSyncDone + threadIdx.x * kDoneWords + word, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

struct LayerGrid {
    int nrb, nsb, ngb, ndb;   // router, shared gate/up, routed gate/up per slot, down blocks
    unsigned *sync;           // kSyncWordsTotal words
    uint64_t wait_ticks;      // a wait's deadline, in ticks of the constant clock
    uint64_t *stamps;         // diagnostics: kStampWords words per workgroup, or null
};

// Diagnostics (phase stamps): thread 0 of each workgroup records the constant
// clock at its phase boundaries in LDS and copies them to
// stamps[block * kStampWords + i] when the workgroup ends (stores to global
// memory would be waited for by the next barrier and lengthen the phase they
// measure); word 0 holds the role (0 router, 1 shared gate/up, 2 routed
// gate/up, 3 down), the slot << 8 and, for the last arrival of a down
// group, 1 << 16.  Words never stamped read all ones.
//   1 start
//   2 router: row dot done; waiters: the routing's done words seen
//   3 router: its stores complete and its done words stored; waiters: top-k done
//   4 gate/up: h computed and stored; down: down-row loads issued
//   5 gate/up: its stores complete and its done words stored; down: the
//     gate/up done words seen
//   6 down: h staged in LDS     7 down: blend stored
//   8 down: its group arrival returned
//   9 down (last of its group): the group's line cleared
//  10 waiters: the logits they select from have arrived
__device__ __forceinline__ uint64_t *stamp_lds() {
    __shared__ uint64_t words[kStampWords];
    return words;
}
__device__ __forceinline__ void stamp_begin(const LayerGrid &g) {
    if (g.stamps && threadIdx.x == 0)
        for (int i = 0; i < kStampWords; ++i) stamp_lds()[i] = ~0ull;
}
__device__ __forceinline__ void stamp(const LayerGrid &g, int i) {
    if (g.stamps && threadIdx.x == 0) stamp_lds()[i] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void stamp_role(const LayerGrid &g, uint64_t tag) {
    if (g.stamps && threadIdx.x == 0) stamp_lds()[0] = tag;
}
__device__ __forceinline__ void stamp_flush(const LayerGrid &g) {
    if (g.stamps && threadIdx.x == 0)
        for (int i = 0; i < kStampWords; ++i) g.stamps[(size_t)blockIdx.x * kStampWords + i] = stamp_lds()[i];
}

// h of every slot into LDS, read coherently (8-byte agent-scope loads, all
// of them issued before any is used) from one replica, and stored in
// chunk-quad order per slot (see DownRow::dot_perm): element i of slot j
// goes to float j*HS + ((f/4) * (HS/CPC) + i/CPC) * 4 + f%4, f = i % CPC.
// HS is the h stride, equal to every slot's intermediate size here.
template <int CPC, int HS, int KS, int NT>
__device__ __forceinline__ void stage_h(const float *h, int nslots, float *hl) {
    constexpr int PER = (KS * HS / 2 + NT - 1) / NT;   // 8-byte loads per thread
    const uint64_t *src = reinterpret_cast<const uint64_t *>(h);
    const int n2 = nslots * HS / 2;
    uint64_t t[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i2 = u * NT + threadIdx.x;
        t[u] = i2 < n2 ? __hip_atomic_load(const_cast<uint64_t *>(src + i2), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)
                       : 0;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i2 = u * NT + threadIdx.x;
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
__device__ __forceinline__ void block_topk(const RouteArgs &r, const float *lrep, int *ids_s, float *w_s,
                                           const LayerGrid &g) {
    if ((threadIdx.x >> 6) == 0) {
        const int lane = threadIdx.x & (kWave - 1);
        const float *l = r.logits_in ? r.logits_in : lrep;
        const bool coherent = r.logits_in == nullptr;
        float raw[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + kWave * i;
            const int ec = e < r.E ? e : r.E - 1;
            raw[i] = coherent ? ld_agent(l + ec) : l[ec];
        }
        if (g.stamps) {
            __builtin_amdgcn_s_waitcnt(0);
            stamp(g, 10);
        }
        int e;
        float w;
        topk_regs<NV>(raw, r.E, r.k, topk_lds<1>(0), e, w);
        if (lane < r.k) {
            ids_s[lane] = e;
            w_s[lane] = w;
        }
    }
    __syncthreads();
}

template <int FMT, int NCH, int NV, int LPR, int DCH, int KS, int HS, int LW>
__global__ __launch_bounds__(LW * kWave) void k_layer_r1(RouteArgs r, FfnArgs a, LayerGrid g) {
    // gate/up chunks per lane follow from the router's: H/1024 (fp8), H/2048 (nvfp4)
    constexpr int CH = byte_codes(FMT) ? (NCH + 1) / 2 : (NCH + 3) / 4;
    constexpr int NCG = gu_lines(KS, HS / (LW * P1));   // lines of gate/up done words
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
    const unsigned *done = sync + kSyncDone + rep_id * kDoneWords;   // this group's replica line
    const float *lrep = a.logits_rep + (size_t)rep_id * r.E;
    const size_t hrep_stride = (size_t)(k + (has_shared ? 1 : 0)) * a.hstride;
    // the routing is ready once every router workgroup's done word is set
    const bool need_router[1] = {lane < g.nrb};
    stamp_begin(g);
    stamp(g, 1);

    // ---------------------------------------------------------------- router
    if (b < g.nrb) {
        stamp_role(g, 0);
        const int n_router = r.logits_in ? 0 : r.E;
        const int n_rows = n_router + (r.wsg ? 1 : 0);
        if (!r.wsg && b == 0 && threadIdx.x == 0) st_agent(r.s, 1.0f);
        const int row = b * LW + wid;
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
        stamp(g, 2);
        // every router block's stores are complete before its done word
        block_publish_done(sync, b);
        stamp(g, 3);
        stamp_flush(g);
        return;
    }
    b -= g.nrb;

    // ---------------------------------------------------------------- shared gate/up
    if (b < g.nsb) {
        stamp_role(g, 1 | ((uint64_t)k << 8));
        const ExpertSet &X = a.shared;
        const int i0 = (b * LW + wid) * P1;
        if (i0 < X.inter) {
            GateUpRows<FMT, CH, P1> rows;
            rows.load(X, 0, i0, a.H);
            rows.template apply<true>(a.x, a.H, X.inter, i0, a.h_rep + (size_t)k * a.hstride, hrep_stride,
                                      kReplicas);
        }
        stamp(g, 4);
        block_publish_done(sync, kDoneGu + k * g.ngb + b);
        stamp(g, 5);
        stamp_flush(g);
        return;
    }
    b -= g.nsb;

    // ---------------------------------------------------------------- routed gate/up
    if (b < k * g.ngb) {
        const int slot = b % k, slice = b / k;
        stamp_role(g, 2 | ((uint64_t)slot << 8));
        block_wait_words<1>(done, need_router, a.err, g.wait_ticks);
        stamp(g, 2);
        block_topk<NV>(r, lrep, ids_s, w_s, g);
        stamp(g, 3);
        const int e = ids_s[slot];
        const ExpertSet &X = a.routed;
        const int i0 = (slice * LW + wid) * P1;
        if (i0 < X.inter) {
            GateUpRows<FMT, CH, P1> rows;
            rows.load(X, e, i0, a.H);
            rows.template apply<true>(a.x, a.H, X.inter, i0, a.h_rep + (size_t)slot * a.hstride, hrep_stride,
                                      kReplicas);
        }
        stamp(g, 4);
        block_publish_done(sync, kDoneGu + slot * g.ngb + slice);
        stamp(g, 5);
        stamp_flush(g);
        return;
    }
    b -= k * g.ngb;

    // ---------------------------------------------------------------- down + blend
    constexpr int RPW = kWave / LPR;
    const int sub = lane % LPR;
    const int o = (b * LW + wid) * RPW + lane / LPR;
    const bool live = o < a.H;
    const int nslots = k + (has_shared ? 1 : 0);
    stamp_role(g, 3);
    // the shared expert's down rows need no routing: with every slot present
    // (the instantiated shape, the shared expert last) they load before the
    // routing wait, ahead of the routed weight stream
    DownRow<FMT, LPR, DCH> rows[KS];
    const bool full = has_shared && k == KS - 1;
    if (full) rows[KS - 1].load(a.shared, 0, o, sub, live);
    block_wait_words<1>(done, need_router, a.err, g.wait_ticks);
    stamp(g, 2);
    block_topk<NV>(r, lrep, ids_s, w_s, g);
    stamp(g, 3);
    if (b == 0 && wid == 0 && lane < k) {
        r.ids[lane] = ids_s[lane];
        r.w[lane] = w_s[lane];
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        if (j < nslots && !(full && j == KS - 1)) {
            const bool sh = j == k;
            rows[j].load(sh ? a.shared : a.routed, sh ? 0 : ids_s[j], o, sub, live);
        }
    }
    const float s_gate = has_shared ? ld_agent(a.s) : 0.0f;
    const float res_in = a.res ? bf16_to_f32(a.res[live ? o : 0]) : 0.0f;   // unconditional load (clamped)
    stamp(g, 4);
    // every slot's h is complete once every gate/up workgroup's done word is set
    bool need_gu[NCG];
#pragma unroll
    for (int c = 0; c < NCG; ++c) need_gu[c] = c * kWave + lane < nslots * g.ngb;
    block_wait_words<NCG>(done + kDoneGu, need_gu, a.err, g.wait_ticks);
    stamp(g, 5);
    stage_h<cols_per_chunk<FMT>(), HS, KS, LW * kWave>(a.h_rep + (size_t)rep_id * hrep_stride, nslots,
                                           reinterpret_cast<float *>(hlds4));
    __syncthreads();
    // Without the norm epilogue the block counts itself on its group's
    // counter now: it has read every done word it reads (and every gate/up
    // block stored its done word after its h stores completed).  The atomic's latency
    // hides behind the blend; the last block of the group clears the group's
    // replica line at the end.  With the epilogue the count comes after the
    // outputs are stored (below).
    const int dsub = b % kGroups;
    const unsigned n_down = group_count(g.ndb, dsub);
    unsigned *down_ctr = sync + kSyncDown + rep_id * kCtrWords;
    unsigned early = 0;
    if (!a.norm_w && threadIdx.x == 0)
        early = __hip_atomic_fetch_add(down_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stamp(g, 6);
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
    stamp(g, 7);
    bool group_last;
    if (a.norm_w) {
        group_last = block_arrive_last(down_ctr, n_down, &ticket_s);
    } else {
        // wave 0 learns from thread 0 whether this block was its group's last
        group_last = wid == 0 && (unsigned)__builtin_amdgcn_readfirstlane((int)early) == n_down - 1;
        if (group_last && lane == 0) __hip_atomic_store(down_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    stamp(g, 8);
    if (group_last && wid == 0) {
        // nobody reads this group's replica line any more in this launch
        unsigned *line = sync + kSyncDone + rep_id * kDoneWords;
#pragma unroll
        for (int c = 0; c <= NCG; ++c)   // the router line, then the gate/up lines
            __hip_atomic_store(line + c * kWave + lane, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        stamp_role(g, 3 | (1u << 16));
        stamp(g, 9);
    }
    stamp_flush(g);
    if (a.norm_w && group_last &&
        block_arrive_last(sync + kSyncNorm, (unsigned)(g.ndb < kGroups ? g.ndb : kGroups), &ticket_s)) {
        // RMSNorm epilogue of the row (the residual after the add, else y):
        // every down workgroup's stores completed before its group counted it
        float *vrow = reinterpret_cast<float *>(hlds4);
        stage_row<true>(a.res ? a.res : a.y, a.H, vrow);
        block_rms_norm(vrow, a.H, a.norm_w, a.norm_eps, a.norm_out);
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

static LayerGrid layer_grid(const RouteArgs &r, const FfnArgs &a, int lpr, int lw, unsigned *sync,
                            uint64_t wait_ticks = 0, uint64_t *stamps = nullptr) {
    LayerGrid g;
    const int n_rows = (r.logits_in ? 0 : r.E) + (r.wsg ? 1 : 0);
    g.nrb = n_rows > 0 ? (n_rows + lw - 1) / lw : 1;
    g.nsb = a.shared.inter > 0 ? (a.shared.inter + lw * P1 - 1) / (lw * P1) : 0;
    g.ngb = (a.routed.inter + lw * P1 - 1) / (lw * P1);
    const int rows_per_block = lw * (kWave / lpr);
    g.ndb = (a.H + rows_per_block - 1) / rows_per_block;
    g.sync = sync;
    g.wait_ticks = wait_ticks;
    g.stamps = stamps;
    return g;
}
static int layer_blocks(const LayerGrid &g, const FfnArgs &a) { return g.nrb + g.nsb + a.k * g.ngb + g.ndb; }
static size_t layer_lds(const FfnArgs &a) {
    const size_t h = (size_t)(a.k + (a.shared.inter > 0 ? 1 : 0)) * a.hstride * 4;
    const size_t row = a.norm_w ? (size_t)a.H * 8 : 0;   // the epilogue's row and weight
    return h > row ? h : row;
}

template <int FMT, int NCH, int NV, int LPR, int DCH, int KS, int HS, int LW>
static hipError_t layer_launch(const RouteArgs &r, const FfnArgs &a, unsigned *sync, uint64_t wait_ticks,
                               uint64_t *stamps, int64_t stamp_words, hipStream_t st) {
    const LayerGrid g = layer_grid(r, a, LPR, LW, sync, wait_ticks, stamps);
    if (stamps && (int64_t)layer_blocks(g, a) * kStampWords > stamp_words) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_layer_r1<FMT, NCH, NV, LPR, DCH, KS, HS, LW>), dim3(layer_blocks(g, a)), dim3(LW * kWave),
                       layer_lds(a), st, r, a, g);
    return hipGetLastError();
}

// Whether every workgroup of the launch can be resident at once on the
// current device: the workgroups that wait are then running while the ones
// they wait on run, and the phases overlap.  (The waits are correct either
// way: a workgroup only waits on lower-indexed ones.)
template <int FMT, int NCH, int NV, int LPR, int DCH, int KS, int HS, int LW>
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
                    &per_cu, reinterpret_cast<const void *>(&k_layer_r1<FMT, NCH, NV, LPR, DCH, KS, HS, LW>), LW * kWave,
                    lds) != hipSuccess)
                return false;
            cache.push_back({dev, lds, per_cu});
        }
    }
    return layer_blocks(layer_grid(r, a, LPR, LW, nullptr), a) <= per_cu * cus;
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
#define MOE_LAYER_SHAPES(X)                \
    X(kFp8, 1, 1, 8, 1, 17, 128, 4)        \
    X(kFp8, 4, 4, 32, 1, 9, 512, 8)        \
    X(kFp8Bf16s, 4, 4, 32, 1, 9, 512, 8)   \
    X(kInt8Row, 4, 4, 32, 1, 9, 512, 8)    \
    X(kInt4Row, 4, 4, 16, 1, 9, 512, 8)    \
    X(kInt4G64, 4, 4, 16, 1, 9, 512, 8)

bool layer_r1_supported(const RouteArgs &r, const FfnArgs &a) {
    const int nslots = a.k + (a.shared.inter > 0 ? 1 : 0);
    if (layer_lds(a) > kLayerMaxHLds || (a.hstride & 1)) return false;
    const LayerShape s = layer_shape(r, a);
    // every replica group needs a down workgroup: its last one clears the
    // group's done words
#define MOE_MATCH(F, N, V, L, D, K, HSV, LWV)                                                          \
    if (s.fmt == F && s.nch == N && s.nv == V && s.lpr == L && s.dch == D && nslots <= K &&              \
        a.routed.inter == HSV && (a.shared.inter == 0 || a.shared.inter == HSV)) {                        \
        const LayerGrid g = layer_grid(r, a, L, LWV, nullptr);                                           \
        return g.ndb >= kGroups && g.nrb <= kMaxRouterBlocks &&                                          \
               kDoneGu + kWave * gu_lines(K, HSV / (LWV * P1)) <= kDoneWords &&                          \
               layer_resident<F, N, V, L, D, K, HSV, LWV>(r, a);                                          \
    }
    MOE_LAYER_SHAPES(MOE_MATCH)
#undef MOE_MATCH
    return false;
}

hipError_t launch_layer_r1(const RouteArgs &r, const FfnArgs &a, unsigned *sync, uint64_t wait_ticks,
                           uint64_t *stamps, int64_t stamp_words, hipStream_t st) {
    const LayerShape s = layer_shape(r, a);
    const int nslots = a.k + (a.shared.inter > 0 ? 1 : 0);
#define MOE_GO(F, N, V, L, D, K, HSV, LWV)                                                             \
    if (s.fmt == F && s.nch == N && s.nv == V && s.lpr == L && s.dch == D && nslots <= K &&              \
        a.routed.inter == HSV && (a.shared.inter == 0 || a.shared.inter == HSV))                          \
        return layer_launch<F, N, V, L, D, K, HSV, LWV>(r, a, sync, wait_ticks, stamps, stamp_words, st);
    MOE_LAYER_SHAPES(MOE_GO)
#undef MOE_GO
    return hipErrorInvalidValue;
}

}  // namespace moe
