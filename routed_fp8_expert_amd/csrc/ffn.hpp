// ffn.hpp -- expert kernels for gfx950 (GEMV arm) and their launchers, one
// instantiation per weight format (ffn_<format>.hip); ffn.hip holds the
// format dispatch, the blend and the RMSNorm kernels.
//
// GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels":
// moe_expert_gate_up_shared_fp8 (routed and shared gate/up in one launch),
// moe_expert_silu_down_shared_fp8, moe_weighted_sum_blend; "Precision":
// fp8/block128x128 weights read bf16 activations (gate/up) and f32
// activations (down).  colibri pull request 1992, "A decode GEMV": a wave per
// output row with 16 bytes per lane reads weights near the bus rate, versus a
// whole block per row; here each wave keeps several 16-byte weight loads per
// lane in flight and reduces across the wave64 with DPP.
//
// One decode row (three launches):
//   lead     router rows (+ shared-gate row) and the shared expert's gate/up,
//            which does not depend on the routing; warms the shared expert's
//            down matrix into the memory-side cache
//   gate/up  each wave takes the top-k of the logits itself, then its slice of
//            a routed expert's gate/up; warms that expert's down rows
//   down     each row group streams row o of all k+1 down matrices, stages h
//            in LDS, and blends in slot order into the residual
#pragma once

#include "mfma.hpp"

namespace moe {

constexpr int P = kPairsPerWave;
constexpr int kWarmLoads = 4;            // 16-byte warming loads per thread (16 KB per block)

// Which expert and which entries (rows of h / dbuf) a task covers.
// R == 1: task j < k is slot j, task k the shared expert.
// R >= 2: task u < max_routed_tasks is the u-th GEMV-arm expert (its rows
// from the grouping), the last task the shared expert over all R rows.
struct Task {
    ExpertSet X;           // the expert family (a copy: no pointer into the kernel arguments)
    int e;                 // expert index within its family
    int n;                 // number of entries
    const int32_t *list;   // entry list (routed, R >= 2) or null
    int first;             // first entry when list is null (entries first .. first+n-1)
    bool valid;
};

__device__ __forceinline__ Task resolve_task(const FfnArgs &a, int task) {
    Task t{a.routed, 0, 0, nullptr, 0, false};
    const int nk = a.R * a.k;
    if (a.R == 1) {
        if (task < a.k) {
            t.e = a.ids[task];
            t.n = 1;
            t.first = task;
            t.valid = t.e >= 0 && t.e < a.E;
            if (!t.valid) flag_error(a.err, kErrBadExpertId);
        } else {
            t.X = a.shared;
            t.n = 1;
            t.first = nk;
            t.valid = a.shared.inter > 0;
        }
        return t;
    }
    if (task < a.max_routed_tasks) {
        if (task >= a.meta[kMetaGemvCount]) return t;
        t.e = a.gemv_list[task];
        t.valid = t.e >= 0 && t.e < a.E;
        if (t.valid) {
            t.n = a.counts[t.e];
            const int off = a.offsets[t.e];
            // caller-supplied grouping must stay inside the R*k entries
            if (t.n < 0 || off < 0 || off + t.n > nk) {
                flag_error(a.err, kErrBadExpertId);
                t.valid = false;
                return t;
            }
            t.list = a.perm + off;
        }
    } else {
        t.X = a.shared;
        t.n = a.R;
        t.first = nk;
        t.valid = a.shared.inter > 0;
    }
    return t;
}

// Entry n of a task; -1 when a caller-supplied permutation points outside
// the step's R*k routed entries.
__device__ __forceinline__ int task_entry(const Task &t, int n, int nk) {
    if (!t.list) return t.first + n;
    const int e = t.list[n];
    return (e >= 0 && e < nk) ? e : -1;
}
__device__ __forceinline__ int entry_row(const FfnArgs &a, int entry) {
    const int nk = a.R * a.k;
    return entry < nk ? entry / a.k : entry - nk;
}

// Warm a (at most 16 KB) slice `part` of `nparts` of a matrix of `bytes`
// bytes into the memory-side cache; returns the folded word.
// A block's share of a matrix read once to warm it into the memory-side
// cache: issue() sends the loads, fold() (after the block's real work, so
// nothing issued later waits behind these loads) folds them into one word.
struct WarmSlice {
    u32x4 v[kWarmLoads];
    __device__ __forceinline__ void issue(const uint8_t *base, size_t bytes, int part, int nparts) {
        size_t chunk = (bytes + nparts - 1) / nparts;
        chunk = (chunk + 15) & ~(size_t)15;
        const size_t cap = (size_t)kWarmLoads * 16 * 256;
        if (chunk > cap) chunk = cap;
        const size_t begin = (size_t)part * chunk;
#pragma unroll
        for (int i = 0; i < kWarmLoads; ++i) {
            const size_t off = begin + ((size_t)i * 256 + threadIdx.x) * 16;
            v[i] = (off + 16 <= bytes && off < begin + chunk) ? ld16(base + off) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ uint32_t fold() const {
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < kWarmLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
        return acc;
    }
};

__device__ __forceinline__ void sink_word(uint32_t *sink, uint32_t acc) {
    if (acc == 0x9E3779B9u && sink) *sink = acc;
}

// ------------------------------------------------------------------ generic gate/up

// gate/up GEMV + silu*mul for the task's rows.  Block = 4 waves; a wave owns
// PM (gate, up) row pairs of one expert in registers and walks the task's
// entries, loading the next entry's activation chunks before reducing the
// current one.
template <int FMT, int CH, int PM>
__device__ __forceinline__ void gate_up_gemv_unit(const FfnArgs &a, int bx, int task) {
    constexpr int XQ = x_quads<FMT>();
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
    const Task t = resolve_task(a, task);
    if (!t.valid || t.n == 0) return;
    const ExpertSet &X = t.X;
    const int i0 = (bx * 4 + wid) * PM;
    if (i0 >= X.inter) return;
    using Rows = GateUpRows<FMT, CH, PM>;
    const int nk = a.R * a.k;
    // the first entry's activation loads go out before the weight loads
    // (which are converted as they arrive, so waited for at once): the
    // activations then travel with the weights instead of after them
    int mine = lane < min(kWave, t.n) ? task_entry(t, lane, nk) : -1;
    int ec = readlane(mine, 0);
    u32x4 xc[CH][XQ], xn[CH][XQ];
    if (ec >= 0) Rows::load_x(a.x + (size_t)entry_row(a, ec) * a.ldx, a.H, xc);
    Rows rows;
    rows.load(X, t.e, i0, a.H);
    for (int n0 = 0; n0 < t.n; n0 += kWave) {
        const int cnt = min(kWave, t.n - n0);
        if (n0 > 0) {
            mine = lane < cnt ? task_entry(t, n0 + lane, nk) : -1;
            ec = readlane(mine, 0);
            if (ec >= 0) Rows::load_x(a.x + (size_t)entry_row(a, ec) * a.ldx, a.H, xc);
        }
        for (int j = 0; j < cnt; ++j) {
            const int en = j + 1 < cnt ? readlane(mine, j + 1) : -1;
            if (en >= 0) Rows::load_x(a.x + (size_t)entry_row(a, en) * a.ldx, a.H, xn);
            if (ec < 0) {
                flag_error(a.err, kErrBadExpertId);
            } else {
                float acc[2 * PM];
                rows.partial(xc, a.H, acc);
                rows.finish(acc, X.inter, i0, a.h + (size_t)ec * a.hstride);
            }
#pragma unroll
            for (int c = 0; c < CH; ++c)
#pragma unroll
                for (int q = 0; q < XQ; ++q) xc[c][q] = xn[c][q];
            ec = en;
        }
    }
}

// gate/up of a step, both arms in one launch: workgroups [0, nm) are
// matrix-core units (column group b % nmx of tile b / nmx, fp8 only), the
// rest GEMV units (slice b % gx of task b / gx).
// (fp8: two waves a SIMD where the registers allow it; the compiler would
// otherwise give the matrix-core unit more and run one.)
template <int FMT, int CH, int PM>
__global__ __launch_bounds__(256, FMT == kFp8 && CH <= 4 ? 2 : 1) void k_gate_up(FfnArgs a, int nmx, int nm, int gx) {
    int b = blockIdx.x;
    if constexpr (FMT == kFp8) {
        if (b < nm) {
            mfma_gate_up_unit(a, b % nmx, b / nmx);
            return;
        }
    }
    b -= nm;
    gate_up_gemv_unit<FMT, CH, PM>(a, b % gx, b / gx);
}

// ------------------------------------------------------------------ one-row fused kernels

// Lead kernel of a one-row layer.  Blocks [0, nrb): one wave per router row
// (the E router rows unless logits are given, then just the shared-gate row);
// the logits are stored write-through (agent scope), each router block then
// takes a ticket, and the last one runs the top-k and publishes ids and
// weights.  No cache writeback or invalidate is needed: the last block reads
// the logits with agent-scope loads.  Blocks [nrb, ...): the shared expert's
// gate/up pairs for the row, each block also warming a slice of the shared
// expert's down matrix into the memory-side cache.
template <int FMT, int NCH, int CH, int NV>
__global__ __launch_bounds__(256) void k_lead_r1(RouteArgs r, FfnArgs a) {
    __shared__ unsigned ticket_s;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    const int n_router = r.logits_in ? 0 : r.E;
    const int n_rows = n_router + (r.wsg ? 1 : 0);
    const int nrb = n_rows > 0 ? (n_rows + 3) / 4 : 1;
    if (!r.wsg && blockIdx.x == 0 && threadIdx.x == 0) r.s[0] = 1.0f;
    if ((int)blockIdx.x < nrb) {
        const int row = blockIdx.x * 4 + wid;
        if (row < n_rows) {
            const bool gate_row = row >= n_router;
            u32x4 wv[NCH];
            load_bf16_row<NCH>(gate_row ? r.wsg : r.wr + (size_t)row * r.H, r.H, wv);
            const float acc = dot_bf16_row<NCH>(wv, r.x, r.H);
            if (lane == 0) {
                if (gate_row)
                    r.s[0] = sigmoid(acc);
                else
                    st_agent(r.logits + row, acc + (r.bias ? r.bias[row] : 0.0f));
            }
        }
        __builtin_amdgcn_s_waitcnt(0);     // this wave's stores have completed
        __syncthreads();
        if (threadIdx.x == 0)
            ticket_s = __hip_atomic_fetch_add(r.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (ticket_s != (unsigned)(nrb - 1) || wid != 0) return;
        int e;
        float w;
        topk_wave<NV>(r.logits_in ? r.logits_in : r.logits, r.E, r.k, r.logits_in == nullptr, topk_lds<1>(0), e, w);
        if (lane < r.k) {
            r.ids[lane] = e;
            r.w[lane] = w;
        }
        if (lane == 0) __hip_atomic_store(r.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const ExpertSet &X = a.shared;
    if (X.inter <= 0) return;
    const int b = blockIdx.x - nrb, nsb = gridDim.x - nrb;
    const int i0 = (b * 4 + wid) * P;
    // activations, then weights, then the warming loads; the dot waits for
    // the first two only (a wave past the expert's rows loads clamped rows
    // as zeros and stores nothing)
    using Rows = GateUpRows<FMT, CH, P>;
    u32x4 x[CH][x_quads<FMT>()];
    Rows::load_x(a.x, a.H, x);
    Rows rows;
    rows.load(X, 0, i0, a.H);
    WarmSlice warm;
    warm.issue(X.dn, (size_t)a.H * row_bytes<FMT>(X.inter), b, nsb);
    float acc[2 * P];
    rows.partial(x, a.H, acc);
    rows.finish(acc, X.inter, i0, a.h + (size_t)a.k * a.hstride);
    sink_word(a.sink, warm.fold());
}

// gate/up of the routed experts of a one-row layer, and of a step of a few
// rows without grouping.  Grid (slices, slots, R): block (b, j, r) takes slot
// j of row r (its expert from the published ids, h row r*k + j) and its slice
// b.  With several rows slot k is the shared expert, run by the blocks of row 0 for
// every row (weights loaded once; h rows R*k + r); at one row the lead kernel
// runs it.
//
// With topk_src set (steps of a few rows), the routed blocks take row r's
// top-k themselves (wave 0, from the logits in memory) instead of reading
// published ids; block (0, 0, r) publishes the row's ids and weights and its
// shared gate (s_mode).
template <int FMT, int CH, int NV>
__global__ __launch_bounds__(256) void k_gate_up_r1(FfnArgs a) {
    __shared__ int e_s;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
    const int slot = blockIdx.y, r = blockIdx.z;
    const int i0 = (blockIdx.x * 4 + wid) * P;
    if (a.topk_src && slot < a.k) {
        const bool publish = blockIdx.x == 0 && slot == 0;
        if (wid == 0) {
            int my_e;
            float my_w;
            topk_wave<NV>(a.topk_src + (size_t)r * a.E, a.E, a.k, false, topk_lds<1>(0), my_e, my_w);
            const int es = __builtin_amdgcn_readlane(my_e, slot);
            if (lane == 0) e_s = es;
            // the routing arrays are the caller's (writable); the other
            // expert kernels only read them, hence the const views
            if (publish && lane < a.k) {
                const_cast<int32_t *>(a.ids)[(size_t)r * a.k + lane] = my_e;
                const_cast<float *>(a.w)[(size_t)r * a.k + lane] = my_w;
            }
        } else if (wid == 1 && publish && a.s_mode != 0) {
            const float s = a.s_mode == 1 ? sigmoid(dot_bf16_row_stream(a.wsg, a.x + (size_t)r * a.ldx, a.H)) : 1.0f;
            if (lane == 0) const_cast<float *>(a.s)[r] = s;
        }
        __syncthreads();
    }
    using Rows = GateUpRows<FMT, CH, P>;
    constexpr int XQ = x_quads<FMT>();
    if (slot == a.k) {
        const ExpertSet &X = a.shared;
        if (r != 0 || i0 >= X.inter) return;
        // every row with this wave's shared rows (the first row's
        // activations issued with the weights)
        u32x4 x[CH][XQ];
        Rows::load_x(a.x, a.H, x);
        Rows rows;
        rows.load(X, 0, i0, a.H);
        for (int rr = 0; rr < a.R; ++rr) {
            if (rr > 0) Rows::load_x(a.x + (size_t)rr * a.ldx, a.H, x);
            float acc[2 * P];
            rows.partial(x, a.H, acc);
            rows.finish(acc, X.inter, i0, a.h + (size_t)(a.R * a.k + rr) * a.hstride);
        }
        return;
    }
    const int e = a.topk_src ? e_s : a.ids[(size_t)r * a.k + slot];
    if (e < 0 || e >= a.E) {
        if (threadIdx.x == 0 && blockIdx.x == 0) flag_error(a.err, kErrBadExpertId);
        return;
    }
    const ExpertSet &X = a.routed;
    // activations and weights in flight before the first wait (a wave past
    // the expert's rows loads clamped rows as zeros and stores nothing).
    // (Warming the expert's down matrix into the memory-side cache from here
    // for the down launch measured slower: 35B-A3B 2 / 4 / 8 rows 19.4 /
    // 31.4 / 54.0 against 16.4 / 26.2 / 45.3 us, 397B-A17B one row 32.1
    // against 29.6 us.)
    u32x4 x[CH][XQ];
    Rows::load_x(a.x + (size_t)r * a.ldx, a.H, x);
    Rows rows;
    rows.load(X, e, i0, a.H);
    float acc[2 * P];
    rows.partial(x, a.H, acc);
    rows.finish(acc, X.inter, i0, a.h + ((size_t)r * a.k + slot) * a.hstride);
}

// Down GEMV fused with the blend, for one row (blockIdx.y) of a one-row
// layer or of a step of a few rows.  A row group of LPR lanes owns output
// element o; it loads row o of every slot's down matrix up front (all k+1
// experts' loads in flight), stages the row's h in LDS (HLDS), then for each
// slot in order reduces d_j and accumulates y = fma(w_j, d_j, y), then
// fma(s, d_shared, y), and adds into the residual.  Slot j's h is row r*k + j,
// the shared expert's row R*k + r.  kDownR1Waves waves a workgroup: the
// row's h is staged once for that many waves' output elements.
constexpr int kDownR1Waves = 8;
// h quads a thread of the per-row down kernel loads per staging pass
__host__ __device__ constexpr int down_r1_stage_loads(int fmt) { return byte_codes(fmt) ? 3 : 6; }
//
// KS > 0: an instantiation for exactly KS slots (k + 1 with the shared
// expert); its slot loops carry no per-slot branch, so the compiler counts
// the loads in flight exactly and each wait below is for the loads it
// needs (with branches it waits for all of them).  KS = 0: any slot count.
template <int FMT, int LPR, int CH, bool HLDS, int KS = 0>
__global__ __launch_bounds__(kDownR1Waves * kWave) void k_down_r1(FfnArgs a) {
    extern __shared__ f32x4 hlds4[];
    constexpr int RPW = kWave / LPR;
    constexpr int NS = KS > 0 ? KS : kMaxSlots;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.y;
    const int sub = lane % LPR;
    const int o = (blockIdx.x * kDownR1Waves + wid) * RPW + lane / LPR;
    const bool live = o < a.H;
    const int nslots = KS > 0 ? KS : a.k + (a.shared.inter > 0 ? 1 : 0);
    auto hrow = [&](int j) { return j == a.k ? (size_t)a.R * a.k + r : (size_t)r * a.k + j; };

    // 32-code chunks (e2m1, int4): h staged in chunk-quad order per slot
    // (DownRow::dot_perm), the quad of slot j starting at element c*CPC + f
    // going to quad (f/4)*(I_j/CPC) + c, so the lanes of a row group read
    // consecutive quads, not quads 128 bytes apart (LDS bank conflicts);
    // measured faster there, slower for 16-code chunks, which keep the plain
    // layout
    constexpr bool PERM = !byte_codes(FMT);
    constexpr int CPC = cols_per_chunk<FMT>();
    constexpr int NT = kDownR1Waves * kWave;
    constexpr int SL = down_r1_stage_loads(FMT);
    const int n4 = a.hstride / 4, total = nslots * n4;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(a.h);
    f32x4 t[SL];
    // staging pass i0: loads from clamped indices, all issued before any is stored
    auto stage_load = [&](int i0) {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int i = i0 + u * NT, ic = i < total ? i : total - 1;
            const int j = ic / n4, q4 = ic - j * n4;
            t[u] = src[hrow(j) * n4 + q4];
        }
    };
    auto stage_store = [&](int i0) {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int i = i0 + u * NT;
            if (i >= total) continue;
            const int j = i / n4, q4 = i - j * n4;
            if (!PERM) {
                hlds4[i] = t[u];
                continue;
            }
            const int ij = j == a.k ? a.shared.inter : a.routed.inter;
            if (4 * q4 < ij) {
                const int c = (4 * q4) / CPC, f = (4 * q4) % CPC;
                hlds4[j * n4 + (f >> 2) * (ij / CPC) + c] = t[u];
            }
        }
    };
    // the row's expert ids in one load (lane j: slot j), read out at once;
    // then the first h staging pass (cache hits), then the down rows (from
    // HBM): loads return in order, so the h stores below wait for the h
    // loads only
    const int idv = a.ids[(size_t)r * a.k + (lane < a.k ? lane : 0)];
    // the blend weights likewise (lane j < k: w_j, lane k: the shared gate),
    // loaded before the rows so that no load issued after them is waited for
    const float cfv = lane < a.k ? a.w[(size_t)r * a.k + lane] : a.s[r];
    int eid[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) eid[j] = readlane(idv, j);
    // and the per-expert global scales (NVFP4; lane j: slot j's expert)
    float gsv = 1.0f;
    if constexpr (KS > 0 && FMT == kNvfp4) {
        const bool ok = idv >= 0 && idv < a.E;
        gsv = lane < a.k ? a.routed.dn_g[ok ? idv : 0] : a.shared.dn_g[0];
    }
    if (HLDS) stage_load(threadIdx.x);
    DownRow<FMT, LPR, CH, true> rows[NS];
    int es[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        if (KS > 0 || j < nslots) {
            const bool sh = j == a.k;
            const ExpertSet &X = sh ? a.shared : a.routed;
            const int e = sh ? 0 : eid[j];
            const bool ok = sh || (e >= 0 && e < a.E);
            es[j] = ok ? e : -1;
            if constexpr (KS > 0)
                rows[j].template load<true>(X, ok ? e : 0, o, sub, live && ok);
            else
                rows[j].load(X, ok ? e : 0, o, sub, live && ok);
        }
    }
    if (HLDS) {
        stage_store(threadIdx.x);
        // (KS > 0 is launched only when one pass stages all of h: a loop here
        // made the compiler wait for every load in flight after it)
        if constexpr (KS == 0) {
            for (int i0 = threadIdx.x + SL * NT; i0 < total; i0 += SL * NT) {
                stage_load(i0);
                stage_store(i0);
            }
        }
        // LDS only: each slot's dot below waits for its own rows, so the
        // dots run while the later slots' rows still stream in
        barrier_lds();
    }
    const float *hl = reinterpret_cast<const float *>(hlds4);
    float y = 0.0f;
    bool bad = false;   // (KS > 0) an invalid id, flagged at the end
    if constexpr (KS > 0) {
        // an invalid id's row was loaded as zeros: its slot adds w * 0
#pragma unroll
        for (int j = 0; j < NS; ++j) bad |= es[j] < 0;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const bool sh = j == a.k;
            const ExpertSet &X = sh ? a.shared : a.routed;
            float d = !HLDS ? rows[j].dot(a.h + hrow(j) * a.hstride, X.inter, sub)
                      : PERM ? rows[j].dot_perm(hl + (size_t)j * a.hstride, X.inter, sub)
                             : rows[j].dot(hl + (size_t)j * a.hstride, X.inter, sub);
            if constexpr (FMT == kNvfp4) d *= readlane(gsv, j);
            y = fmaf(readlane(cfv, j), d, y);
        }
    } else {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (j < nslots) {
                const bool sh = j == a.k;
                const ExpertSet &X = sh ? a.shared : a.routed;
                if (es[j] < 0) {
                    if (threadIdx.x == 0 && blockIdx.x == 0) flag_error(a.err, kErrBadExpertId);
                    continue;
                }
                float d = !HLDS ? rows[j].dot(a.h + hrow(j) * a.hstride, X.inter, sub)
                          : PERM ? rows[j].dot_perm(hl + (size_t)j * a.hstride, X.inter, sub)
                                 : rows[j].dot(hl + (size_t)j * a.hstride, X.inter, sub);
                d *= global_scale<FMT>(X.dn_g, es[j]);
                y = fmaf(sh ? a.s[r] : a.w[(size_t)r * a.k + j], d, y);
            }
        }
    }
    if (live && sub == 0) store_out(a.y, a.res, a.ldy, r, o, y);
    // (a branch with an atomic before the dots made the compiler wait there
    // for every load in flight)
    if (bad && threadIdx.x == 0 && blockIdx.x == 0) flag_error(a.err, kErrBadExpertId);
}

// Down GEMV for one expert of a multi-row step.  A row group of LPR lanes
// keeps RPL consecutive rows of the expert's down matrix in registers; per
// entry it loads the lane's h chunks once (the next entry's while reducing
// the current one), forms the RPL partial sums and reduces them together,
// row i ending in the group's lanes [i * LPR/RPL, (i+1) * LPR/RPL).
template <int FMT, int LPR, int CH, int RPL>
__device__ __forceinline__ void down_gemv_unit(const FfnArgs &a, int bx, int task) {
    constexpr int G = kWave / LPR, HQ = h_quads<FMT>(), SPAN = LPR / RPL;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
    const Task t = resolve_task(a, task);
    if (!t.valid || t.n == 0) return;
    const ExpertSet &X = t.X;
    const int wave_row0 = (bx * 4 + wid) * G * RPL;
    if (wave_row0 >= a.H) return;
    const int sub = lane % LPR;
    const int o0 = wave_row0 + (lane / LPR) * RPL;
    using Row = DownRow<FMT, LPR, CH>;
    const int nk = a.R * a.k;
    // the first entry's h loads before the weight loads (as in the gate/up unit)
    int mine = lane < min(kWave, t.n) ? task_entry(t, lane, nk) : -1;
    int ec = readlane(mine, 0);
    f32x4 hc[CH][HQ], hn[CH][HQ];
    if (ec >= 0) Row::load_h(a.h + (size_t)ec * a.hstride, X.inter, sub, hc);
    Row rows[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) rows[i].template load<true>(X, t.e, o0 + i, sub, o0 + i < a.H);
    const float g = global_scale<FMT>(X.dn_g, t.e);
    const int orow = o0 + sub / SPAN;
    const bool writer = sub % SPAN == 0 && orow < a.H;
    for (int n0 = 0; n0 < t.n; n0 += kWave) {
        const int cnt = min(kWave, t.n - n0);
        if (n0 > 0) {
            mine = lane < cnt ? task_entry(t, n0 + lane, nk) : -1;
            ec = readlane(mine, 0);
            if (ec >= 0) Row::load_h(a.h + (size_t)ec * a.hstride, X.inter, sub, hc);
        }
        for (int j = 0; j < cnt; ++j) {
            const int en = j + 1 < cnt ? readlane(mine, j + 1) : -1;
            if (en >= 0) Row::load_h(a.h + (size_t)en * a.hstride, X.inter, sub, hn);
            if (ec >= 0) {
                float v[RPL];
#pragma unroll
                for (int i = 0; i < RPL; ++i) v[i] = rows[i].partial(hc, X.inter, sub);
                xreduce<LPR, RPL, 1>(v);
                if (writer) a.dbuf[(size_t)ec * a.H + orow] = v[0] * g;
            }
#pragma unroll
            for (int c = 0; c < CH; ++c)
#pragma unroll
                for (int q = 0; q < HQ; ++q) hc[c][q] = hn[c][q];
            ec = en;
        }
    }
}

// Down projection of a multi-row step, both arms in one launch (the layout
// of k_gate_up): matrix-core units of the plan's 16-row down tiles first
// (nm blocks, column group b % nmx of tile b / nmx; nm = 0 when the 64-row
// launch below takes the matrix-core arm), then GEMV units (slice b % gx of
// task b / gx).
template <int FMT, int LPR, int CH, int RPL>
__global__ __launch_bounds__(256) void k_down_grouped(FfnArgs a, int nmx, int nm, int gx) {
    int b = blockIdx.x;
    if constexpr (FMT == kFp8) {
        if (b < nm) {
            mfma_down_unit<kMfmaTileRows / 16>(a, b % nmx, b / nmx);
            return;
        }
    }
    b -= nm;
    down_gemv_unit<FMT, LPR, CH, RPL>(a, b % gx, b / gx);
}

// The matrix-core arm of the down projection on the plan's 64-row (gate/up)
// tiles, for steps of kDownTallRows rows and more: an expert's down matrix is
// then read once per 64 rows instead of once per 16.  A launch of its own,
// before the GEMV units': its tiles take more registers and LDS than those
// units, which would otherwise run at its occupancy.
constexpr int kDownTallRows = 512;

template <int FMT>
__global__ __launch_bounds__(256, 2) void k_down_mfma(FfnArgs a, int nmx) {
    const int b = blockIdx.x;
    mfma_down_unit<kMfmaGuTileRows / 16>(a, b % nmx, b / nmx);
}

// Blend for multi-row steps: y[r][o] = sum_j w[r][j] dbuf[r*k+j][o] (slot
// order) + s[r] dbuf[shared r][o], with the same operation sequence as the
// one-row fused kernel.
// (The slot loads are unconditional and a skipped slot is a select, so the
// k + 1 loads of a column are in flight together; a slot with an expert id
// outside [0, E) leaves y unchanged, as in the one-row kernels.)
// ------------------------------------------------------------------ launchers

static inline int routed_tasks(const FfnArgs &a) { return a.R == 1 ? a.k : a.max_routed_tasks; }
static inline int n_tasks(const FfnArgs &a) { return routed_tasks(a) + (a.shared.inter > 0 && !a.shared_mfma ? 1 : 0); }
static inline int gate_up_chunks(int fmt, int H) { return (fmt_row_bytes(fmt, H) / 16 + kWave - 1) / kWave; }

static inline int max_inter(const FfnArgs &a) { return a.routed.inter > a.shared.inter ? a.routed.inter : a.shared.inter; }

#define MOE_CH_DISPATCH(CH_VALUE, LAUNCH)                                                             \
    do {                                                                                              \
        const int ch_ = (CH_VALUE);                                                                   \
        if (ch_ <= 1) { constexpr int CH = 1; LAUNCH; }                                               \
        else if (ch_ <= 2) { constexpr int CH = 2; LAUNCH; }                                          \
        else if (ch_ <= 4) { constexpr int CH = 4; LAUNCH; }                                          \
        else { constexpr int CH = 8; LAUNCH; }                                                        \
    } while (0)

template <int FMT>
hipError_t gate_up_fmt(const FfnArgs &a, hipStream_t st) {
    const int ch = gate_up_chunks(FMT, a.H);
    const int pm = ch <= 2 ? 4 : P;        // 4 pairs per wave while the registers allow
    const int gx = (max_inter(a) + 4 * pm - 1) / (4 * pm);
    const int nmx = mfma_gate_up_groups(max_inter(a));
    const int nm = FMT == kFp8 && a.mfma_gu_max_tiles > 0 ? nmx * a.mfma_gu_max_tiles : 0;
    const long long nb = nm + (long long)gx * n_tasks(a);
    if (nb == 0) return hipSuccess;
    dim3 grid((unsigned)nb), block(256);
    if (pm == 4) {
        if (ch <= 1) hipLaunchKernelGGL((k_gate_up<FMT, 1, 4>), grid, block, 0, st, a, nmx, nm, gx);
        else hipLaunchKernelGGL((k_gate_up<FMT, 2, 4>), grid, block, 0, st, a, nmx, nm, gx);
    } else {
        if (ch <= 4) hipLaunchKernelGGL((k_gate_up<FMT, 4, P>), grid, block, 0, st, a, nmx, nm, gx);
        else hipLaunchKernelGGL((k_gate_up<FMT, 8, P>), grid, block, 0, st, a, nmx, nm, gx);
    }
    return hipGetLastError();
}


template <int FMT, int NCH, int NV>
hipError_t lead_fmt(const RouteArgs &r, const FfnArgs &a, hipStream_t st) {
    const int n_rows = (r.logits_in ? 0 : r.E) + (r.wsg ? 1 : 0);
    const int nrb = n_rows > 0 ? (n_rows + 3) / 4 : 1;
    const int nsb = a.shared.inter > 0 ? (a.shared.inter + 4 * P - 1) / (4 * P) : 0;
    dim3 grid(nrb + nsb), block(256);
    MOE_CH_DISPATCH(gate_up_chunks(FMT, a.H),
                    hipLaunchKernelGGL((k_lead_r1<FMT, NCH, CH, NV>), grid, block, 0, st, r, a));
    return hipGetLastError();
}

template <int FMT, int NCH>
hipError_t lead_nv(const RouteArgs &r, const FfnArgs &a, hipStream_t st) {
    switch (topk_nv(r.E)) {
        case 1: return lead_fmt<FMT, NCH, 1>(r, a, st);
        case 2: return lead_fmt<FMT, NCH, 2>(r, a, st);
        case 4: return lead_fmt<FMT, NCH, 4>(r, a, st);
        case 8: return lead_fmt<FMT, NCH, 8>(r, a, st);
        default: return lead_fmt<FMT, NCH, 16>(r, a, st);
    }
}

template <int FMT>
hipError_t lead_nch(const RouteArgs &r, const FfnArgs &a, hipStream_t st) {
    const int nch = ((r.H >> 3) + kWave - 1) / kWave;
    if (nch <= 1) return lead_nv<FMT, 1>(r, a, st);
    if (nch <= 2) return lead_nv<FMT, 2>(r, a, st);
    if (nch <= 4) return lead_nv<FMT, 4>(r, a, st);
    if (nch <= 8) return lead_nv<FMT, 8>(r, a, st);
    return lead_nv<FMT, 16>(r, a, st);
}


template <int FMT>
hipError_t gate_up_r1_fmt(const FfnArgs &a, hipStream_t st) {
    const int inter = a.R > 1 ? max_inter(a) : a.routed.inter;
    const int slots = a.k + (a.R > 1 && a.shared.inter > 0 ? 1 : 0);
    dim3 grid((inter + 4 * P - 1) / (4 * P), slots, a.R), block(256);
    // the in-kernel top-k holds NV logits a lane: 4 up to 256 experts, 8, 16
    const int nv = topk_nv(a.E);
    if (nv <= 4)
        MOE_CH_DISPATCH(gate_up_chunks(FMT, a.H), hipLaunchKernelGGL((k_gate_up_r1<FMT, CH, 4>), grid, block, 0, st, a));
    else if (nv <= 8)
        MOE_CH_DISPATCH(gate_up_chunks(FMT, a.H), hipLaunchKernelGGL((k_gate_up_r1<FMT, CH, 8>), grid, block, 0, st, a));
    else
        MOE_CH_DISPATCH(gate_up_chunks(FMT, a.H), hipLaunchKernelGGL((k_gate_up_r1<FMT, CH, 16>), grid, block, 0, st, a));
    return hipGetLastError();
}


constexpr size_t kMaxHLds = 64 * 1024;

#define MOE_DOWN_CH(...)                                                                           \
    do {                                                                                              \
        if (ch_ <= 1) { constexpr int CH = 1; __VA_ARGS__; }                                          \
        else if (ch_ <= 2) { constexpr int CH = 2; __VA_ARGS__; }                                     \
        else { constexpr int CH = 4; __VA_ARGS__; }                                                   \
    } while (0)
#define MOE_DOWN_DISPATCH(...)                                                                     \
    do {                                                                                              \
        int lpr_, ch_;                                                                                \
        down_lane_shape(FMT, a.routed.inter, a.shared.inter, lpr_, ch_);                              \
        if (ch_ > 4) return hipErrorInvalidValue;                                                     \
        const int rows_per_block = 4 * (kWave / lpr_);                                                \
        if (lpr_ == 8) { constexpr int LPR = 8; MOE_DOWN_CH(__VA_ARGS__); }                                \
        else if (lpr_ == 16) { constexpr int LPR = 16; MOE_DOWN_CH(__VA_ARGS__); }                         \
        else if (lpr_ == 32) { constexpr int LPR = 32; MOE_DOWN_CH(__VA_ARGS__); }                         \
        else { constexpr int LPR = 64; MOE_DOWN_CH(__VA_ARGS__); }                                         \
        return hipGetLastError();                                                                     \
    } while (0)

template <int FMT>
hipError_t down_r1_fmt(const FfnArgs &a, hipStream_t st) {
    const int nslots = a.k + (a.shared.inter > 0 ? 1 : 0);
    const size_t hbytes = (size_t)nslots * a.hstride * 4;
    // one staging pass covers h (the slot-count instantiations need it)
    const bool one_pass = (size_t)nslots * (a.hstride / 4) <= (size_t)down_r1_stage_loads(FMT) * kDownR1Waves * kWave;
    MOE_DOWN_DISPATCH({
        const int rpb = kDownR1Waves * (kWave / LPR);
        dim3 grid((a.H + rpb - 1) / rpb, a.R), block(kDownR1Waves * kWave);
        (void)rows_per_block;
        if (hbytes > kMaxHLds)
            hipLaunchKernelGGL((k_down_r1<FMT, LPR, CH, false>), grid, block, 0, st, a);
        else if (CH == 1 && nslots == 9 && one_pass)
            hipLaunchKernelGGL((k_down_r1<FMT, LPR, CH, true, 9>), grid, block, hbytes, st, a);
        else if (CH == 1 && nslots == 11 && one_pass)
            hipLaunchKernelGGL((k_down_r1<FMT, LPR, CH, true, 11>), grid, block, hbytes, st, a);
        else
            hipLaunchKernelGGL((k_down_r1<FMT, LPR, CH, true>), grid, block, hbytes, st, a);
    });
}
// Rows per row group of the grouped down kernel: 8 register rows per lane
// in all (RPL rows of CH chunks).
constexpr int down_rpl(int ch) { return ch <= 1 ? 8 : ch <= 2 ? 4 : 2; }

template <int FMT>
hipError_t down_grouped_fmt(const FfnArgs &a, hipStream_t st) {
    const int nmx = mfma_down_groups(a.H);
    int nm = 0;
    if constexpr (FMT == kFp8) {
        if (a.mfma_max_tiles > 0 && a.R >= kDownTallRows) {
            hipLaunchKernelGGL((k_down_mfma<FMT>), dim3((unsigned)(nmx * a.mfma_gu_max_tiles)), dim3(256), 0, st, a,
                               nmx);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        } else if (a.mfma_max_tiles > 0) {
            nm = nmx * a.mfma_max_tiles;
        }
    }
    MOE_DOWN_DISPATCH({
        constexpr int RPL = down_rpl(CH);
        const int rows = rows_per_block * RPL;
        const int gx = (a.H + rows - 1) / rows;
        const long long nb = nm + (long long)gx * n_tasks(a);
        if (nb == 0) return hipSuccess;
        hipLaunchKernelGGL((k_down_grouped<FMT, LPR, CH, RPL>), dim3((unsigned)nb), dim3(256), 0, st, a, nmx, nm, gx);
    });
}

// The per-format launchers, instantiated once each in ffn_<format>.hip.
#define MOE_FFN_FORMAT_LAUNCHERS(X, FMT)                                              \
    X hipError_t gate_up_fmt<FMT>(const FfnArgs &, hipStream_t);                      \
    X hipError_t lead_nch<FMT>(const RouteArgs &, const FfnArgs &, hipStream_t);       \
    X hipError_t gate_up_r1_fmt<FMT>(const FfnArgs &, hipStream_t);                   \
    X hipError_t down_r1_fmt<FMT>(const FfnArgs &, hipStream_t);                      \
    X hipError_t down_grouped_fmt<FMT>(const FfnArgs &, hipStream_t);

}  // namespace moe
