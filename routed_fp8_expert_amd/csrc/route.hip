// route.hip -- routing kernels for gfx950: the bf16 router GEMV with the
// shared-expert gate, the wave64 top-k softmax, and the token-by-expert
// grouping (histogram, exclusive scan, deterministic ranks).
//
// GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels": gemv::dense_gemv_bf16
// (the router; "Precision": bf16 weight, bf16 activation) and
// moe_topk::moe_topk_softmax (node output f32,i32).  colibri pull request
// 1992, "What it is": the shared expert's gate.  The grouping serves the
// multi-row plan arms ("Plan arms": multi_seq rows 2..64) so that each
// touched expert's weights are read once per step.
#include "gemv.hpp"

namespace moe {

// Router GEMV for multi-row steps: one wave per router row (row E is the
// shared-gate vector) holds it in registers.  The workgroup stages blocks of
// RB activation rows in LDS (each read from memory once per workgroup); every
// wave forms its row's RB partial sums and reduces them together (the
// transposing reduction: the same bits as the one-row wave sum), so lane
// group i of the wave ends with row r0 + i.
#ifndef MOE_ROUTER_WAVES
#define MOE_ROUTER_WAVES 8
#endif
// Waves (router rows) per workgroup: every workgroup stages the activation
// rows, so more rows a workgroup stage less in all.
constexpr int kRouterWaves = MOE_ROUTER_WAVES;

template <int NCH, int RB>
__global__ __launch_bounds__(kRouterWaves * kWave) void k_router(RouteArgs a) {
    extern __shared__ u32x4 xs[];    // [RB][H/8] 16-byte activation chunks
    constexpr int SPAN = kWave / RB, NT = kRouterWaves * kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * kRouterWaves + (threadIdx.x >> 6);
    const bool live = row < a.E + (a.wsg ? 1 : 0);
    const bool gate_row = row >= a.E;
    const int nch = a.H >> 3;
    u32x4 wv[NCH];
    if (live) load_bf16_row<NCH>(gate_row ? a.wsg : a.wr + (size_t)row * a.H, a.H, wv);
    const float bias = (live && !gate_row && a.bias) ? a.bias[row] : 0.0f;
    for (int r0 = 0; r0 < a.R; r0 += RB) {
        const int nr = min(RB, a.R - r0);
        __syncthreads();
        // every staging load issued before the first store (a load feeding a
        // store in a loop with a run-time trip count ran one latency per
        // iteration); loads past the block read chunk 0 of row r0, unused
        constexpr int PER = (RB * NCH * kWave + NT - 1) / NT;
        u32x4 t[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int i = u * NT + (int)threadIdx.x;
            const int ic = i < nr * nch ? i : 0;
            const int rr = ic / nch, c = ic - rr * nch;
            t[u] = ld16(a.x + (size_t)(r0 + rr) * a.ldx + (size_t)c * 8);
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int i = u * NT + (int)threadIdx.x;
            if (i < nr * nch) xs[i] = t[u];
        }
        __syncthreads();
        if (!live) continue;
        float p[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
            float acc = 0.0f;
            if (rr < nr) {
#pragma unroll
                for (int t = 0; t < NCH; ++t) {
                    const int c = lane + kWave * t;
                    if (c < nch) acc = dot8_bf16(wv[t], xs[rr * nch + c], acc);
                }
            }
            p[rr] = acc;
        }
        xreduce<kWave, RB, 1>(p);
        const int mine = lane / SPAN;
        if (lane % SPAN == 0 && mine < nr) {
            if (gate_row) a.s[r0 + mine] = sigmoid(p[0]);
            else a.logits[(size_t)(r0 + mine) * a.E + row] = p[0] + bias;
        }
    }
}

// Top-k from logits (given, or written by the router launch): one wave per
// row.  s_mode 1 also computes the shared gate here, 2 writes s = 1.
template <int NV>
__global__ __launch_bounds__(256) void k_topk(RouteArgs a, int s_mode) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.R) return;
    const float *l = a.logits_in ? a.logits_in + (size_t)r * a.E : a.logits + (size_t)r * a.E;
    // the shared gate's first loads go out with the logits' (same bits as
    // the one-row router's dot; 12 / 16 rows 60.1 / 75.0 -> 58.0 / 73.3 us)
    float raw[NV];
    load_logits<NV>(l, a.E, false, raw);
    RowStreamHead sq;
    if (s_mode == 1) row_stream_head(a.wsg, a.x + (size_t)r * a.ldx, a.H, sq);
    int e;
    float w;
    topk_regs<NV>(raw, a.E, a.k, topk_lds<4>(threadIdx.x >> 6), e, w);
    if (lane < a.k) {
        a.ids[(size_t)r * a.k + lane] = e;
        a.w[(size_t)r * a.k + lane] = w;
    }
    if (s_mode == 1) {
        const float d = row_stream_dot(sq, a.wsg, a.x + (size_t)r * a.ldx, a.H);
        if (lane == 0) a.s[r] = sigmoid(d);
    } else if (s_mode == 2 && lane == 0) {
        a.s[r] = 1.0f;
    }
}

// Inclusive prefix sum over the wave: row shifts by 1, 2, 4, 8 within each
// 16-lane row, then the two row broadcasts carry rows 0 and 1 into the rows
// above them.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp<0x111>(0, v);           // row_shr:1
    v += dpp<0x112>(0, v);           // row_shr:2
    v += dpp<0x114>(0, v);           // row_shr:4
    v += dpp<0x118>(0, v);           // row_shr:8
    v += dpp<kDppBcast15, 0xa>(0, v);
    v += dpp<kDppBcast31, 0xc>(0, v);
    return v;
}

// Exclusive prefix sum over the 1024-thread block; every thread calls it.
// Each wave scans itself, publishes its total, and then scans the 16 totals
// itself (no second round through LDS).
__device__ int block_excl_scan(int v, int *wave_tot, int *total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int inc = wave_incl_scan(v);
    if (lane == kWave - 1) wave_tot[wid] = inc;
    __syncthreads();
    const int t = lane < 16 ? wave_tot[lane] : 0;
    const int ti = wave_incl_scan(t);
    const int before = readlane(ti, wid) - readlane(t, wid);
    *total = readlane(ti, 15);
    __syncthreads();   // wave_tot is reused by the next scan
    return inc - v + before;
}

// Splits the touched experts into the GEMV-arm list and the MFMA-arm list
// (rows >= threshold), both ascending, and the MFMA row-tile prefixes: of
// kMfmaTileRows-row tiles at mfma_tiles[0 .. n], of kMfmaGuTileRows-row
// tiles at mfma_tiles[E+1 .. E+1+n].  Thread e of a 1024-thread block holds
// expert e's row count c.
__device__ void plan_lists(const RouteArgs &a, int e, int c, int *wave_tot) {
    const int E = a.E;
    const bool mf = e < E && c > 0 && a.mfma_min_rows > 0 && c >= a.mfma_min_rows;
    const bool gv = e < E && c > 0 && !mf;
    int n_gemv, n_mfma, n_tiles, n_gu_tiles;
    const int pg = block_excl_scan(gv ? 1 : 0, wave_tot, &n_gemv);
    const int pm = block_excl_scan(mf ? 1 : 0, wave_tot, &n_mfma);
    const int tiles = mf ? (c + kMfmaTileRows - 1) / kMfmaTileRows : 0;
    const int gu_tiles = mf ? (c + kMfmaGuTileRows - 1) / kMfmaGuTileRows : 0;
    // both tile counts in one scan: the down tiles in the low 16 bits (their
    // total is at most R*k/16 + E < 2^16), the gate/up tiles above
    const int packed = block_excl_scan(tiles | (gu_tiles << 16), wave_tot, &n_tiles);
    const int pt = packed & 0xFFFF, pgt = packed >> 16;
    n_gu_tiles = n_tiles >> 16;
    n_tiles &= 0xFFFF;
    int32_t *gu_prefix = a.mfma_tiles + E + 1;
    if (gv) a.gemv_list[pg] = e;
    if (mf) {
        a.mfma_list[pm] = e;
        a.mfma_tiles[pm] = pt;
        gu_prefix[pm] = pgt;
    }
    if (threadIdx.x == 0) {
        a.meta[kMetaGemvCount] = n_gemv;
        a.meta[kMetaMfmaCount] = n_mfma;
        a.meta[kMetaMfmaTiles] = n_tiles;
        a.meta[kMetaMfmaGuTiles] = n_gu_tiles;
        a.mfma_tiles[n_mfma] = n_tiles;
        gu_prefix[n_mfma] = n_gu_tiles;
    }
}

// Planning alone, from grouping counts made elsewhere.
__global__ __launch_bounds__(1024) void k_plan(RouteArgs a) {
    __shared__ int wave_tot[40];
    const int e = threadIdx.x;
    int c = 0;
    if (e < a.E) {
        c = a.counts[e];
        if (c < 0 || c > a.R) {
            flag_error(a.err, kErrBadExpertId);
            c = 0;
        }
    }
    plan_lists(a, e, c, wave_tot);
}

// Grouping by expert: a bitmap of rows per expert (rows ascending), counts
// by popcount (with each word's count of the expert's earlier rows kept in
// pre), an exclusive scan for the offsets, and each (row, slot) placed at
// offset + (rows before it that chose the same expert).  With `do_plan` it
// also writes the arm lists.  One 1024-thread workgroup; COHERENT reads the
// ids at agent scope (written by other workgroups of the same launch).  LDS:
// bm and pre, E * ceil(R/32) words each.
constexpr int kGroupIds = 16;   // (row, slot) entries a grouping thread holds: R*k <= 16 * 1024
template <bool COHERENT>
__device__ void group_rows(const RouteArgs &a, int do_plan, uint32_t *bm, int *wave_tot, int *soff) {
    const int tid = threadIdx.x;
    const int R = a.R, E = a.E, k = a.k, W = (R + 31) >> 5;
    const int n = R * k;
    auto id_at = [&](int i) { return COHERENT ? ld_agent(a.ids + i) : a.ids[i]; };
    // the step's ids, kGroupIds a thread (entry tid + 1024 u), all loads in
    // flight at once and kept for both passes
    int idr[kGroupIds];
#pragma unroll
    for (int u = 0; u < kGroupIds; ++u) {
        const int i = tid + 1024 * u;
        idr[u] = i < n ? id_at(i) : -1;
    }
    for (int i = tid; i < E * W; i += 1024) bm[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kGroupIds; ++u) {
        const int i = tid + 1024 * u;
        if (i >= n) continue;
        const int e = idr[u];
        const int r = i / k;
        if (e >= 0 && e < E)
            atomicOr(&bm[e * W + (r >> 5)], 1u << (r & 31));
        else
            flag_error(a.err, kErrBadExpertId);
    }
    __syncthreads();
    int *pre = reinterpret_cast<int *>(bm + E * W);
    const int e = tid;
    int c = 0;
    if (e < E)
        for (int q = 0; q < W; ++q) {
            pre[e * W + q] = c;
            c += __popc(bm[e * W + q]);
        }
    int total;
    const int off = block_excl_scan(e < E ? c : 0, wave_tot, &total);
    if (e < E) {
        a.counts[e] = c;
        a.offsets[e] = off;
        soff[e] = off;
    }
    if (e == 0) a.offsets[E] = total;
    if (do_plan) plan_lists(a, e, c, wave_tot);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kGroupIds; ++u) {
        const int i = tid + 1024 * u;
        const int ee = idr[u];
        if (i >= n || ee < 0 || ee >= E) continue;
        const int r = i / k;
        const int rank = pre[ee * W + (r >> 5)] + __popc(bm[ee * W + (r >> 5)] & ((1u << (r & 31)) - 1u));
        a.perm[soff[ee] + rank] = i;
    }
}

__global__ __launch_bounds__(1024) void k_group(RouteArgs a, int do_plan) {
    extern __shared__ uint32_t bm[];          // [E][W], then pre [E][W]
    __shared__ int wave_tot[40];
    __shared__ int soff[1024];
    group_rows<false>(a, do_plan, bm, wave_tot, soff);
}

// Top-k of a grouped step and its grouping in one launch: one wave a row, 16
// rows a workgroup (ids and weights stored write-through), then each
// workgroup counts itself done once its stores have completed, and the last
// one to do so groups the step (reading the ids at agent scope) and resets
// the count for the next call.  No workgroup waits on another.
template <int NV>
__global__ __launch_bounds__(1024) void k_topk_group(RouteArgs a, int s_mode, int do_plan) {
    extern __shared__ uint32_t bm[];          // [E][W] and pre [E][W], the grouping's
    __shared__ int wave_tot[40];
    __shared__ int soff[1024];
    __shared__ unsigned ticket_s;
    const int lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.x * 16 + (threadIdx.x >> 6);
    if (r < a.R) {
        const float *l = a.logits_in ? a.logits_in + (size_t)r * a.E : a.logits + (size_t)r * a.E;
        int e;
        float w;
        // (issuing the shared gate's loads with the logits', as k_topk does,
        // measured 0.2-0.3 us slower here: 64 rows 155.8 -> 156.0, Zipf 64
        // rows 103.0 -> 103.3)
        topk_wave<NV>(l, a.E, a.k, false, topk_lds<16>(threadIdx.x >> 6), e, w);
        if (lane < a.k) {
            st_agent(a.ids + (size_t)r * a.k + lane, e);
            st_agent(a.w + (size_t)r * a.k + lane, w);
        }
        if (s_mode == 1) {
            // chunks in order, the wave sum last: the bits of the one-row router
            const float d = dot_bf16_row_stream(a.wsg, a.x + (size_t)r * a.ldx, a.H);
            if (lane == 0) a.s[r] = sigmoid(d);
        } else if (s_mode == 2 && lane == 0) {
            a.s[r] = 1.0f;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        ticket_s = __hip_atomic_fetch_add(a.group_ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket_s != gridDim.x - 1) return;
    if (threadIdx.x == 0) __hip_atomic_store(a.group_ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    group_rows<true>(a, do_plan, bm, wave_tot, soff);
}

// ------------------------------------------------------------------ launchers

size_t group_lds_bytes(int E, int R) { return (size_t)E * (size_t)((R + 31) / 32) * 8u; }

// Activation rows staged per block: 64 KB of LDS at most.
static int router_rows_per_block(int H, int R) {
    int rb = H <= 2048 ? 16 : H <= 4096 ? 8 : 4;
    while (rb > 2 && rb / 2 >= R) rb /= 2;
    return rb;
}

template <int NCH>
static hipError_t router_nch(const RouteArgs &a, hipStream_t st) {
    const int rows = a.E + (a.wsg ? 1 : 0);
    const int rb = router_rows_per_block(a.H, a.R);
    const size_t lds = (size_t)rb * (size_t)a.H * 2;
    dim3 grid((rows + kRouterWaves - 1) / kRouterWaves), block(kRouterWaves * kWave);
    switch (rb) {
        case 2: hipLaunchKernelGGL((k_router<NCH, 2>), grid, block, lds, st, a); break;
        case 4: hipLaunchKernelGGL((k_router<NCH, 4>), grid, block, lds, st, a); break;
        case 8: hipLaunchKernelGGL((k_router<NCH, 8>), grid, block, lds, st, a); break;
        default: hipLaunchKernelGGL((k_router<NCH, 16>), grid, block, lds, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_router(const RouteArgs &a, hipStream_t st) {
    const int nch = ((a.H >> 3) + kWave - 1) / kWave;
    if (nch <= 1) return router_nch<1>(a, st);
    if (nch <= 2) return router_nch<2>(a, st);
    if (nch <= 4) return router_nch<4>(a, st);
    if (nch <= 8) return router_nch<8>(a, st);
    return router_nch<16>(a, st);
}

hipError_t launch_topk(const RouteArgs &a, bool compute_s, hipStream_t st) {
    const int s_mode = a.wsg ? (compute_s ? 1 : 0) : 2;
    dim3 grid((a.R + 3) / 4), block(256);
    switch (topk_nv(a.E)) {
        case 1: hipLaunchKernelGGL(k_topk<1>, grid, block, 0, st, a, s_mode); break;
        case 2: hipLaunchKernelGGL(k_topk<2>, grid, block, 0, st, a, s_mode); break;
        case 4: hipLaunchKernelGGL(k_topk<4>, grid, block, 0, st, a, s_mode); break;
        case 8: hipLaunchKernelGGL(k_topk<8>, grid, block, 0, st, a, s_mode); break;
        default: hipLaunchKernelGGL(k_topk<16>, grid, block, 0, st, a, s_mode); break;
    }
    return hipGetLastError();
}

hipError_t launch_group(const RouteArgs &a, bool plan, hipStream_t st) {
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), group_lds_bytes(a.E, a.R), st, a, (int)plan);
    return hipGetLastError();
}

hipError_t launch_topk_group(const RouteArgs &a, bool compute_s, bool plan, hipStream_t st) {
    const int s_mode = a.wsg ? (compute_s ? 1 : 0) : 2;
    dim3 grid((a.R + 15) / 16), block(1024);
    const size_t lds = group_lds_bytes(a.E, a.R);
    switch (topk_nv(a.E)) {
        case 1: hipLaunchKernelGGL(k_topk_group<1>, grid, block, lds, st, a, s_mode, (int)plan); break;
        case 2: hipLaunchKernelGGL(k_topk_group<2>, grid, block, lds, st, a, s_mode, (int)plan); break;
        case 4: hipLaunchKernelGGL(k_topk_group<4>, grid, block, lds, st, a, s_mode, (int)plan); break;
        case 8: hipLaunchKernelGGL(k_topk_group<8>, grid, block, lds, st, a, s_mode, (int)plan); break;
        default: hipLaunchKernelGGL(k_topk_group<16>, grid, block, lds, st, a, s_mode, (int)plan); break;
    }
    return hipGetLastError();
}

hipError_t launch_plan(const RouteArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
