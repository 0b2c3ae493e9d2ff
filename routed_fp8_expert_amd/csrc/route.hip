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
#include "device.hpp"
#include "kernels.hpp"

#include <math.h>

namespace moe {

constexpr int kMaxTopkPerLane = 16;   // E <= 1024

__device__ __forceinline__ void st_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Softmax over E logits, the k largest (value descending, lower index first
// on equal values), and their renormalised weights, by one wave.  The
// weights are exp(l_j - m) / sum_j exp(l_j - m): the softmax denominator over
// all E cancels in the renormalisation.  `coherent` reads the logits with
// agent-scope loads (they were written by other workgroups of this launch).
__device__ void topk_row(const float *l, int E, int k, int32_t *ids, float *w, bool coherent) {
    const int lane = threadIdx.x & (kWave - 1);
    float v[kMaxTopkPerLane];
    uint32_t taken = 0;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxTopkPerLane; ++i) {
        const int e = lane + kWave * i;
        float t = -INFINITY;
        if (e < E) {
            t = coherent ? ld_agent(l + e) : l[e];
            if (t != t) t = -INFINITY;
        } else {
            taken |= 1u << i;
        }
        v[i] = t;
        m = fmaxf(m, t);
    }
    m = wave_max(m);
    float my_v = 0.0f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxTopkPerLane; ++i) {
            const int e = lane + kWave * i;
            if (!((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, kWave);
            const int oe = __shfl_xor(be, o, kWave);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if (be < E && (be & (kWave - 1)) == lane) taken |= 1u << (be >> 6);
        if (lane == j) {
            my_v = bv;
            my_e = be < E ? be : 0;
        }
    }
    const float ex = lane < k ? expf(my_v - m) : 0.0f;
    const float sum = group_sum<kWave>(ex);
    if (lane < k) {
        ids[lane] = my_e;
        w[lane] = ex / sum;
    }
}

// x . v over H bf16 elements by one wave (16-byte chunks, lane-strided).
__device__ __forceinline__ float wave_dot_bf16(const uint16_t *a, const uint16_t *b, int H) {
    const int lane = threadIdx.x & (kWave - 1);
    float acc = 0.0f;
    for (int c = lane; c < (H >> 3); c += kWave) acc = dot8_bf16(ld16(a + c * 8), ld16(b + c * 8), acc);
    return group_sum<kWave>(acc);
}

__device__ __forceinline__ float sigmoid(float t) { return 1.0f / (1.0f + expf(-t)); }

// Router GEMV: one wave per router row (row E is the shared-gate vector).
// The row stays in registers while the wave walks the R activation rows.
// With `fuse_topk`, the last workgroup to finish runs the top-k for every
// row (a ticket counter in the ctx, reset by that workgroup).
template <int NCH>
__global__ __launch_bounds__(64) void k_router(RouteArgs a, int fuse_topk, int s_mode) {
    const int lane = threadIdx.x;
    const int row = blockIdx.x;
    const int nch = a.H >> 3;
    const uint16_t *wrow = row < a.E ? a.wr + (size_t)row * a.H : a.wsg;
    u32x4 wv[NCH];
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
        const int c = lane + kWave * t;
        wv[t] = c < nch ? ld16_stream(wrow + (size_t)c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    const float bias = (row < a.E && a.bias) ? a.bias[row] : 0.0f;
    for (int r = 0; r < a.R; ++r) {
        const uint16_t *xr = a.x + (size_t)r * a.ldx;
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int c = lane + kWave * t;
            if (c < nch) acc = dot8_bf16(wv[t], ld16(xr + (size_t)c * 8), acc);
        }
        acc = group_sum<kWave>(acc);
        if (lane == 0) {
            if (row < a.E)
                st_agent(a.logits + (size_t)r * a.E + row, acc + bias);
            else
                st_agent(a.s + r, sigmoid(acc));
        }
    }
    if (!fuse_topk) return;
    __threadfence();
    unsigned ticket = 0;
    if (lane == 0)
        ticket = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    ticket = __shfl(ticket, 0, kWave);
    if (ticket != gridDim.x - 1) return;
    __threadfence();
    for (int r = 0; r < a.R; ++r) {
        topk_row(a.logits + (size_t)r * a.E, a.E, a.k, a.ids + (size_t)r * a.k,
                 a.w + (size_t)r * a.k, true);
        if (s_mode == 2 && lane == 0) a.s[r] = 1.0f;
    }
    if (lane == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Top-k from logits (given, or written by an earlier router launch): one
// wave per row.  s_mode 1 computes the shared gate here, 2 writes s = 1.
__global__ __launch_bounds__(256) void k_topk(RouteArgs a, int s_mode) {
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.R) return;
    const float *l = a.logits_in ? a.logits_in + (size_t)r * a.E : a.logits + (size_t)r * a.E;
    topk_row(l, a.E, a.k, a.ids + (size_t)r * a.k, a.w + (size_t)r * a.k, false);
    if (s_mode == 1) {
        const float d = wave_dot_bf16(a.x + (size_t)r * a.ldx, a.wsg, a.H);
        if ((threadIdx.x & 63) == 0) a.s[r] = sigmoid(d);
    } else if (s_mode == 2 && (threadIdx.x & 63) == 0) {
        a.s[r] = 1.0f;
    }
}

// Exclusive scan of one int per thread over a 1024-thread block.
__device__ int block_excl_scan(int v, int *wave_tot, int *total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += t;
    }
    if (lane == kWave - 1) wave_tot[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        int t = lane < 16 ? wave_tot[lane] : 0;
        int ti = t;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int u = __shfl_up(ti, o, kWave);
            if (lane >= o) ti += u;
        }
        if (lane < 16) wave_tot[16 + lane] = ti - t;
        if (lane == 15) wave_tot[32] = ti;
    }
    __syncthreads();
    const int excl = inc - v + wave_tot[16 + wid];
    *total = wave_tot[32];
    __syncthreads();
    return excl;
}

constexpr int kMfmaTileRows = 32;

// Splits the touched experts into the GEMV-arm list and the MFMA-arm list
// (rows >= threshold), both ascending, and the MFMA row-tile prefix.  Thread
// e of a 1024-thread block holds expert e's row count c.
__device__ void plan_lists(const RouteArgs &a, int e, int c, int *wave_tot) {
    const int E = a.E;
    const bool mf = e < E && c > 0 && a.mfma_min_rows > 0 && c >= a.mfma_min_rows;
    const bool gv = e < E && c > 0 && !mf;
    int n_gemv, n_mfma, n_tiles;
    const int pg = block_excl_scan(gv ? 1 : 0, wave_tot, &n_gemv);
    const int pm = block_excl_scan(mf ? 1 : 0, wave_tot, &n_mfma);
    const int tiles = mf ? (c + kMfmaTileRows - 1) / kMfmaTileRows : 0;
    const int pt = block_excl_scan(tiles, wave_tot, &n_tiles);
    if (gv) a.gemv_list[pg] = e;
    if (mf) {
        a.mfma_list[pm] = e;
        a.mfma_tiles[pm] = pt;
    }
    if (threadIdx.x == 0) {
        a.meta[kMetaGemvCount] = n_gemv;
        a.meta[kMetaMfmaCount] = n_mfma;
        a.meta[kMetaMfmaTiles] = n_tiles;
        a.mfma_tiles[n_mfma] = n_tiles;
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
// by popcount, an exclusive scan for the offsets, and each (row, slot) placed
// at offset + (rows before it that chose the same expert).  With `do_plan`
// it also writes the arm lists.  One 1024-thread workgroup.
__global__ __launch_bounds__(1024) void k_group(RouteArgs a, int do_plan) {
    extern __shared__ uint32_t bm[];          // [E][W]
    __shared__ int wave_tot[40];
    __shared__ int soff[1024];
    const int tid = threadIdx.x;
    const int R = a.R, E = a.E, k = a.k, W = (R + 31) >> 5;
    const int n = R * k;
    for (int i = tid; i < E * W; i += 1024) bm[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += 1024) {
        const int e = a.ids[i];
        const int r = i / k;
        if (e >= 0 && e < E)
            atomicOr(&bm[e * W + (r >> 5)], 1u << (r & 31));
        else
            flag_error(a.err, kErrBadExpertId);
    }
    __syncthreads();
    const int e = tid;
    int c = 0;
    if (e < E)
        for (int q = 0; q < W; ++q) c += __popc(bm[e * W + q]);
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
    for (int i = tid; i < n; i += 1024) {
        const int ee = a.ids[i];
        if (ee < 0 || ee >= E) continue;
        const int r = i / k;
        const uint32_t *row = bm + ee * W;
        int rank = __popc(row[r >> 5] & ((1u << (r & 31)) - 1u));
        for (int q = 0; q < (r >> 5); ++q) rank += __popc(row[q]);
        a.perm[soff[ee] + rank] = i;
    }
}

// ------------------------------------------------------------------ launchers

size_t group_lds_bytes(int E, int R) { return (size_t)E * (size_t)((R + 31) / 32) * 4u; }

hipError_t launch_router(const RouteArgs &a, bool fuse_topk, hipStream_t st) {
    const int nch = ((a.H >> 3) + kWave - 1) / kWave;
    const int rows = a.E + (a.wsg ? 1 : 0);
    const int s_mode = a.wsg ? 0 : 2;
    dim3 grid(rows), block(64);
    if (nch <= 1)
        hipLaunchKernelGGL(k_router<1>, grid, block, 0, st, a, (int)fuse_topk, s_mode);
    else if (nch <= 2)
        hipLaunchKernelGGL(k_router<2>, grid, block, 0, st, a, (int)fuse_topk, s_mode);
    else if (nch <= 4)
        hipLaunchKernelGGL(k_router<4>, grid, block, 0, st, a, (int)fuse_topk, s_mode);
    else if (nch <= 8)
        hipLaunchKernelGGL(k_router<8>, grid, block, 0, st, a, (int)fuse_topk, s_mode);
    else
        hipLaunchKernelGGL(k_router<16>, grid, block, 0, st, a, (int)fuse_topk, s_mode);
    return hipGetLastError();
}

hipError_t launch_topk(const RouteArgs &a, bool compute_s, hipStream_t st) {
    const int s_mode = a.wsg ? (compute_s ? 1 : 0) : 2;
    hipLaunchKernelGGL(k_topk, dim3((a.R + 3) / 4), dim3(256), 0, st, a, s_mode);
    return hipGetLastError();
}

hipError_t launch_group(const RouteArgs &a, bool plan, hipStream_t st) {
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), group_lds_bytes(a.E, a.R), st, a, (int)plan);
    return hipGetLastError();
}

hipError_t launch_plan(const RouteArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
