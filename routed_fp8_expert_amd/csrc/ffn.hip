// ffn.hip -- expert kernels for gfx950 (GEMV arm): gate/up GEMV with
// silu*mul, the down GEMV fused with the routing-weighted blend and the
// residual add, and the grouped variants for multi-row steps.
//
// GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels":
// moe_expert_gate_up_shared_fp8 (routed and shared gate/up in one launch),
// moe_expert_silu_down_shared_fp8, moe_weighted_sum_blend; "Precision":
// fp8/block128x128 weights read bf16 activations (gate/up) and f32
// activations (down).  colibri pull request 1992, "A decode GEMV": a wave per
// output row with 16 bytes per lane reads weights near the bus rate, versus a
// whole block per row; here each wave keeps several 16-byte weight loads per
// lane in flight and reduces across the wave64.
//
// Weight layouts (see moe.h): fp8 rows of H (gate/up) or I (down) codes with
// f32 scales per 128x128 block; nvfp4 rows of packed e2m1 nibbles with one
// e4m3 scale per 16 columns and an f32 global per matrix.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {

enum : int { kFp8 = 0, kNvfp4 = 1 };
constexpr int kMaxSlots = 17;   // top_k <= 16, plus the shared expert

// Bytes of one stored weight row of `cols` columns, and columns per 16-byte chunk.
template <int FMT> __device__ __forceinline__ int row_bytes(int cols) { return FMT == kFp8 ? cols : cols / 2; }
template <int FMT> constexpr int cols_per_chunk() { return FMT == kFp8 ? 16 : 32; }

// Scale(s) of chunk `c` of weight row `row` in a matrix of `cols` columns.
// fp8: one f32 per 128x128 block; nvfp4: two e4m3 bytes (two 16-column groups).
template <int FMT>
__device__ __forceinline__ f32x2 chunk_scale(const uint8_t *s, int row, int cols, int c) {
    if (FMT == kFp8) {
        const float *sf = reinterpret_cast<const float *>(s);
        const float v = sf[(size_t)(row >> 7) * (cols >> 7) + ((c * 16) >> 7)];
        return f32x2{v, v};
    } else {
        const uint16_t b = *reinterpret_cast<const uint16_t *>(s + (size_t)row * (cols >> 4) + 2 * c);
        return f32x2{e4m3_f32(b, 0), e4m3_f32(b, 1)};
    }
}

// Partial dot of one 16-byte weight chunk with bf16 activations at `xp`
// (the chunk's first column), scaled by its block scale(s).
template <int FMT>
__device__ __forceinline__ float chunk_dot_bf16(u32x4 w, f32x2 sc, const uint16_t *xp) {
    if (FMT == kFp8) {
        return sc.x * dot16_e4m3_bf16(w, ld16(xp), ld16(xp + 8));
    } else {
        float a = dot8_e2m1_bf16(w.x, ld16(xp), 0.0f);
        a = dot8_e2m1_bf16(w.y, ld16(xp + 8), a);
        float b = dot8_e2m1_bf16(w.z, ld16(xp + 16), 0.0f);
        b = dot8_e2m1_bf16(w.w, ld16(xp + 24), b);
        return sc.x * a + sc.y * b;
    }
}

// Partial dot of one 16-byte weight chunk with f32 activations at `hp`.
template <int FMT>
__device__ __forceinline__ float chunk_dot_f32(u32x4 w, f32x2 sc, const float *hp) {
    const f32x4 *h4 = reinterpret_cast<const f32x4 *>(hp);
    if (FMT == kFp8) {
        f32x4 hv[4] = {h4[0], h4[1], h4[2], h4[3]};
        return sc.x * dot16_e4m3_f32(w, hv);
    } else {
        float a = dot8_e2m1_f32(w.x, h4[0], h4[1], 0.0f);
        a = dot8_e2m1_f32(w.y, h4[2], h4[3], a);
        float b = dot8_e2m1_f32(w.z, h4[4], h4[5], 0.0f);
        b = dot8_e2m1_f32(w.w, h4[6], h4[7], b);
        return sc.x * a + sc.y * b;
    }
}

template <int FMT> __device__ __forceinline__ float global_scale(const float *g, int e) {
    return FMT == kNvfp4 ? g[e] : 1.0f;
}

// Which expert and which entries (rows of h / dbuf) a task covers.
// R == 1: task j < k is slot j, task k the shared expert.
// R >= 2: task u < max_routed_tasks is the u-th GEMV-arm expert (its rows
// from the grouping), the last task the shared expert over all R rows.
struct Task {
    const ExpertSet *X;
    int e;          // expert index within its family
    int n;          // number of entries
    const int32_t *list;   // entry list (routed, R >= 2) or null
    int first;      // first entry when list is null (entries first .. first+n-1)
    bool valid;
};

__device__ __forceinline__ Task resolve_task(const FfnArgs &a, int task) {
    Task t{&a.routed, 0, 0, nullptr, 0, false};
    const int nk = a.R * a.k;
    if (a.R == 1) {
        if (task < a.k) {
            t.e = a.ids[task];
            t.n = 1;
            t.first = task;
            t.valid = t.e >= 0 && t.e < a.E;
            if (!t.valid) flag_error(a.err, kErrBadExpertId);
        } else {
            t.X = &a.shared;
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
        t.X = &a.shared;
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

// gate/up GEMV + silu*mul.  Block = 4 waves; a wave owns P (gate, up) row
// pairs (i, I+i) of one expert, keeps their 2P rows in registers (CH 16-byte
// chunks per lane per row, lane-strided along the row) and walks the task's
// activation rows.  h[entry][i] = silu(g_i) * u_i in f32.
template <int FMT, int CH, int P>
__global__ __launch_bounds__(256) void k_gate_up(FfnArgs a) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
    const Task t = resolve_task(a, blockIdx.y);
    if (!t.valid || t.n == 0) return;
    const ExpertSet &X = *t.X;
    const int I = X.inter, H = a.H;
    const int i0 = (blockIdx.x * 4 + wid) * P;
    if (i0 >= I) return;
    const int rb = row_bytes<FMT>(H);
    const int nch = rb >> 4;
    const uint8_t *wbase = X.gu + (size_t)t.e * X.gu_stride;
    const uint8_t *sbase = X.gu_s + (size_t)t.e * X.gu_s_stride;

    u32x4 wv[2 * P][CH];
    f32x2 sc[2 * P][CH];
#pragma unroll
    for (int q = 0; q < 2 * P; ++q) {
        const int p = q >> 1;
        const int row = (q & 1) ? I + i0 + p : i0 + p;
        const bool live = i0 + p < I;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = lane + kWave * c;
            const bool ok = live && ch < nch;
            wv[q][c] = ok ? ld16_stream(wbase + (size_t)row * rb + (size_t)ch * 16) : u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int q = 0; q < 2 * P; ++q) {
        const int p = q >> 1;
        const int row = (q & 1) ? I + i0 + p : i0 + p;
        const bool live = i0 + p < I;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = lane + kWave * c;
            sc[q][c] = (live && ch < nch) ? chunk_scale<FMT>(sbase, row, H, ch) : f32x2{0.0f, 0.0f};
        }
    }
    const float g = global_scale<FMT>(X.gu_g, t.e);

    for (int n = 0; n < t.n; ++n) {
        const int entry = task_entry(t, n, a.R * a.k);
        if (entry < 0) {
            if (lane == 0) flag_error(a.err, kErrBadExpertId);
            continue;
        }
        const uint16_t *xr = a.x + (size_t)entry_row(a, entry) * a.ldx;
        float acc[2 * P];
#pragma unroll
        for (int q = 0; q < 2 * P; ++q) acc[q] = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = lane + kWave * c;
            if (ch < nch) {
                const uint16_t *xp = xr + (size_t)ch * cols_per_chunk<FMT>();
#pragma unroll
                for (int q = 0; q < 2 * P; ++q) acc[q] += chunk_dot_bf16<FMT>(wv[q][c], sc[q][c], xp);
            }
        }
#pragma unroll
        for (int q = 0; q < 2 * P; ++q) acc[q] = group_sum<kWave>(acc[q]);
        if (lane < P && i0 + lane < I) {
            float gv = acc[0], uv = acc[1];
#pragma unroll
            for (int p = 1; p < P; ++p)
                if (lane == p) {
                    gv = acc[2 * p];
                    uv = acc[2 * p + 1];
                }
            a.h[(size_t)entry * a.hstride + i0 + lane] = silu_mul(gv * g, uv * g);
        }
    }
}

// One down-projection output element: row `o` of expert `e`, dotted with
// h[entry], reduced over the LPR lanes of the row group.  Weight chunks and
// scales are preloaded by the caller.
template <int FMT, int LPR, int CH>
__device__ __forceinline__ float down_dot(const u32x4 (&wv)[CH], const f32x2 (&sc)[CH], const float *hrow,
                                          int sub, int nch) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int ch = sub + LPR * c;
        if (ch < nch) acc += chunk_dot_f32<FMT>(wv[c], sc[c], hrow + (size_t)ch * cols_per_chunk<FMT>());
    }
    return group_sum<LPR>(acc);
}

template <int FMT, int LPR, int CH>
__device__ __forceinline__ void load_down_row(const ExpertSet &X, int e, int o, int sub, int nch, int rb,
                                              bool live, u32x4 (&wv)[CH], f32x2 (&sc)[CH]) {
    const uint8_t *wrow = X.dn + (size_t)e * X.dn_stride + (size_t)o * rb;
    const uint8_t *sbase = X.dn_s + (size_t)e * X.dn_s_stride;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int ch = sub + LPR * c;
        const bool ok = live && ch < nch;
        wv[c] = ok ? ld16_stream(wrow + (size_t)ch * 16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int ch = sub + LPR * c;
        sc[c] = (live && ch < nch) ? chunk_scale<FMT>(sbase, o, X.inter, ch) : f32x2{0.0f, 0.0f};
    }
}

__device__ __forceinline__ void store_out(const FfnArgs &a, int r, int o, float y) {
    if (a.y) a.y[(size_t)r * a.ldy + o] = f32_to_bf16(y);
    if (a.res) {
        uint16_t *p = a.res + (size_t)r * a.ldy + o;
        *p = f32_to_bf16(bf16_to_f32(*p) + y);
    }
}

// Down GEMV fused with the blend, one activation row.  A row group of LPR
// lanes owns output element o; it loads row o of every slot's down matrix up
// front (all k+1 experts' loads in flight), then for each slot in order
// reduces d_j and accumulates y = fma(w_j, d_j, y), then fma(s, d_shared, y).
template <int FMT, int LPR, int CH>
__global__ __launch_bounds__(256) void k_down_r1(FfnArgs a) {
    constexpr int RPW = kWave / LPR;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
    const int sub = lane % LPR;
    const int o = (blockIdx.x * 4 + wid) * RPW + lane / LPR;
    const bool live = o < a.H;
    const int nslots = a.k + (a.shared.inter > 0 ? 1 : 0);

    u32x4 wv[kMaxSlots][CH];
    f32x2 sc[kMaxSlots][CH];
    int es[kMaxSlots];
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
        if (j < nslots) {
            const bool sh = j == a.k;
            const ExpertSet &X = sh ? a.shared : a.routed;
            int e = sh ? 0 : a.ids[j];
            const bool ok = sh || (e >= 0 && e < a.E);
            if (!ok) e = -1;
            es[j] = e;
            const int rb = row_bytes<FMT>(X.inter);
            load_down_row<FMT, LPR, CH>(X, ok ? e : 0, o, sub, rb >> 4, rb, live && ok, wv[j], sc[j]);
        }
    }
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
        if (j < nslots) {
            const bool sh = j == a.k;
            const ExpertSet &X = sh ? a.shared : a.routed;
            if (es[j] < 0) {
                if (lane == 0 && blockIdx.x == 0 && wid == 0) flag_error(a.err, kErrBadExpertId);
                continue;
            }
            const int rb = row_bytes<FMT>(X.inter);
            float d = down_dot<FMT, LPR, CH>(wv[j], sc[j], a.h + (size_t)j * a.hstride, sub, rb >> 4);
            d *= global_scale<FMT>(X.dn_g, es[j]);
            y = fmaf(sh ? a.s[0] : a.w[j], d, y);
        }
    }
    if (live && sub == 0) store_out(a, 0, o, y);
}

// Down GEMV for one expert of a multi-row step: a row group keeps row o of
// the expert in registers and writes dbuf[entry][o] for each of its rows.
template <int FMT, int LPR, int CH>
__global__ __launch_bounds__(256) void k_down_grouped(FfnArgs a) {
    constexpr int RPW = kWave / LPR;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
    const Task t = resolve_task(a, blockIdx.y);
    if (!t.valid || t.n == 0) return;
    const ExpertSet &X = *t.X;
    const int sub = lane % LPR;
    const int o = (blockIdx.x * 4 + wid) * RPW + lane / LPR;
    const bool live = o < a.H;
    const int rb = row_bytes<FMT>(X.inter);
    u32x4 wv[CH];
    f32x2 sc[CH];
    load_down_row<FMT, LPR, CH>(X, t.e, o, sub, rb >> 4, rb, live, wv, sc);
    const float g = global_scale<FMT>(X.dn_g, t.e);
    for (int n = 0; n < t.n; ++n) {
        const int entry = task_entry(t, n, a.R * a.k);
        if (entry < 0) continue;
        const float d = down_dot<FMT, LPR, CH>(wv, sc, a.h + (size_t)entry * a.hstride, sub, rb >> 4) * g;
        if (live && sub == 0) a.dbuf[(size_t)entry * a.H + o] = d;
    }
}

// Blend for multi-row steps: y[r][o] = sum_j w[r][j] dbuf[r*k+j][o] (slot
// order) + s[r] dbuf[shared r][o], then the residual add and bf16 rounding,
// with the same operation sequence as the one-row fused kernel.
__global__ __launch_bounds__(256) void k_blend(FfnArgs a) {
    const int o = blockIdx.x * 256 + threadIdx.x;
    const int r = blockIdx.y;
    if (o >= a.H) return;
    float y = 0.0f;
    for (int j = 0; j < a.k; ++j) {
        const int i = r * a.k + j;
        const int e = a.ids[i];
        if (e < 0 || e >= a.E) continue;
        y = fmaf(a.w[i], a.dbuf[(size_t)i * a.H + o], y);
    }
    if (a.shared.inter > 0) y = fmaf(a.s[r], a.dbuf[(size_t)(a.R * a.k + r) * a.H + o], y);
    store_out(a, r, o, y);
}

// Decode probe: every code through the kernels' converters.
//   fmt 0: 4 e4m3 codes per thread -> out[2i] via the bf16 path, out[2i+1] via the f32 path
//   fmt 1: 4 bytes per thread -> per byte b: out[4b..4b+1] bf16 path (low, high nibble),
//          out[4b+2..4b+3] f32 path
__global__ void k_decode_probe(int fmt, const uint8_t *codes, float *out, int n) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (4 * t >= n) return;
    const uint32_t w = *reinterpret_cast<const uint32_t *>(codes + 4 * t);
    if (fmt == 0) {
        const bf16x2 b0 = e4m3x2_bf16<false>(w), b1 = e4m3x2_bf16<true>(w);
        const f32x2 f0 = e4m3x2_f32<false>(w), f1 = e4m3x2_f32<true>(w);
        const float bv[4] = {(float)b0.x, (float)b0.y, (float)b1.x, (float)b1.y};
        const float fv[4] = {f0.x, f0.y, f1.x, f1.y};
        for (int i = 0; i < 4; ++i) {
            out[2 * (4 * t + i)] = bv[i];
            out[2 * (4 * t + i) + 1] = fv[i];
        }
    } else {
        const bf16x2 b[4] = {e2m1x2_bf16<0>(w), e2m1x2_bf16<1>(w), e2m1x2_bf16<2>(w), e2m1x2_bf16<3>(w)};
        const f32x2 f[4] = {e2m1x2_f32<0>(w), e2m1x2_f32<1>(w), e2m1x2_f32<2>(w), e2m1x2_f32<3>(w)};
        for (int i = 0; i < 4; ++i) {
            float *q = out + 4 * (4 * t + i);
            q[0] = (float)b[i].x;
            q[1] = (float)b[i].y;
            q[2] = f[i].x;
            q[3] = f[i].y;
        }
    }
}

// ------------------------------------------------------------------ launchers

static int routed_tasks(const FfnArgs &a) { return a.R == 1 ? a.k : a.max_routed_tasks; }
static int n_tasks(const FfnArgs &a) { return routed_tasks(a) + (a.shared.inter > 0 ? 1 : 0); }

template <int FMT>
static hipError_t gate_up_fmt(const FfnArgs &a, hipStream_t st) {
    constexpr int P = 2;
    const int imax = a.routed.inter > a.shared.inter ? a.routed.inter : a.shared.inter;
    const int nch = (FMT == kFp8 ? a.H : a.H / 2) / 16;
    const int ch = (nch + kWave - 1) / kWave;
    dim3 grid((imax + 4 * P - 1) / (4 * P), n_tasks(a)), block(256);
    if (ch <= 1)
        hipLaunchKernelGGL((k_gate_up<FMT, 1, P>), grid, block, 0, st, a);
    else if (ch <= 2)
        hipLaunchKernelGGL((k_gate_up<FMT, 2, P>), grid, block, 0, st, a);
    else if (ch <= 4)
        hipLaunchKernelGGL((k_gate_up<FMT, 4, P>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((k_gate_up<FMT, 8, P>), grid, block, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gate_up(const FfnArgs &a, hipStream_t st) {
    return a.fmt == kFp8 ? gate_up_fmt<kFp8>(a, st) : gate_up_fmt<kNvfp4>(a, st);
}

// Lanes per down row: enough 16-byte chunks to cover the routed expert's row
// (capped at the wave); chunks per lane cover the longer of routed and shared.
template <int FMT>
static void down_shape(const FfnArgs &a, int &lpr, int &ch) {
    const int nch = (FMT == kFp8 ? a.routed.inter : a.routed.inter / 2) / 16;
    const int ie = a.routed.inter > a.shared.inter ? a.routed.inter : a.shared.inter;
    const int nchmax = (FMT == kFp8 ? ie : ie / 2) / 16;
    lpr = nch >= 64 ? 64 : nch >= 32 ? 32 : nch >= 16 ? 16 : 8;
    ch = (nchmax + lpr - 1) / lpr;
}

#define MOE_DOWN_DISPATCH(KERNEL, FMT, GRID)                                                          \
    do {                                                                                              \
        int lpr, ch;                                                                                  \
        down_shape<FMT>(a, lpr, ch);                                                                  \
        const int rows_per_block = 4 * (kWave / lpr);                                                 \
        dim3 grid GRID;                                                                               \
        dim3 block(256);                                                                              \
        if (ch > 4) return hipErrorInvalidValue;                                                      \
        if (lpr == 8) {                                                                               \
            if (ch <= 1) hipLaunchKernelGGL((KERNEL<FMT, 8, 1>), grid, block, 0, st, a);              \
            else if (ch <= 2) hipLaunchKernelGGL((KERNEL<FMT, 8, 2>), grid, block, 0, st, a);         \
            else hipLaunchKernelGGL((KERNEL<FMT, 8, 4>), grid, block, 0, st, a);                      \
        } else if (lpr == 16) {                                                                       \
            if (ch <= 1) hipLaunchKernelGGL((KERNEL<FMT, 16, 1>), grid, block, 0, st, a);             \
            else if (ch <= 2) hipLaunchKernelGGL((KERNEL<FMT, 16, 2>), grid, block, 0, st, a);        \
            else hipLaunchKernelGGL((KERNEL<FMT, 16, 4>), grid, block, 0, st, a);                     \
        } else if (lpr == 32) {                                                                       \
            if (ch <= 1) hipLaunchKernelGGL((KERNEL<FMT, 32, 1>), grid, block, 0, st, a);             \
            else if (ch <= 2) hipLaunchKernelGGL((KERNEL<FMT, 32, 2>), grid, block, 0, st, a);        \
            else hipLaunchKernelGGL((KERNEL<FMT, 32, 4>), grid, block, 0, st, a);                     \
        } else {                                                                                      \
            if (ch <= 1) hipLaunchKernelGGL((KERNEL<FMT, 64, 1>), grid, block, 0, st, a);             \
            else if (ch <= 2) hipLaunchKernelGGL((KERNEL<FMT, 64, 2>), grid, block, 0, st, a);        \
            else hipLaunchKernelGGL((KERNEL<FMT, 64, 4>), grid, block, 0, st, a);                     \
        }                                                                                             \
        return hipGetLastError();                                                                     \
    } while (0)

template <int FMT>
static hipError_t down_r1_fmt(const FfnArgs &a, hipStream_t st) {
    MOE_DOWN_DISPATCH(k_down_r1, FMT, ((a.H + rows_per_block - 1) / rows_per_block));
}
template <int FMT>
static hipError_t down_grouped_fmt(const FfnArgs &a, hipStream_t st) {
    MOE_DOWN_DISPATCH(k_down_grouped, FMT, ((a.H + rows_per_block - 1) / rows_per_block, n_tasks(a)));
}

hipError_t launch_down_blend_r1(const FfnArgs &a, hipStream_t st) {
    return a.fmt == kFp8 ? down_r1_fmt<kFp8>(a, st) : down_r1_fmt<kNvfp4>(a, st);
}
hipError_t launch_down_grouped(const FfnArgs &a, hipStream_t st) {
    return a.fmt == kFp8 ? down_grouped_fmt<kFp8>(a, st) : down_grouped_fmt<kNvfp4>(a, st);
}
hipError_t launch_blend(const FfnArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_blend, dim3((a.H + 255) / 256, a.R), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_decode_probe(int fmt, const uint8_t *codes, float *out, int n, hipStream_t st) {
    const int threads = (n + 3) / 4;
    hipLaunchKernelGGL(k_decode_probe, dim3((threads + 255) / 256), dim3(256), 0, st, fmt, codes, out, n);
    return hipGetLastError();
}

}  // namespace moe
