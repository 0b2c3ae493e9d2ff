// mfma.hip -- the grouped-GEMM arm on gfx950 matrix cores, for experts that
// receive many rows in a multi-row step (the same arithmetic as the GEMV arm).
//
// GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels": w8a16_gemm_pipelined_m32
// (fp8 block-128 weights times bf16 activations on tensor cores), and "Plan
// arms": the plan changes shape at the larger multi-row arms.  Here the fp8
// codes are converted exactly to bf16 and fed to v_mfma_f32_16x16x32_bf16
// with f32 accumulation; the block scale (one per 128x128 block) multiplies a
// per-K-block partial sum.  The down projection's f32 intermediate h enters
// as a bf16 pair hi + lo (hi = bf16(h), lo = bf16(h - hi)), two MFMAs, so h
// keeps about 16 significant bits.
//
// Work unit: (an expert's 32-row tile, 64 output columns); a workgroup is 4
// waves, each wave 16 columns (gate/up: 16 gate and the 16 matching up
// columns) for both 16-row halves of the tile.  Operand layout of the
// 16x16x32 MFMA: A[i][k] in lane i + 16*(k/8) element k%8, B[k][j] in lane
// j + 16*(k/8) element k%8, D[i][j] in lane j + 16*(i/4) element i%4.  The K
// order inside a 64-wide chunk is permuted the same way for A and B (lane
// group g holds k = 16g..16g+15, split over two MFMAs), which leaves the
// products unchanged.
#include "gemv.hpp"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 32;

// 8 e4m3 codes (2 dwords) to 8 bf16, exact.
__device__ __forceinline__ bf16x8 e4m3x8_bf16(uint32_t w0, uint32_t w1) {
    const bf16x2 a = e4m3x2_bf16<false>(w0), b = e4m3x2_bf16<true>(w0);
    const bf16x2 c = e4m3x2_bf16<false>(w1), d = e4m3x2_bf16<true>(w1);
    return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The tile a workgroup row (blockIdx.y) covers: an expert of the MFMA list
// and 32 of its rows, or 32 rows of the shared expert.
struct MTile {
    const ExpertSet *X;
    int e, row0, n;           // expert, first row within the expert, rows in the tile
    const int32_t *list;      // routed: the expert's entries; shared: null (entries first + m)
    int first;
    bool valid;
};

__device__ __forceinline__ MTile resolve_mtile(const FfnArgs &a, int t) {
    MTile m{&a.routed, 0, 0, 0, nullptr, 0, false};
    const int nk = a.R * a.k;
    const int n_routed = a.meta[kMetaMfmaTiles];
    if (t < n_routed) {
        // the expert whose tile range holds t (prefix over the MFMA list)
        int lo = 0, hi = a.meta[kMetaMfmaCount] - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.mfma_tiles[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int e = a.mfma_list[lo];
        if (e < 0 || e >= a.E) return m;
        const int cnt = a.counts[e], off = a.offsets[e];
        if (cnt < 0 || off < 0 || off + cnt > nk) return m;
        m.e = e;
        m.row0 = (t - a.mfma_tiles[lo]) * kTileRows;
        m.n = min(kTileRows, cnt - m.row0);
        m.list = a.perm + off + m.row0;
        m.valid = m.n > 0;
        return m;
    }
    if (!a.shared_mfma) return m;
    const int ts = t - n_routed;
    if (ts * kTileRows >= a.R) return m;
    m.X = &a.shared;
    m.row0 = ts * kTileRows;
    m.n = min(kTileRows, a.R - m.row0);
    m.first = nk + m.row0;
    m.valid = true;
    return m;
}

__device__ __forceinline__ int mtile_entry(const MTile &m, int i, int nk) {
    if (i >= m.n) return -1;
    if (!m.list) return m.first + i;
    const int e = m.list[i];
    return (e >= 0 && e < nk) ? e : -1;
}

// ------------------------------------------------------------------ gate/up

// Y = X_tile . W_gu^T for 16 gate and 16 up columns per wave, then
// h = silu(gate) * up for the tile's rows.
__global__ __launch_bounds__(256) void k_mfma_gate_up(FfnArgs a) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    const MTile t = resolve_mtile(a, blockIdx.y);
    if (!t.valid) return;
    const ExpertSet &X = *t.X;
    const int I = X.inter, H = a.H, nk = a.R * a.k;
    const int n0 = (blockIdx.x * 4 + wid) * 16;
    if (n0 >= I) return;
    const int col = lane & 15, grp = lane >> 4;
    // A rows: the two 16-row halves of the tile; a row past the tile reads row 0 (zeroed)
    int ent[2];
    const uint16_t *xr[2];
    bool rv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        ent[h] = mtile_entry(t, h * 16 + col, nk);
        rv[h] = ent[h] >= 0;
        const int row = rv[h] ? (ent[h] < nk ? ent[h] / a.k : ent[h] - nk) : 0;
        xr[h] = a.x + (size_t)row * a.ldx;
    }
    const uint8_t *wg = X.gu + (size_t)t.e * X.gu_stride + (size_t)(n0 + col) * H;
    const uint8_t *wu = X.gu + (size_t)t.e * X.gu_stride + (size_t)(I + n0 + col) * H;
    const float *sg = reinterpret_cast<const float *>(X.gu_s + (size_t)t.e * X.gu_s_stride) + (size_t)(n0 >> 7) * (H >> 7);
    const float *su = reinterpret_cast<const float *>(X.gu_s + (size_t)t.e * X.gu_s_stride) + (size_t)((I + n0) >> 7) * (H >> 7);

    f32x4 cg[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, cu[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    for (int kb = 0; kb < (H >> 7); ++kb) {
        // one 128-wide K block: two 64-wide chunks per lane group
        u32x4 bgw[2], buw[2], ax[2][2][2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int k0 = kb * 128 + c * 64 + grp * 16;
            bgw[c] = ld16_stream(wg + k0);
            buw[c] = ld16_stream(wu + k0);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                ax[h][c][0] = rv[h] ? ld16(xr[h] + k0) : u32x4{0u, 0u, 0u, 0u};
                ax[h][c][1] = rv[h] ? ld16(xr[h] + k0 + 8) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        f32x4 tg[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, tu[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bf16x8 g0 = e4m3x8_bf16(bgw[c].x, bgw[c].y), g1 = e4m3x8_bf16(bgw[c].z, bgw[c].w);
            const bf16x8 u0 = e4m3x8_bf16(buw[c].x, buw[c].y), u1 = e4m3x8_bf16(buw[c].z, buw[c].w);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8 x0 = as_bf16x8(ax[h][c][0]), x1 = as_bf16x8(ax[h][c][1]);
                tg[h] = mfma(x0, g0, tg[h]);
                tg[h] = mfma(x1, g1, tg[h]);
                tu[h] = mfma(x0, u0, tu[h]);
                tu[h] = mfma(x1, u1, tu[h]);
            }
        }
        const float s_g = sg[kb], s_u = su[kb];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cg[h][i] = fmaf(s_g, tg[h][i], cg[h][i]);
                cu[h][i] = fmaf(s_u, tu[h][i], cu[h][i]);
            }
    }
    // D[i][j]: lane holds column j = col, rows 4*grp .. 4*grp+3 of each half
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = mtile_entry(t, h * 16 + 4 * grp + i, nk);
            if (e >= 0) a.h[(size_t)e * a.hstride + n0 + col] = silu_mul(cg[h][i], cu[h][i]);
        }
}

// ------------------------------------------------------------------ down

// D = h_tile . W_dn^T for 16 output columns per wave; h enters as hi + lo.
__global__ __launch_bounds__(256) void k_mfma_down(FfnArgs a) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    const MTile t = resolve_mtile(a, blockIdx.y);
    if (!t.valid) return;
    const ExpertSet &X = *t.X;
    const int I = X.inter, H = a.H, nk = a.R * a.k;
    const int n0 = (blockIdx.x * 4 + wid) * 16;
    if (n0 >= H) return;
    const int col = lane & 15, grp = lane >> 4;
    int ent[2];
    const float *hr[2];
    bool rv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        ent[h] = mtile_entry(t, h * 16 + col, nk);
        rv[h] = ent[h] >= 0;
        hr[h] = a.h + (size_t)(rv[h] ? ent[h] : 0) * a.hstride;
    }
    const uint8_t *wd = X.dn + (size_t)t.e * X.dn_stride + (size_t)(n0 + col) * I;
    const float *sd = reinterpret_cast<const float *>(X.dn_s + (size_t)t.e * X.dn_s_stride) + (size_t)(n0 >> 7) * (I >> 7);

    f32x4 cd[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    for (int kb = 0; kb < (I >> 7); ++kb) {
        u32x4 bw[2];
        f32x4 hv[2][2][4];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int k0 = kb * 128 + c * 64 + grp * 16;
            bw[c] = ld16_stream(wd + k0);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    hv[h][c][q] = rv[h] ? *reinterpret_cast<const f32x4 *>(hr[h] + k0 + 4 * q) : f32x4{0, 0, 0, 0};
        }
        f32x4 td[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bf16x8 w0 = e4m3x8_bf16(bw[c].x, bw[c].y), w1 = e4m3x8_bf16(bw[c].z, bw[c].w);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8 hi0, lo0, hi1, lo1;
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v0 = hv[h][c][q][i], v1 = hv[h][c][q + 2][i];
                        const __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1;
                        hi0[q * 4 + i] = b0;
                        lo0[q * 4 + i] = (__bf16)(v0 - (float)b0);
                        hi1[q * 4 + i] = b1;
                        lo1[q * 4 + i] = (__bf16)(v1 - (float)b1);
                    }
                td[h] = mfma(hi0, w0, td[h]);
                td[h] = mfma(lo0, w0, td[h]);
                td[h] = mfma(hi1, w1, td[h]);
                td[h] = mfma(lo1, w1, td[h]);
            }
        }
        const float s = sd[kb];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) cd[h][i] = fmaf(s, td[h][i], cd[h][i]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = mtile_entry(t, h * 16 + 4 * grp + i, nk);
            if (e >= 0) a.dbuf[(size_t)e * a.H + n0 + col] = cd[h][i];
        }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_mfma_gate_up(const FfnArgs &a, hipStream_t st) {
    if (a.mfma_max_tiles <= 0) return hipSuccess;
    const int imax = a.routed.inter > a.shared.inter ? a.routed.inter : a.shared.inter;
    hipLaunchKernelGGL(k_mfma_gate_up, dim3((imax + 63) / 64, a.mfma_max_tiles), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_mfma_down(const FfnArgs &a, hipStream_t st) {
    if (a.mfma_max_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_mfma_down, dim3((a.H + 63) / 64, a.mfma_max_tiles), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
