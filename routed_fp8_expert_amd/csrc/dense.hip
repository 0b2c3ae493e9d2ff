// dense.hip -- dense fp8 block-128 projection on gfx950: y = x . dequant(W)^T
// for bf16 activation rows, W in e4m3 codes with one f32 scale per 128x128
// block, f32 accumulation, one bf16 rounding of each output.
//
// GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels": w8a16_gemm_pipelined_m32
// (fp8 block-128 weights times bf16 activations on tensor cores, rows 1 to
// 128 by the "Plan arms" table); "Precision": fp8/block128x128 weights read
// bf16 activations.  Two arms, as for the experts:
//
//   GEMV (fewer than 8 rows)    a wave holds NR weight rows (16-byte lane
//                               chunks, one scale per chunk: the NR rows share
//                               a 128-row scale block) and walks the
//                               activation rows, loading the next row while
//                               reducing the current one; the NR outputs are
//                               reduced together (transposing reduction).
//   matrix cores (>= 8 rows)    a workgroup of 8 waves owns 16 or 32
//                               output columns for one group of 16-row tiles
//                               (the groups sized so the grid covers the
//                               chip); its waves split K (at most eight
//                               128-wide blocks each, the codes held in
//                               registers from entry); fp8 codes converted
//                               exactly to bf16 for v_mfma_f32_16x16x32_bf16,
//                               each block's products scaled, the partial
//                               tiles summed through LDS in K-slice order.
//                               The row groups of a column tile run on one
//                               XCD, so its weights come from HBM once.
#include "mfma.hpp"

namespace moe {

// ------------------------------------------------------------------ GEMV arm

template <int CH, int NR>
__global__ __launch_bounds__(256) void k_dense_gemv(DenseArgs a) {
    constexpr int SPAN = kWave / NR;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    const int n0 = (blockIdx.x * 4 + wid) * NR;
    if (n0 >= a.N) return;
    const int nch = a.K >> 4, nkb = a.K >> 7;
    // weights (unconditional loads from clamped chunks; N is a multiple of 128)
    u32x4 w[NR][CH];
    float sc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int ch = lane + kWave * c, cc = ch < nch ? ch : nch - 1;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const u32x4 v = ld16_stream(a.w + (size_t)(n0 + i) * a.w_stride + (size_t)cc * 16);
            w[i][c] = ch < nch ? v : u32x4{0u, 0u, 0u, 0u};
        }
        sc[c] = a.s[(size_t)(n0 >> 7) * nkb + ((cc * 16) >> 7)];
    }
    u32x4 xc[CH][2], xn[CH][2];
    auto load_x = [&](int r, u32x4 (&xd)[CH][2]) {
        const uint16_t *xr = a.x + (size_t)r * a.ldx;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = lane + kWave * c, cc = ch < nch ? ch : nch - 1;
            xd[c][0] = ld16(xr + (size_t)cc * 16);
            xd[c][1] = ld16(xr + (size_t)cc * 16 + 8);
        }
    };
    load_x(0, xc);
    for (int r = 0; r < a.R; ++r) {
        if (r + 1 < a.R) load_x(r + 1, xn);
        float p[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < CH; ++c)
                acc += sc[c] * dot16_e4m3_bf16(w[i][c], xc[c][0], xc[c][1]);   // zero codes past K
            p[i] = acc;
        }
        xreduce<kWave, NR, 1>(p);
        if (lane % SPAN == 0) a.y[(size_t)r * a.ldy + n0 + lane / SPAN] = f32_to_bf16(p[0]);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            xc[c][0] = xn[c][0];
            xc[c][1] = xn[c][1];
        }
    }
}

// ------------------------------------------------------------------ matrix-core arm

// A workgroup of KS x RS waves owns 16*CT output columns for the 16-row tiles
// of one row group (tpg tiles).  Wave (ks, rg) owns K slice ks (at most KBMAX
// 128-wide blocks, contiguous; its weight codes loaded once, at entry, kept
// in registers) and the group's tiles rg, rg + RS, ...; it walks them with
// the next tiles' activations in flight, each tile's K-block products scaled
// and summed in K order, and leaves its partial tiles in LDS.  Every CHUNK
// tiles the partials are summed over the K slices in slice order and rounded
// once.  A row's result depends on nothing but the row (not on the column
// tile width or the grouping), so any row count gives the same bits for it.
//
// Blocks map to (column tile, row group) through a virtual index that is
// contiguous per XCD (blocks are dispatched to the 8 XCDs round robin):
// consecutive virtual indices are the row groups of one column tile, so
// they share its weight lines in that XCD's L2.
// A tile's activations for this wave's K slice, as loaded: block b, load i
// holds rows 4i + lane/16 of the tile, values 8*(lane%16) .. +7 of the
// block (whole 256-byte row pieces; fragment-shaped loads, 16 rows x 64
// bytes each, run at about a third of the rate from L2).
template <int KBMAX>
struct DenseXs {
    u32x4 v[KBMAX][4];
};

constexpr int kDXRow = 128 + 8;   // bf16 per row of a wave's staged K block (8 of padding)

template <int KBMAX>
__device__ __forceinline__ void dense_load_x(DenseXs<KBMAX> &xs, const DenseArgs &a, int rt, int kb0, int nkb,
                                             int lane) {
    const int piece = lane & 15;
#pragma unroll
    for (int b = 0; b < KBMAX; ++b) {
        const int kb = kb0 + b < nkb ? kb0 + b : nkb - 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ra = rt * 16 + i * 4 + (lane >> 4);
            const uint16_t *xr = a.x + (size_t)(ra < a.R ? ra : 0) * a.ldx;   // rows past R: row 0, results dropped
            xs.v[b][i] = ld16(xr + kb * 128 + piece * 8);
        }
    }
}

// This wave's K-slice products for one tile; nmine is wave-uniform (FULL:
// nmine == KBMAX, no branch between the blocks, so their LDS staging,
// fragment reads, conversions and MFMAs can interleave).  Each K block goes
// through one of the wave's two LDS blocks (alternating; rows padded: the
// fragment reads of 16 lanes hit distinct banks) into MFMA fragments.
template <int CT, int KBMAX, bool FULL>
__device__ __forceinline__ void dense_products(f32x4 (&acc)[CT], u32x4 (&w)[KBMAX][CT][2], float sl,
                                               const DenseXs<KBMAX> &cur, int nmine, uint16_t *xw, int lane) {
    const int col = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < KBMAX; ++b) {
        if (FULL || b < nmine) {
            uint16_t *xbuf = xw + (b & 1) * 16 * kDXRow;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4 *>(xbuf + (i * 4 + (lane >> 4)) * kDXRow + (lane & 15) * 8) = cur.v[b][i];
            f32x4 td[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) td[ct] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const u32x4 *xp = reinterpret_cast<const u32x4 *>(xbuf + col * kDXRow + c * 64 + grp * 16);
                const bf16x8 xa = as_bf16x8(xp[0]), xb = as_bf16x8(xp[1]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    // more than four 16x128 code tiles a wave: convert per
                    // tile (converted codes kept across tiles would not fit
                    // beside the activations); the empty asm on the codes
                    // themselves keeps the conversion in the loop without a
                    // register copy
                    if (KBMAX * CT > 4) asm volatile("" : "+v"(w[b][ct][c]));
                    const u32x4 q = w[b][ct][c];
                    td[ct] = mfma(xa, e4m3x8_bf16(q.x, q.y), td[ct]);
                    td[ct] = mfma(xb, e4m3x8_bf16(q.z, q.w), td[ct]);
                }
            }
            const float sc = readlane(sl, b);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[ct][i] = fmaf(sc, td[ct][i], acc[ct][i]);
        }
    }
}

template <int CT, int KS, int RS, int KBMAX, int D, int CHUNK>
__global__ __launch_bounds__(KS * RS * 64) void k_dense_mfma(DenseArgs a, int tpg, int ngroups) {
    static_assert((CHUNK / RS) % D == 0, "the activation ring turns whole within a chunk");
    constexpr int NT = KS * RS * 64;
    extern __shared__ float part[];   // [CHUNK][KS][CT][256], then the waves' [2][16][kDXRow] bf16 blocks
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wid % KS, rg = wid / KS;
    const int col = lane & 15, grp = lane >> 4;
    const int v = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);   // grid: a multiple of 8 blocks
    if (v >= (a.N / (16 * CT)) * ngroups) return;                            // padding blocks
    const int ctile = v / ngroups, grpi = v - ctile * ngroups;
    const int n0 = ctile * (16 * CT);
    const int nrt_all = (a.R + 15) >> 4;
    const int tb = grpi * tpg, te = tb + tpg < nrt_all ? tb + tpg : nrt_all;   // this group's tiles [tb, te)
    const int nkb = a.K >> 7;
    const int kb0 = ks * nkb / KS, nmine = (ks + 1) * nkb / KS - kb0;   // nmine <= KBMAX (host)
    uint16_t *xw = reinterpret_cast<uint16_t *>(part + CHUNK * KS * CT * 256) + wid * 2 * 16 * kDXRow;

    u32x4 w[KBMAX][CT][2];
#pragma unroll
    for (int b = 0; b < KBMAX; ++b) {
        const int kb = kb0 + b < nkb ? kb0 + b : nkb - 1;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                w[b][ct][c] = ld16_stream(a.w + (size_t)(n0 + ct * 16 + col) * a.w_stride + kb * 128 + c * 64 + grp * 16);
    }
    // one scale per K block: the CT column tiles share a 128-row block
    const float sl = a.s[(size_t)(n0 >> 7) * nkb + (kb0 + lane < nkb ? kb0 + lane : nkb - 1)];

    // a ring of D activation buffers: this wave's next D tiles in flight (a
    // buffer is refilled as soon as its tile's values are in LDS)
    DenseXs<KBMAX> xb[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (D > 1 && tb + rg + d * RS < te) dense_load_x(xb[d], a, tb + rg + d * RS, kb0, nkb, lane);
    for (int t0 = tb; t0 < te; t0 += CHUNK) {
#pragma unroll
        for (int j = 0; j < CHUNK / RS; ++j) {
            const int t = t0 + rg + j * RS;
            if (t < te) {
                if (D == 1) dense_load_x(xb[0], a, t, kb0, nkb, lane);   // no ring: this tile now
                f32x4 acc[CT];
                // the branch-free form only where its longer live ranges fit
                // the registers (no spills)
                if (KBMAX * CT <= 4 && nmine == KBMAX)
                    dense_products<CT, KBMAX, true>(acc, w, sl, xb[j % D], nmine, xw, lane);
                else
                    dense_products<CT, KBMAX, false>(acc, w, sl, xb[j % D], nmine, xw, lane);
                const int tn = t + D * RS;
                if (D > 1 && tn < te) dense_load_x(xb[j % D], a, tn, kb0, nkb, lane);
                float *pp = part + ((j * RS + rg) * KS + ks) * CT * 256;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pp[ct * 256 + i * 64 + lane] = acc[ct][i];
            }
        }
        barrier_lds();   // the partial tiles in LDS; the activation loads stay in flight
        const int ntile = te - t0 < CHUNK ? te - t0 : CHUNK;
        for (int v = threadIdx.x; v < ntile * CT * 256; v += NT) {
            const int tt = v / (CT * 256), rem = v - tt * (CT * 256);
            float sum = 0.0f;
#pragma unroll
            for (int k2 = 0; k2 < KS; ++k2) sum += part[(tt * KS + k2) * CT * 256 + rem];
            const int ct = rem >> 8, i = (rem >> 6) & 3, l = rem & 63;
            const int r = (t0 + tt) * 16 + 4 * (l >> 4) + i;
            if (r < a.R) a.y[(size_t)r * a.ldy + n0 + ct * 16 + (l & 15)] = f32_to_bf16(sum);
        }
        barrier_lds();
    }
}

// ------------------------------------------------------------------ launcher

// Rows from which the matrix-core arm runs.  Below it the GEMV arm, whose
// bits for a row do not depend on the call's row count (so one-row calls and
// calls of up to seven rows agree bit for bit).
constexpr int kDenseMfmaRows = 8;

template <int CH, int NR>
static void dense_gemv_launch(const DenseArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((k_dense_gemv<CH, NR>), dim3((a.N + 4 * NR - 1) / (4 * NR)), dim3(256), 0, st, a);
}

// Grid of the matrix-core arm: ncol column tiles times row groups of tpg
// tiles, the groups as few as give at least one workgroup per CU (one
// workgroup fills a CU's LDS share), rounded up to a multiple of 8 blocks.
template <int CT, int KS, int RS, int KBMAX, int D, int CHUNK>
static void dense_mfma_launch(const DenseArgs &a, hipStream_t st) {
    constexpr int kTargetBlocks = 256;
    const size_t lds = (size_t)CHUNK * KS * CT * 256 * sizeof(float) + (size_t)KS * RS * 2 * 16 * kDXRow * sizeof(uint16_t);
    const int ncol = a.N / (16 * CT), nrt = (a.R + 15) >> 4;
    int ngroups = (kTargetBlocks + ncol - 1) / ncol;
    if (ngroups > nrt) ngroups = nrt;
    const int tpg = (nrt + ngroups - 1) / ngroups;
    ngroups = (nrt + tpg - 1) / tpg;
    const int nb = (ncol * ngroups + 7) / 8 * 8;
    hipLaunchKernelGGL((k_dense_mfma<CT, KS, RS, KBMAX, D, CHUNK>), dim3(nb), dim3(KS * RS * 64), lds, st, a, tpg,
                       ngroups);
}

hipError_t launch_dense(const DenseArgs &a, hipStream_t st) {
    const int nkb = a.K >> 7;
    if (a.R >= kDenseMfmaRows) {
        // eight waves splitting K: two 128-wide blocks a wave (two tiles'
        // activations in flight) up to K 2048, four up to 4096, eight beyond.
        // 32 columns a workgroup up to K 4096 (its codes and two tiles'
        // activations fit the registers of two waves a SIMD) once that still
        // gives a workgroup per CU; 16 below (more workgroups; measured)
        const int nrt = (a.R + 15) >> 4;
        const bool wide = (a.N / 32) * nrt >= 256;
        if (nkb <= 16) {
            if (wide) dense_mfma_launch<2, 8, 1, 2, 2, 4>(a, st);
            else dense_mfma_launch<1, 8, 1, 2, 2, 8>(a, st);
        } else if (nkb <= 32) {
            if (wide) dense_mfma_launch<2, 8, 1, 4, 2, 4>(a, st);
            else dense_mfma_launch<1, 8, 1, 4, 2, 8>(a, st);
        } else {
            dense_mfma_launch<1, 8, 1, 8, 1, 8>(a, st);
        }
        return hipGetLastError();
    }
    // 16-byte weight chunks per lane and row: K/1024 rounded up to a power of
    // two; four weight rows a wave up to K 2048, two beyond (measured)
    const int ch = (a.K + 1023) / 1024;
    if (ch <= 1) dense_gemv_launch<1, 4>(a, st);
    else if (ch <= 2) dense_gemv_launch<2, 4>(a, st);
    else if (ch <= 4) dense_gemv_launch<4, 2>(a, st);
    else dense_gemv_launch<8, 2>(a, st);
    return hipGetLastError();
}

}  // namespace moe
