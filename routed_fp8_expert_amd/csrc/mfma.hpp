// mfma.hpp -- the grouped-GEMM arm on gfx950 matrix cores, for experts that
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
// Work unit: an expert's 64-row tile by 16 gate (+ 16 up) columns per wave
// (gate/up; each K block's weight codes are converted once and multiplied
// into up to four 16-row subtiles) or a 16-row tile by 32 output columns per
// wave (down), over all of K, with the next K block's loads in flight while
// one is multiplied; the activation (or h) tile staged through LDS for the
// workgroup's four waves; no cross-wave reduction.
// The units run as the leading workgroups of the grouped gate/up and down
// launches (ffn.hip), beside the GEMV arm's.  Operand layout of the
// 16x16x32 MFMA: A[i][k] in lane i + 16*(k/8) element k%8, B[k][j] in lane
// j + 16*(k/8) element k%8, D[i][j] in lane j + 16*(i/4) element i%4.  The K
// order inside a 64-wide chunk is permuted the same way for A and B (lane
// group g holds k = 16g..16g+15, split over two MFMAs), which leaves the
// products unchanged.
#pragma once
#include "gemv.hpp"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// The tile a unit covers: an expert of the MFMA list and TR of its rows, or
// TR rows of the shared expert.  TR selects the tile prefix: kMfmaTileRows
// (down) at mfma_tiles[0 ..], kMfmaGuTileRows (gate/up) at mfma_tiles[E+1 ..].
struct MTile {
    ExpertSet X;           // the expert family (a copy: no pointer into the kernel arguments)
    int e, row0, n;           // expert, first row within the expert, rows in the tile
    const int32_t *list;      // routed: the expert's entries; shared: null (entries first + m)
    int first;
    bool valid;
};

template <int TR>
__device__ __forceinline__ MTile resolve_mtile(const FfnArgs &a, int t) {
    static_assert(TR == kMfmaTileRows || TR == kMfmaGuTileRows, "a planned tile height");
    MTile m{a.routed, 0, 0, 0, nullptr, 0, false};
    const int nk = a.R * a.k;
    const int n_routed = a.meta[TR == kMfmaTileRows ? kMetaMfmaTiles : kMetaMfmaGuTiles];
    const int32_t *prefix = TR == kMfmaTileRows ? a.mfma_tiles : a.mfma_tiles + a.E + 1;
    if (t < n_routed) {
        // the expert whose tile range holds t (prefix over the MFMA list)
        int lo = 0, hi = a.meta[kMetaMfmaCount] - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (prefix[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int e = a.mfma_list[lo];
        if (e < 0 || e >= a.E) return m;
        const int cnt = a.counts[e], off = a.offsets[e];
        if (cnt < 0 || off < 0 || off + cnt > nk) return m;
        m.e = e;
        m.row0 = (t - prefix[lo]) * TR;
        m.n = min(TR, cnt - m.row0);
        m.list = a.perm + off + m.row0;
        m.valid = m.n > 0;
        return m;
    }
    if (!a.shared_mfma) return m;
    const int ts = t - n_routed;
    if (ts * TR >= a.R) return m;
    m.X = a.shared;
    m.row0 = ts * TR;
    m.n = min(TR, a.R - m.row0);
    m.first = nk + m.row0;
    m.valid = true;
    return m;
}

// Entry of row i of the tile, -1 past the tile's rows or for a listed entry
// outside the step's R*k routed entries (shared-expert entries, first + i,
// lie past them by construction).  The list load is unconditional, from a
// clamped index: a valid tile has at least one row.
__device__ __forceinline__ int mtile_entry(const MTile &m, int i, int nk) {
    const int ic = i < m.n ? i : 0;
    if (!m.list) return i < m.n ? m.first + ic : -1;
    const int e = m.list[ic];
    return (i < m.n && e >= 0 && e < nk) ? e : -1;
}

// ------------------------------------------------------------------ gate/up

constexpr int kMfmaWaves = 4;    // waves per workgroup; each owns its own columns over all of K

// Activation tiles go through LDS.  A fragment load straight from memory
// (16 rows x 64 bytes per instruction, the rows H elements apart) runs at
// about a third of the rate of whole-row pieces (measured on MI355X: ~37
// against ~120 GB/s per compute unit from L2), and the workgroup's four
// waves read the same tile; so the workgroup loads each 128-wide K block of
// the tile once, 16 bytes a thread in whole 256-byte row pieces, into a
// double-buffered LDS tile whose rows are padded so that the fragment reads
// of 16 lanes hit distinct banks.
constexpr int kXRow = 128 + 8;   // bf16 per staged activation row (8 of padding)

// The gate and up weight chunks of one 128-wide K block (16 codes each, two
// 64-wide halves).
struct GuStage {
    u32x4 g[2], u[2];
};

__device__ __forceinline__ void gu_load(GuStage &s, const uint8_t *wg, const uint8_t *wu, int kb, int grp) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int k0 = kb * 128 + c * 64 + grp * 16;
        s.g[c] = ld16_stream(wg + k0);
        s.u[c] = ld16_stream(wu + k0);
    }
}

constexpr int kGuSub = kMfmaGuTileRows / 16;   // 16-row subtiles of a gate/up tile

// acc[q] += scale * (X_q . W^T) over one K block, gate and up, for the
// tile's first nsub 16-row subtiles q (nsub is the same for the whole
// workgroup): the block's codes are converted once and multiplied into every
// subtile.  The lane's activation fragments (row 16q + col, k = c*64 +
// grp*16 .. +15) come from the LDS tile.  Per subtile the MFMA chain is the
// one a lone 16-row tile takes, so a row's result does not depend on its
// subtile.
__device__ __forceinline__ void gu_step(const GuStage &s, const uint16_t (*xs)[kXRow], int col, int grp, float sg,
                                        float su, int nsub, f32x4 (&accg)[kGuSub], f32x4 (&accu)[kGuSub]) {
    f32x4 tg[kGuSub], tu[kGuSub];
#pragma unroll
    for (int q = 0; q < kGuSub; ++q) tg[q] = tu[q] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const bf16x8 g0 = e4m3x8_bf16(s.g[c].x, s.g[c].y), g1 = e4m3x8_bf16(s.g[c].z, s.g[c].w);
        const bf16x8 u0 = e4m3x8_bf16(s.u[c].x, s.u[c].y), u1 = e4m3x8_bf16(s.u[c].z, s.u[c].w);
#pragma unroll
        for (int q = 0; q < kGuSub; ++q) {
            if (q < nsub) {
                const u32x4 *xp = reinterpret_cast<const u32x4 *>(&xs[q * 16 + col][c * 64 + grp * 16]);
                const bf16x8 x0 = as_bf16x8(xp[0]), x1 = as_bf16x8(xp[1]);
                tg[q] = mfma(x0, g0, tg[q]);
                tg[q] = mfma(x1, g1, tg[q]);
                tu[q] = mfma(x0, u0, tu[q]);
                tu[q] = mfma(x1, u1, tu[q]);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < kGuSub; ++q) {
        if (q < nsub) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                accg[q][i] = fmaf(sg, tg[q][i], accg[q][i]);
                accu[q][i] = fmaf(su, tu[q][i], accu[q][i]);
            }
        }
    }
}

// h = silu(X_tile . Wg^T) * (X_tile . Wu^T) for a tile of up to 64 rows and
// 16 gate columns (+ the 16 matching up columns) per wave, all of K; two K
// blocks of weight loads in flight, the next K block of activations staged
// while one is multiplied.  The weights are read once per 64 rows: an
// expert's gate/up matrix is the bulk of what a unit loads.
__device__ __forceinline__ void mfma_gate_up_unit(const FfnArgs &a, int bx, int tile) {
    __shared__ uint16_t xs[2][kMfmaGuTileRows][kXRow];
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    const MTile t = resolve_mtile<kMfmaGuTileRows>(a, tile);
    if (!t.valid) return;
    const ExpertSet &X = t.X;
    const int I = X.inter, H = a.H, nk = a.R * a.k;
    // I is a multiple of 128, so a workgroup's 64 columns are all in range or
    // all past it: the exit is uniform (the waves share the barriers below)
    if (bx * kMfmaWaves * 16 >= I) return;
    const int nsub = (t.n + 15) >> 4;   // 1 .. kGuSub
    const int n0 = (bx * kMfmaWaves + wid) * 16;
    const int col = lane & 15, grp = lane >> 4;
    const int nkb = H >> 7;
    // this thread's staging pieces: 16 bytes (8 values) of tile rows
    // threadIdx/16 + 16q; rows without an entry stage row 0 (results dropped)
    const int srow = threadIdx.x >> 4, spiece = threadIdx.x & 15;
    const uint16_t *sx0 = a.x + spiece * 8;
    int srx[kGuSub];   // activation row of each staged tile row
#pragma unroll
    for (int q = 0; q < kGuSub; ++q) {
        srx[q] = 0;
        if (q < nsub) {
            const int sent = mtile_entry(t, srow + 16 * q, nk);
            srx[q] = sent >= 0 ? (sent < nk ? sent / a.k : sent - nk) : 0;
        }
    }
    auto xrow = [&](int q) { return sx0 + (size_t)srx[q] * a.ldx; };
    const uint8_t *wg = X.gu + (size_t)t.e * X.gu_stride + (size_t)(n0 + col) * H;
    const uint8_t *wu = X.gu + (size_t)t.e * X.gu_stride + (size_t)(I + n0 + col) * H;
    // the K block's scales, lane j holding block j (H <= 8192: at most 64)
    const float *sbase = reinterpret_cast<const float *>(X.gu_s + (size_t)t.e * X.gu_s_stride);
    const float sgl = lane < nkb ? sbase[(size_t)(n0 >> 7) * nkb + lane] : 0.0f;
    const float sul = lane < nkb ? sbase[(size_t)((I + n0) >> 7) * nkb + lane] : 0.0f;

    f32x4 accg[kGuSub], accu[kGuSub];
#pragma unroll
    for (int q = 0; q < kGuSub; ++q) accg[q] = accu[q] = f32x4{0, 0, 0, 0};
    // Pipeline: the weights two K blocks ahead, the activations one block
    // ahead in registers (stored into LDS at the start of the step that
    // precedes their use).  The barriers wait for LDS only, so loads in
    // flight stay in flight across them (a full barrier would wait for the
    // next blocks' weights every step); in the steady loop every load is
    // unconditional (row 0 for rows past the tile), so the compiler's wait
    // counts stay exact.
    GuStage s0, s1;
    auto load_w = [&](GuStage &st, int kb) { gu_load(st, wg, wu, kb, grp); };
    u32x4 xr[kGuSub];
    auto load_x = [&](int kb) {
#pragma unroll
        for (int q = 0; q < kGuSub; ++q) xr[q] = ld16(xrow(q) + kb * 128);
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int q = 0; q < kGuSub; ++q)
            if (q < nsub) *reinterpret_cast<u32x4 *>(&xs[buf][srow + 16 * q][spiece * 8]) = xr[q];
    };
    load_w(s0, 0);
    if (nkb > 1) load_w(s1, 1);
    load_x(0);
    store_x(0);
    if (nkb > 1) load_x(1);
    barrier_lds();
    // one K block: the next block's activations (in xr) stored into the other
    // LDS buffer, the block after that loaded, this block multiplied from LDS
    auto step = [&](int kb, const GuStage &st, bool tail) {
        if (!tail || kb + 1 < nkb) store_x((kb + 1) & 1);
        if (!tail || kb + 2 < nkb) load_x(kb + 2);
        gu_step(st, xs[kb & 1], col, grp, readlane(sgl, kb), readlane(sul, kb), nsub, accg, accu);
        barrier_lds();
    };
    int kb = 0;
    for (; kb + 3 < nkb; kb += 2) {   // every load of the two steps is real
        step(kb, s0, false);
        load_w(s0, kb + 2);
        step(kb + 1, s1, false);
        load_w(s1, kb + 3);
    }
    for (; kb < nkb; kb += 2) {       // the last one to three blocks
        step(kb, s0, true);
        if (kb + 2 < nkb) load_w(s0, kb + 2);
        if (kb + 1 < nkb) {
            step(kb + 1, s1, true);
            if (kb + 3 < nkb) load_w(s1, kb + 3);
        }
    }
    // D[i][j]: lane holds column j = col, rows 16q + 4*grp .. +3
#pragma unroll
    for (int q = 0; q < kGuSub; ++q) {
        if (q < nsub) {
            int oent[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) oent[i] = mtile_entry(t, 16 * q + 4 * grp + i, nk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (oent[i] >= 0) a.h[(size_t)oent[i] * a.hstride + n0 + col] = silu_mul(accg[q][i], accu[q][i]);
        }
    }
}

// ------------------------------------------------------------------ down

// The weight chunks of one 128-wide K block of the down tile: the wave's two
// 16-column tiles, two 64-wide halves.
struct DnStage {
    u32x4 w[2][2];
};

__device__ __forceinline__ void dn_load(DnStage &s, const uint8_t *const (&wd)[2], int kb, int grp) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int k0 = kb * 128 + c * 64 + grp * 16;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s.w[nt][c] = ld16_stream(wd[nt] + k0);
    }
}

constexpr int kHbRow = 128 + 8;   // bf16 per staged h row (8 of padding)

// One K block of a down tile's h (SUB 16-row subtiles) in LDS, split as hi +
// lo bf16 (hi = bf16(h), lo = bf16(h - hi)) once, when staged, for all four
// waves.
template <int SUB>
struct DnHs {
    uint16_t hi[16 * SUB][kHbRow];
    uint16_t lo[16 * SUB][kHbRow];
};

// acc[q][nt] += scale[nt] * (h_q . W^T) over one K block for the tile's
// first nsub 16-row subtiles q (nsub is the same for the whole workgroup):
// the block's codes are converted once and multiplied into every subtile.
// The lane's h fragments (row 16q + col, k = c*64 + grp*16 .. +15) are read
// as hi and lo from LDS.  Per subtile the MFMA chain is the one a lone
// 16-row tile takes (hi0, lo0, hi1, lo1 for each half), so a row's result
// does not depend on its subtile.
template <int SUB>
__device__ __forceinline__ void dn_step(const DnStage &s, const DnHs<SUB> &hs, int col, int grp, const float (&sc)[2],
                                        int nsub, f32x4 (&acc)[SUB][2]) {
    bf16x8 w0[2][2], w1[2][2];   // [c][nt]
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            w0[c][nt] = e4m3x8_bf16(s.w[nt][c].x, s.w[nt][c].y);
            w1[c][nt] = e4m3x8_bf16(s.w[nt][c].z, s.w[nt][c].w);
        }
#pragma unroll
    for (int q = 0; q < SUB; ++q) {
        if (q < nsub) {
            f32x4 td[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const u32x4 *hp = reinterpret_cast<const u32x4 *>(&hs.hi[q * 16 + col][c * 64 + grp * 16]);
                const u32x4 *lp = reinterpret_cast<const u32x4 *>(&hs.lo[q * 16 + col][c * 64 + grp * 16]);
                const bf16x8 hi0 = as_bf16x8(hp[0]), hi1 = as_bf16x8(hp[1]);
                const bf16x8 lo0 = as_bf16x8(lp[0]), lo1 = as_bf16x8(lp[1]);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    td[nt] = mfma(hi0, w0[c][nt], td[nt]);
                    td[nt] = mfma(lo0, w0[c][nt], td[nt]);
                    td[nt] = mfma(hi1, w1[c][nt], td[nt]);
                    td[nt] = mfma(lo1, w1[c][nt], td[nt]);
                }
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[q][nt][i] = fmaf(sc[nt], td[nt][i], acc[q][nt][i]);
        }
    }
}

// D = h_tile . W_dn^T for a tile of up to 16*SUB rows (SUB 16-row subtiles:
// 1, the down tiles of the plan, or 4, its 64-row gate/up tiles) and 32
// output columns per wave (two 16-column tiles), all of K = I.  The expert's
// down matrix is read once per tile.  Pipeline as in the gate/up unit: the
// weights two K blocks ahead, h one block ahead in registers (split into
// hi + lo when stored into the other LDS buffer, at the start of the step
// before its use), LDS-only barriers, unconditional loads (entry 0's h for
// rows past the tile) in the steady loop.
template <int SUB>
__device__ __forceinline__ void mfma_down_unit(const FfnArgs &a, int bx, int tile) {
    static_assert(SUB == kMfmaTileRows / 16 || SUB == kMfmaGuTileRows / 16, "a planned tile height");
    __shared__ DnHs<SUB> hs[2];
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    const MTile t = resolve_mtile<16 * SUB>(a, tile);
    if (!t.valid) return;
    const ExpertSet &X = t.X;
    const int I = X.inter, H = a.H, nk = a.R * a.k;
    // H is a multiple of 128: a workgroup's 128 columns are all in range or
    // all past it (uniform exit; the waves share the barriers below)
    if (bx * kMfmaWaves * 32 >= H) return;
    const int nsub = (t.n + 15) >> 4;   // 1 .. SUB
    const int n0 = (bx * kMfmaWaves + wid) * 32;
    const int col = lane & 15, grp = lane >> 4;
    const int nkb = I >> 7;
    // staging: thread t loads values 4*(t%16) .. +3 and 64 + 4*(t%16) .. +3 of
    // the K block for tile rows t/16 + 16q
    const int srow = threadIdx.x >> 4, spiece = threadIdx.x & 15;
    const float *sh[SUB];
#pragma unroll
    for (int q = 0; q < SUB; ++q) {
        const int sent = mtile_entry(t, srow + 16 * q, nk);   // -1 past the tile: entry 0's h (results dropped)
        sh[q] = a.h + (size_t)(sent >= 0 ? sent : 0) * a.hstride + spiece * 4;
    }
    const uint8_t *wd[2];
    float sl[2];
    const float *sbase = reinterpret_cast<const float *>(X.dn_s + (size_t)t.e * X.dn_s_stride);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        wd[nt] = X.dn + (size_t)t.e * X.dn_stride + (size_t)(n0 + nt * 16 + col) * I;
        sl[nt] = lane < nkb ? sbase[(size_t)((n0 + nt * 16) >> 7) * nkb + lane] : 0.0f;
    }
    f32x4 acc[SUB][2];
#pragma unroll
    for (int q = 0; q < SUB; ++q) acc[q][0] = acc[q][1] = f32x4{0, 0, 0, 0};
    DnStage s0, s1;
    f32x4 hr[SUB][2];
    auto load_h = [&](int kb) {
#pragma unroll
        for (int q = 0; q < SUB; ++q) {
            hr[q][0] = *reinterpret_cast<const f32x4 *>(sh[q] + kb * 128);
            hr[q][1] = *reinterpret_cast<const f32x4 *>(sh[q] + kb * 128 + 64);
        }
    };
    auto store_h = [&](int buf) {
#pragma unroll
        for (int q = 0; q < SUB; ++q) {
            if (q < nsub) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    uint32_t hi2[2], lo2[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const float v0 = hr[q][half][2 * i], v1 = hr[q][half][2 * i + 1];
                        const __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1;
                        const __bf16 l0 = (__bf16)(v0 - (float)b0), l1 = (__bf16)(v1 - (float)b1);
                        hi2[i] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
                        lo2[i] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
                    }
                    const int k0 = half * 64 + spiece * 4;
                    *reinterpret_cast<u32x2 *>(&hs[buf].hi[srow + 16 * q][k0]) = u32x2{hi2[0], hi2[1]};
                    *reinterpret_cast<u32x2 *>(&hs[buf].lo[srow + 16 * q][k0]) = u32x2{lo2[0], lo2[1]};
                }
            }
        }
    };
    dn_load(s0, wd, 0, grp);
    if (nkb > 1) dn_load(s1, wd, 1, grp);
    load_h(0);
    store_h(0);
    if (nkb > 1) load_h(1);
    barrier_lds();
    auto step = [&](int kb, const DnStage &st, bool tail) {
        if (!tail || kb + 1 < nkb) store_h((kb + 1) & 1);
        if (!tail || kb + 2 < nkb) load_h(kb + 2);
        const float sc[2] = {readlane(sl[0], kb), readlane(sl[1], kb)};
        dn_step(st, hs[kb & 1], col, grp, sc, nsub, acc);
        barrier_lds();
    };
    int kb = 0;
    for (; kb + 3 < nkb; kb += 2) {   // every load of the two steps is real
        step(kb, s0, false);
        dn_load(s0, wd, kb + 2, grp);
        step(kb + 1, s1, false);
        dn_load(s1, wd, kb + 3, grp);
    }
    for (; kb < nkb; kb += 2) {       // the last one to three blocks
        step(kb, s0, true);
        if (kb + 2 < nkb) dn_load(s0, wd, kb + 2, grp);
        if (kb + 1 < nkb) {
            step(kb + 1, s1, true);
            if (kb + 3 < nkb) dn_load(s1, wd, kb + 3, grp);
        }
    }
    // D[i][j]: lane holds column j = col, rows 16q + 4*grp .. +3
#pragma unroll
    for (int q = 0; q < SUB; ++q) {
        if (q < nsub) {
            int oent[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) oent[i] = mtile_entry(t, 16 * q + 4 * grp + i, nk);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int o = n0 + nt * 16 + col;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (oent[i] >= 0) a.dbuf[(size_t)oent[i] * a.H + o] = acc[q][nt][i];
            }
        }
    }
}

// Workgroups of matrix-core units in a grouped launch: column groups of 64
// gate/up pairs (gate/up) or 128 output columns (down), times the tile bound.
__host__ __device__ inline int mfma_gate_up_groups(int imax) { return (imax + kMfmaWaves * 16 - 1) / (kMfmaWaves * 16); }
__host__ __device__ inline int mfma_down_groups(int H) { return (H + kMfmaWaves * 32 - 1) / (kMfmaWaves * 32); }

}  // namespace moe
