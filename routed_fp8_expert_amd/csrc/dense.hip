// dense.hip -- dense fp8 block-128 projection on gfx950: y = x . dequant(W)^T
// for bf16 activation rows, W in e4m3 codes with one f32 scale per 128x128
// block, f32 accumulation, one bf16 rounding of each output.
//
// GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels": w8a16_gemm_pipelined_m32
// (fp8 block-128 weights times bf16 activations on tensor cores, rows 1 to
// 128 by the "Plan arms" table); "Precision": fp8/block128x128 weights read
// bf16 activations.  Two arms, as for the experts:
//
//   GEMV (fewer than 32 rows)   a wave holds NR weight rows (16-byte lane
//                               chunks, one scale per chunk: the NR rows share
//                               a 128-row scale block) and walks the
//                               activation rows, loading the next row while
//                               reducing the current one; the NR outputs are
//                               reduced together (transposing reduction).
//   matrix cores (>= 32 rows)   a wave owns a 16-row tile by 32 output
//                               columns over all of K; fp8 codes converted
//                               exactly to bf16, v_mfma_f32_16x16x32_bf16,
//                               the block scale applied per 128-wide K block,
//                               two K blocks of loads in flight.
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

struct DenseStage {
    u32x4 w[2][2];      // [column tile][64-wide half of the K block]
    u32x4 x[2][2];      // [half][8-value piece]
};

__device__ __forceinline__ void dense_load(DenseStage &s, const uint8_t *const (&wd)[2], const uint16_t *xr, int kb,
                                           int grp) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int k0 = kb * 128 + c * 64 + grp * 16;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s.w[nt][c] = ld16_stream(wd[nt] + k0);
        s.x[c][0] = ld16(xr + k0);
        s.x[c][1] = ld16(xr + k0 + 8);
    }
}

__device__ __forceinline__ void dense_step(const DenseStage &s, const float (&sc)[2], f32x4 (&acc)[2]) {
    f32x4 td[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const bf16x8 x0 = as_bf16x8(s.x[c][0]), x1 = as_bf16x8(s.x[c][1]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            td[nt] = mfma(x0, e4m3x8_bf16(s.w[nt][c].x, s.w[nt][c].y), td[nt]);
            td[nt] = mfma(x1, e4m3x8_bf16(s.w[nt][c].z, s.w[nt][c].w), td[nt]);
        }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] = fmaf(sc[nt], td[nt][i], acc[nt][i]);
}

// Grid (N/128, ceil(R/16)); a workgroup is 4 waves x 32 output columns.
__global__ __launch_bounds__(256) void k_dense_mfma(DenseArgs a) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6;
    const int n0 = (blockIdx.x * 4 + wid) * 32;
    if (n0 >= a.N) return;
    const int r0 = blockIdx.y * 16;
    const int col = lane & 15, grp = lane >> 4;
    const int nkb = a.K >> 7;
    const int ra = r0 + col;   // the A-operand row this lane loads (row 0 past R: its outputs are dropped)
    const uint16_t *xr = a.x + (size_t)(ra < a.R ? ra : 0) * a.ldx;
    const uint8_t *wd[2];
    float sl[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        wd[nt] = a.w + (size_t)(n0 + nt * 16 + col) * a.w_stride;
        sl[nt] = a.s[(size_t)((n0 + nt * 16) >> 7) * nkb + (lane < nkb ? lane : 0)];
    }
    f32x4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    DenseStage s0, s1;
    dense_load(s0, wd, xr, 0, grp);
    if (nkb > 1) dense_load(s1, wd, xr, 1, grp);
    for (int kb = 0; kb < nkb; kb += 2) {
        {
            const float sc[2] = {readlane(sl[0], kb), readlane(sl[1], kb)};
            dense_step(s0, sc, acc);
        }
        if (kb + 2 < nkb) dense_load(s0, wd, xr, kb + 2, grp);
        if (kb + 1 < nkb) {
            const float sc[2] = {readlane(sl[0], kb + 1), readlane(sl[1], kb + 1)};
            dense_step(s1, sc, acc);
            if (kb + 3 < nkb) dense_load(s1, wd, xr, kb + 3, grp);
        }
    }
    // D[i][j]: lane holds column j = col, rows 4*grp .. 4*grp+3
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + 4 * grp + i;
            if (r < a.R) a.y[(size_t)r * a.ldy + n0 + nt * 16 + col] = f32_to_bf16(acc[nt][i]);
        }
}

// ------------------------------------------------------------------ launcher

constexpr int kDenseMfmaRows = 32;   // rows from which the matrix-core arm runs

template <int CH, int NR>
static void dense_gemv_launch(const DenseArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((k_dense_gemv<CH, NR>), dim3((a.N + 4 * NR - 1) / (4 * NR)), dim3(256), 0, st, a);
}

hipError_t launch_dense(const DenseArgs &a, hipStream_t st) {
    if (a.R >= kDenseMfmaRows) {
        hipLaunchKernelGGL(k_dense_mfma, dim3((a.N + 127) / 128, (a.R + 15) / 16), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    // 16-byte weight chunks per lane and row: K/1024 rounded up to a power of
    // two; at most 16 weight chunks per lane in all (K <= 8192)
    const int ch = (a.K + 1023) / 1024;
    if (ch <= 1) dense_gemv_launch<1, 8>(a, st);
    else if (ch <= 2) dense_gemv_launch<2, 8>(a, st);
    else if (ch <= 4) dense_gemv_launch<4, 4>(a, st);
    else dense_gemv_launch<8, 2>(a, st);
    return hipGetLastError();
}

}  // namespace moe
