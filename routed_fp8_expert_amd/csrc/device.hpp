// device.hpp -- device helpers shared by the gfx950 kernels: vector loads,
// the stored number formats, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ loads

__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
// Weights are read once per step: stream them past the caches.
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// ------------------------------------------------------------------ formats

// bf16 is the top half of a binary32, so widening is a shift.
__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest bf16, ties to even; NaN kept quiet.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// Two OCP e4m3 codes (byte pair 0-1 or 2-3 of `w`) to two bf16.  Every e4m3
// value is exact in bf16 (3 mantissa bits, exponents 2^-9 .. 2^8).
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_bf16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}
// Two OCP e4m3 codes to two f32.
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}
// One e4m3 code (byte `b` of `w`) to f32.
__device__ __forceinline__ float e4m3_f32(uint32_t w, int b) {
    f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(w >> (16 * (b >> 1)), false);
    return (b & 1) ? v.y : v.x;
}
// Two e2m1 codes (byte `B` of `w`, the low nibble first) to two bf16.
template <int B>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
}
// Two e2m1 codes to two f32.
template <int B>
__device__ __forceinline__ f32x2 e2m1x2_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}

__device__ __forceinline__ float dot2(bf16x2 a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, as_bf16x2(b), c, false);
}

// 16 e4m3 codes (one 16-byte chunk) . 16 bf16 activations (two 16-byte chunks).
__device__ __forceinline__ float dot16_e4m3_bf16(u32x4 w, u32x4 xa, u32x4 xb) {
    float a = 0.0f;
    a = dot2(e4m3x2_bf16<false>(w.x), xa.x, a);
    a = dot2(e4m3x2_bf16<true>(w.x), xa.y, a);
    a = dot2(e4m3x2_bf16<false>(w.y), xa.z, a);
    a = dot2(e4m3x2_bf16<true>(w.y), xa.w, a);
    a = dot2(e4m3x2_bf16<false>(w.z), xb.x, a);
    a = dot2(e4m3x2_bf16<true>(w.z), xb.y, a);
    a = dot2(e4m3x2_bf16<false>(w.w), xb.z, a);
    a = dot2(e4m3x2_bf16<true>(w.w), xb.w, a);
    return a;
}

// 8 e2m1 codes (one dword) . 8 bf16 activations (one 16-byte chunk).
__device__ __forceinline__ float dot8_e2m1_bf16(uint32_t w, u32x4 x, float a) {
    a = dot2(e2m1x2_bf16<0>(w), x.x, a);
    a = dot2(e2m1x2_bf16<1>(w), x.y, a);
    a = dot2(e2m1x2_bf16<2>(w), x.z, a);
    a = dot2(e2m1x2_bf16<3>(w), x.w, a);
    return a;
}

// 16 e4m3 codes . 16 f32 activations (four 16-byte chunks).
__device__ __forceinline__ float dot16_e4m3_f32(u32x4 w, const f32x4 *h) {
    float a = 0.0f;
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f32x2 lo = e4m3x2_f32<false>(ws[q]), hi = e4m3x2_f32<true>(ws[q]);
        a = fmaf(lo.x, h[q].x, a);
        a = fmaf(lo.y, h[q].y, a);
        a = fmaf(hi.x, h[q].z, a);
        a = fmaf(hi.y, h[q].w, a);
    }
    return a;
}

// 8 e2m1 codes (one dword) . 8 f32 activations (two 16-byte chunks).
__device__ __forceinline__ float dot8_e2m1_f32(uint32_t w, f32x4 h0, f32x4 h1, float a) {
    f32x2 v0 = e2m1x2_f32<0>(w), v1 = e2m1x2_f32<1>(w), v2 = e2m1x2_f32<2>(w),
          v3 = e2m1x2_f32<3>(w);
    a = fmaf(v0.x, h0.x, a);
    a = fmaf(v0.y, h0.y, a);
    a = fmaf(v1.x, h0.z, a);
    a = fmaf(v1.y, h0.w, a);
    a = fmaf(v2.x, h1.x, a);
    a = fmaf(v2.y, h1.y, a);
    a = fmaf(v3.x, h1.z, a);
    a = fmaf(v3.y, h1.w, a);
    return a;
}

// Two's-complement integer codes (the integer expert formats).  A
// sign-extending bit-field extract and an int -> f32 convert give the exact
// value; integers of at most 8 significant bits are exact in bf16, so the
// upper half of the f32 is the bf16, and two of them pack into a pair.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
    return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xffff0000u);
}
// int8 code in byte B of w.
template <int B>
__device__ __forceinline__ float i8_f32(uint32_t w) {
    return (float)((int)(w << (24 - 8 * B)) >> 24);
}
// int4 code in nibble N of w (nibble 0 = bits 0..3).
template <int N>
__device__ __forceinline__ float i4_f32(uint32_t w) {
    return (float)((int)(w << (28 - 4 * N)) >> 28);
}

// 16 int8 codes (one 16-byte chunk) . 16 bf16 activations (two 16-byte chunks).
__device__ __forceinline__ float dot16_i8_bf16(u32x4 w, u32x4 xa, u32x4 xb) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    const uint32_t xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    float a = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        a = dot2(as_bf16x2(pack_bf16_exact(i8_f32<0>(ws[q]), i8_f32<1>(ws[q]))), xs[2 * q], a);
        a = dot2(as_bf16x2(pack_bf16_exact(i8_f32<2>(ws[q]), i8_f32<3>(ws[q]))), xs[2 * q + 1], a);
    }
    return a;
}
// 16 int8 codes . 16 f32 activations (four 16-byte chunks).
__device__ __forceinline__ float dot16_i8_f32(u32x4 w, const f32x4 *h) {
    float a = 0.0f;
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        a = fmaf(i8_f32<0>(ws[q]), h[q].x, a);
        a = fmaf(i8_f32<1>(ws[q]), h[q].y, a);
        a = fmaf(i8_f32<2>(ws[q]), h[q].z, a);
        a = fmaf(i8_f32<3>(ws[q]), h[q].w, a);
    }
    return a;
}
// 8 int4 codes (one dword, the even column in the low nibble) . 8 bf16
// activations (one 16-byte chunk).
__device__ __forceinline__ float dot8_i4_bf16(uint32_t w, u32x4 x, float a) {
    a = dot2(as_bf16x2(pack_bf16_exact(i4_f32<0>(w), i4_f32<1>(w))), x.x, a);
    a = dot2(as_bf16x2(pack_bf16_exact(i4_f32<2>(w), i4_f32<3>(w))), x.y, a);
    a = dot2(as_bf16x2(pack_bf16_exact(i4_f32<4>(w), i4_f32<5>(w))), x.z, a);
    a = dot2(as_bf16x2(pack_bf16_exact(i4_f32<6>(w), i4_f32<7>(w))), x.w, a);
    return a;
}
// 8 int4 codes . 8 f32 activations (two 16-byte chunks).
__device__ __forceinline__ float dot8_i4_f32(uint32_t w, f32x4 h0, f32x4 h1, float a) {
    a = fmaf(i4_f32<0>(w), h0.x, a);
    a = fmaf(i4_f32<1>(w), h0.y, a);
    a = fmaf(i4_f32<2>(w), h0.z, a);
    a = fmaf(i4_f32<3>(w), h0.w, a);
    a = fmaf(i4_f32<4>(w), h1.x, a);
    a = fmaf(i4_f32<5>(w), h1.y, a);
    a = fmaf(i4_f32<6>(w), h1.z, a);
    a = fmaf(i4_f32<7>(w), h1.w, a);
    return a;
}

// 8 bf16 weights . 8 bf16 activations (one 16-byte chunk each).
__device__ __forceinline__ float dot8_bf16(u32x4 w, u32x4 x, float a) {
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.x), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.w), a, false);
    return a;
}

// ------------------------------------------------------------------ reductions
//
// Cross-lane steps use DPP (data-parallel primitives on the VALU: quad
// permutes, half-row and row mirrors, row broadcasts) rather than
// ds_bpermute, so a reduction is a short chain of VALU ops with no LDS round
// trip.  All lanes of the wave must be active.

enum : int {
    kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141, // lane i <- lane 7-i within each 8-lane half-row
    kDppMirror = 0x140,     // lane i <- lane 15-i within each 16-lane row
    kDppBcast15 = 0x142,    // row r <- lane 15 of row r-1 (rows selected by the row mask)
    kDppBcast31 = 0x143,    // rows 2,3 <- lane 31
};

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp(float old, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, v), CTRL, ROWS, 0xf,
                                                                 false));
}
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// The two results of a lane-swap builtin, as floats.  Each result is copied
// into a named integer before the bit cast: hipcc miscompiles bit casts of
// both subscripts inside one expression (it reads element 0 twice).
template <int M>
__device__ __forceinline__ void lane_swap(float a, float b, float &ra, float &rb) {
    static_assert(M == 32 || M == 16, "swap stride");
    const unsigned ua = __builtin_bit_cast(unsigned, a), ub = __builtin_bit_cast(unsigned, b);
    unsigned x, y;
    if constexpr (M == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
        x = r[0];
        y = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
        x = r[0];
        y = r[1];
    }
    ra = __builtin_bit_cast(float, x);
    rb = __builtin_bit_cast(float, y);
}

// One butterfly stage over lane pairs l, l ^ m (m = 32, 16: the gfx950
// lane-swap instructions; m = 8, 4: row and half-row mirrors, which pair
// l with the lane whose low 4 or 3 bits are inverted; m = 2, 1: quad
// permutes).  Every lane adds its partner's value to its own.
template <int M>
__device__ __forceinline__ float bfly(float v) {
    if constexpr (M == 32 || M == 16) {
        float x, y;
        lane_swap<M>(v, v, x, y);
        return x + y;
    } else {
        constexpr int CTRL = M == 8 ? kDppMirror : M == 4 ? kDppHalfMirror : M == 2 ? kDppXor2 : kDppXor1;
        return v + dpp<CTRL>(0.0f, v);
    }
}

// Transposing stage over lane pairs l, l ^ m for two values a, b: lanes with
// bit m clear end with a + a(partner), lanes with it set with b + b(partner).
// Per kept value this is the same addition bfly<M> makes.
template <int M>
__device__ __forceinline__ float bfly_split(float a, float b) {
    if constexpr (M == 32 || M == 16) {
        float x, y;
        lane_swap<M>(a, b, x, y);
        return x + y;
    } else {
        constexpr int CTRL = M == 8 ? kDppMirror : M == 4 ? kDppHalfMirror : M == 2 ? kDppXor2 : kDppXor1;
        const bool hi = (threadIdx.x & M) != 0;
        const float keep = hi ? b : a, send = hi ? a : b;
        return keep + dpp<CTRL>(0.0f, send);
    }
}

// Sum over aligned groups of W lanes (W = 8, 16, 32 or 64) by butterfly
// stages from stride W/2 down to 1; every lane of a group ends with the same
// value, and the addition tree is the one xreduce uses, so a dot product
// comes out bit-identical wherever it is computed.
template <int W, int M = W / 2>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
    if constexpr (M == 0) {
        return v;
    } else {
        return group_sum<W, M / 2>(bfly<M>(v));
    }
}

// Reduce NU units of U values each over aligned groups of W lanes at once:
// the first log2(NU) stages transpose (each halves the units a lane keeps),
// the rest are plain butterflies.  On return v[0 .. U-1] hold unit
// (lane % W) / (W / NU), summed over the group, with the same bits
// group_sum would give for that value alone.
template <int W, int NU, int U, int M = W / 2>
__device__ __forceinline__ void xreduce(float *v) {
    static_assert(NU >= 1 && NU <= W, "units");
    if constexpr (M == 0) {
        return;
    } else if constexpr (NU > 1) {
        constexpr int H = NU / 2;
#pragma unroll
        for (int u = 0; u < H; ++u)
#pragma unroll
            for (int e = 0; e < U; ++e) v[u * U + e] = bfly_split<M>(v[u * U + e], v[(u + H) * U + e]);
        xreduce<W, H, U, M / 2>(v);
    } else {
#pragma unroll
        for (int e = 0; e < U; ++e) v[e] = bfly<M>(v[e]);
        xreduce<W, 1, U, M / 2>(v);
    }
}

__device__ __forceinline__ float wave_max(float v) {
    const float ninf = -__builtin_inff();
    v = fmaxf(v, dpp<kDppXor1>(ninf, v));
    v = fmaxf(v, dpp<kDppXor2>(ninf, v));
    v = fmaxf(v, dpp<kDppHalfMirror>(ninf, v));
    v = fmaxf(v, dpp<kDppMirror>(ninf, v));
    v = fmaxf(v, dpp<kDppBcast15, 0xa>(ninf, v));
    v = fmaxf(v, dpp<kDppBcast31, 0xc>(ninf, v));
    return readlane(v, 63);
}

// Wave argmax under the total order (larger value first, lower index first
// among equal values).  Returns the winner in every lane.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ void argmax_step(float &v, int &i) {
    const float ov = dpp<CTRL, ROWS>(-__builtin_inff(), v);
    const int oi = dpp<CTRL, ROWS>(0x7fffffff, i);
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
    argmax_step<kDppXor1>(v, i);
    argmax_step<kDppXor2>(v, i);
    argmax_step<kDppHalfMirror>(v, i);
    argmax_step<kDppMirror>(v, i);
    argmax_step<kDppBcast15, 0xa>(v, i);
    argmax_step<kDppBcast31, 0xc>(v, i);
    v = readlane(v, 63);
    i = readlane(i, 63);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

// Workgroup barrier for data exchanged through LDS: waits for the wave's
// LDS operations, not for its global loads in flight (__syncthreads waits
// for both).  The memory clobber keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void flag_error(uint32_t *err, uint32_t bit) {
    if (err) __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
