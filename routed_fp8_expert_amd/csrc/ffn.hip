// ffn.hip -- the expert kernels' format dispatch (the kernels themselves are
// in ffn.hpp, instantiated per weight format in ffn_<format>.hip), the
// blend of multi-row steps, the RMSNorm epilogue kernels and the decode probe.
//
// GB10 blueprint for Qwen3.6-35B-A3B-FP8, "Kernels": moe_weighted_sum_blend,
// residual_add_rms_norm.
#include "ffn.hpp"

namespace moe {

MOE_FFN_FORMAT_LAUNCHERS(extern template, kFp8)
MOE_FFN_FORMAT_LAUNCHERS(extern template, kNvfp4)
MOE_FFN_FORMAT_LAUNCHERS(extern template, kInt8Row)
MOE_FFN_FORMAT_LAUNCHERS(extern template, kInt4Row)
MOE_FFN_FORMAT_LAUNCHERS(extern template, kInt4G64)
MOE_FFN_FORMAT_LAUNCHERS(extern template, kFp8Bf16s)

__device__ __forceinline__ float blend_value(const FfnArgs &a, int r, int o) {
    float d[kMaxSlots];
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j)
        if (j < a.k) d[j] = a.dbuf[(size_t)(r * a.k + j) * a.H + o];
    const float ds = a.shared.inter > 0 ? a.dbuf[(size_t)(a.R * a.k + r) * a.H + o] : 0.0f;
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
        if (j < a.k) {
            const int i = r * a.k + j;
            const int e = a.ids[i];
            const float t = fmaf(a.w[i], d[j], y);
            y = (e >= 0 && e < a.E) ? t : y;
        }
    }
    if (a.shared.inter > 0) y = fmaf(a.s[r], ds, y);
    return y;
}

// ... then the residual add and bf16 rounding.
__global__ __launch_bounds__(256) void k_blend(FfnArgs a) {
    const int o = blockIdx.x * 256 + threadIdx.x;
    const int r = blockIdx.y;
    if (o >= a.H) return;
    store_out(a.y, a.res, a.ldy, r, o, blend_value(a, r, o));
}

// The same with the RMSNorm epilogue: one workgroup per row (the norm needs
// the whole row); the normalised row is the residual after the add (the
// output y without a residual).  The row's routing is read once, and each
// thread loads a batch of columns' down outputs before using any.
__global__ __launch_bounds__(256) void k_blend_norm(FfnArgs a) {
    extern __shared__ float vrow[];   // [2H]: the row, then the staged weight
    __shared__ int ids_s[kMaxSlots];
    __shared__ float w_s[kMaxSlots];
    const int r = blockIdx.x;
    if (threadIdx.x < a.k) {
        ids_s[threadIdx.x] = a.ids[r * a.k + threadIdx.x];
        w_s[threadIdx.x] = a.w[r * a.k + threadIdx.x];
    }
    __syncthreads();
    const bool sh = a.shared.inter > 0;
    const float sr = sh ? a.s[r] : 0.0f;
    for (int o0 = threadIdx.x; o0 < a.H; o0 += 256 * kNormBatch) {
        float y[kNormBatch];
#pragma unroll
        for (int u = 0; u < kNormBatch; ++u) y[u] = 0.0f;
        for (int j = 0; j < a.k; ++j) {
            const int e = ids_s[j];
            const bool ok = e >= 0 && e < a.E;
            const float *d = a.dbuf + (size_t)(r * a.k + j) * a.H;
            float t[kNormBatch];
#pragma unroll
            for (int u = 0; u < kNormBatch; ++u) {
                const int o = o0 + 256 * u;
                t[u] = d[o < a.H ? o : a.H - 1];
            }
#pragma unroll
            for (int u = 0; u < kNormBatch; ++u) {
                const float v = fmaf(w_s[j], t[u], y[u]);
                y[u] = ok ? v : y[u];
            }
        }
        if (sh) {
            const float *d = a.dbuf + (size_t)(a.R * a.k + r) * a.H;
            float t[kNormBatch];
#pragma unroll
            for (int u = 0; u < kNormBatch; ++u) {
                const int o = o0 + 256 * u;
                t[u] = d[o < a.H ? o : a.H - 1];
            }
#pragma unroll
            for (int u = 0; u < kNormBatch; ++u) y[u] = fmaf(sr, t[u], y[u]);
        }
        uint16_t rin[kNormBatch];
#pragma unroll
        for (int u = 0; u < kNormBatch; ++u) {
            const int o = o0 + 256 * u;
            rin[u] = a.res ? a.res[(size_t)r * a.ldy + (o < a.H ? o : a.H - 1)] : (uint16_t)0;
        }
#pragma unroll
        for (int u = 0; u < kNormBatch; ++u) {
            const int o = o0 + 256 * u;
            if (o >= a.H) continue;
            const uint16_t yb = f32_to_bf16(y[u]);
            uint16_t src = yb;
            if (a.y) a.y[(size_t)r * a.ldy + o] = yb;
            if (a.res) {
                src = f32_to_bf16(bf16_to_f32(rin[u]) + y[u]);
                a.res[(size_t)r * a.ldy + o] = src;
            }
            vrow[o] = bf16_to_f32(src);
        }
    }
    __syncthreads();
    block_rms_norm(vrow, a.H, a.norm_w, a.norm_eps, a.norm_out + (size_t)r * a.ldn);
}

// The RMSNorm epilogue alone, on rows a previous launch wrote (one workgroup
// per row).
__global__ __launch_bounds__(256) void k_rmsnorm(FfnArgs a) {
    extern __shared__ float vrow[];   // [2H]
    const int r = blockIdx.x;
    stage_row<false>((a.res ? a.res : a.y) + (size_t)r * a.ldy, a.H, vrow);
    block_rms_norm(vrow, a.H, a.norm_w, a.norm_eps, a.norm_out + (size_t)r * a.ldn);
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

// One instantiation per weight format: FN<FMT>(args...).
#define MOE_FMT_DISPATCH(FMT_VALUE, FN, ...)                                                      \
    do {                                                                                          \
        switch (FMT_VALUE) {                                                                      \
            case kFp8: return FN<kFp8>(__VA_ARGS__);                                              \
            case kNvfp4: return FN<kNvfp4>(__VA_ARGS__);                                          \
            case kInt8Row: return FN<kInt8Row>(__VA_ARGS__);                                      \
            case kInt4Row: return FN<kInt4Row>(__VA_ARGS__);                                      \
            case kInt4G64: return FN<kInt4G64>(__VA_ARGS__);                                      \
            case kFp8Bf16s: return FN<kFp8Bf16s>(__VA_ARGS__);                                    \
            default: return hipErrorInvalidValue;                                                 \
        }                                                                                         \
    } while (0)

hipError_t launch_gate_up(const FfnArgs &a, hipStream_t st) {
    MOE_FMT_DISPATCH(a.fmt, gate_up_fmt, a, st);
}

hipError_t launch_lead_r1(const RouteArgs &r, const FfnArgs &a, hipStream_t st) {
    MOE_FMT_DISPATCH(a.fmt, lead_nch, r, a, st);
}

hipError_t launch_gate_up_r1(const FfnArgs &a, hipStream_t st) {
    MOE_FMT_DISPATCH(a.fmt, gate_up_r1_fmt, a, st);
}

hipError_t launch_down_blend_r1(const FfnArgs &a, hipStream_t st) {
    MOE_FMT_DISPATCH(a.fmt, down_r1_fmt, a, st);
}

hipError_t launch_down_grouped(const FfnArgs &a, hipStream_t st) {
    MOE_FMT_DISPATCH(a.fmt, down_grouped_fmt, a, st);
}

hipError_t launch_blend(const FfnArgs &a, hipStream_t st) {
    if (a.norm_w)
        hipLaunchKernelGGL(k_blend_norm, dim3(a.R), dim3(256), (size_t)a.H * 8, st, a);
    else
        hipLaunchKernelGGL(k_blend, dim3((a.H + 255) / 256, a.R), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const FfnArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_rmsnorm, dim3(a.R), dim3(256), (size_t)a.H * 8, st, a);
    return hipGetLastError();
}

hipError_t launch_decode_probe(int fmt, const uint8_t *codes, float *out, int n, hipStream_t st) {
    const int threads = (n + 3) / 4;
    hipLaunchKernelGGL(k_decode_probe, dim3((threads + 255) / 256), dim3(256), 0, st, fmt, codes, out, n);
    return hipGetLastError();
}

}  // namespace moe
