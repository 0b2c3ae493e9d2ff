// gemv.hpp -- the per-wave building blocks every kernel is made of: a bf16
// router row, the wave64 top-k softmax, the fp8 / nvfp4 weight chunks of the
// gate/up and down GEMVs.  Kernels that compute the same quantity call the
// same function, so the fused one-row kernels and the generic multi-row
// kernels give bit-identical values.
#pragma once

#include "device.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace moe {


constexpr int kPairsPerWave = 2;       // gate/up (i, I+i) row pairs per wave

__device__ __forceinline__ float sigmoid(float t) { return 1.0f / (1.0f + expf(-t)); }

// ------------------------------------------------------------------ router

// One bf16 router row (H values, resident in registers as NCH 16-byte chunks
// per lane) dotted with activation row xr: the lane-strided chunks, fdot2
// with f32 accumulation, a wave sum.
// Every load below is unconditional, from a clamped chunk index, with the
// bounds applied to the value: a load under a per-lane condition compiles to
// a branch that waits for it, which serialises the loads.
template <int NCH>
__device__ __forceinline__ void load_bf16_row(const uint16_t *row, int H, u32x4 (&wv)[NCH]) {
    const int lane = threadIdx.x & (kWave - 1), nch = H >> 3;
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
        const int c = lane + kWave * t;
        const u32x4 v = ld16_stream(row + (size_t)(c < nch ? c : nch - 1) * 8);
        wv[t] = c < nch ? v : u32x4{0u, 0u, 0u, 0u};
    }
}
template <int NCH>
__device__ __forceinline__ float dot_bf16_row(const u32x4 (&wv)[NCH], const uint16_t *xr, int H) {
    const int lane = threadIdx.x & (kWave - 1), nch = H >> 3;
    u32x4 xv[NCH];
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
        const int c = lane + kWave * t;
        xv[t] = ld16(xr + (size_t)(c < nch ? c : nch - 1) * 8);
    }
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
        const int c = lane + kWave * t;
        if (c < nch) acc = dot8_bf16(wv[t], xv[t], acc);
    }
    return group_sum<kWave>(acc);
}

// x_r . w with the bits of load_bf16_row<16> + dot_bf16_row<16> (the same
// lane-strided chunks in the same order, the same wave sum), four chunks per
// lane in flight instead of sixteen held in registers.  In two parts, so a
// caller can issue the first four chunks' loads (all of them for H <= 2048)
// ahead of other work: row_stream_head, then row_stream_dot.
struct RowStreamHead {
    u32x4 wv[4], xv[4];
};
__device__ __forceinline__ void row_stream_load(const uint16_t *wrow, const uint16_t *xr, int nch, int t0,
                                                RowStreamHead &q) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int c = lane + kWave * (t0 + t), cc = c < nch ? c : nch - 1;
        q.wv[t] = ld16_stream(wrow + (size_t)cc * 8);
        q.xv[t] = ld16(xr + (size_t)cc * 8);
    }
}
__device__ __forceinline__ void row_stream_head(const uint16_t *wrow, const uint16_t *xr, int H, RowStreamHead &q) {
    row_stream_load(wrow, xr, H >> 3, 0, q);
}
__device__ __forceinline__ float row_stream_dot(RowStreamHead &q, const uint16_t *wrow, const uint16_t *xr, int H) {
    const int lane = threadIdx.x & (kWave - 1), nch = H >> 3;
    float acc = 0.0f;
#pragma unroll
    for (int t0 = 0; t0 < 16; t0 += 4) {
        if (kWave * t0 >= nch) break;
        if (t0 > 0) row_stream_load(wrow, xr, nch, t0, q);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (lane + kWave * (t0 + t) < nch) acc = dot8_bf16(q.wv[t], q.xv[t], acc);
    }
    return group_sum<kWave>(acc);
}
__device__ __forceinline__ float dot_bf16_row_stream(const uint16_t *wrow, const uint16_t *xr, int H) {
    RowStreamHead q;
    row_stream_head(wrow, xr, H, q);
    return row_stream_dot(q, wrow, xr, H);
}

// ------------------------------------------------------------------ top-k

__device__ __forceinline__ float ld_agent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int ld_agent(const int *p) {
    return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_agent(const unsigned *p) {
    return __hip_atomic_load(const_cast<unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A logit as an order-preserving unsigned 32-bit key (larger value, larger
// key; -0 and +0 share one key, NaN counts as -inf).  Key 0 sorts below
// every real logit.
__device__ __forceinline__ uint32_t logit_key(float v) {
    v = v != v ? -__builtin_inff() : (v == 0.0f ? 0.0f : v);
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Largest (smallest) unsigned value of the wave, uniform: row stages by DPP,
// then the two lane swaps.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
    const int id = MAX ? 0 : -1;
    auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, (uint32_t)dpp<kDppXor1>(id, (int)v));
    v = op(v, (uint32_t)dpp<kDppXor2>(id, (int)v));
    v = op(v, (uint32_t)dpp<kDppHalfMirror>(id, (int)v));
    v = op(v, (uint32_t)dpp<kDppMirror>(id, (int)v));
    float x, y;
    lane_swap<16>(__uint_as_float(v), __uint_as_float(v), x, y);
    v = op(__float_as_uint(x), __float_as_uint(y));
    lane_swap<32>(__uint_as_float(v), __uint_as_float(v), x, y);
    v = op(__float_as_uint(x), __float_as_uint(y));
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Per lane: b where bit `lane` of the wave mask m is set, else a.  (Chains
// of selects on one lane-index test compile into longer code than these
// mask tests.)
__device__ __forceinline__ uint32_t lane_select(uint32_t a, uint32_t b, uint64_t m) {
    return ((m >> (threadIdx.x & (kWave - 1))) & 1ull) ? b : a;
}

// Largest unsigned value of the wave, uniform: DPP row stages, the two row
// broadcasts carry it into lane 63, which is read out.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    v = mx(v, (uint32_t)dpp<kDppXor1>(0, (int)v));
    v = mx(v, (uint32_t)dpp<kDppXor2>(0, (int)v));
    v = mx(v, (uint32_t)dpp<kDppHalfMirror>(0, (int)v));
    v = mx(v, (uint32_t)dpp<kDppMirror>(0, (int)v));
    v = mx(v, (uint32_t)dpp<kDppBcast15, 0xa>(0, (int)v));
    v = mx(v, (uint32_t)dpp<kDppBcast31, 0xc>(0, (int)v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// The k largest of the wave's keys (key[i] of lane l: expert l + 64 i, key
// 0 for none) under the top-k order, by rounds: each lane's keys sorted
// once, stable, with their positions packed four bits each into `perm`;
// every round the wave takes the largest lane head by a 32-bit wave max, the
// lane holding it (the lowest expert index among equal heads: a second,
// rarely taken pass) pops its head.  Lane j < k gets round j's key and
// expert.  The general path of topk_regs (any number of ties).
template <int NV>
__device__ __forceinline__ void topk_rounds(uint32_t (&key)[NV], int k, int &sel_key, int &sel_idx) {
    using Perm = typename std::conditional<(NV <= 8), uint32_t, uint64_t>::type;
    const int lane = threadIdx.x & (kWave - 1);
    int pos[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) pos[i] = i;
    // stable sort by key, descending: equal keys keep ascending index
#pragma unroll
    for (int i = 1; i < NV; ++i) {
#pragma unroll
        for (int j = i; j > 0; --j) {
            const bool sw = key[j] > key[j - 1];
            const uint32_t ka = key[j - 1], kb = key[j];
            const int ia = pos[j - 1], ib = pos[j];
            key[j - 1] = sw ? kb : ka;
            key[j] = sw ? ka : kb;
            pos[j - 1] = sw ? ib : ia;
            pos[j] = sw ? ia : ib;
        }
    }
    Perm perm = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) perm |= (Perm)pos[i] << (4 * i);
    sel_key = 0;
    sel_idx = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t best = wave_max_u32(key[0]);
        uint64_t hit = __builtin_amdgcn_ballot_w64(key[0] == best);
        if (__builtin_popcountll(hit) > 1) {
            const uint32_t head = (uint32_t)lane + kWave * (uint32_t)(perm & 15);
            const uint32_t least = wave_ext_u32<false>(key[0] == best ? head : 0xffffffffu);
            hit = __builtin_amdgcn_ballot_w64(key[0] == best && head == least);
        }
        const int wl = __builtin_ctzll(hit);
        const int bi = wl + kWave * (__builtin_amdgcn_readlane((int)(uint32_t)perm, wl) & 15);
        // lane wl pops its head; lane j takes the round's key and expert
        const uint64_t pop = 1ull << wl, put = 1ull << j;
        key[0] = lane == wl ? (NV > 1 ? key[1] : 0u) : key[0];
#pragma unroll
        for (int i = 1; i + 1 < NV; ++i) key[i] = lane_select(key[i], key[i + 1], pop);
        if constexpr (NV > 1) key[NV - 1] = lane_select(key[NV - 1], 0u, pop);
        if constexpr (NV > 1) {
            if constexpr (NV <= 8) {
                perm = lane_select((uint32_t)perm, (uint32_t)perm >> 4, pop);
            } else {
                const Perm sh = perm >> 4;
                perm = (Perm)lane_select((uint32_t)perm, (uint32_t)sh, pop) |
                       ((Perm)lane_select((uint32_t)(perm >> 32), (uint32_t)(sh >> 32), pop) << 32);
            }
        }
        sel_key = (int)lane_select((uint32_t)sel_key, best, put);
        sel_idx = (int)lane_select((uint32_t)sel_idx, (uint32_t)bi, put);
    }
}

// Lanes below bit `lane` set in m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// LDS words (64-bit) one selecting wave uses in topk_regs: the packed
// candidates and their zero padding in [0, kTopkOut), the selected ones in
// [kTopkOut, kTopkOut + kMaxTopK).
constexpr int kTopkOut = 80;
constexpr int kTopkLds = kTopkOut + kMaxTopK;

// Per-wave top-k scratch of a kernel whose waves 0 .. MAXW-1 may select at
// the same time (16-byte aligned; one array per kernel and MAXW).
template <int MAXW>
__device__ __forceinline__ uint64_t *topk_lds(int wave) {
    __shared__ __attribute__((aligned(16))) uint64_t words[MAXW * kTopkLds];
    return words + wave * kTopkLds;
}

// Softmax over the E logits of one row, the k largest under the top-k order
// (larger value first, lower index first among equal values) and their
// renormalised weights, by one wave (all 64 lanes active).
//
// Selection: split the lanes into G >= k groups and take T, the smallest of
// the G group maxima (for 8 < k < 16: the k-th largest of the 16 maxima).
// Those are G (k) distinct experts with keys >= T, so the k-th largest key
// is >= T and every expert of the top-k is a candidate (key >= T).  The candidates (usually a few times k) are written, as 64-bit
// order keys (key, then the complemented expert index: distinct, larger
// first in the top-k order), to consecutive words of the wave's LDS scratch
// (a ballot prefix gives each its word); each candidate's rank is the number
// of candidates with a larger order key, counted by every lane against the
// whole list read back as broadcasts (every lane reads the same words); the
// candidate of rank j < k is written to output word j, which lane j reads.
// More than 64 candidates (mass ties) take the round-by-round path.
// The wave's LDS accesses execute in issue order, so no wait separates the
// writes from the reads; the compiler barriers keep their program order.
// w_j = exp(l_j - m) / sum_j exp(l_j - m), m the largest logit: the softmax
// denominator over all E cancels in the renormalisation.  Lane j < k returns
// slot j.  raw[i] is the logit of expert lane + 64 i (entries past E unused);
// scr is this wave's kTopkLds words of LDS (16-byte aligned).
template <int NV>
__device__ __forceinline__ void topk_regs(const float (&raw)[NV], int E, int k, uint64_t *scr, int &my_e,
                                          float &my_w) {
    static_assert(NV >= 1 && NV <= 16, "logits per lane");
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t key[NV];
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        key[i] = e < E ? logit_key(raw[i]) : 0u;
        lmax = key[i] > lmax ? key[i] : lmax;
    }
    // group maxima (8 lanes a group for k <= 8, else 4), then their minimum
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
    uint32_t g = lmax;
    g = mx(g, (uint32_t)dpp<kDppXor1>(0, (int)g));
    g = mx(g, (uint32_t)dpp<kDppXor2>(0, (int)g));
    uint32_t thr;
    if (k > 8 && k < 16) {
        // T = the k-th largest of the 16 group maxima (lane 4h holds group
        // h's; ties ranked by group index): k distinct experts are >= T, and
        // T is much tighter than the smallest maximum (about 15 candidates
        // against 50 at 512 experts, top-10)
        const int gi = lane >> 2;
        int rank = 0;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)g, 4 * h);
            rank += (o > g || (o == g && h < gi)) ? 1 : 0;
        }
        const uint64_t at = __builtin_amdgcn_ballot_w64(rank == k - 1 && (lane & 3) == 0);
        thr = (uint32_t)__builtin_amdgcn_readlane((int)g, __builtin_ctzll(at));
    } else {
        if (k <= 8) {
            g = mx(g, (uint32_t)dpp<kDppHalfMirror>(0, (int)g));
        } else {
            g = mn(g, (uint32_t)dpp<kDppHalfMirror>(-1, (int)g));
        }
        g = mn(g, (uint32_t)dpp<kDppMirror>(-1, (int)g));
        g = mn(g, (uint32_t)dpp<kDppBcast15, 0xa>(-1, (int)g));
        g = mn(g, (uint32_t)dpp<kDppBcast31, 0xc>(-1, (int)g));
        thr = (uint32_t)__builtin_amdgcn_readlane((int)g, kWave - 1);
    }
    uint64_t cm[NV];
    int cn = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        cm[i] = __builtin_amdgcn_ballot_w64(key[i] >= thr && key[i] != 0u);
        cn += __builtin_popcountll(cm[i]);
    }
    int sel_key, sel_idx;
    if (cn <= kWave) {
        int base = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if ((cm[i] >> lane) & 1ull)
                scr[base + lanes_below(cm[i])] = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(lane + kWave * i);
            base += __builtin_popcountll(cm[i]);
        }
        // zeros after the list up to the next multiple of 8 (precede nothing)
        if (lane < 8) scr[cn + lane] = 0ull;
        asm volatile("" ::: "memory");
        const uint64_t me = scr[lane];
        typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
        const u64x2 *list = reinterpret_cast<const u64x2 *>(scr);
        int r0 = 0, r1 = 0;
        for (int q = 0; q < cn; q += 8) {
            u64x2 o[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] = list[q / 2 + u];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                r0 += o[u].x > me ? 1 : 0;
                r1 += o[u].y > me ? 1 : 0;
            }
        }
        const int rank = r0 + r1;
        asm volatile("" ::: "memory");
        if (lane < cn && rank < k) scr[kTopkOut + rank] = me;
        asm volatile("" ::: "memory");
        const uint64_t sel = scr[kTopkOut + (lane < k ? lane : 0)];
        sel_key = (int)(uint32_t)(sel >> 32);
        sel_idx = (int)~(uint32_t)sel;
    } else {
        topk_rounds<NV>(key, k, sel_key, sel_idx);
    }
    const float v = key_logit((uint32_t)sel_key);
    const float m = readlane(v, 0);
    const float ex = lane < k ? expf(v - m) : 0.0f;
    const float sum = group_sum<kWave>(ex);
    my_e = (lane < k && sel_idx >= 0 && sel_idx < E) ? sel_idx : 0;
    my_w = ex / sum;
}

// The same from logits in memory; `coherent` reads them with agent-scope
// loads (written by other workgroups of the same launch).
template <int NV>
__device__ __forceinline__ void load_logits(const float *l, int E, bool coherent, float (&raw)[NV]) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + kWave * i;
        const int ec = e < E ? e : E - 1;
        raw[i] = coherent ? ld_agent(l + ec) : l[ec];
    }
}
template <int NV>
__device__ __forceinline__ void topk_wave(const float *l, int E, int k, bool coherent, uint64_t *scr, int &my_e,
                                          float &my_w) {
    float raw[NV];
    load_logits<NV>(l, E, coherent, raw);
    topk_regs<NV>(raw, E, k, scr, my_e, my_w);
}

// Logits per lane for E experts: 1, 2, 4, 8 or 16.
__host__ __device__ constexpr int topk_nv(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

// ------------------------------------------------------------------ RMSNorm epilogue

// Columns a 256-thread block loads per batch of the norm epilogue: eight per
// thread, issued before any is used (a loop that used each load at once
// would pay the memory latency once per column).
constexpr int kNormBatch = 8;

// out[o] = bf16(v[o] * rsqrt(mean v^2 + eps) * gamma[o]) for one row whose
// f32 values v (already bf16-rounded) are in LDS, with room for H more
// floats after them (the weight is staged there); every thread of the block
// (256 to 1024 threads) calls it.  The sum of squares runs in one fixed order
// whatever the block size: threads 0..255 each over the columns t, t + 256,
// ..., the wave sum, then the four waves in order (further waves add zero),
// so the result does not depend on timing or on the calling kernel.
__device__ __forceinline__ void block_rms_norm(float *v, int H, const uint16_t *gamma, float eps, uint16_t *out) {
    __shared__ float part[16];
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x >> 6, nt = blockDim.x;
    float *gs = v + H;
    for (int o0 = threadIdx.x; o0 < H; o0 += nt * kNormBatch) {
        uint16_t t[kNormBatch];
#pragma unroll
        for (int u = 0; u < kNormBatch; ++u) {
            const int o = o0 + nt * u;
            t[u] = gamma[o < H ? o : H - 1];
        }
#pragma unroll
        for (int u = 0; u < kNormBatch; ++u) {
            const int o = o0 + nt * u;
            if (o < H) gs[o] = bf16_to_f32(t[u]);
        }
    }
    float ss = 0.0f;
    if (threadIdx.x < 256)
        for (int o = threadIdx.x; o < H; o += 256) ss = fmaf(v[o], v[o], ss);
    ss = group_sum<kWave>(ss);
    if (lane == 0) part[wid] = ss;
    __syncthreads();
    float tot = ((part[0] + part[1]) + part[2]) + part[3];
    for (int w = 4; w < nt / kWave; ++w) tot += part[w];
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    for (int o = threadIdx.x; o < H; o += nt) out[o] = f32_to_bf16(v[o] * r * gs[o]);
    __syncthreads();
}

// Stage a bf16 row into LDS as f32, kNormBatch loads in flight per thread
// (COHERENT: agent-scope loads of values other workgroups of the launch wrote).
template <bool COHERENT>
__device__ __forceinline__ void stage_row(const uint16_t *src, int H, float *v) {
    const int nt = blockDim.x;
    for (int o0 = threadIdx.x; o0 < H; o0 += nt * kNormBatch) {
        uint16_t t[kNormBatch];
#pragma unroll
        for (int u = 0; u < kNormBatch; ++u) {
            const int o = o0 + nt * u;
            const int oc = o < H ? o : H - 1;
            if constexpr (COHERENT)
                t[u] = __hip_atomic_load(const_cast<uint16_t *>(src + oc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                t[u] = src[oc];
        }
#pragma unroll
        for (int u = 0; u < kNormBatch; ++u) {
            const int o = o0 + nt * u;
            if (o < H) v[o] = bf16_to_f32(t[u]);
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------------ weight chunks

template <int FMT> __device__ __forceinline__ int row_bytes(int cols) { return fmt_row_bytes(FMT, cols); }
template <int FMT> constexpr int cols_per_chunk() { return byte_codes(FMT) ? 16 : 32; }

// Scale(s) of 16-byte chunk `c` of weight row `row` of a matrix with `cols`
// columns.  fp8: one f32 (or bf16) per 128x128 block; nvfp4: two e4m3 bytes (two
// 16-column groups); int8/int4 per row: the row's f32; int4-g64: the f32 of
// the 64-column group holding the chunk's 32 columns.
// The stored bits of a chunk's scale (a float, a bf16 or two e4m3 bytes),
// loaded as they are and decoded by scale_of where the chunk is used: a
// conversion right after the load would wait for it there, and the loads of
// a unit's rows (or of a row's slots) would then go out one at a time.
template <int FMT>
__device__ __forceinline__ uint32_t chunk_scale_raw(const uint8_t *s, int row, int cols, int c) {
    const uint32_t *sf = reinterpret_cast<const uint32_t *>(s);
    if constexpr (FMT == kFp8) {
        return sf[(size_t)(row >> 7) * (cols >> 7) + ((c * 16) >> 7)];
    } else if constexpr (FMT == kFp8Bf16s) {
        const uint16_t *sb = reinterpret_cast<const uint16_t *>(s);
        return sb[(size_t)(row >> 7) * (cols >> 7) + ((c * 16) >> 7)];
    } else if constexpr (FMT == kNvfp4) {
        return *reinterpret_cast<const uint16_t *>(s + (size_t)row * (cols >> 4) + 2 * c);
    } else if constexpr (FMT == kInt4G64) {
        return sf[(size_t)row * (cols >> 6) + (c >> 1)];
    } else {
        return sf[row];
    }
}
template <int FMT>
__device__ __forceinline__ f32x2 scale_of(uint32_t raw) {
    if constexpr (FMT == kFp8Bf16s) {
        const float v = bf16_to_f32((uint16_t)raw);
        return f32x2{v, v};
    } else if constexpr (FMT == kNvfp4) {
        return f32x2{e4m3_f32(raw, 0), e4m3_f32(raw, 1)};
    } else {
        const float v = __uint_as_float(raw);
        return f32x2{v, v};
    }
}
template <int FMT>
__device__ __forceinline__ f32x2 chunk_scale(const uint8_t *s, int row, int cols, int c) {
    const float *sf = reinterpret_cast<const float *>(s);
    if constexpr (FMT == kFp8) {
        const float v = sf[(size_t)(row >> 7) * (cols >> 7) + ((c * 16) >> 7)];
        return f32x2{v, v};
    } else if constexpr (FMT == kFp8Bf16s) {
        const uint16_t *sb = reinterpret_cast<const uint16_t *>(s);
        const float v = bf16_to_f32(sb[(size_t)(row >> 7) * (cols >> 7) + ((c * 16) >> 7)]);
        return f32x2{v, v};
    } else if constexpr (FMT == kNvfp4) {
        const uint16_t b = *reinterpret_cast<const uint16_t *>(s + (size_t)row * (cols >> 4) + 2 * c);
        return f32x2{e4m3_f32(b, 0), e4m3_f32(b, 1)};
    } else if constexpr (FMT == kInt4G64) {
        const float v = sf[(size_t)row * (cols >> 6) + (c >> 1)];
        return f32x2{v, v};
    } else {
        const float v = sf[row];
        return f32x2{v, v};
    }
}

// 16-byte loads of activation per weight chunk: bf16 (gate/up) and f32 (down).
template <int FMT> constexpr int x_quads() { return byte_codes(FMT) ? 2 : 4; }
template <int FMT> constexpr int h_quads() { return byte_codes(FMT) ? 4 : 8; }

// One 16-byte weight chunk . the chunk's bf16 activations (in registers).
template <int FMT>
__device__ __forceinline__ float chunk_dot_bf16(u32x4 w, f32x2 sc, const u32x4 (&x)[x_quads<FMT>()]) {
    if constexpr (fp8_block(FMT)) {
        return sc.x * dot16_e4m3_bf16(w, x[0], x[1]);
    } else if constexpr (FMT == kInt8Row) {
        return sc.x * dot16_i8_bf16(w, x[0], x[1]);
    } else if constexpr (FMT == kNvfp4) {
        float a = dot8_e2m1_bf16(w.x, x[0], 0.0f);
        a = dot8_e2m1_bf16(w.y, x[1], a);
        float b = dot8_e2m1_bf16(w.z, x[2], 0.0f);
        b = dot8_e2m1_bf16(w.w, x[3], b);
        return sc.x * a + sc.y * b;
    } else {
        float a = dot8_i4_bf16(w.x, x[0], 0.0f);
        a = dot8_i4_bf16(w.y, x[1], a);
        a = dot8_i4_bf16(w.z, x[2], a);
        a = dot8_i4_bf16(w.w, x[3], a);
        return sc.x * a;
    }
}
template <int FMT>
__device__ __forceinline__ void load_x_chunk(const uint16_t *xp, u32x4 (&x)[x_quads<FMT>()]) {
#pragma unroll
    for (int q = 0; q < x_quads<FMT>(); ++q) x[q] = ld16(xp + 8 * q);
}
// ... with the activations at xp (the chunk's first column).
template <int FMT>
__device__ __forceinline__ float chunk_dot_bf16(u32x4 w, f32x2 sc, const uint16_t *xp) {
    u32x4 x[x_quads<FMT>()];
    load_x_chunk<FMT>(xp, x);
    return chunk_dot_bf16<FMT>(w, sc, x);
}

// One 16-byte weight chunk . the chunk's f32 activations (in registers).
template <int FMT>
__device__ __forceinline__ float chunk_dot_f32(u32x4 w, f32x2 sc, const f32x4 (&h)[h_quads<FMT>()]) {
    if constexpr (fp8_block(FMT)) {
        return sc.x * dot16_e4m3_f32(w, h);
    } else if constexpr (FMT == kInt8Row) {
        return sc.x * dot16_i8_f32(w, h);
    } else if constexpr (FMT == kNvfp4) {
        float a = dot8_e2m1_f32(w.x, h[0], h[1], 0.0f);
        a = dot8_e2m1_f32(w.y, h[2], h[3], a);
        float b = dot8_e2m1_f32(w.z, h[4], h[5], 0.0f);
        b = dot8_e2m1_f32(w.w, h[6], h[7], b);
        return sc.x * a + sc.y * b;
    } else {
        float a = dot8_i4_f32(w.x, h[0], h[1], 0.0f);
        a = dot8_i4_f32(w.y, h[2], h[3], a);
        a = dot8_i4_f32(w.z, h[4], h[5], a);
        a = dot8_i4_f32(w.w, h[6], h[7], a);
        return sc.x * a;
    }
}
// ... with the activations at hp (global or LDS).
template <int FMT>
__device__ __forceinline__ float chunk_dot_f32(u32x4 w, f32x2 sc, const float *hp) {
    const f32x4 *h4 = reinterpret_cast<const f32x4 *>(hp);
    f32x4 h[h_quads<FMT>()];
#pragma unroll
    for (int q = 0; q < h_quads<FMT>(); ++q) h[q] = h4[q];
    return chunk_dot_f32<FMT>(w, sc, h);
}

template <int FMT> __device__ __forceinline__ float global_scale(const float *g, int e) {
    return FMT == kNvfp4 ? g[e] : 1.0f;
}

// ------------------------------------------------------------------ gate/up

// The 2P gate/up rows (i0+p, I+i0+p) of expert e held by one wave: CH
// lane-strided 16-byte chunks per row, with their scales.
template <int FMT, int CH, int P>
struct GateUpRows {
    // fp8: the P gate rows (and the P up rows) sit in one 128-row scale
    // block (i0 is a multiple of P, which divides 128), so one scale per
    // chunk serves each half; the other formats' scales are per row.
    static constexpr int NS = fp8_block(FMT) ? 2 : 2 * P;
    static_assert(128 % P == 0, "pairs per wave must divide the scale block");
    u32x4 w[2 * P][CH];
    f32x2 sc[NS][CH];
    float g;

    __device__ __forceinline__ static constexpr int sidx(int q) { return fp8_block(FMT) ? (q & 1) : q; }

    __device__ __forceinline__ void load(const ExpertSet &X, int e, int i0, int H) {
        const int lane = threadIdx.x & (kWave - 1);
        const int I = X.inter, rb = row_bytes<FMT>(H), nch = rb >> 4;
        const uint8_t *wbase = X.gu + (size_t)e * X.gu_stride;
        const uint8_t *sbase = X.gu_s + (size_t)e * X.gu_s_stride;
#pragma unroll
        for (int q = 0; q < 2 * P; ++q) {
            const int p = q >> 1;
            const bool live = i0 + p < I;
            const int row = ((q & 1) ? I : 0) + (live ? i0 + p : i0);
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int ch = lane + kWave * c;
                const u32x4 v = ld16_stream(wbase + (size_t)row * rb + (size_t)(ch < nch ? ch : nch - 1) * 16);
                w[q][c] = (live && ch < nch) ? v : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int p = q >> 1;
            const bool live = i0 + p < I;
            const int row = ((q & 1) ? I : 0) + (live ? i0 + p : i0);
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int ch = lane + kWave * c;
                const f32x2 v = chunk_scale<FMT>(sbase, row, H, ch < nch ? ch : nch - 1);
                sc[q][c] = (live && ch < nch) ? v : f32x2{0.0f, 0.0f};
            }
        }
        g = global_scale<FMT>(X.gu_g, e);
    }

    // Per-lane partial sums of the 2P rows (gate p at 2p, up p at 2p+1)
    // against the lane's activation chunks x[c] (chunk lane + 64c).
    __device__ __forceinline__ void partial(const u32x4 (&x)[CH][x_quads<FMT>()], int H, float (&acc)[2 * P]) const {
        const int lane = threadIdx.x & (kWave - 1), nch = row_bytes<FMT>(H) >> 4;
#pragma unroll
        for (int q = 0; q < 2 * P; ++q) acc[q] = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (lane + kWave * c < nch) {
#pragma unroll
                for (int q = 0; q < 2 * P; ++q) acc[q] += chunk_dot_bf16<FMT>(w[q][c], sc[sidx(q)][c], x[c]);
            }
        }
    }

    // The lane's activation chunks of row xr.
    __device__ __forceinline__ static void load_x(const uint16_t *xr, int H, u32x4 (&x)[CH][x_quads<FMT>()]) {
        const int lane = threadIdx.x & (kWave - 1), nch = row_bytes<FMT>(H) >> 4;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = lane + kWave * c;   // chunks past the row are loaded clamped, never used
            load_x_chunk<FMT>(xr + (size_t)(ch < nch ? ch : nch - 1) * cols_per_chunk<FMT>(), x[c]);
        }
    }

    // Reduce the partials over the wave (pair p ends in lanes
    // [p * 64/P, (p+1) * 64/P)) and write h[i0 + p] = silu(g) * u.  Plain:
    // the first lane of the pair's span writes.  COHERENT (another workgroup
    // of the same launch reads it): the value is written at agent scope
    // (write-through) into `nrep` replicas `rep` floats apart, lane c of the
    // span writing replica c.
    template <bool COHERENT = false>
    __device__ __forceinline__ void finish(float (&acc)[2 * P], int I, int i0, float *hrow, size_t rep = 0,
                                           int nrep = 1) const {
        constexpr int SPAN = kWave / P;
        const int lane = threadIdx.x & (kWave - 1);
        xreduce<kWave, P, 2>(acc);
        const int p = lane / SPAN, copy = lane % SPAN;
        if (i0 + p >= I) return;
        const float hv = silu_mul(acc[0] * g, acc[1] * g);
        if (COHERENT) {
            if (copy < nrep)
                __hip_atomic_store(hrow + (size_t)copy * rep + i0 + p, hv, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else if (copy == 0) {
            hrow[i0 + p] = hv;
        }
    }

    // h[i0 + p] = silu(g) * u for activation row xr.
    template <bool COHERENT = false>
    __device__ __forceinline__ void apply(const uint16_t *xr, int H, int I, int i0, float *hrow,
                                          size_t rep = 0, int nrep = 1) const {
        u32x4 x[CH][x_quads<FMT>()];
        load_x(xr, H, x);
        float acc[2 * P];
        partial(x, H, acc);
        finish<COHERENT>(acc, I, i0, hrow, rep, nrep);
    }
};

// ------------------------------------------------------------------ down

// Row o of expert e's down matrix as seen by one lane of its LPR-lane row
// group: CH chunks (lane-strided by LPR) with their scales.
//
// RAW: keep each chunk's scale as its stored bits, loaded unconditionally
// from a clamped position and decoded where used (the per-row down kernel:
// its NVFP4 rows otherwise load one slot at a time, each scale conversion
// waiting for its load); otherwise decode at the load, masked (the one-launch
// layer measured faster so).
template <int FMT, int LPR, int CH, bool RAW = false>
struct DownRow {
    u32x4 w[CH];
    uint32_t sr[CH];   // RAW: scale bits (scale_of)
    f32x2 sc[CH];      // !RAW: decoded scales, zero past the row

    // CLAMPED: unconditional loads from a clamped row and chunk, zeroed past
    // the matrix (the grouped kernel: its loads then overlap, 176 against
    // 192 us per 8-row 397B-A17B layer); otherwise loads under the row/chunk
    // condition (the one-row kernels: measured faster there, 19.1 against
    // 20.2 us per 35B-A3B layer).
    template <bool CLAMPED = false>
    __device__ __forceinline__ void load(const ExpertSet &X, int e, int o, int sub, bool live) {
        const int rb = row_bytes<FMT>(X.inter), nch = rb >> 4;
        const int oc = CLAMPED && !live ? 0 : o;
        const uint8_t *wrow = X.dn + (size_t)e * X.dn_stride + (size_t)oc * rb;
        const uint8_t *sbase = X.dn_s + (size_t)e * X.dn_s_stride;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = sub + LPR * c;
            if constexpr (CLAMPED) {
                const u32x4 v = ld16_stream(wrow + (size_t)(ch < nch ? ch : nch - 1) * 16);
                w[c] = (live && ch < nch) ? v : u32x4{0u, 0u, 0u, 0u};
            } else {
                w[c] = (live && ch < nch) ? ld16_stream(wrow + (size_t)ch * 16) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = sub + LPR * c;
            if constexpr (RAW) {
                // unmasked: a chunk past the row or a dead row has zero codes
                sr[c] = chunk_scale_raw<FMT>(sbase, live ? o : 0, X.inter, ch < nch ? ch : nch - 1);
            } else if constexpr (CLAMPED) {
                const f32x2 v = chunk_scale<FMT>(sbase, oc, X.inter, ch < nch ? ch : nch - 1);
                sc[c] = (live && ch < nch) ? v : f32x2{0.0f, 0.0f};
            } else {
                sc[c] = (live && ch < nch) ? chunk_scale<FMT>(sbase, o, X.inter, ch) : f32x2{0.0f, 0.0f};
            }
        }
    }
    __device__ __forceinline__ f32x2 scale(int c) const {
        if constexpr (RAW)
            return scale_of<FMT>(sr[c]);
        else
            return sc[c];
    }

    // Per-lane partial sum against the lane's h chunks hq[c] (chunk sub + LPR c).
    __device__ __forceinline__ float partial(const f32x4 (&hq)[CH][h_quads<FMT>()], int inter, int sub) const {
        const int nch = row_bytes<FMT>(inter) >> 4;
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            if (sub + LPR * c < nch) acc += chunk_dot_f32<FMT>(w[c], scale(c), hq[c]);
        return acc;
    }

    // The lane's h chunks of h (global or LDS, plain layout).
    __device__ __forceinline__ static void load_h(const float *h, int inter, int sub, f32x4 (&hq)[CH][h_quads<FMT>()]) {
        const int nch = row_bytes<FMT>(inter) >> 4;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = sub + LPR * c;   // chunks past the row: loaded clamped, never used
            const f32x4 *h4 =
                reinterpret_cast<const f32x4 *>(h + (size_t)(ch < nch ? ch : nch - 1) * cols_per_chunk<FMT>());
#pragma unroll
            for (int q = 0; q < h_quads<FMT>(); ++q) hq[c][q] = h4[q];
        }
    }

    // d = row . h (h: the expert's f32 intermediate, global or LDS), reduced
    // over the row group; every lane of the group gets it.
    __device__ __forceinline__ float dot(const float *h, int inter, int sub) const {
        f32x4 hq[CH][h_quads<FMT>()];
        load_h(h, inter, sub, hq);
        return group_sum<LPR>(partial(hq, inter, sub));
    }

    // The same dot product over h held in LDS in chunk-quad order (quad q of
    // chunk c at float (q * nchunks + c) * 4), so consecutive lanes read
    // consecutive 16-byte words: the same products in the same order.
    __device__ __forceinline__ float dot_perm(const float *hl, int inter, int sub) const {
        constexpr int CPC = cols_per_chunk<FMT>();
        const int nch = row_bytes<FMT>(inter) >> 4;
        const int nct = inter / CPC;
        f32x4 hq[CH][h_quads<FMT>()];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = sub + LPR * c;
            if (ch < nch) {
#pragma unroll
                for (int q = 0; q < h_quads<FMT>(); ++q)
                    hq[c][q] = *reinterpret_cast<const f32x4 *>(hl + ((size_t)q * nct + ch) * 4);
            }
        }
        return group_sum<LPR>(partial(hq, inter, sub));
    }
};

// Lanes per down row and chunks per lane for a layer (the launchers and the
// host-side shape check agree on this rule): lanes cover the routed expert's
// row, capped at the wave; chunks per lane cover the longer of the two rows.
__host__ __device__ inline void down_lane_shape(int fmt, int inter, int shared_inter, int &lpr, int &ch) {
    const int nch = fmt_row_bytes(fmt, inter) / 16;
    const int ie = inter > shared_inter ? inter : shared_inter;
    const int nchmax = fmt_row_bytes(fmt, ie) / 16;
    lpr = nch >= 64 ? 64 : nch >= 32 ? 32 : nch >= 16 ? 16 : 8;
    ch = (nchmax + lpr - 1) / lpr;
}

__device__ __forceinline__ void store_out(uint16_t *y, uint16_t *res, int64_t ldy, int r, int o, float v) {
    if (y) y[(size_t)r * ldy + o] = f32_to_bf16(v);
    if (res) {
        uint16_t *p = res + (size_t)r * ldy + o;
        *p = f32_to_bf16(bf16_to_f32(*p) + v);
    }
}

// Reads `bytes` (a multiple of 16) starting at p, spread over the block's
// threads, and folds them into one word so the loads cannot be dropped: a
// plain (cache-allocating) read that leaves the lines in the memory-side
// cache for a later kernel.
__device__ __forceinline__ uint32_t warm_bytes(const uint8_t *p, size_t bytes) {
    uint32_t acc = 0;
    for (size_t off = (size_t)threadIdx.x * 16; off < bytes; off += (size_t)blockDim.x * 16) {
        const u32x4 v = ld16(p + off);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    return acc;
}

}  // namespace moe
