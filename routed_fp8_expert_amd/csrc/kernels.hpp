// kernels.hpp -- host-side launch interface between the C ABI (api.cpp) and
// the gfx950 kernels (route.hip, ffn.hip).  Plain structs of device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct ExpertSet {
    const uint8_t *gu, *gu_s, *dn, *dn_s;     // codes and scales (bytes)
    const float *gu_g, *dn_g;                 // nvfp4 globals (per expert), else null
    int64_t gu_stride, gu_s_stride, dn_stride, dn_s_stride;
    int inter;                                 // I of this family (0 = absent)
};

// Per-step bookkeeping written by the grouping kernel, read by the expert
// kernels (int32 words in the workspace).
constexpr int kReplicas = 8;   // one copy per XCD (workgroups map to XCDs by index)
constexpr int kMaxTopK = 16;
constexpr int kMaxSlots = kMaxTopK + 1;   // routed slots plus the shared expert

// A ctx's synchronisation words (uint32, device memory of the ctx pool), in
// groups that each start a 256-byte line: the router ticket of the one-row
// lead kernel, the device error word, the cache-warming sink, the ticket of
// the fused top-k + grouping launch, then the one-launch layer's words
// (layer.hip: per-replica done-word lines and the arrival sub-counters).
constexpr int kSyncLine = 64;   // words per 256-byte line
constexpr int kLayerSyncWords = 71 * kSyncLine;
enum CtxWord : int {
    kWordRouterTicket = 0,
    kWordError = 1 * kSyncLine,
    kWordSink = 2 * kSyncLine,
    kWordGroupTicket = 3 * kSyncLine,
    kWordLayerSync = 4 * kSyncLine,
    kCtxWords = kWordLayerSync + kLayerSyncWords
};
// Bits of the ctx's device error word.
enum : uint32_t { kErrBadExpertId = 1u, kErrWaitTimeout = 2u };

constexpr int kMfmaTileRows = 16;   // rows of an expert per matrix-core tile (down, fewer-row steps)
constexpr int kMfmaGuTileRows = 64; // rows of an expert per gate/up matrix-core tile

// Weight formats (the values of the C ABI's moe_weight_format).
enum : int { kFp8 = 0, kNvfp4 = 1, kInt8Row = 2, kInt4Row = 3, kInt4G64 = 4, kFp8Bf16s = 5 };
// e4m3 codes with one scale per 128x128 block (f32 or bf16).
__host__ __device__ constexpr bool fp8_block(int fmt) { return fmt == kFp8 || fmt == kFp8Bf16s; }
// One code per byte (fp8, int8) or two (e2m1, int4).
__host__ __device__ constexpr bool byte_codes(int fmt) { return fp8_block(fmt) || fmt == kInt8Row; }
__host__ __device__ constexpr int fmt_row_bytes(int fmt, int cols) { return byte_codes(fmt) ? cols : cols / 2; }

enum MetaWord : int {
    kMetaGemvCount = 0,   // routed experts on the GEMV arm
    kMetaMfmaCount = 1,   // routed experts on the MFMA arm
    kMetaMfmaTiles = 2,   // MFMA row tiles (routed)
    kMetaMfmaGuTiles = 3, // gate/up MFMA row tiles of kMfmaGuTileRows (routed)
    kMetaWords = 16
};

struct RouteArgs {
    const uint16_t *x; int64_t ldx; int R;
    const uint16_t *wr; const float *bias; const uint16_t *wsg;
    int H, E, k;
    const float *logits_in;     // when non-null the router GEMV is skipped
    float *logits;              // [R][E] (router output or scratch)
    int32_t *ids; float *w; float *s;
    int32_t *counts, *offsets, *perm;   // grouping (R >= 2)
    int32_t *meta, *gemv_list, *mfma_list, *mfma_tiles;
    int mfma_min_rows;          // experts with count >= this go to the MFMA arm (0 = never)
    uint32_t *err;
    unsigned *ticket;           // ctx word: router workgroups done (one-row lead kernel)
    unsigned *group_ticket;     // ctx word: top-k workgroups done (fused top-k + grouping)
};

struct FfnArgs {
    const uint16_t *x; int64_t ldx; int R; int H; int E; int k; int fmt;
    ExpertSet routed, shared;
    const int32_t *ids; const float *w; const float *s;
    const int32_t *counts, *offsets, *perm;
    const int32_t *meta, *gemv_list, *mfma_list, *mfma_tiles;
    float *h;        // [NE][hstride] silu*mul products, NE = R*k (+ R shared)
    int hstride;     // max(I, Is)
    float *dbuf;     // [NE][H] per-entry down outputs (R >= 2)
    uint16_t *y; uint16_t *res; int64_t ldy;
    uint32_t *err;
    int max_routed_tasks;       // grid bound on routed experts for R >= 2
    int mfma_max_tiles;         // grid bound on MFMA row tiles (0 = MFMA arm off)
    int mfma_gu_max_tiles;      // grid bound on gate/up MFMA row tiles
    int shared_mfma;            // the shared expert's rows go to the MFMA arm
    uint32_t *sink;             // word the cache-warming reads fold into
    // single-launch one-row layer: per-XCD replicas of values crossing workgroups
    float *logits_rep;          // [kReplicas][E]
    float *h_rep;               // [kReplicas][k+1][hstride]
    // optional epilogue: RMSNorm of each output row (res after the add, else y)
    const uint16_t *norm_w;     // bf16 [H] weight; null = no epilogue
    float norm_eps;
    uint16_t *norm_out;         // bf16 [R][ldn]
    int64_t ldn;
    // few-rows steps: the gate/up blocks take their row's top-k themselves
    const float *topk_src;      // logits [R][E] to select from; null = ids already published
    const uint16_t *wsg;        // shared-gate vector (s_mode 1)
    int s_mode;                 // 0: s written by the router, 1: s = sigmoid(x . wsg), 2: s = 1
};

// Dense fp8 block-128 projection y = x . dequant(W)^T.
struct DenseArgs {
    const uint8_t *w; int64_t w_stride;   // e4m3 codes [N][w_stride bytes]
    const float *s;                       // f32 scales [N/128][K/128]
    const uint16_t *x; int64_t ldx;       // bf16 [R][ldx]
    uint16_t *y; int64_t ldy;             // bf16 [R][ldy]
    int N, K, R;
};

// Each launcher returns the hipError_t of its launch (hipGetLastError).
hipError_t launch_router(const RouteArgs &a, hipStream_t st);
hipError_t launch_topk(const RouteArgs &a, bool compute_s, hipStream_t st);
hipError_t launch_group(const RouteArgs &a, bool plan, hipStream_t st);
hipError_t launch_topk_group(const RouteArgs &a, bool compute_s, bool plan, hipStream_t st);
hipError_t launch_plan(const RouteArgs &a, hipStream_t st);
size_t group_lds_bytes(int E, int R);

hipError_t launch_gate_up(const FfnArgs &a, hipStream_t st);
// One-row layer: router rows + shared expert, then top-k + routed gate/up.
hipError_t launch_lead_r1(const RouteArgs &r, const FfnArgs &a, hipStream_t st);
hipError_t launch_gate_up_r1(const FfnArgs &a, hipStream_t st);
// One-row layer in a single launch (layer.hip); `sync` = the ctx's
// kLayerSyncWords layer words, all zero between launches; a wait for another
// workgroup gives up after `wait_ticks` ticks of the device's constant clock
// (s_memrealtime).
// `stamps` (diagnostics, or null): kStampWords words per workgroup of phase
// timestamps; a launch needing more than `stamp_words` fails.
constexpr int kStampWords = 16;
bool layer_r1_supported(const RouteArgs &r, const FfnArgs &a);
hipError_t launch_layer_r1(const RouteArgs &r, const FfnArgs &a, unsigned *sync, uint64_t wait_ticks,
                           uint64_t *stamps, int64_t stamp_words, hipStream_t st);
hipError_t launch_down_blend_r1(const FfnArgs &a, hipStream_t st);
hipError_t launch_down_grouped(const FfnArgs &a, hipStream_t st);
hipError_t launch_blend(const FfnArgs &a, hipStream_t st);
hipError_t launch_rmsnorm(const FfnArgs &a, hipStream_t st);
hipError_t launch_dense(const DenseArgs &a, hipStream_t st);

// The ctx pool (ctx_pool.hip): kMaxCtxPerDevice slots of kCtxWords words per
// device in static device memory.  ctx_slot_acquire makes `device` current's
// pool address known (hipGetSymbolAddress, once per device), takes a free
// slot, resets it (synchronously) and returns its words; release frees it.
// ctx_layer_words_reset returns a slot's layer words to their state between
// launches (zero).
constexpr int kMaxCtxPerDevice = 64;
hipError_t ctx_slot_acquire(int device, int *slot, uint32_t **words);
void ctx_slot_release(int device, int slot);
hipError_t ctx_layer_words_reset(uint32_t *words);

// The static workspace of moe_layer_forward_static (static_scratch.hip):
// kStaticScratchBytes per device.  static_scratch_init resolves its address
// on `device`, which must be current (once per device; at ctx creation);
// static_scratch_ptr returns it (null before init).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch_init(int device);
void *static_scratch_ptr(int device);

// Diagnostics: decode n codes with the kernels' own converters.
hipError_t launch_decode_probe(int fmt, const uint8_t *codes, float *out, int n, hipStream_t st);

}  // namespace moe
