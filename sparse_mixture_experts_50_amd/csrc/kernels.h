// Launch interfaces of the MoE layer kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

// Tokens per router block.
#define MOE_ROUTER_TOKENS 32
// Most depth ranges the bf16 router's logits are split into.
#define MOE_ROUTER_MAX_SPLITS 8
// Most assignments (T*k) that the single-block permute takes.
#define MOE_PERMUTE_ONE_BLOCK 256

struct RouterParams {
    const void *x;        // [T][d]
    const void *wr;       // [E][d]
    const float *add;     // [E] or null
    const float *sub;     // [E] or null
    int32_t *topk_idx;    // [T][k]
    float *topk_w;        // [T][k]
    float *p_part;        // [ceil(T/32)][E]
    float *zh_part;       // [ceil(T/32)][2]: sum lse^2, sum entropy (nats)
    float *scores;        // expert choice: logits [E][T]; null for top-k
    int32_t *slot_of;     // expert choice: [T][E], set to -1 here
    int32_t *blk;         // top-k: [ceil(T/32)][E] picks of each expert
                          // among the block's 32 tokens (the dispatch's
                          // per-chunk counts)
    float *part;          // split bf16 router: [S][T][E] fp32 partial sums
                          // over S consecutive depth ranges of kc each
    int S, kc;            // S = 0: the fused kernel
    int T, d, E, k;
};

// How the bf16 router runs: fused (one kernel, 32 tokens per block) or
// split (partial logits over S depth ranges of kc each, then routing).
struct RouterPlan {
    int ep, tokens, S, kc;
    bool split;
};
RouterPlan router_plan(int T, int d, int E, int cus);

struct PermuteParams {
    const int32_t *topk_idx;  // [T*k]
    const float *p_part;      // [n_rtiles][E]
    const float *zh_part;     // [n_rtiles][2]
    const int32_t *blk;       // [n_chunks][E]: per-chunk expert counts from
                              // the router
    const float *scores;      // expert choice: logits [E][T]; else null
    int32_t *counts, *kept, *offsets, *slot_token, *slot_of;
    float *f, *p, *l_aux;
    float *monitor;           // [6] or null
    // top-k: chunk c = the assignments of router token tile c,
    // [32 k c, 32 k (c + 1)); n_chunks = n_rtiles (0 for expert choice)
    int T, E, k, capacity, n_rtiles, n_chunks;
    float alpha;
};

struct CombineParams {
    const void *yp;           // [slots][d]
    const int32_t *slot_of;   // [T][k]
    const float *topk_w;      // [T][k]
    void *y;                  // [T][d]
    int T, d, k, n_shared, shared_base;
};

// GEMM kernel variants.
enum GemmVariant {
    GEMM_BF16_256x256 = 0,
    GEMM_BF16_128x256 = 1,
    GEMM_BF16_32x256 = 2,
    GEMM_BF16_64x64 = 3,
    GEMM_F32_64x64 = 4,
    GEMM_BF16_DMA_256x256 = 5,
    GEMM_BF16_DMA_128x256 = 6,
    GEMM_BF16_STREAM_32x64 = 7,
    GEMM_BF16_DMA64_256x256 = 8,
    GEMM_BF16_DMA64_128x256 = 9,
    GEMM_FP8_STREAM_32x64 = 10,   // FP8 (E4M3) weights, bf16 activations
    GEMM_BF16_STREAM_64x64 = 11,  // streaming with 64-column units
    GEMM_FP8_STREAM_64x64 = 12,
    GEMM_BF16_DMA64_320x256 = 13,  // 320-row tiles: one per ~257-320-row group
    GEMM_BF16_W4_256x256 = 14,     // four waves of 128 x 128, K % 128 == 0
    GEMM_BF16_W4_128x256 = 15,     // the same kernel, every tile 128 x 256
    GEMM_BF16_RING_16x16 = 16,     // weight ring through LDS, 16-row passes
    GEMM_FP8_RING_16x16 = 17,
    GEMM_BF16_RING2_16x16 = 18,    // 1 KB row runs, two blocks per CU
    GEMM_FP8_RING2_16x16 = 19,
    GEMM_BF16_X2_128x256 = 20,     // two blocks per CU, 32-deep stages, K % 32 == 0
    GEMM_BF16_W4X_256x256 = 21,    // variant 14 with 32x32x16 MFMAs, mixed tile heights
    GEMM_BF16_W4X_128x256 = 22,    // variant 15 with 32x32x16 MFMAs
    GEMM_BF16_W4_256x192 = 23,     // variant 14 with 192-column tiles (ungated, N % 192 == 0)
    GEMM_BF16_TALL_320x192 = 24,   // four waves of 160 x 96: one tile per group of <= 320 rows (ungated)
    GEMM_BF16_TALL_288x224 = 25,   // four waves of 144 x 112: one tile per group of <= 288 rows (ungated)
};

inline bool tall_variant(int v) {
    return v == GEMM_BF16_TALL_320x192 || v == GEMM_BF16_TALL_288x224;
}

// Weight-ring kernels: bytes of each weight row per stage (bf16 / FP8),
// and the most routed slots whose tokens they stage in LDS.
constexpr int MOE_RING_CB_BF16 = 2048;
constexpr int MOE_RING_CB_FP8 = 1024;
constexpr int MOE_RING_MAXTOK = 1024;

inline bool ring_variant(int v) {
    return v == GEMM_BF16_RING_16x16 || v == GEMM_FP8_RING_16x16 ||
           v == GEMM_BF16_RING2_16x16 || v == GEMM_FP8_RING2_16x16;
}

// Blocks per CU of a weight-ring variant, and its bytes of each row per
// stage.
inline int ring_occupancy(int v) {
    return v == GEMM_BF16_RING2_16x16 || v == GEMM_FP8_RING2_16x16 ? 2 : 1;
}
inline int ring_cb(int v) {
    return v == GEMM_BF16_RING_16x16 ? MOE_RING_CB_BF16 : v == GEMM_FP8_RING_16x16 ? MOE_RING_CB_FP8 : 1024;
}

// Variants that stream weights over persistent (group, column-slab) units.
inline bool stream_variant(int v) {
    return v == GEMM_BF16_STREAM_32x64 || v == GEMM_FP8_STREAM_32x64 ||
           v == GEMM_BF16_STREAM_64x64 || v == GEMM_FP8_STREAM_64x64;
}

struct GemmVariantInfo {
    int bm, bn, threads, lds_bytes;
};

GemmVariantInfo gemm_variant_info(int variant);

hipError_t launch_router(const RouterParams &p, int dtype, hipStream_t s);
hipError_t launch_permute(const PermuteParams &p, hipStream_t s);
// Router and permute of a decode-sized step in two launches instead of
// three (bf16 split router plan, E <= 32, T <= 32, T*k <= 256, top-k
// routing): the partial logits, then routing and dispatch in one block;
// the same results as launch_router followed by launch_permute.
bool route_permute_small_ok(const RouterParams &p);
hipError_t launch_route_permute_small(const RouterParams &p,
                                      const PermuteParams &q, hipStream_t s);
hipError_t launch_expert_choice(const PermuteParams &p, hipStream_t s);
hipError_t launch_gemm(const GemmParams &p, int variant, bool up, int grid,
                       hipStream_t s);
// The tall-tile kernel (variants 24 and 25): bn = 192 or 224 columns.
hipError_t launch_gemm_tall(const GemmParams &p, int bn, bool up, int grid,
                            hipStream_t s);
hipError_t launch_combine(const CombineParams &p, int dtype, hipStream_t s);
hipError_t launch_bias_update(int E, const int32_t *counts, float target,
                              float gamma, float *bias, hipStream_t s);
