// Host-side launchers of the library's kernels (internal, C++ linkage).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_TOPK = 32;

// counts == nullptr (only for T > 64): ids and weights only, no histogram
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, hipStream_t s);

bool router_shape_ok(int T, int E, int H);
hipError_t launch_router_topk(const uint16_t* x, const uint16_t* w_router, int T, int E, int H, int k,
                              int32_t* topk_ids, float* topk_w, int32_t* counts, float* logits, float* scratch_logits,
                              hipStream_t s);

size_t permute_ws_bytes(int T, int E);
hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_to_sorted, int32_t* block_hist,
                          hipStream_t s);

struct FfnLaunch {
    const uint16_t* x;
    int wfmt;                       // 0 = bf16, 1 = 3-bit groups of 128, 2 = bf16 in the row-pair layout
    const void* wg;
    const void* wu;
    const void* wd;
    const uint16_t* sg;
    const uint16_t* su;
    const uint16_t* sd;
    const int32_t* offsets;
    const int32_t* sorted_pair;
    int T, E, k, H, I, fat_threshold;
    uint16_t* y;
    void* ws;                       // FFN part of the workspace
    int32_t* counts;                // plan only: per-expert row counts written too (nullable)
};

size_t ffn_ws_bytes(int T, int E, int k, int H, int I, int wfmt);
hipError_t launch_ffn_plan(const FfnLaunch& a, hipStream_t s);
hipError_t launch_ffn_phase(const FfnLaunch& a, int phase, hipStream_t s);   // 1 = gate/up, 2 = down

// bf16 matrices [mats, rows, cols] -> the row-pair layout (pack.hip)
hipError_t launch_pack_pairs(const uint16_t* src, uint16_t* dst, int64_t mats, int rows, int cols, int to_fp16,
                             hipStream_t s);

hipError_t launch_combine(const uint16_t* y, const float* w, const int32_t* p2s, int T, int k, int H,
                          float* out, hipStream_t s);

}  // namespace moe
