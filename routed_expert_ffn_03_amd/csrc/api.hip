// C ABI of the routed-expert layer library: argument checks, workspace
// layout, and the launches.  Every check here happens on the host before
// anything is enqueued; nothing here synchronises with the device.
// Failing loudly instead of falling back: "dsv41-flash-engram-disk-prestage",
// section "The prestage, per decode step", point 4.
#include "../../include/moe_mi355x.h"
#include "ffn_shared.h"
#include "kernels.h"

#include <mutex>

namespace {

// Workspace of moe_grouped_ffn_noalloc: one array per GPU, held by the code
// object for the life of the process.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// The device address of `scratch` on the current device.
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool bad_tek(int T, int E, int k) {
    if (T < 1 || E < 1 || E > moe::MAX_EXPERTS || k < 1) return true;
    if (k > moe::MAX_TOPK || k > E) return true;
    if ((long long)T * (long long)k >= (1LL << 31)) return true;
    return false;
}

// The fat kernels address x, the activation a and one expert's matrix with
// 32-bit buffer offsets: each must stay below 4 GiB.
bool ffn_shape_ok(int T, int k, int H, int I) {
    if (H < 256 || I < 128 || H % 256 != 0 || I % 128 != 0) return false;
    const unsigned long long lim = 1ULL << 32;
    return (unsigned long long)T * H * 2 < lim && (unsigned long long)T * k * I * 2 < lim &&
           (unsigned long long)I * H * 2 < lim;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool wfmt_known(int wfmt) {
    return wfmt == MOE_WFMT_BF16 || wfmt == MOE_WFMT_Q3G128 || wfmt == MOE_WFMT_BF16_PAIRS;
}

// Shape rules of a format beyond ffn_shape_ok: the row-pair layout is read
// by the MFMA-tile and the whole-line streaming kernels only, and the latter
// needs each wave's quarter of the reduction index (H / 4 and I / 4) to be a
// multiple of 64.
bool wfmt_shape_ok(int wfmt, int T, int k, int H, int I) {
    if (wfmt != MOE_WFMT_BF16_PAIRS) return true;
    return moe::stream_fits(1, T, k, H, I) && moe::stream_fits(2, T, k, H, I);
}

// Scales come with the 3-bit format and only with it.
bool scales_ok(int wfmt, const void* a, const void* b) {
    return wfmt == MOE_WFMT_Q3G128 ? (a && b) : (!a && !b);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or format not supported by the kernels";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch or runtime error";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_version(void) { return "0.1.0"; }

size_t moe_workspace_size(int T, int E, int k, int H, int I, int wfmt) {
    if (bad_tek(T, E, k) || !ffn_shape_ok(T, k, H, I)) return 0;
    if (!wfmt_known(wfmt) || !wfmt_shape_ok(wfmt, T, k, H, I)) return 0;
    return align256(moe::permute_ws_bytes(T, E)) + moe::ffn_ws_bytes(T, E, k, H, I, wfmt);
}

moe_status moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                          int32_t* expert_counts, void* stream) {
    if (!logits || !topk_ids || !topk_w || !expert_counts) return MOE_ERR_INVALID_ARG;
    if (bad_tek(T, E, k)) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_route_topk(logits, T, E, k, topk_ids, topk_w, expert_counts,
                                             reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_router_topk(const uint16_t* x, const uint16_t* w_router, int T, int E, int H, int k,
                           int32_t* topk_ids, float* topk_w, int32_t* expert_counts, float* logits, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!x || !w_router || !topk_ids || !topk_w || !expert_counts) return MOE_ERR_INVALID_ARG;
    if (bad_tek(T, E, k) || H < 1) return MOE_ERR_INVALID_ARG;
    if (!moe::router_shape_ok(T, E, H)) return MOE_ERR_UNSUPPORTED;
    // a workspace, when given, must hold the logits of the batch
    if (workspace && workspace_bytes < (size_t)T * (size_t)E * sizeof(float)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_router_topk(x, w_router, T, E, H, k, topk_ids, topk_w, expert_counts, logits,
                                              reinterpret_cast<float*>(workspace),
                                              reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_permute(const int32_t* topk_ids, int T, int E, int k, int32_t* expert_offsets,
                       int32_t* sorted_pair, int32_t* pair_to_sorted, void* workspace, size_t workspace_bytes,
                       void* stream) {
    if (!topk_ids || !expert_offsets || !sorted_pair || !pair_to_sorted) return MOE_ERR_INVALID_ARG;
    if (bad_tek(T, E, k)) return MOE_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < moe::permute_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_permute(topk_ids, T, E, k, expert_offsets, sorted_pair, pair_to_sorted,
                                          reinterpret_cast<int32_t*>(workspace),
                                          reinterpret_cast<hipStream_t>(stream)));
}

// Shared checks of the FFN entry points; fills `a` on success.
static moe_status ffn_prepare(moe::FfnLaunch& a, int wfmt, int T, int E, int k, int H, int I,
                              void* workspace, size_t workspace_bytes) {
    if (bad_tek(T, E, k) || H < 1 || I < 1) return MOE_ERR_INVALID_ARG;
    if (!wfmt_known(wfmt)) return MOE_ERR_UNSUPPORTED;
    if (!ffn_shape_ok(T, k, H, I) || !wfmt_shape_ok(wfmt, T, k, H, I)) return MOE_ERR_UNSUPPORTED;
    const size_t need = moe_workspace_size(T, E, k, H, I, wfmt);
    if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    a = moe::FfnLaunch{};
    a.wfmt = wfmt;
    a.T = T; a.E = E; a.k = k; a.H = H; a.I = I;
    a.ws = reinterpret_cast<char*>(workspace) + align256(moe::permute_ws_bytes(T, E));
    return MOE_OK;
}

moe_status moe_ffn_plan(const int32_t* expert_offsets, int T, int E, int k, int H, int I, int wfmt,
                        int fat_threshold, void* workspace, size_t workspace_bytes, void* stream) {
    if (!expert_offsets || fat_threshold < 1) return MOE_ERR_INVALID_ARG;
    moe::FfnLaunch a;
    moe_status st = ffn_prepare(a, wfmt, T, E, k, H, I, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    a.offsets = expert_offsets;
    a.fat_threshold = fat_threshold;
    return hip_status(moe::launch_ffn_plan(a, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_ffn_gate_up(const uint16_t* x, int wfmt, const void* w_gate, const void* w_up,
                           const uint16_t* s_gate, const uint16_t* s_up, const int32_t* sorted_pair,
                           int T, int E, int k, int H, int I, int fat_threshold, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!x || !w_gate || !w_up || !sorted_pair || fat_threshold < 1) return MOE_ERR_INVALID_ARG;
    if (wfmt_known(wfmt) && !scales_ok(wfmt, s_gate, s_up))
        return MOE_ERR_INVALID_ARG;
    moe::FfnLaunch a;
    moe_status st = ffn_prepare(a, wfmt, T, E, k, H, I, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    a.x = x;
    a.wg = w_gate; a.wu = w_up;
    a.sg = s_gate; a.su = s_up;
    a.sorted_pair = sorted_pair;
    a.fat_threshold = fat_threshold;
    return hip_status(moe::launch_ffn_phase(a, 1, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_ffn_down(int wfmt, const void* w_down, const uint16_t* s_down, int T, int E, int k, int H, int I,
                        int fat_threshold, uint16_t* y_sorted, void* workspace, size_t workspace_bytes,
                        void* stream) {
    if (!w_down || !y_sorted || fat_threshold < 1) return MOE_ERR_INVALID_ARG;
    if (wfmt_known(wfmt) && !scales_ok(wfmt, s_down, s_down))
        return MOE_ERR_INVALID_ARG;
    moe::FfnLaunch a;
    moe_status st = ffn_prepare(a, wfmt, T, E, k, H, I, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    a.wd = w_down;
    a.sd = s_down;
    a.y = y_sorted;
    a.fat_threshold = fat_threshold;
    return hip_status(moe::launch_ffn_phase(a, 2, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn(const uint16_t* x, int wfmt, const void* w_gate, const void* w_up, const void* w_down,
                           const uint16_t* s_gate, const uint16_t* s_up, const uint16_t* s_down,
                           const int32_t* expert_offsets, const int32_t* sorted_pair, int T, int E, int k, int H,
                           int I, int fat_threshold, uint16_t* y_sorted, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (!x || !w_gate || !w_up || !w_down || !expert_offsets || !sorted_pair || !y_sorted)
        return MOE_ERR_INVALID_ARG;
    if (fat_threshold < 1) return MOE_ERR_INVALID_ARG;
    if (wfmt_known(wfmt)) {
        if (!scales_ok(wfmt, s_gate, s_up) || !scales_ok(wfmt, s_down, s_down)) return MOE_ERR_INVALID_ARG;
    }
    moe::FfnLaunch a;
    moe_status st = ffn_prepare(a, wfmt, T, E, k, H, I, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    st = moe_ffn_plan(expert_offsets, T, E, k, H, I, wfmt, fat_threshold, workspace, workspace_bytes, stream);
    if (st != MOE_OK) return st;
    st = moe_ffn_gate_up(x, wfmt, w_gate, w_up, s_gate, s_up, sorted_pair, T, E, k, H, I, fat_threshold, workspace,
                         workspace_bytes, stream);
    if (st != MOE_OK) return st;
    return moe_ffn_down(wfmt, w_down, s_down, T, E, k, H, I, fat_threshold, y_sorted, workspace, workspace_bytes,
                        stream);
}

moe_status moe_route_permute_plan(const float* logits, int T, int E, int k, int H, int I, int wfmt,
                                  int fat_threshold, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                                  int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_to_sorted,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (!logits || !topk_ids || !topk_w || !expert_counts || !expert_offsets || !sorted_pair || !pair_to_sorted)
        return MOE_ERR_INVALID_ARG;
    if (fat_threshold < 1) return MOE_ERR_INVALID_ARG;
    moe::FfnLaunch a;
    moe_status st = ffn_prepare(a, wfmt, T, E, k, H, I, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (T <= moe::FRONT_MAX_T) {
        const moe::FfnPlanPtrs pp = moe::ffn_plan_ptrs(T, E, k, H, I, wfmt, a.ws);
        return hip_status(moe::launch_route_permute_plan(logits, T, E, k, fat_threshold, topk_ids, topk_w,
                                                         expert_counts, expert_offsets, sorted_pair, pair_to_sorted,
                                                         pp, s));
    }
    // larger batches: the gate (ids and weights only), the permute, then the
    // plan, which also writes the histogram from the route lists (the gate's
    // own histogram would merge ~T/16 block histograms by global atomics)
    if (moe::launch_route_topk(logits, T, E, k, topk_ids, topk_w, nullptr, s) != hipSuccess) return MOE_ERR_HIP;
    st = moe_permute(topk_ids, T, E, k, expert_offsets, sorted_pair, pair_to_sorted, workspace, workspace_bytes,
                     stream);
    if (st != MOE_OK) return st;
    a.offsets = expert_offsets;
    a.fat_threshold = fat_threshold;
    a.counts = expert_counts;
    return hip_status(moe::launch_ffn_plan(a, s));
}

moe_status moe_grouped_ffn_noalloc(const uint16_t* x, int wfmt, const void* w_gate, const void* w_up,
                                   const void* w_down, const uint16_t* s_gate, const uint16_t* s_up,
                                   const uint16_t* s_down, const int32_t* expert_offsets, const int32_t* sorted_pair,
                                   int T, int E, int k, int H, int I, int fat_threshold, uint16_t* y_sorted,
                                   void* stream) {
    if (!x || !w_gate || !w_up || !w_down || !expert_offsets || !sorted_pair || !y_sorted)
        return MOE_ERR_INVALID_ARG;
    if (fat_threshold < 1 || bad_tek(T, E, k) || H < 1 || I < 1) return MOE_ERR_INVALID_ARG;
    if (!wfmt_known(wfmt)) return MOE_ERR_UNSUPPORTED;
    if (!scales_ok(wfmt, s_gate, s_up) || !scales_ok(wfmt, s_down, s_down)) return MOE_ERR_INVALID_ARG;
    if (!ffn_shape_ok(T, k, H, I) || !wfmt_shape_ok(wfmt, T, k, H, I)) return MOE_ERR_UNSUPPORTED;
    if (moe::ffn_ws_bytes(T, E, k, H, I, wfmt) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    hipError_t err = scratch_address(&ws);
    if (err != hipSuccess) return MOE_ERR_HIP;
    moe::FfnLaunch a{};
    a.x = x;
    a.wfmt = wfmt;
    a.wg = w_gate; a.wu = w_up; a.wd = w_down;
    a.sg = s_gate; a.su = s_up; a.sd = s_down;
    a.offsets = expert_offsets;
    a.sorted_pair = sorted_pair;
    a.T = T; a.E = E; a.k = k; a.H = H; a.I = I;
    a.fat_threshold = fat_threshold;
    a.y = y_sorted;
    a.ws = ws;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // the plan rewrites the list header, totals and the tail counters of
    // the shared array before the two phases read them
    err = moe::launch_ffn_plan(a, s);
    if (err == hipSuccess) err = moe::launch_ffn_phase(a, 1, s);
    if (err == hipSuccess) err = moe::launch_ffn_phase(a, 2, s);
    return hip_status(err);
}

moe_status moe_pack_bf16_pairs(const uint16_t* src, uint16_t* dst, int64_t mats, int rows, int cols, int to_fp16,
                               void* stream) {
    if (!src || !dst || mats < 1 || rows < 2 || rows % 2 != 0 || cols < 32 || cols % 32 != 0)
        return MOE_ERR_INVALID_ARG;
    if (to_fp16 != 0 && to_fp16 != 1) return MOE_ERR_INVALID_ARG;
    if (((uintptr_t)src | (uintptr_t)dst) & 15) return MOE_ERR_INVALID_ARG;
    const unsigned long long per = (unsigned long long)rows * (unsigned long long)cols * 2ull;
    if ((unsigned long long)mats > (1ull << 62) / per) return MOE_ERR_INVALID_ARG;
    const uintptr_t bytes = (uintptr_t)((unsigned long long)mats * per);
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_ERR_INVALID_ARG;     // overlapping buffers
    return hip_status(moe::launch_pack_pairs(src, dst, mats, rows, cols, to_fp16, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const uint16_t* y_sorted, const float* topk_w, const int32_t* pair_to_sorted, int T, int k,
                       int H, float* out, void* stream) {
    if (!y_sorted || !topk_w || !pair_to_sorted || !out) return MOE_ERR_INVALID_ARG;
    if (T < 1 || k < 1 || k > moe::MAX_TOPK || H < 1 || (long long)T * k >= (1LL << 31))
        return MOE_ERR_INVALID_ARG;
    if (H % 8) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_combine(y_sorted, topk_w, pair_to_sorted, T, k, H, out,
                                          reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
