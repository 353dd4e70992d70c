// The front of a small layer call in one launch: top-k gate, per-expert
// route lists and the FFN's batch plan for T <= 64 tokens.
//
// The three steps and their sources are those of moe_route_topk (routing to
// a few of the layer's routed experts: dsv41-flash-offload wiki, opening
// paragraph), moe_permute (one route list per expert, experts with a positive
// count only: wiki file table, staged cold-expert prefill entry) and
// moe_ffn_plan (lists cut into batches; busy lists of at least the fat
// threshold as MFMA tiles: wiki file table, segment and busy-expert GEMM
// entries).  A decode step runs them back to back on a few dozen pairs, where
// each launch costs a few microseconds of fixed latency; one block does all
// three here, keeping the route lists in LDS between them.
//
// With at most 64 tokens every token is one bit of a 64-bit mask per expert
// (bit t: token t picked the expert); the histogram is each mask's population
// count, and the rank of pair (t, j) inside its expert's list is the number
// of lower bits, which is its ascending-token (= ascending-pair) position.
// Results are identical to the three separate calls.
#include "common.h"
#include "ffn_shared.h"
#include "kernels.h"
#include "route_keys.h"

namespace moe {
namespace {

constexpr int FRONT_THREADS = 1024;
constexpr int FRONT_WAVES = FRONT_THREADS / WAVE;

template <int NV>                                   // keys per lane (>= E / 64)
__global__ __launch_bounds__(FRONT_THREADS)
void route_permute_plan_kernel(const float* __restrict__ logits, int T, int E, int k, int thr,
                               int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                               int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_to_sorted,
                               FfnHeader* __restrict__ hdr, MTile* __restrict__ fat, MTile* __restrict__ thin) {
    __shared__ unsigned long long mask[MAX_EXPERTS];
    __shared__ int ids_s[FRONT_MAX_T * MAX_TOPK];
    __shared__ int base[MAX_EXPERTS];
    __shared__ int scratch[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += FRONT_THREADS) mask[e] = 0ull;
    __syncthreads();

    // 1. gate: one wave per token, the keys and k rounds of moe_route_topk
    for (int t = wave; t < T; t += FRONT_WAVES) {
        const float* row = logits + (size_t)t * E;
        uint32_t ord[1][NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + WAVE * i;
            ord[0][i] = e < E ? ordered_bits(row[e]) : 0u;
        }
        int me[1] = {0};
        float mv[1] = {0.0f};
        wave_topk<NV, 1>(ord, k, lane, me, mv);
        const int my_e = me[0];
        const float my_v = mv[0];
        const float v0 = __shfl(my_v, 0, 64);
        const float z = lane < k ? expf(my_v - v0) : 0.0f;
        const float s = wave_sum(z);
        if (lane < k) {
            topk_ids[(size_t)t * k + lane] = my_e;
            topk_w[(size_t)t * k + lane] = z / s;
            ids_s[t * k + lane] = my_e;
            atomicOr(&mask[my_e], 1ull << t);
        }
    }
    __syncthreads();

    // 2. histogram and list offsets, one expert per thread
    const int e = tid;
    const int n = e < E ? __popcll(mask[e]) : 0;
    const int incl = block_inclusive_scan(n, scratch);
    if (e < E) {
        counts[e] = n;
        offsets[e] = incl - n;
        base[e] = incl - n;
    }
    if (tid == 0) offsets[E] = T * k;
    __syncthreads();

    // 3. the route lists: pair (t, j) at its expert's offset plus the number
    //    of lower tokens that picked the same expert
    for (int p = tid; p < T * k; p += FRONT_THREADS) {
        const int t = p / k, ep = ids_s[p];
        const int pos = base[ep] + __popcll(mask[ep] & ((1ull << t) - 1ull));
        sorted_pair[pos] = p;
        pair_to_sorted[p] = pos;
    }

    // 4. the batch plan of the expert FFN
    int nf = 0, nt = 0;
    if (e < E) {
        if (n >= thr) nf = (n + FAT_BM - 1) / FAT_BM;
        else nt = (n + THIN_BM - 1) / THIN_BM;
    }
    const int fi = block_inclusive_scan(nf, scratch);
    const int ti = block_inclusive_scan(nt, scratch);
    if (e < E) write_expert_tiles(e, incl - n, n, nf, nt, fi - nf, ti - nt, fat, thin);
    if (tid == FRONT_THREADS - 1) {
        hdr->n_fat = fi;
        hdr->n_thin = ti;
        hdr->tail_next[0] = hdr->tail_next[1] = 0;
        hdr->tail_done[0] = hdr->tail_done[1] = 0;
    }
}

template <int NV>
void front_launch(const float* logits, int T, int E, int k, int thr, int32_t* ids, float* w, int32_t* counts,
                  int32_t* offsets, int32_t* sp, int32_t* p2s, const FfnPlanPtrs& pp, hipStream_t s) {
    route_permute_plan_kernel<NV><<<1, FRONT_THREADS, 0, s>>>(logits, T, E, k, thr, ids, w, counts, offsets, sp,
                                                               p2s, pp.hdr, pp.fat, pp.thin);
}

}  // namespace

hipError_t launch_route_permute_plan(const float* logits, int T, int E, int k, int fat_threshold, int32_t* topk_ids,
                                     float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                     int32_t* pair_to_sorted, const FfnPlanPtrs& pp, hipStream_t s) {
    if (T < 1 || T > FRONT_MAX_T) return hipErrorInvalidValue;
    const int nv = (E + WAVE - 1) / WAVE;
    auto go = [&](auto nv_c) {
        front_launch<decltype(nv_c)::value>(logits, T, E, k, fat_threshold, topk_ids, topk_w, counts, offsets,
                                            sorted_pair, pair_to_sorted, pp, s);
    };
    if (nv <= 1) go(std::integral_constant<int, 1>{});
    else if (nv <= 2) go(std::integral_constant<int, 2>{});
    else if (nv <= 4) go(std::integral_constant<int, 4>{});
    else if (nv <= 6) go(std::integral_constant<int, 6>{});       // E = 384
    else if (nv <= 8) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 16>{});
    return hipGetLastError();
}

}  // namespace moe
