// Permute: per-expert route lists as a stable counting sort of the pairs
// p = t*k + j by expert id.
//
// One route list per expert, only experts with a positive count run:
// dsv41-flash-offload wiki, repository file table, entry for the staged
// cold-expert prefill patch.  Reading for a unique order: lists in expert
// order, ascending pair index inside a list.
//
// Three passes, no global atomics, every position a pure function of the ids:
//   1. block histogram: block b (256 consecutive tokens) counts its pairs per
//      expert in LDS and writes hist[b][e];
//   2. scan (one block): per expert, totals -> offsets (exclusive scan over
//      experts) and hist[b][e] -> offsets[e] + sum_{b'<b} hist[b'][e];
//   3. scatter: inside block b the rank of pair (t, j) among the block's
//      pairs of the same expert is (pairs of lower waves) + (lower lanes of
//      its own wave), read off 64-bit lane masks built with LDS atomic OR.
//      Since a token picks an expert at most once, lane order = pair order.
// Up to 1024 tokens the same three steps run inside one block.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int PB_TOKENS = 256;            // tokens (= threads) per block
constexpr int PB_WAVES = PB_TOKENS / WAVE;
constexpr int PB_SMALL_T = 1024;          // one-block path up to this many tokens

__global__ __launch_bounds__(PB_TOKENS)
void permute_hist_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                         int32_t* __restrict__ block_hist) {
    __shared__ int hist[MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += PB_TOKENS) hist[e] = 0;
    __syncthreads();
    const int t = blockIdx.x * PB_TOKENS + threadIdx.x;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicAdd(&hist[ids[(size_t)t * k + j]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += PB_TOKENS) block_hist[(size_t)blockIdx.x * E + e] = hist[e];
}

__global__ __launch_bounds__(1024)
void permute_scan_kernel(int32_t* __restrict__ block_hist, int nblocks, int E, int P,
                         int32_t* __restrict__ offsets) {
    // each thread walks its expert's column of block counts in chunks of CH
    // loads issued together (a plain loop waits for every load in turn)
    constexpr int CH = 16;
    __shared__ int scratch[16];
    const int e = threadIdx.x;
    int total = 0;
    if (e < E)
        for (int b0 = 0; b0 < nblocks; b0 += CH) {
            int v[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) v[i] = b0 + i < nblocks ? block_hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < CH; ++i) total += v[i];
        }
    const int incl = block_inclusive_scan(total, scratch);
    if (e < E) {
        int base = incl - total;
        offsets[e] = base;
        for (int b0 = 0; b0 < nblocks; b0 += CH) {
            int v[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) v[i] = b0 + i < nblocks ? block_hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < CH; ++i)
                if (b0 + i < nblocks) {
                    block_hist[(size_t)(b0 + i) * E + e] = base;
                    base += v[i];
                }
        }
    }
    if (e == 0) offsets[E] = P;
}

__global__ __launch_bounds__(PB_TOKENS)
void permute_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                            const int32_t* __restrict__ block_base, int32_t* __restrict__ sorted_pair,
                            int32_t* __restrict__ pair_to_sorted) {
    __shared__ unsigned long long mask[PB_WAVES][MAX_EXPERTS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < PB_WAVES * E; i += PB_TOKENS) mask[i / E][i % E] = 0ull;
    __syncthreads();
    const int t = blockIdx.x * PB_TOKENS + threadIdx.x;
    const unsigned long long bit = 1ull << lane;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicOr(&mask[wave][ids[(size_t)t * k + j]], bit);
    __syncthreads();
    if (t < T) {
        const int32_t* base = block_base + (size_t)blockIdx.x * E;
        for (int j = 0; j < k; ++j) {
            const int p = t * k + j;
            const int e = ids[p];
            int pos = base[e] + __popcll(mask[wave][e] & (bit - 1ull));
            for (int w = 0; w < wave; ++w) pos += __popcll(mask[w][e]);
            sorted_pair[pos] = p;
            pair_to_sorted[p] = pos;
        }
    }
}

// Small batches (T <= PB_SMALL_T): the three passes in one block.  Counts,
// the scan and the running per-expert bases stay in LDS; tokens go through in
// chunks of 256 with the same lane-mask ranking as the scatter pass.
__global__ __launch_bounds__(PB_TOKENS)
void permute_small_kernel(const int32_t* __restrict__ ids, int T, int E, int k, int32_t* __restrict__ offsets,
                          int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_to_sorted) {
    __shared__ int base[MAX_EXPERTS];
    __shared__ unsigned long long mask[PB_WAVES][MAX_EXPERTS];
    __shared__ int scratch[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += PB_TOKENS) base[e] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += PB_TOKENS)
        for (int j = 0; j < k; ++j) atomicAdd(&base[ids[(size_t)t * k + j]], 1);
    __syncthreads();
    // exclusive scan of the counts: 4 consecutive experts per thread
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        c[i] = e < E ? base[e] : 0;
        sum += c[i];
    }
    int run = block_inclusive_scan(sum, scratch) - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        if (e < E) {
            base[e] = run;
            offsets[e] = run;
        }
        run += c[i];
    }
    if (tid == 0) offsets[E] = T * k;
    __syncthreads();
    const unsigned long long bit = 1ull << lane;
    for (int t0 = 0; t0 < T; t0 += PB_TOKENS) {
        for (int i = tid; i < PB_WAVES * E; i += PB_TOKENS) mask[i / E][i % E] = 0ull;
        __syncthreads();
        const int t = t0 + tid;
        if (t < T)
            for (int j = 0; j < k; ++j) atomicOr(&mask[wave][ids[(size_t)t * k + j]], bit);
        __syncthreads();
        if (t < T) {
            for (int j = 0; j < k; ++j) {
                const int p = t * k + j;
                const int e = ids[p];
                int pos = base[e] + __popcll(mask[wave][e] & (bit - 1ull));
                for (int w = 0; w < wave; ++w) pos += __popcll(mask[w][e]);
                sorted_pair[pos] = p;
                pair_to_sorted[p] = pos;
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += PB_TOKENS) {
            int n = 0;
            for (int w = 0; w < PB_WAVES; ++w) n += __popcll(mask[w][e]);
            base[e] += n;
        }
        __syncthreads();
    }
}

}  // namespace

size_t permute_ws_bytes(int T, int E) {
    const size_t nb = (size_t)(T + PB_TOKENS - 1) / PB_TOKENS;
    return nb * (size_t)E * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_to_sorted, int32_t* block_hist,
                          hipStream_t s) {
    if (T <= PB_SMALL_T) {
        permute_small_kernel<<<1, PB_TOKENS, 0, s>>>(ids, T, E, k, offsets, sorted_pair, pair_to_sorted);
        return hipGetLastError();
    }
    const int nb = (T + PB_TOKENS - 1) / PB_TOKENS;
    permute_hist_kernel<<<nb, PB_TOKENS, 0, s>>>(ids, T, E, k, block_hist);
    permute_scan_kernel<<<1, 1024, 0, s>>>(block_hist, nb, E, T * k, offsets);
    permute_scatter_kernel<<<nb, PB_TOKENS, 0, s>>>(ids, T, E, k, block_hist, sorted_pair, pair_to_sorted);
    return hipGetLastError();
}

}  // namespace moe
