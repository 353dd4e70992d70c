// Router: per-token top-k over the layer's experts, gate weights and the
// load histogram.
//
// Routing to a few of the layer's routed experts per token: dsv41-flash-offload
// wiki, opening paragraph.  The gate is not written on the pages; this is the
// reading the library implements: the k largest logits (ties -> lower expert
// index, -0 == +0), weights = softmax over the selected logits.
//
// One wavefront per token.  Lane i holds experts i, i+64, ... as 64-bit keys
//   key = (order-preserving bits of the logit) << 32 | ~expert
// so one unsigned max over the wave yields the largest logit and, among equal
// logits, the lowest expert index.  k rounds of (lane-local max, 6-step
// butterfly max, owner clears the winner) give the ordered top-k.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int ROUTE_THREADS = 256;
constexpr int ROUTE_WAVES = ROUTE_THREADS / WAVE;

__device__ __forceinline__ uint32_t ordered_bits(float v) {
    if (v == 0.0f) v = 0.0f;                        // -0 -> +0
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o ^ 0x80000000u) : ~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// tokens_per_block tokens per block; waves take tokens round-robin.
// direct_counts: the grid is one block covering all tokens, so the block
// histogram is the answer (no zeroing pass, no atomics).
template <int NV>                                   // keys per lane (>= E / 64)
__global__ __launch_bounds__(ROUTE_THREADS)
void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k, int tokens_per_block,
                       int direct_counts, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                       int32_t* __restrict__ counts) {
    __shared__ int hist[MAX_EXPERTS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) hist[e] = 0;
    __syncthreads();

    const int t0 = blockIdx.x * tokens_per_block;
    const int t1 = min(T, t0 + tokens_per_block);
    for (int t = t0 + wave; t < t1; t += ROUTE_WAVES) {
        const float* row = logits + (size_t)t * E;
        uint64_t key[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + WAVE * i;
            key[i] = 0;
            if (e < E) key[i] = ((uint64_t)ordered_bits(row[e]) << 32) | (uint32_t)(~e);
        }
        int my_e = 0;
        float my_v = 0.0f;
        for (int j = 0; j < k; ++j) {
            uint64_t m = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i) m = key[i] > m ? key[i] : m;
            m = wave_max_u64(m);
            const int win = (int)(~(uint32_t)m);
            if ((win & 63) == lane) {
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    if (i == (win >> 6)) key[i] = 0;
            }
            if (lane == j) {
                my_e = win;
                my_v = from_ordered((uint32_t)(m >> 32));
            }
        }
        const float v0 = __shfl(my_v, 0, 64);
        const float z = lane < k ? expf(my_v - v0) : 0.0f;
        const float s = wave_sum(z);
        if (lane < k) {
            topk_ids[(size_t)t * k + lane] = my_e;
            topk_w[(size_t)t * k + lane] = z / s;
            atomicAdd(&hist[my_e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) {
        if (direct_counts) counts[e] = hist[e];
        else if (hist[e]) atomicAdd(&counts[e], hist[e]);
    }
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

template <int NV>
void route_launch(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w, int32_t* counts,
                  hipStream_t s) {
    // Small batches: one block owns every token and writes the histogram
    // directly.  Larger ones: 16 tokens per block (4 per wave) keeps ~1k
    // blocks in flight at 16k tokens; bins merge with integer atomics after a
    // zeroing pass (integer sums are order-independent, so the result is
    // deterministic).
    const int single_max = 64;
    if (T <= single_max) {
        route_topk_kernel<NV><<<1, ROUTE_THREADS, 0, s>>>(logits, T, E, k, T, 1, topk_ids, topk_w, counts);
        return;
    }
    const int tpb = 16;
    zero_i32_kernel<<<(E + 255) / 256, 256, 0, s>>>(counts, E);
    const int blocks = (T + tpb - 1) / tpb;
    route_topk_kernel<NV><<<blocks, ROUTE_THREADS, 0, s>>>(logits, T, E, k, tpb, 0, topk_ids, topk_w, counts);
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, hipStream_t s) {
    const int nv = (E + WAVE - 1) / WAVE;
    if (nv <= 1) route_launch<1>(logits, T, E, k, topk_ids, topk_w, counts, s);
    else if (nv <= 2) route_launch<2>(logits, T, E, k, topk_ids, topk_w, counts, s);
    else if (nv <= 4) route_launch<4>(logits, T, E, k, topk_ids, topk_w, counts, s);
    else if (nv <= 8) route_launch<8>(logits, T, E, k, topk_ids, topk_w, counts, s);
    else route_launch<16>(logits, T, E, k, topk_ids, topk_w, counts, s);
    return hipGetLastError();
}

}  // namespace moe
