// Combine: out[t, :] = sum_j w[t, j] * y_sorted[pair_to_sorted[t*k + j], :].
//
// Routed work is split per expert and the results are combined back per
// token on the GPU: dsv41-flash-offload wiki, repository file table,
// CPU-tier entry.  Reading: the combine is the gate-weighted sum.
//
// A gather-sum, not a scatter: every output element is owned by one thread
// that adds its k terms in ascending j in fp32 (one fma each), so the result is bit-identical
// from run to run (no atomics).  Each thread moves 16-byte fp16 loads and
// 32-byte fp32 stores; the per-token indices and weights are wave-uniform.
// y is read once, a wave's loads covering whole lines: with the
// non-temporal hint (16k chunk: 248 -> 218 us; the same hint on the stores
// measured slower).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int CB_THREADS = 128;
constexpr int CB_COLS = CB_THREADS * 8;     // columns per block
constexpr int CB_J = 8;                     // rows loaded ahead

__global__ __launch_bounds__(CB_THREADS)
void combine_kernel(const uint16_t* __restrict__ y, const float* __restrict__ w,
                    const int32_t* __restrict__ p2s, int k, int H, int col_blocks,
                    float* __restrict__ out) {
    const int t = blockIdx.x / col_blocks;
    const int col = (blockIdx.x % col_blocks) * CB_COLS + threadIdx.x * 8;
    if (col >= H) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // CB_J rows at a time, all loaded before the first product so that their
    // latencies overlap; then the rest one by one
    const float* wt = w + (size_t)t * k;
    const int32_t* pt = p2s + (size_t)t * k;
    auto term = [&](float wj, u32x4 h) {
        const f16x8 v = __builtin_bit_cast(f16x8, h);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, (float)v[i], acc[i]);
    };
    int j0 = 0;
    for (; j0 + CB_J <= k; j0 += CB_J) {
        float wj[CB_J];
        u32x4 h[CB_J];
#pragma unroll
        for (int jj = 0; jj < CB_J; ++jj) {
            wj[jj] = wt[j0 + jj];
            h[jj] = ldg16_stream(y + (size_t)pt[j0 + jj] * H + col);
        }
#pragma unroll
        for (int jj = 0; jj < CB_J; ++jj) term(wj[jj], h[jj]);
    }
    for (; j0 < k; ++j0) term(wt[j0], ldg16_stream(y + (size_t)pt[j0] * H + col));
    float* o = out + (size_t)t * H + col;
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = __float_as_uint(acc[i]);
        b[i] = __float_as_uint(acc[4 + i]);
    }
    stg16(o, a);
    stg16(o + 4, b);
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, const float* w, const int32_t* p2s, int T, int k, int H,
                          float* out, hipStream_t s) {
    const int col_blocks = (H + CB_COLS - 1) / CB_COLS;
    const size_t blocks = (size_t)T * col_blocks;
    combine_kernel<<<(unsigned)blocks, CB_THREADS, 0, s>>>(y, w, p2s, k, H, col_blocks, out);
    return hipGetLastError();
}

}  // namespace moe
