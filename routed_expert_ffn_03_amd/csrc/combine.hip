// Combine: out[t, :] = sum_j w[t, j] * y_sorted[pair_to_sorted[t*k + j], :].
//
// Routed work is split per expert and the results are combined back per
// token on the GPU: dsv41-flash-offload wiki, repository file table,
// CPU-tier entry.  Reading: the combine is the gate-weighted sum.
//
// A gather-sum, not a scatter: every output element is owned by one thread
// that adds its k terms in ascending j in fp32, so the result is bit-identical
// from run to run (no atomics).  Each thread moves 16-byte fp16 loads and
// 32-byte fp32 stores; the per-token indices and weights are wave-uniform.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int CB_THREADS = 128;
constexpr int CB_COLS = CB_THREADS * 8;     // columns per block

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
    for (int j = 0; j < k; ++j) {
        const size_t p = (size_t)t * k + j;
        const float wj = w[p];
        const size_t row = (size_t)p2s[p];
        const f16x8 h = __builtin_bit_cast(f16x8, ldg16(y + row * H + col));
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wj * (float)h[i];
    }
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
