// Top-k selection keys shared by the router kernels (internal header).
//
// A logit and its expert index packed into one 64-bit key,
//   key = (order-preserving bits of the logit) << 32 | ~expert,
// so that one unsigned max over a wave yields the largest logit and, among
// equal logits, the lowest expert index (-0 and +0 compare equal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ __forceinline__ uint32_t ordered_bits(float v) {
    if (v == 0.0f) v = 0.0f;                        // -0 -> +0
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o ^ 0x80000000u) : ~o);
}

// Wave-wide max of a 64-bit key without LDS round trips: four DPP steps give
// every lane the max of its 16-lane row (lane ^ 1, lane ^ 2, the other quad
// of its 8 by the half-row mirror, the other 8 by the row mirror), then the
// row swaps of gfx950 combine rows 0/1 and 2/3, and the two halves.  Called
// with every lane active.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_u64<0xB1>(v);                         // quad_perm [1, 0, 3, 2]
    v = dpp_max_u64<0x4E>(v);                         // quad_perm [2, 3, 0, 1]
    v = dpp_max_u64<0x141>(v);                        // row_half_mirror
    v = dpp_max_u64<0x140>(v);                        // row_mirror
    {
        // both operands the same register: one result holds rows (0, 0, 2, 2),
        // the other rows (1, 1, 3, 3)
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        const uint64_t a = ((uint64_t)hi[0] << 32) | lo[0], b = ((uint64_t)hi[1] << 32) | lo[1];
        v = a > b ? a : b;
    }
    {
        // lower and upper 32 lanes
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        const uint64_t a = ((uint64_t)hi[0] << 32) | lo[0], b = ((uint64_t)hi[1] << 32) | lo[1];
        v = a > b ? a : b;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace moe
