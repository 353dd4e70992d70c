// Top-k selection shared by the router kernels (internal header).
//
// A logit becomes its order-preserving 32-bit pattern (-0 and +0 equal), so
// that an unsigned max picks the largest logit; among equal logits the
// lowest expert index is taken.
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

// Wave-wide max of a 32-bit value, the same in every lane (a scalar): four
// DPP max steps leave every lane of a 16-lane row with the row's max, then
// the four rows' maxima are read out and combined on the scalar unit.  Called
// with every lane active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1, 0, 3, 2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2, 3, 0, 1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// Top-k of Q tokens' logits held by one wave, the tokens' rounds interleaved:
// ord[q][i] = ordered_bits of the logit of expert lane + 64 i of token q (0
// for padding and for entries already taken).  Round j takes, per token, the
// largest ord and among equal ones the lowest expert index -- the same order
// as one unsigned max over the 64-bit keys (ord << 32 | ~expert): M = wave
// max of ord; the winner is the smallest i whose ballot of (ord == M) is not
// empty, and the lowest lane in that ballot.  Lane j keeps round j's expert
// and logit.  Called with every lane active; logits must not be NaN.
template <int NV, int Q>
__device__ __forceinline__ void wave_topk(uint32_t (&ord)[Q][NV], int k, int lane, int (&my_e)[Q], float (&my_v)[Q]) {
    for (int j = 0; j < k; ++j) {
        uint32_t M[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            uint32_t m = ord[q][0];
#pragma unroll
            for (int i = 1; i < NV; ++i) m = max(m, ord[q][i]);
            M[q] = wave_max_u32(m);
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            int wi = 0;
            uint64_t b = 0;
#pragma unroll
            for (int i = NV - 1; i >= 0; --i) {                  // the smallest i with a match wins
                const uint64_t bi = __builtin_amdgcn_ballot_w64(ord[q][i] == M[q]);
                if (bi) {
                    wi = i;
                    b = bi;
                }
            }
            const int wl = (int)__builtin_ctzll(b);
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (i == wi && lane == wl) ord[q][i] = 0;
            if (lane == j) {
                my_e[q] = wl + 64 * wi;
                my_v[q] = from_ordered(M[q]);
            }
        }
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace moe
