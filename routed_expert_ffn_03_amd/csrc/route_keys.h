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

// A sorted list of a token's 8 largest logits (ordered bits, expert), kept
// by one lane: top-k with one token per lane.  A logit enters by a
// branch-free insertion after the entries it does not exceed, so logits
// offered in ascending expert order keep equal values in ascending expert
// order, the order of the selection above.
struct Top8 {
    uint32_t v[8];
    int e[8];
};

__device__ __forceinline__ void top8_init(Top8& t) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        t.v[j] = 0u;                                       // below every finite logit's pattern
        t.e[j] = 0;
    }
}

__device__ __forceinline__ void top8_insert(Top8& t, uint32_t v, int e) {
    bool c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = v > t.v[j];
#pragma unroll
    for (int j = 7; j >= 1; --j) {
        // the list is sorted, so v lands at the first j with c[j]
        t.v[j] = max(min(t.v[j - 1], v), t.v[j]);
        t.e[j] = c[j - 1] ? t.e[j - 1] : (c[j] ? e : t.e[j]);
    }
    t.v[0] = max(t.v[0], v);
    t.e[0] = c[0] ? e : t.e[0];
}

// Softmax weights of the first k entries (k <= 8), summed in the order of
// wave_sum's butterfly over lanes 0..7, so that they equal the per-wave
// selection's weights bit for bit.
__device__ __forceinline__ void top8_weights(const Top8& t, int k, float (&w)[8]) {
    const float v0 = from_ordered(t.v[0]);
    float z[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = j < k ? expf(from_ordered(t.v[j]) - v0) : 0.0f;
    const float sum = ((z[0] + z[4]) + (z[2] + z[6])) + ((z[1] + z[5]) + (z[3] + z[7]));
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = z[j] / sum;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace moe
