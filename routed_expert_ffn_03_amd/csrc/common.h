// Device-side helpers shared by the library's kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> fp16 bits.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// Eight bf16 values (one 16-byte chunk) re-encoded as fp16.  Exact for
// magnitudes in fp16's normal range [2^-14, 65504]; smaller magnitudes are
// truncated toward zero (error < 2^-24); larger ones saturate.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float lo = __uint_as_float(v[i] << 16);
        float hi = __uint_as_float(v[i] & 0xFFFF0000u);
        auto h = __builtin_amdgcn_cvt_pkrtz(lo, hi);   // two __fp16
        r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
}

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(4))) float f32x4;

// 16x16x32 fp16: lane L holds row (A) or column (B) L % 16, k 8 (L / 16) ..
// 8 (L / 16) + 7; result element i of lane L is row 4 (L / 16) + i, column L % 16
__device__ __forceinline__ f32x4 mfma16_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// A 16-byte load with the non-temporal hint, for data read once in whole
// lines (the wave's 64 lanes cover contiguous lines).
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void stg16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

// silu(g) * u with the hardware reciprocal (1 ulp) in place of a division.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Inclusive prefix sum of one int per thread over a block of up to 1024
// threads (blockDim.x a multiple of 64).  `scratch` holds >= 16 ints.
__device__ __forceinline__ int block_inclusive_scan(int v, int* scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int n = __shfl_up(v, off, 64);
        if (lane >= off) v += n;
    }
    if (lane == 63) scratch[wave] = v;
    __syncthreads();
    if (wave == 0) {
        const int nw = blockDim.x >> 6;
        int s = lane < nw ? scratch[lane] : 0;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            int n = __shfl_up(s, off, 64);
            if (lane >= off) s += n;
        }
        if (lane < nw) scratch[lane] = s;
    }
    __syncthreads();
    int r = v + (wave > 0 ? scratch[wave - 1] : 0);
    __syncthreads();
    return r;
}

}  // namespace moe
