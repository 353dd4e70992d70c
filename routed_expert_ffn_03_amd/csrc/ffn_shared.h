// Work lists and kernel arguments shared by the grouped-FFN kernels
// (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "lds_dma.h"

namespace moe {

// One M-tile of an expert's route list: rows [row0, row0 + rows) of the
// sorted pairs; `first` / `count` locate all M-tiles of the same expert.
struct MTile {
    int32_t e, row0, rows, first, count, pad[3];
};

struct FfnHeader {
    int32_t n_fat, n_thin;
    int32_t tail_next[2];         // fat items handed out past the static rounds, per phase
    int32_t tail_done[2];         // blocks past their last item; the last one re-zeroes both counters
    int32_t pad[58];
};

// The fat kernels walk their items in static rounds (block b: item b, b + G,
// ...).  In the gate/up phase the last partial round and the three full
// rounds before it are handed out instead one item at a time from a counter,
// as blocks finish: item costs vary with the M-tile's row tiles, and the
// static split alone leaves the busiest CU ~7% above the mean at the 16k chunk
// (the dynamic tail gains 2% there; the shorter down kernel loses 1-2% with
// it and stays static).
constexpr int FAT_TAIL_ROUNDS = 3;

constexpr int FAT_BM = 256;              // rows per fat M-tile
constexpr int FAT_THREADS = 256;
constexpr int THIN_BM = 32;
constexpr int THIN_THREADS = 256;

constexpr int Q3_WORDS = 13;

struct FfnArgs {
    const uint16_t* x;
    const void* wg;
    const void* wu;
    const void* wd;
    const uint16_t* sg;
    const uint16_t* su;
    const uint16_t* sd;
    const int32_t* sorted_pair;
    int T, k, H, I, E;
    int pairs;                    // weight format 2: row-pair layout, gate/up bf16, W_down fp16
    uint16_t* act;
    uint16_t* y;
    uint16_t* xq;                 // 3-bit thin path: x rows in pair-slot order per 128-group
    uint32_t* xs;                 // ... and each (token, group) sum of x as a bf16 hi, lo pair
    const FfnHeader* hdr;
    const MTile* fat;
    const MTile* thin;
};

__device__ __forceinline__ int logical_block() {
    const int G = gridDim.x, b = blockIdx.x;
    return (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
}


// Fat work item -> (M-tile, N-tile).  The items of one expert (count M-tiles
// x NT N-tiles) are contiguous: its M-tiles are split into ceil(count / 8)
// blocks of near-equal size s (at most 8), and within a block the items run
// N-tile by N-tile with the s M-tiles of each N-tile next to each other.  The
// 32 consecutive items that the blocks of one XCD take at a time then cover s
// activation tiles and about 32 / s weight tiles, each fetched once into that
// XCD's L2 and shared.
__device__ __forceinline__ void fat_item(const MTile* __restrict__ fat, int item, int NT, MTile& t, int& nt) {
    const int q0 = item / NT;
    const MTile t0 = fat[q0];
    const int me = t0.count, local = item - t0.first * NT;
    const int nblk = (me + 7) >> 3;
    const int q = me / nblk, r = me - q * nblk;              // r blocks of q + 1 M-tiles, then blocks of q
    const int big = (q + 1) * NT;
    int s, m0, off;
    if (local < r * big) {
        const int b = local / big;
        s = q + 1; m0 = b * s; off = local - b * big;
    } else {
        const int l2 = local - r * big, b = l2 / (q * NT);
        s = q; m0 = r * (q + 1) + b * q; off = l2 - b * q * NT;
    }
    nt = off / s;
    t = fat[t0.first + m0 + (off - nt * s)];
}

// The M-tiles of expert e (route list rows [r0, r0 + n)): nf fat tiles from
// index f0 of the fat list or nt thin (32-row) tiles from index t0 of the
// thin list.  The expert's 32-row tiles are spread evenly over its nf
// M-tiles, so the M-tiles of one expert cost the same and walk the weights in
// step.
__device__ __forceinline__ void write_expert_tiles(int e, int r0, int n, int nf, int nt, int f0, int t0,
                                                   MTile* __restrict__ fat, MTile* __restrict__ thin) {
    const int rt = (n + 31) >> 5;
    for (int i = 0; i < nf; ++i) {
        const int rt0 = i * (rt / nf) + min(i, rt % nf);
        const int rti = rt / nf + (i < rt % nf ? 1 : 0);
        MTile m = {};
        m.e = e; m.row0 = r0 + 32 * rt0; m.rows = min(32 * rti, n - 32 * rt0);
        m.first = f0; m.count = nf;
        fat[f0 + i] = m;
    }
    for (int i = 0; i < nt; ++i) {
        MTile m = {};
        m.e = e; m.row0 = r0 + i * THIN_BM; m.rows = min(THIN_BM, n - i * THIN_BM);
        m.first = t0; m.count = nt;
        thin[t0 + i] = m;
    }
}

// The four waves' partial 32 x 32 tiles of one thin item are summed through
// LDS; wave 0 stores the result (the barriers wait for LDS traffic only,
// so loads of later work issued before them stay in flight): phase 1 silu(gate) * up for the 16 gate
// columns (the up partner sits 16 lanes over), phase 2 the 32 y columns.
template <int PHASE>
__device__ __forceinline__ void thin_reduce_store(const FfnArgs& a, const f32x16& acc, const MTile& t, int nt,
                                                  float (&red)[4][16][64], int wave, int lane) {
    const int m = lane & 31, g = lane >> 5;
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
    lds_barrier();
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float v = red[0][r][lane] + red[1][r][lane] + red[2][r][lane] + red[3][r][lane];
            const int row = 8 * (r >> 2) + 4 * g + (r & 3);
            if (PHASE == 1) {
                const float u = __shfl(v, (lane + 16) & 63, 64);
                if (m < 16 && row < t.rows)
                    a.act[(size_t)(t.row0 + row) * a.I + nt * 16 + m] = f32_to_f16_bits(silu_mul(v, u));
            } else {
                if (row < t.rows) a.y[(size_t)(t.row0 + row) * a.H + nt * 32 + m] = f32_to_f16_bits(v);
            }
        }
    }
    lds_barrier();
}

// bf16 thin phases with the weights streamed through LDS (stream.hip)
bool stream_fits(int phase, int T, int k, int H, int I);
hipError_t launch_stream_phase(const FfnArgs& fa, int phase, int blocks, hipStream_t s);
int stream_occupancy(int phase);

// Wait until at most `stages` stages of this wave's loads are outstanding
// (loads complete in issue order, L load instructions per stage).
template <int L>
__device__ __forceinline__ void vm_wait_stages(int stages) {
    switch (stages) {
        case 0: vm_wait<0>(); break;
        case 1: vm_wait<L>(); break;
        case 2: vm_wait<2 * L>(); break;
        case 3: vm_wait<3 * L>(); break;
        case 4: vm_wait<4 * L>(); break;
        default: vm_wait<5 * L>(); break;
    }
}

constexpr int DMA_BK = 32;                                  // k per LDS stage
constexpr uint32_t DMA_ROW = DMA_BK * 2;                    // bytes of one row per stage
constexpr uint32_t DMA_OPER = FAT_BM * DMA_ROW;             // 16 KB: 256 rows of one operand

// ------------------------------------------------------------ 3-bit pair slots
//
// The gate/up thin path for tiles of at most 16 rows feeds the MFMA with the
// 3-bit codes themselves: the bf16 number 128 + u (bits 0x4300 | u) is exact,
// and two of them come out of one packed 16-bit shift and one and-or when the
// pair is fields i and i + 5 of a word (bits 3i and 3i + 15).  Slot 2P and
// 2P + 1 of a 128-group hold pair P: fields 10w + i and 10w + i + 5 for
// P = 5w + i < 60, fields 120 + i and 125 + i for P = 60 + i < 63, and fields
// 123, 124 for P = 63.  The activations are stored in the same slot order
// (the MFMA sums over k in any order), and
//   sum_k x_k (u_k - 4) = sum_k x_k (128 + u_k) - 132 sum_k x_k,
// the last term through one more MFMA step against the group sum of x.
__host__ __device__ constexpr int pair_field(int slot) {
    const int P = slot >> 1, hi = slot & 1;
    if (P == 63) return 123 + hi;
    const int a = P < 60 ? 10 * (P / 5) + P % 5 : 120 + (P - 60);
    return a + 5 * hi;
}

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

// bf16 pair (128 + u_a, 128 + u_b) of pair P from the group's 13 words;
// `magic` holds 0x43004300 in a VGPR, so the mask and the or are one
// v_and_or_b32 (a VOP3 instruction reads at most one SGPR or constant here)
template <int P>
__device__ __forceinline__ uint32_t magic_pair(const uint32_t (&w)[Q3_WORDS], uint32_t magic) {
    if constexpr (P == 63) {
        return ((w[12] >> 9) & 7u) | (((w[12] >> 12) & 7u) << 16) | magic;
    } else {
        constexpr int W = P < 60 ? P / 5 : 12, I = P < 60 ? P % 5 : P - 60;
        const u16x2 v = __builtin_bit_cast(u16x2, w[W] << 1);
        const u16x2 sh = {(unsigned short)(3 * I + 1), (unsigned short)(3 * I)};
        return (__builtin_bit_cast(uint32_t, v >> sh) & 0x00070007u) | magic;
    }
}


// One 128-group of a token's x row in pair-slot order (dst) and the group's
// sum of x, summed in fp64 and stored as a bf16 hi, lo pair (sum_dst).  src
// and dst may be global or LDS; both 16-byte aligned.
__device__ __forceinline__ void q3_prep_group(const uint16_t* src16, uint16_t* dst16, uint32_t* sum_dst) {
    const u32x4* src = reinterpret_cast<const u32x4*>(src16);
    u32x4* dst = reinterpret_cast<u32x4*>(dst16);
    uint32_t v[64];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const u32x4 q = src[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = q[j];
    }
    auto half = [&](int f) -> uint32_t { return (v[f >> 1] >> (16 * (f & 1))) & 0xFFFFu; };
    double sum = 0.0;
#pragma unroll
    for (int f = 0; f < 128; ++f) sum += (double)__uint_as_float(half(f) << 16);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = 4 * i + j;
            o[j] = half(pair_field(2 * d)) | (half(pair_field(2 * d + 1)) << 16);
        }
        dst[i] = o;
    }
    const __bf16 hi = (__bf16)(float)sum;
    const __bf16 lo = (__bf16)(float)(sum - (double)(float)hi);
    *sum_dst = (uint32_t)__builtin_bit_cast(uint16_t, hi) | ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
}

// Part `part` of `parts` (a power of two up to 16) of q3_prep_group for a
// bf16 row already in LDS: the slot chunks 16 part / parts .. of one group,
// and the fp64 sum of those chunks' fields, returned for the caller to add
// across the parts (exact, so in any order, while a group's magnitudes span
// less than about 2^38; beyond that the order of the partial sums decides
// the rounding of the group sum).
__device__ __forceinline__ double q3_prep_part_lds(const uint16_t* src16, uint16_t* dst16, int part, int parts) {
    u32x4* dst = reinterpret_cast<u32x4*>(dst16);
    const int per = 16 / parts, i0 = part * per;
    double sum = 0.0;
    for (int i = i0; i < i0 + per; ++i) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = 4 * i + j;
            const uint32_t lo = src16[pair_field(2 * d)], hi = src16[pair_field(2 * d + 1)];
            sum += (double)__uint_as_float(lo << 16) + (double)__uint_as_float(hi << 16);
            o[j] = lo | (hi << 16);
        }
        dst[i] = o;
    }
    return sum;
}

// A bf16 group sum as the (hi, lo) pair of q3_prep_group
__device__ __forceinline__ uint32_t q3_sum_pair_bf16(double sum) {
    const __bf16 h = (__bf16)(float)sum;
    const __bf16 l = (__bf16)(float)(sum - (double)(float)h);
    return (uint32_t)__builtin_bit_cast(uint16_t, h) | ((uint32_t)__builtin_bit_cast(uint16_t, l) << 16);
}

// The same for an fp16 row (the activations of the down phase): the slots
// for the fp16 products with the codes as the exact fp16 numbers 1024 + u
// (bits 0x6400 | u), and the group sum as an fp16 hi, lo pair.  Each field
// is read where it lies, one 16-bit load per field in slot order, so no
// 128-value group is held in registers; the fp64 sum of 128 fp16 values is
// exact, so the order of the additions does not matter.
__device__ __forceinline__ void q3_prep_group_f16(const uint16_t* src16, uint16_t* dst16, uint32_t* sum_dst) {
    u32x4* dst = reinterpret_cast<u32x4*>(dst16);
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = 4 * i + j;
            const uint16_t lo = src16[pair_field(2 * d)], hi = src16[pair_field(2 * d + 1)];
            sum += (double)(float)__builtin_bit_cast(_Float16, lo) + (double)(float)__builtin_bit_cast(_Float16, hi);
            o[j] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        dst[i] = o;
    }
    const _Float16 h = (_Float16)(float)sum;
    const _Float16 l = (_Float16)(float)(sum - (double)h);
    *sum_dst = (uint32_t)__builtin_bit_cast(uint16_t, h) | ((uint32_t)__builtin_bit_cast(uint16_t, l) << 16);
}

// Where the FFN part of a workspace keeps its header and tile lists.
struct FfnPlanPtrs {
    FfnHeader* hdr;
    MTile* fat;
    MTile* thin;
};
FfnPlanPtrs ffn_plan_ptrs(int T, int E, int k, int H, int I, int wfmt, void* ffn_ws);

// The 3-bit gate/up streaming kernel for decode batches (q3dec.hip): every
// tile thin, at most Q3DEC_MAX_T tokens whose x rows fit in LDS.  Returns
// false (and launches nothing) for shapes it does not take.
constexpr int Q3DEC_MAX_T = 14;
bool q3dec_fits(int T, int E, int k, int H);
hipError_t launch_q3dec_gate_up(const FfnArgs& fa, int cus, hipStream_t s);

// Route + permute + plan in one block (front.hip), for 1 <= T <= FRONT_MAX_T.
constexpr int FRONT_MAX_T = 64;
hipError_t launch_route_permute_plan(const float* logits, int T, int E, int k, int fat_threshold, int32_t* topk_ids,
                                     float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                     int32_t* pair_to_sorted, const FfnPlanPtrs& pp, hipStream_t s);

// The bf16 MFMA-tile kernels with two waves per SIMD (fat8.hip): the device's
// LDS limit is raised for them on first use; `phase` 1 = gate/up, 2 = down.
hipError_t launch_fat8_phase(const FfnArgs& fa, int phase, int cus, hipStream_t s);

}  // namespace moe
