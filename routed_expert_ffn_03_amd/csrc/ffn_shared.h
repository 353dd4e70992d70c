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
    int T, k, H, I;
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

// Where the FFN part of a workspace keeps its header and tile lists.
struct FfnPlanPtrs {
    FfnHeader* hdr;
    MTile* fat;
    MTile* thin;
};
FfnPlanPtrs ffn_plan_ptrs(int T, int E, int k, int H, int I, int wfmt, void* ffn_ws);

// Route + permute + plan in one block (front.hip), for 1 <= T <= FRONT_MAX_T.
constexpr int FRONT_MAX_T = 64;
hipError_t launch_route_permute_plan(const float* logits, int T, int E, int k, int fat_threshold, int32_t* topk_ids,
                                     float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                     int32_t* pair_to_sorted, const FfnPlanPtrs& pp, hipStream_t s);

// The bf16 MFMA-tile kernels with two waves per SIMD (fat8.hip): the device's
// LDS limit is raised for them on first use; `phase` 1 = gate/up, 2 = down.
hipError_t launch_fat8_phase(const FfnArgs& fa, int phase, int cus, hipStream_t s);

}  // namespace moe
