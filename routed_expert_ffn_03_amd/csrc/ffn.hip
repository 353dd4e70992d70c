// Grouped expert FFN: y_sorted[i] = (silu(x_t W_gate^T) * (x_t W_up^T)) W_down^T
// for every sorted row i of every expert's route list.
//
// Sources: busy experts run as GEMMs on reconstructed weights and the others
// on a separate path (dsv41-flash-offload wiki, opening paragraph and
// repository file table: busy-expert GEMM and stock group-kernel entries);
// the split point is the "fat threshold", 32 rows by default (recipe page
// "DeepSeek-V4.1-Flash / RTX 3090", step 3 environment block); oversized
// route lists are cut into batches that share one read of the expert's
// weights (wiki file table, segment patch entry).  The SwiGLU form of the
// expert is this library's reading; the pages do not give it.
//
// Schedule (all on the caller's stream, counts known only on the device):
//   build_tiles   one block: per-expert row counts -> 128-row "fat" M-tiles for
//                 experts with >= fat_threshold rows, 32-row "thin" M-tiles
//                 for the rest; tile lists + totals into the workspace.
//   phase 1       gate/up: fat kernel, then thin kernel; SwiGLU fused in the
//                 epilogue; the activation a is stored fp16 [P, I].
//   phase 2       down: fat kernel, then thin kernel; y stored fp16 [P, H].
//
// Fat kernel (MFMA-bound at large M): persistent, one 256-thread block per CU,
// work item = (N-tile, M-tile) with the M-tile index fastest so consecutive
// items share one expert weight tile; items are spread so each XCD walks a
// contiguous range of them (its own L2 sees the shared weight tile).  Tile
// 128 rows x 256 weight rows x 64 k, double-buffered in LDS (96 KB) with an
// XOR swizzle that keeps 16-byte reads conflict-free; each wave owns 64 rows
// x 128 weight rows = 2 x 4 MFMA 32x32x16 accumulators.  Phase 1's 256
// weight rows are 128 gate rows and the matching 128 up rows, so every wave
// holds gate and up for the same outputs and applies SwiGLU in registers.
//
// Thin kernel (HBM-bound): persistent, several blocks per CU, work item =
// (32 weight rows, thin M-tile); the four waves split the reduction index and
// stream weights straight from HBM into MFMA operands (no LDS staging: every
// weight element is used once), 4 chunks in flight per lane, then reduce the
// four partial tiles through LDS.  Phase 1 items carry 16 gate + 16 up rows.
//
// Precision: fp32 accumulation; a in fp16; the down projection runs on fp16
// MFMA with W_down converted to fp16 when staged.  3-bit weights are decoded
// to bf16 (phase 1) or fp16 (phase 2) as they are staged.
#include "common.h"
#include "kernels.h"

#include <mutex>

namespace moe {
namespace {

struct MTile {
    int32_t e, row0, rows, pad;
};

struct FfnHeader {
    int32_t n_fat, n_thin;
    int32_t pad[62];
};

constexpr int FAT_BM = 128;
constexpr int FAT_BN_ROWS = 256;          // weight rows per fat tile
constexpr int FAT_BK = 64;
constexpr int FAT_THREADS = 256;
constexpr int FAT_STAGE = (FAT_BM + FAT_BN_ROWS) * 8;   // 16-byte chunks per stage
constexpr int THIN_BM = 32;
constexpr int THIN_THREADS = 256;
constexpr int THIN_DEPTH = 4;             // chunks in flight per lane

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
    int k, H, I;
    uint16_t* act;
    uint16_t* y;
    const FfnHeader* hdr;
    const MTile* fat;
    const MTile* thin;
};

// ------------------------------------------------------------ tile builder

__global__ __launch_bounds__(1024)
void build_tiles_kernel(const int32_t* __restrict__ offsets, int E, int thr, FfnHeader* __restrict__ hdr,
                        MTile* __restrict__ fat, MTile* __restrict__ thin) {
    __shared__ int scratch[16];
    const int e = threadIdx.x;
    int n = 0, nf = 0, nt = 0, r0 = 0;
    if (e < E) {
        r0 = offsets[e];
        n = offsets[e + 1] - r0;
        if (n >= thr) nf = (n + FAT_BM - 1) / FAT_BM;
        else nt = (n + THIN_BM - 1) / THIN_BM;
    }
    const int fi = block_inclusive_scan(nf, scratch);
    const int ti = block_inclusive_scan(nt, scratch);
    for (int i = 0; i < nf; ++i) {
        MTile m;
        m.e = e; m.row0 = r0 + i * FAT_BM; m.rows = min(FAT_BM, n - i * FAT_BM); m.pad = 0;
        fat[fi - nf + i] = m;
    }
    for (int i = 0; i < nt; ++i) {
        MTile m;
        m.e = e; m.row0 = r0 + i * THIN_BM; m.rows = min(THIN_BM, n - i * THIN_BM); m.pad = 0;
        thin[ti - nt + i] = m;
    }
    if (e == (int)blockDim.x - 1) {
        hdr->n_fat = fi;
        hdr->n_thin = ti;
    }
}

// ------------------------------------------------------------ weight loaders

// 3-bit group decode: the 8 weights k..k+7 (k % 8 == 0) of one output row.
// A group of 128 weights is 13 words; field f sits in word f/10 at bits
// 3*(f%10).  Eight consecutive fields span at most two words; they are
// gathered into one 24-bit run first.  weight = scale * (field - 4), computed
// exactly in fp32 as fma(field, s, -4s) and rounded once to the MFMA type.
template <bool TO_F16>
__device__ __forceinline__ u32x4 q3_chunk(const uint32_t* __restrict__ wrow, const uint16_t* __restrict__ srow,
                                          int k) {
    const int g = k >> 7, f0 = k & 127;
    const uint32_t* gw = wrow + g * Q3_WORDS;
    const int wlo = f0 / 10, n0 = f0 - wlo * 10;
    uint32_t bits = (gw[wlo] & 0x3FFFFFFFu) >> (3 * n0);   // bits 30-31 are not fields
    if (n0 > 2) bits |= gw[wlo + 1] << (30 - 3 * n0);
    const float s = (float)__builtin_bit_cast(_Float16, srow[g]);
    const float m4 = -4.0f * s;
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float v0 = fmaf((float)((bits >> (6 * i)) & 7u), s, m4);
        const float v1 = fmaf((float)((bits >> (6 * i + 3)) & 7u), s, m4);
        if (TO_F16) {
            const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
            r[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        } else {
            // round to nearest even bf16 (values are finite)
            uint32_t u0 = __float_as_uint(v0), u1 = __float_as_uint(v1);
            u0 += 0x7FFFu + ((u0 >> 16) & 1u);
            u1 += 0x7FFFu + ((u1 >> 16) & 1u);
            r[i] = (u0 >> 16) | (u1 & 0xFFFF0000u);
        }
    }
    return r;
}

// One weight row as seen by a loader: bf16 row pointer, or 3-bit words + scales.
struct WRow {
    const void* w;
    const uint16_t* s;
};

template <int WFMT>
__device__ __forceinline__ WRow weight_row(const void* base, const uint16_t* sbase, size_t row, int K) {
    WRow r;
    if (WFMT == 0) {
        r.w = reinterpret_cast<const uint16_t*>(base) + row * (size_t)K;
        r.s = nullptr;
    } else {
        const size_t groups = (size_t)(K >> 7);
        r.w = reinterpret_cast<const uint32_t*>(base) + row * groups * Q3_WORDS;
        r.s = sbase + row * groups;
    }
    return r;
}

// 8 weights k..k+7 of a row as an MFMA operand chunk: bf16 for phase 1, fp16
// for phase 2.
template <int WFMT, int PHASE>
__device__ __forceinline__ u32x4 load_w8(const WRow& r, int k) {
    if (WFMT == 0) {
        u32x4 v = ldg16(reinterpret_cast<const uint16_t*>(r.w) + k);
        return PHASE == 2 ? bf16x8_to_f16x8(v) : v;
    } else {
        return q3_chunk<PHASE == 2>(reinterpret_cast<const uint32_t*>(r.w), r.s, k);
    }
}

template <int PHASE>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return PHASE == 1 ? mfma_bf16(a, b, c) : mfma_f16(a, b, c);
}

__device__ __forceinline__ int logical_block() {
    const int G = gridDim.x, b = blockIdx.x;
    return (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
}

// ------------------------------------------------------------ fat kernel

template <int PHASE, int WFMT>
__global__ __launch_bounds__(FAT_THREADS, 1)
void ffn_fat_kernel(FfnArgs a) {
    __shared__ u32x4 smem[2 * FAT_STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int K = PHASE == 1 ? a.H : a.I;
    const int NT = PHASE == 1 ? a.I / 128 : a.H / 256;
    const int n_mt = a.hdr->n_fat;
    const int n_items = n_mt * NT;
    const int c = tid & 7, rb = tid >> 3;
    const int swz = (rb >> 1) & 7;          // rows rb + 32 i share it
    const int KT = K / FAT_BK;
    // weight-row groups of this wave (two 64-row groups of the 256 staged)
    const int bgrp0 = PHASE == 1 ? wn * 64 : wn * 128;
    const int bgrp1 = PHASE == 1 ? 128 + wn * 64 : wn * 128 + 64;

    for (int item = logical_block(); item < n_items; item += gridDim.x) {
        const int nt = item / n_mt, mt = item % n_mt;
        const MTile t = a.fat[mt];
        const uint16_t* arow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rb + 32 * i;
            arow[i] = nullptr;
            if (r < t.rows) {
                if (PHASE == 1) {
                    const int tok = a.sorted_pair[t.row0 + r] / a.k;
                    arow[i] = a.x + (size_t)tok * a.H;
                } else {
                    arow[i] = a.act + (size_t)(t.row0 + r) * a.I;
                }
            }
        }
        WRow brow[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = rb + 32 * i;
            if (PHASE == 1) {
                const int n = nt * 128 + (r & 127);
                brow[i] = r < 128 ? weight_row<WFMT>(a.wg, a.sg, (size_t)t.e * a.I + n, K)
                                  : weight_row<WFMT>(a.wu, a.su, (size_t)t.e * a.I + n, K);
            } else {
                brow[i] = weight_row<WFMT>(a.wd, a.sd, (size_t)t.e * a.H + nt * 256 + r, K);
            }
        }
        const bool act0 = wm * 64 < t.rows;        // this wave has rows to compute
        const bool act1 = wm * 64 + 32 < t.rows;

        u32x4 ar[4], br[8];
        auto gload = [&](int kt) {
            const int off = kt * FAT_BK + c * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ar[i] = u32x4{0, 0, 0, 0};
                if (arow[i]) ar[i] = ldg16(arow[i] + off);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) br[i] = load_w8<WFMT, PHASE>(brow[i], off);
        };
        auto sstore = [&](int stage) {
            u32x4* sA = smem + stage * FAT_STAGE;
            u32x4* sB = sA + FAT_BM * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) sA[(rb + 32 * i) * 8 + (c ^ swz)] = ar[i];
#pragma unroll
            for (int i = 0; i < 8; ++i) sB[(rb + 32 * i) * 8 + (c ^ swz)] = br[i];
        };

        f32x16 acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

        auto compute = [&](int stage) {
            const u32x4* sA = smem + stage * FAT_STAGE;
            const u32x4* sB = sA + FAT_BM * 8;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ch = 2 * s + (lane >> 5);
                u32x4 af[2], bfr[4];
#pragma unroll
                for (int ri = 0; ri < 2; ++ri) {
                    const int ra = wm * 64 + ri * 32 + (lane & 31);
                    af[ri] = sA[ra * 8 + (ch ^ ((ra >> 1) & 7))];
                }
#pragma unroll
                for (int cj = 0; cj < 4; ++cj) {
                    const int rw = ((cj >> 1) ? bgrp1 : bgrp0) + (cj & 1) * 32 + (lane & 31);
                    bfr[cj] = sB[rw * 8 + (ch ^ ((rw >> 1) & 7))];
                }
#pragma unroll
                for (int cj = 0; cj < 4; ++cj) {
                    acc[0][cj] = mma<PHASE>(af[0], bfr[cj], acc[0][cj]);
                    if (act1) acc[1][cj] = mma<PHASE>(af[1], bfr[cj], acc[1][cj]);
                }
            }
        };

        gload(0);
        sstore(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            if (kt + 1 < KT) gload(kt + 1);
            if (act0) compute(kt & 1);
            if (kt + 1 < KT) sstore((kt + 1) & 1);
            __syncthreads();
        }

        // epilogue: registers -> LDS (fp16) -> 16-byte row stores
        // MFMA 32x32 output layout: lane holds column (lane & 31) and rows
        // 8*(r>>2) + 4*(lane>>5) + (r&3) for r = 0..15.
        if (PHASE == 1) {
            constexpr int LD = 72;                               // halves per staged row
            uint16_t* sO = reinterpret_cast<uint16_t*>(smem) + wave * 64 * LD;
#pragma unroll
            for (int ri = 0; ri < 2; ++ri)
#pragma unroll
                for (int cj = 0; cj < 2; ++cj)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = ri * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        const int n = cj * 32 + (lane & 31);
                        sO[m * LD + n] = f32_to_f16_bits(silu_mul(acc[ri][cj][r], acc[ri][cj + 2][r]));
                    }
            __syncthreads();
            const int n0 = nt * 128 + wn * 64;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int m = it * 8 + (lane >> 3), ch = lane & 7;
                const int row = wm * 64 + m;
                if (row < t.rows)
                    stg16(a.act + (size_t)(t.row0 + row) * a.I + n0 + ch * 8,
                          *reinterpret_cast<const u32x4*>(sO + m * LD + ch * 8));
            }
        } else {
            constexpr int LD = 136;
            uint16_t* sO = reinterpret_cast<uint16_t*>(smem) + wave * 64 * LD;
#pragma unroll
            for (int ri = 0; ri < 2; ++ri)
#pragma unroll
                for (int cj = 0; cj < 4; ++cj)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = ri * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        const int n = cj * 32 + (lane & 31);
                        sO[m * LD + n] = f32_to_f16_bits(acc[ri][cj][r]);
                    }
            __syncthreads();
            const int n0 = nt * 256 + wn * 128;
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int m = it * 4 + (lane >> 4), ch = lane & 15;
                const int row = wm * 64 + m;
                if (row < t.rows)
                    stg16(a.y + (size_t)(t.row0 + row) * a.H + n0 + ch * 8,
                          *reinterpret_cast<const u32x4*>(sO + m * LD + ch * 8));
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ thin kernel

template <int PHASE, int WFMT>
__global__ __launch_bounds__(THIN_THREADS)
void ffn_thin_kernel(FfnArgs a) {
    __shared__ float red[4][16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 31, g = lane >> 5;
    const int K = PHASE == 1 ? a.H : a.I;
    const int NT = PHASE == 1 ? a.I / 16 : a.H / 32;
    const int n_mt = a.hdr->n_thin;
    const int n_items = n_mt * NT;
    const int Kw = K / 4;                   // reduction slice of this wave
    const int nch = Kw / 32;                // 32-k chunks: lane half g covers 16 of them
    const int kbase = wave * Kw + g * 16;

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int nt = item / n_mt, mt = item % n_mt;
        const MTile t = a.thin[mt];
        const uint16_t* arow = nullptr;
        if (m < t.rows) {
            if (PHASE == 1) arow = a.x + (size_t)(a.sorted_pair[t.row0 + m] / a.k) * a.H;
            else arow = a.act + (size_t)(t.row0 + m) * a.I;
        }
        WRow brow;
        if (PHASE == 1) {
            const size_t n = (size_t)t.e * a.I + nt * 16 + (m & 15);
            brow = m < 16 ? weight_row<WFMT>(a.wg, a.sg, n, K) : weight_row<WFMT>(a.wu, a.su, n, K);
        } else {
            brow = weight_row<WFMT>(a.wd, a.sd, (size_t)t.e * a.H + nt * 32 + m, K);
        }

        u32x4 ra[THIN_DEPTH][2], rw[THIN_DEPTH][2];
        auto load = [&](int ch, u32x4 (&xa)[2], u32x4 (&xw)[2]) {
            const int k0 = kbase + ch * 32;
            xa[0] = u32x4{0, 0, 0, 0};
            xa[1] = u32x4{0, 0, 0, 0};
            if (arow) {
                xa[0] = ldg16(arow + k0);
                xa[1] = ldg16(arow + k0 + 8);
            }
            xw[0] = load_w8<WFMT, PHASE>(brow, k0);
            xw[1] = load_w8<WFMT, PHASE>(brow, k0 + 8);
        };
        f32x16 acc = f32x16{};
#pragma unroll
        for (int d = 0; d < THIN_DEPTH - 1; ++d)
            if (d < nch) load(d, ra[d], rw[d]);
        for (int c0 = 0; c0 < nch; c0 += THIN_DEPTH) {
#pragma unroll
            for (int d = 0; d < THIN_DEPTH; ++d) {
                const int ch = c0 + d;
                if (ch + THIN_DEPTH - 1 < nch)
                    load(ch + THIN_DEPTH - 1, ra[(d + THIN_DEPTH - 1) % THIN_DEPTH],
                         rw[(d + THIN_DEPTH - 1) % THIN_DEPTH]);
                if (ch < nch) {
                    acc = mma<PHASE>(ra[d][0], rw[d][0], acc);
                    acc = mma<PHASE>(ra[d][1], rw[d][1], acc);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
        __syncthreads();
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
        __syncthreads();
    }
}

// ------------------------------------------------------------ host side

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct FfnLayout {
    size_t hdr, fat, thin, act, total;
    size_t max_fat, max_thin;
};

FfnLayout ffn_layout(int T, int E, int k, int H, int I) {
    (void)H;
    const size_t P = (size_t)T * k;
    const size_t nz = P < (size_t)E ? P : (size_t)E;        // experts that can be non-empty
    FfnLayout L;
    L.max_fat = P / FAT_BM + nz + 1;
    L.max_thin = P / THIN_BM + nz + 1;
    L.hdr = 0;
    L.fat = align256(sizeof(FfnHeader));
    L.thin = L.fat + align256(L.max_fat * sizeof(MTile));
    L.act = L.thin + align256(L.max_thin * sizeof(MTile));
    L.total = L.act + align256(P * (size_t)I * sizeof(uint16_t));
    return L;
}

struct DevInfo {
    int cus = 0;
    int thin_blocks[2][2] = {{0, 0}, {0, 0}};   // [wfmt][phase-1]
};

std::mutex g_dev_mu;
DevInfo g_dev[64];

template <int PHASE, int WFMT>
int thin_occupancy() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ffn_thin_kernel<PHASE, WFMT>, THIN_THREADS, 0) !=
        hipSuccess || n < 1)
        n = 1;
    return n;
}

hipError_t dev_info(DevInfo& out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DevInfo& d = g_dev[dev];
    if (d.cus == 0) {
        int cus = 0;
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return err;
        d.thin_blocks[0][0] = thin_occupancy<1, 0>();
        d.thin_blocks[0][1] = thin_occupancy<2, 0>();
        d.thin_blocks[1][0] = thin_occupancy<1, 1>();
        d.thin_blocks[1][1] = thin_occupancy<2, 1>();
        d.cus = cus;
    }
    out = d;
    return hipSuccess;
}

FfnArgs make_args(const FfnLaunch& a) {
    const FfnLayout L = ffn_layout(a.T, a.E, a.k, a.H, a.I);
    char* ws = reinterpret_cast<char*>(a.ws);
    FfnArgs fa;
    fa.x = a.x;
    fa.wg = a.wg; fa.wu = a.wu; fa.wd = a.wd;
    fa.sg = a.sg; fa.su = a.su; fa.sd = a.sd;
    fa.sorted_pair = a.sorted_pair;
    fa.k = a.k; fa.H = a.H; fa.I = a.I;
    fa.act = reinterpret_cast<uint16_t*>(ws + L.act);
    fa.y = a.y;
    fa.hdr = reinterpret_cast<FfnHeader*>(ws + L.hdr);
    fa.fat = reinterpret_cast<MTile*>(ws + L.fat);
    fa.thin = reinterpret_cast<MTile*>(ws + L.thin);
    return fa;
}

template <int PHASE, int WFMT>
void launch_phase_t(const FfnArgs& fa, const DevInfo& d, hipStream_t s) {
    ffn_fat_kernel<PHASE, WFMT><<<d.cus, FAT_THREADS, 0, s>>>(fa);
    ffn_thin_kernel<PHASE, WFMT><<<d.cus * d.thin_blocks[WFMT][PHASE - 1], THIN_THREADS, 0, s>>>(fa);
}

}  // namespace

size_t ffn_ws_bytes(int T, int E, int k, int H, int I) { return ffn_layout(T, E, k, H, I).total; }

hipError_t launch_ffn_plan(const FfnLaunch& a, hipStream_t s) {
    const FfnLayout L = ffn_layout(a.T, a.E, a.k, a.H, a.I);
    char* ws = reinterpret_cast<char*>(a.ws);
    build_tiles_kernel<<<1, 1024, 0, s>>>(a.offsets, a.E, a.fat_threshold,
                                          reinterpret_cast<FfnHeader*>(ws + L.hdr),
                                          reinterpret_cast<MTile*>(ws + L.fat),
                                          reinterpret_cast<MTile*>(ws + L.thin));
    return hipGetLastError();
}

hipError_t launch_ffn_phase(const FfnLaunch& a, int phase, hipStream_t s) {
    DevInfo d;
    hipError_t err = dev_info(d);
    if (err != hipSuccess) return err;
    const FfnArgs fa = make_args(a);
    if (phase == 1) {
        if (a.wfmt == 0) launch_phase_t<1, 0>(fa, d, s);
        else launch_phase_t<1, 1>(fa, d, s);
    } else {
        if (a.wfmt == 0) launch_phase_t<2, 0>(fa, d, s);
        else launch_phase_t<2, 1>(fa, d, s);
    }
    return hipGetLastError();
}

}  // namespace moe
