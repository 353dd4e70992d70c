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
//   build_tiles   one block: per-expert row counts -> "fat" M-tiles of up to
//                 256 rows (equal multiples of 32) for experts with at least
//                 fat_threshold rows, 32-row "thin" M-tiles for the rest; tile
//                 lists + totals into the workspace (front.hip does the same
//                 inside its single-block route + permute + plan launch).
//   phase 1       gate/up: fat kernel, then thin kernel; SwiGLU fused in the
//                 epilogue; the activation a is stored fp16 [P, I].
//   phase 2       down: fat kernel, then thin kernel; y stored fp16 [P, H].
//
// Fat kernels (MFMA-bound at large M): persistent, one block per CU, 256-row
// M-tiles x 256 weight rows (phase 1: 128 gate rows + the matching 128 up
// rows, so SwiGLU is applied to accumulators in registers), operands staged
// in LDS by direct-to-LDS buffer loads.  bf16 weights: fat8.hip (eight waves,
// two per SIMD taking turns between MFMA clusters and operand traffic).  3-bit
// weights: ffn_fat_kernel below (four waves side by side, the 3-bit words
// decoded into MFMA operands between the MFMAs).  Work items of one expert
// are walked so that 32 consecutive items, which run on one XCD, share
// activation and weight tiles in that XCD's L2.
//
// Thin kernels (HBM-bound): persistent, several blocks per CU, work item =
// (32 weight rows, thin M-tile); the four waves split the reduction index,
// stream the weights and reduce the four partial tiles through LDS.  Phase 1
// items carry 16 gate + 16 up rows.  bf16 weights: stream.hip (whole-line
// non-temporal loads through a per-wave LDS ring); the kernel below, which
// loads the MFMA operand layout straight into registers, only where a wave's
// quarter of K is not a multiple of 64.  3-bit: ffn_thin_q3_kernel below, and
// q3dec.hip for the gate/up of decode batches (every tile thin, at most 14
// tokens).
//
// Precision: fp32 accumulation; a in fp16; the down projection runs on fp16
// MFMA with W_down converted to fp16 when staged.  3-bit weights are decoded
// to bf16 (phase 1) or fp16 (phase 2), or enter the MFMA as exact codes
// (pair-slot path).
#include "common.h"
#include "ffn_shared.h"
#include "kernels.h"
#include "lds_dma.h"

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace moe {
namespace {

// ------------------------------------------------------------ tile builder

__global__ __launch_bounds__(1024)
void build_tiles_kernel(const int32_t* __restrict__ offsets, int E, int thr, FfnHeader* __restrict__ hdr,
                        MTile* __restrict__ fat, MTile* __restrict__ thin, int32_t* __restrict__ counts) {
    __shared__ int scratch[16];
    const int e = threadIdx.x;
    int n = 0, nf = 0, nt = 0, r0 = 0;
    if (e < E) {
        r0 = offsets[e];
        n = offsets[e + 1] - r0;
        if (counts) counts[e] = n;                       // the load histogram, when asked for
        if (n >= thr) nf = (n + FAT_BM - 1) / FAT_BM;
        else nt = (n + THIN_BM - 1) / THIN_BM;
    }
    const int fi = block_inclusive_scan(nf, scratch);
    const int ti = block_inclusive_scan(nt, scratch);
    write_expert_tiles(e, r0, n, nf, nt, fi - nf, ti - nt, fat, thin);
    if (e == (int)blockDim.x - 1) {
        hdr->n_fat = fi;
        hdr->n_thin = ti;
        hdr->tail_next[0] = hdr->tail_next[1] = 0;
        hdr->tail_done[0] = hdr->tail_done[1] = 0;
    }
}

template <int PHASE>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return PHASE == 1 ? mfma_bf16(a, b, c) : mfma_f16(a, b, c);
}

// ------------------------------------------------------------ fat kernel

// Wait until at most N of this wave's LDS reads are outstanding; the operand
// registers the wait is for are tied to it, so no use of them is scheduled
// before it.
template <int N>
__device__ __forceinline__ void lds_wait_frag(u32x4 (&x)[8], u32x4 (&y)[2]) {
    asm volatile("s_waitcnt lgkmcnt(%10)"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]),
                   "+v"(y[0]), "+v"(y[1])
                 : "n"(N)
                 : "memory");
}

// 3-bit field at bit OFF as one v_bfe_u32 (left to the compiler, a constant
// offset becomes a shift, a mask and a byte conversion: one more instruction)
template <int OFF>
__device__ __forceinline__ uint32_t field3(uint32_t bits) {
    uint32_t r;
    asm("v_bfe_u32 %0, %1, %2, 3" : "=v"(r) : "v"(bits), "n"(OFF));
    return r;
}

// Ring stage layout of the fat kernel per weight format.  bf16: activations
// and weight rows, 16 KB each, 64-byte rows.  3-bit: activations, the four
// packed words of each weight row that hold the stage's 32 k (16 bytes) and
// the dword holding the row's group scale.  LOADS: load instructions per wave
// per stage; AHEAD: how many stages past the one being computed must have
// landed at its barrier (the 3-bit kernel decodes one stage ahead).
template <int WFMT>
struct FatStage;
template <>
struct FatStage<0> {
    static constexpr uint32_t BYTES = 2 * DMA_OPER;
    static constexpr int LOADS = 8, AHEAD = 1;
};
template <>
struct FatStage<1> {
    static constexpr uint32_t RAW = FAT_BM * 16, SCL = FAT_BM * 4;
    static constexpr uint32_t BYTES = DMA_OPER + RAW + SCL;
    static constexpr int LOADS = 6, AHEAD = 2;
};

template <int WFMT, int NS>
constexpr size_t fat_lds_bytes() {
    return (size_t)NS * FatStage<WFMT>::BYTES;
}

// Epilogue: wave w holds every row tile of its 64 weight rows (phase 1: 32
// gate rows and the matching 32 up rows, i.e. 32 output columns; phase 2: 64
// output columns).  Passes of 64 rows through LDS, 16-byte row stores (MFMA
// 32x32 output: lane holds column n, rows 8 (r >> 2) + 4 g + (r & 3)).  Phase
// 1 stores silu(gate) * up as fp16 activations, phase 2 fp16 y rows.  RT is a
// compile-time constant and the epilogue runs inside the K-loop instantiation
// of that count, so the accumulators never merge across instantiations (a
// merge would route all of them through VGPRs).
template <int PHASE, int RT>
__device__ __forceinline__ void fat_epilogue(const FfnArgs& a, const f32x16 (&acc)[8][2], const MTile& t, int nt,
                                             u32x4* smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int N = PHASE == 1 ? a.I : a.H;
    constexpr int OC = PHASE == 1 ? 32 : 64;            // output columns per wave
    constexpr int LD = OC + 8;                          // staged row length (halves)
    uint16_t* sO = reinterpret_cast<uint16_t*>(smem) + wave * 64 * LD;
    uint16_t* dst = PHASE == 1 ? a.act : a.y;
    const int col0 = PHASE == 1 ? nt * 128 + 32 * wave : nt * 256 + 64 * wave;
    static_for<(RT + 1) / 2>([&](auto pass_c) {
        constexpr int PASS = decltype(pass_c)::value;
        static_for<2>([&](auto h_c) {
            constexpr int H = decltype(h_c)::value, RI = 2 * PASS + H;
            if constexpr (RI < RT) {
                static_for<PHASE == 1 ? 1 : 2>([&](auto cj_c) {
                    constexpr int CJ = decltype(cj_c)::value;
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = H * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                        const float v = PHASE == 1 ? silu_mul(acc[RI][0][r], acc[RI][1][r]) : acc[RI][CJ][r];
                        sO[m * LD + CJ * 32 + n] = f32_to_f16_bits(v);
                    }
                });
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        __syncthreads();
        constexpr int LPR = OC / 8;                     // lanes per staged row
#pragma unroll
        for (int it = 0; it < LPR; ++it) {
            const int m = it * (64 / LPR) + lane / LPR, ch = lane % LPR;
            const int row = PASS * 64 + m;
            if (row < t.rows)
                stg16(dst + (size_t)(t.row0 + row) * N + col0 + ch * 8,
                      *reinterpret_cast<const u32x4*>(sO + m * LD + ch * 8));
        }
        __syncthreads();
    });
}

// One 16-k step: MFMA slot i (row tile i / 2, column tile i % 2) for the RT
// row tiles, each preceded by side(i); slots past the last MFMA still run
// their side work, in order.  Scheduling barriers keep exactly this order,
// so the side work (LDS reads, loads, the stage barrier, conversions, 3-bit
// decode) issues while the MFMA before it executes.
template <int PHASE, int RT, class Side>
__device__ __forceinline__ void step_slots(f32x16 (&acc)[8][2], const u32x4 (&af)[8], const u32x4 (&bf)[2],
                                           Side&& side) {
    static_for<16>([&](auto i) {
        constexpr int I = decltype(i)::value;
        side(i);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (I / 2 < RT) {
            acc[I / 2][I % 2] = mma<PHASE>(af[I / 2], bf[I % 2], acc[I / 2][I % 2]);
            __builtin_amdgcn_sched_barrier(0);
        }
    });
}

// The packed words and scale dwords one lane reads to decode its weights of
// one stage: for 16-k step s and column tile c, the word holding its first
// field (lo) and the next one (hi); the scale dword of each of its two rows.
struct Q3Raw {
    uint32_t lo[2][2], hi[2][2], sc[2];
};

// Fat tile: 256 rows x 256 weight rows with the four waves side by side
// (1 x 4).  Wave w owns weight rows [64 w, 64 w + 64) of the tile as two
// 32-row column tiles (phase 1: gate rows 32 w.. and the matching up rows
// 128 + 32 w.., so SwiGLU is applied in registers) against every 32-row tile
// of the M-tile; all waves therefore have the same number of row tiles, and
// each wave prepares only the weight operands its own MFMAs use (the bf16 ->
// fp16 conversion of phase 2, or the 3-bit decode).  Operands stream through
// a ring of NS stages of 32 k filled by direct-to-LDS buffer loads (16 rows x
// 64 bytes per instruction for activations and bf16 weights); LDS rows are 64
// bytes with the 16-byte chunk c of row r at position c ^ ((r >> 2) & 3), so
// each 16-lane group of a fragment read covers all banks once.  Stages
// kt+1 .. kt+NS-1 are in flight while stage kt is computed; one barrier per
// stage frees the slot just read.
//
// 3-bit weights: during stage kt every lane reads, for both of its weight rows
// and both 16-k steps of stage kt+1, the packed word holding its first field
// and the next one (field f of a group sits in word f / 10 at bit 3 (f % 10)),
// and decodes the 32 weights (scale * (field - 4), exact in fp32, rounded once)
// in 16 pieces placed between the MFMAs of stage kt.  No decoded weight goes
// through LDS: b128 LDS writes are the scarce LDS resource.
template <int PHASE, int WFMT, int NS>
__global__ __launch_bounds__(FAT_THREADS, 1)
void ffn_fat_kernel(FfnArgs a) {
    using Stage = FatStage<WFMT>;
    static_assert(NS >= 2 + Stage::AHEAD - 1 && NS - 1 <= 5, "ring depth outside the wait table");
    extern __shared__ u32x4 smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int n = lane & 31, g = lane >> 5;
    const int K = PHASE == 1 ? a.H : a.I;
    const int N = PHASE == 1 ? a.I : a.H;
    constexpr int BN = PHASE == 1 ? 128 : 256;
    const int NT = N / BN;
    const int n_items = a.hdr->n_fat * NT;
    const int KT = K / DMA_BK;                                // a multiple of 4 (K % 128 == 0)
    const __amdgpu_buffer_rsrc_t asrc = PHASE == 1
        ? make_rsrc(a.x, (uint32_t)((size_t)a.T * a.H * 2))
        : make_rsrc(a.act, (uint32_t)((size_t)a.T * a.k * a.I * 2));
    const size_t wmat = (size_t)a.I * a.H;
    const size_t wbytes = WFMT == 0 ? wmat * 2 : wmat / 128 * Q3_WORDS * 4;
    const size_t sbytes = wmat / 128 * 2;
    const int GR = K >> 7;                                    // 3-bit scale groups per weight row
    const uint32_t q3_row_bytes = (uint32_t)GR * (Q3_WORDS * 4);
    // load roles: activation instruction q of this wave fills rows 64 q + 16
    // wave + L/4 (so the first (RT + 1) / 2 instructions cover the RT row tiles
    // of a tile, on every wave alike), weight instruction q rows 64 wave + 16 q
    // + L/4; the chunk landing at position L%4 is (L%4) ^ ((row >> 2) & 3)
    const int lrow = 64 * wave + (lane >> 2);
    const uint32_t lch16 = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
    const uint32_t sbase = lds_addr(smem);
    // fragment reads: chunk 2 s + g of row r, swizzled by (r >> 2) & 3 = (n >> 2) & 3
    uint32_t aoffs[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) aoffs[s] = (uint32_t)n * DMA_ROW + (uint32_t)(((2 * s + g) ^ ((n >> 2) & 3)) * 16);
    // the two weight rows (tile rows) of this lane's B operands: column tiles 0 and 1
    const int brow[2] = {PHASE == 1 ? 32 * wave + n : 64 * wave + n,
                         PHASE == 1 ? 128 + 32 * wave + n : 64 * wave + 32 + n};

    const int n_static = PHASE == 1 ? max(0, n_items / (int)gridDim.x - FAT_TAIL_ROUNDS) * (int)gridDim.x : n_items;
    FfnHeader* const hdr = const_cast<FfnHeader*>(a.hdr);
    volatile int* const bcast = reinterpret_cast<volatile int*>(smem);   // ring slot 0 is free between items
    int item = logical_block();
    for (;;) {
        if (PHASE == 1 && item >= n_static) {
            // tail round: the next unclaimed item, the same for the whole block
            __syncthreads();
            if (threadIdx.x == 0) bcast[0] = n_static + atomicAdd(&hdr->tail_next[PHASE - 1], 1);
            __syncthreads();
            item = __builtin_amdgcn_readfirstlane(bcast[0]);
            __syncthreads();                                  // every wave has it before the ring is refilled
        }
        if (item >= n_items) break;
        MTile t;
        int nt;
        fat_item(a.fat, item, NT, t, nt);
        const int rt = (t.rows + 31) >> 5;                   // row tiles with data, the same for every wave

        // waves 0-1 load gate rows, waves 2-3 the matching up rows (phase 1)
        const char* wmatp = reinterpret_cast<const char*>(PHASE == 1 ? (wave < 2 ? a.wg : a.wu) : a.wd);
        const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(wmatp + t.e * wbytes, (uint32_t)wbytes);
        // activation rows and bf16 weight rows this lane loads (rows past the
        // M-tile repeat its last row; their results are never stored)
        uint32_t aoff[4], boff[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = lrow + 16 * q;
            const int r = min(64 * q + 16 * wave + (lane >> 2), t.rows - 1);
            const uint32_t src = PHASE == 1 ? (uint32_t)(a.sorted_pair[t.row0 + r] / a.k) : (uint32_t)(t.row0 + r);
            aoff[q] = src * (uint32_t)K * 2u + lch16;
            const uint32_t wrow = PHASE == 1 ? (uint32_t)(nt * 128 + (row & 127)) : (uint32_t)(nt * 256 + row);
            boff[q] = wrow * (uint32_t)K * 2u + lch16;
        }
        // 3-bit: this lane loads the words and the scale of tile row 64 wave + lane
        __amdgpu_buffer_rsrc_t ssrc = wsrc;
        uint32_t roff = 0, sidx = 0, spar[2] = {0, 0};
        if constexpr (WFMT == 1) {
            const char* smatp = reinterpret_cast<const char*>(PHASE == 1 ? (wave < 2 ? a.sg : a.su) : a.sd);
            ssrc = make_rsrc(smatp + t.e * sbytes, (uint32_t)sbytes);
            const int lr = 64 * wave + lane;
            const uint32_t lgr = PHASE == 1 ? (uint32_t)(nt * 128 + (lr & 127)) : (uint32_t)(nt * 256 + lr);
            roff = lgr * q3_row_bytes;
            sidx = lgr * (uint32_t)GR;
            // the scale of group grp sits in the high half of its dword when (row * GR + grp) is odd
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint32_t gr = PHASE == 1 ? (uint32_t)(nt * 128 + (brow[c] & 127)) : (uint32_t)(nt * 256 + brow[c]);
                spar[c] = (gr * (uint32_t)GR) & 1u;
            }
        }

        f32x16 acc[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

        // load instruction q of stage kt into ring slot `slot`: q < 4 the
        // activation rows; then bf16: the weight rows (q = 4..7); 3-bit: the
        // packed words (q = 4) and the scale dwords (q = 5)
        auto issue_one = [&](int kt, int slot, int q) {
            char* st = reinterpret_cast<char*>(smem) + slot * Stage::BYTES;
            if (q < 4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(asrc, (lds_ptr_t)(st + (4 * q + wave) * 1024), 16, aoff[q],
                                                         kt * DMA_ROW, 0, 0);
            else if constexpr (WFMT == 0)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc, (lds_ptr_t)(st + DMA_OPER + (4 * wave + q - 4) * 1024),
                                                         16, boff[q - 4], kt * DMA_ROW, 0, 0);
            else if (q == 4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc, (lds_ptr_t)(st + DMA_OPER + wave * 1024), 16, roff,
                                                         (kt >> 2) * (Q3_WORDS * 4) + (kt & 3) * 12, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ssrc, (lds_ptr_t)(st + DMA_OPER + Stage::RAW + wave * 256), 4,
                                                         ((sidx + (uint32_t)(kt >> 2)) >> 1) * 4u, 0, 0, 0);
        };
        // bf16: fragment j of 16-k step s in ring slot `slot` (j < RT: activation
        // row tile j; RT + c: weight column tile c; larger j: nothing)
        auto read_one = [&](auto rt_c, auto j_c, int slot, int s, u32x4 (&af)[8], u32x4 (&bf)[2]) {
            constexpr int RT = decltype(rt_c)::value, J = decltype(j_c)::value;
            const uint32_t st = sbase + slot * Stage::BYTES;
            if constexpr (J < RT)
                af[J] = ds_read16<J * 32 * DMA_ROW>(st + aoffs[s]);
            else if constexpr (J < RT + 2)
                bf[J - RT] = ds_read16<0>(st + DMA_OPER + (uint32_t)brow[J - RT] * DMA_ROW +
                                          (uint32_t)(((2 * s + g) ^ ((n >> 2) & 3)) * 16));
        };
        // activation fragments of 16-k step s (row tiles 0..RT-1) and, for
        // bf16 weights, the two weight fragments
        auto reads = [&](auto rt_c, int slot, int s, u32x4 (&af)[8], u32x4 (&bf)[2]) {
            constexpr int RT = decltype(rt_c)::value;
            const uint32_t st = sbase + slot * Stage::BYTES;
            const uint32_t aa = st + aoffs[s];
            static_for<RT>([&](auto r_c) {
                constexpr int R = decltype(r_c)::value;
                af[R] = ds_read16<R * 32 * DMA_ROW>(aa);
            });
            if constexpr (WFMT == 0) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    bf[c] = ds_read16<0>(st + DMA_OPER + (uint32_t)brow[c] * DMA_ROW +
                                         (uint32_t)(((2 * s + g) ^ ((n >> 2) & 3)) * 16));
            }
        };
        // 3-bit: packed words and scales of stage kt (in `slot`) for this lane;
        // a `hi` word past the row's four (never used: its fields land above
        // bit 23) is the next row's first word
        auto rreads = [&](int slot, int kt, Q3Raw& rw) {
            const uint32_t rb = sbase + slot * Stage::BYTES + DMA_OPER;
            const int j = kt & 3;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int f0 = 32 * j + 16 * s + 8 * g;        // first field (group-relative)
                const uint32_t wo = (uint32_t)(f0 / 10 - 3 * j) * 4u;
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    rw.lo[s][c] = ds_read4(rb + (uint32_t)brow[c] * 16u + wo);
                    rw.hi[s][c] = ds_read4(rb + (uint32_t)brow[c] * 16u + wo + 4u);
                }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) rw.sc[c] = ds_read4(rb + FatStage<1>::RAW + (uint32_t)brow[c] * 4u);
        };
        auto rwait = [&](Q3Raw& rw) {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(rw.lo[0][0]), "+v"(rw.lo[0][1]), "+v"(rw.lo[1][0]), "+v"(rw.lo[1][1]),
                           "+v"(rw.hi[0][0]), "+v"(rw.hi[0][1]), "+v"(rw.hi[1][0]), "+v"(rw.hi[1][1]),
                           "+v"(rw.sc[0]), "+v"(rw.sc[1])
                         :
                         : "memory");
        };
        // 3-bit decode piece P of stage kt: chunk C = P / 4 (step C / 2, column
        // tile C % 2), weights 2 Q and 2 Q + 1 of its 8 (Q = P % 4); one
        // bit-field extract, one conversion and one fma per weight
        auto piece = [&](auto p_c, int kt, const Q3Raw& rw, uint32_t (&bits)[4], float (&sf)[2], float (&m4)[2],
                         u32x4 (&bo)[2][2]) {
            constexpr int P = decltype(p_c)::value, C = P / 4, Q = P % 4, S = C / 2, CJ = C % 2;
            if constexpr (P == 0) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const uint32_t sb = ((spar[c] + (uint32_t)(kt >> 2)) & 1u) ? (rw.sc[c] >> 16) : (rw.sc[c] & 0xFFFFu);
                    sf[c] = (float)__builtin_bit_cast(_Float16, (uint16_t)sb);
                    m4[c] = -4.0f * sf[c];
                }
            }
            if constexpr (Q == 0) {
                const int sh = 3 * ((32 * (kt & 3) + 16 * S + 8 * g) % 10);
                bits[C] = ((rw.lo[S][CJ] & 0x3FFFFFFFu) >> sh) | (rw.hi[S][CJ] << (30 - sh));
            }
            const float v0 = fmaf((float)field3<6 * Q>(bits[C]), sf[CJ], m4[CJ]);
            const float v1 = fmaf((float)field3<6 * Q + 3>(bits[C]), sf[CJ], m4[CJ]);
            if constexpr (PHASE == 2) {
                const f16x2 h = {(_Float16)v0, (_Float16)v1};
                bo[S][CJ][Q] = __builtin_bit_cast(uint32_t, h);
            } else {
                const bf16x2 h = {(__bf16)v0, (__bf16)v1};
                bo[S][CJ][Q] = __builtin_bit_cast(uint32_t, h);
            }
        };

        u32x4 B0[2][2], B1[2][2];
        auto kloop = [&](auto rt_c) {
            constexpr int RT = decltype(rt_c)::value, S = 2 * RT;
            constexpr int BAR = S / 4;                               // step-1 slot of the stage barrier
            // loads per stage: the activation instructions that reach the RT
            // row tiles, then the weight (or packed word and scale) instructions
            constexpr int LA = (RT + 1) / 2;
            constexpr int LOADS = LA + Stage::LOADS - 4;
            auto issue_i = [&](int kt, int slot, int i) { issue_one(kt, slot, i < LA ? i : i - LA + 4); };
            auto issue_all = [&](int kt, int slot) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) issue_i(kt, slot, i);
            };
            // prologue: the whole ring in flight; stage 0 (and for 3-bit weights
            // stage 1) landed; 3-bit: stage 0 decoded into B0
            const int pro = min(NS, KT);
            for (int s = 0; s < pro; ++s) issue_all(s, s);
            vm_wait_stages<LOADS>(pro - Stage::AHEAD);
            __builtin_amdgcn_s_barrier();
            if constexpr (WFMT == 1) {
                Q3Raw rw;
                uint32_t bits[4];
                float sf[2], m4[2];
                rreads(0, 0, rw);
                rwait(rw);
                static_for<16>([&](auto p) { piece(p, 0, rw, bits, sf, m4, B0); });
            }

            static_assert(BAR + LOADS < 16, "the refill loads follow the barrier inside step 1");
            static_assert(WFMT != 0 || (LOADS <= 8 && 2 * (15 - BAR) >= RT + 2),
                          "bf16: one refill load per odd slot of step 0, next-step reads after the barrier");
            u32x4 x0[8], x1[8], y0[2], y1[2];
            reads(rt_c, 0, 0, x0, y0);
            int slot = 0;
            if constexpr (WFMT == 0) {
                // per stage kt: the even slots of step 0 read step 1's fragments
                // (two per slot) and the odd slots refill the slot that stage kt-1
                // used with stage kt-1+NS (one load per slot; every wave finished
                // reading it before the previous barrier); step 1 waits for stage
                // kt+1, passes the barrier and reads stage kt+1's first step, two
                // fragments per slot.  No slot issues a burst of loads or reads
                // that would hold the wave while its MFMA pipe drains (the four
                // waves leave a barrier together and would queue all their
                // loads at once).
                auto stage = [&](int kt, auto more_c) {
                    constexpr bool more = decltype(more_c)::value;
                    const int nslot = slot + 1 == NS ? 0 : slot + 1;
                    const int pslot = slot == 0 ? NS - 1 : slot - 1;
                    const bool refill = kt >= 1 && kt - 1 + NS < KT;
                    lds_wait_frag<0>(x0, y0);
                    __builtin_amdgcn_sched_barrier(0);
                    step_slots<PHASE, RT>(acc, x0, y0, [&](auto i) {
                        constexpr int I = decltype(i)::value;
                        if constexpr (PHASE == 2 && I < 2) y0[I] = bf16x8_to_f16x8(y0[I]);
                        if constexpr (I % 2 == 0) {
                            read_one(rt_c, std::integral_constant<int, I>{}, slot, 1, x1, y1);
                            read_one(rt_c, std::integral_constant<int, I + 1>{}, slot, 1, x1, y1);
                        } else {
                            if constexpr (I / 2 < LOADS)
                                if (refill) issue_i(kt - 1 + NS, pslot, I / 2);
                        }
                    });
                    lds_wait_frag<0>(x1, y1);
                    __builtin_amdgcn_sched_barrier(0);
                    step_slots<PHASE, RT>(acc, x1, y1, [&](auto i) {
                        constexpr int I = decltype(i)::value;
                        if constexpr (PHASE == 2 && I < 2) y1[I] = bf16x8_to_f16x8(y1[I]);
                        if constexpr (I == BAR && more) {
                            vm_wait_stages<LOADS>(min(NS - 2, KT - 2 - kt));   // stage kt+1 landed here
                            __builtin_amdgcn_s_barrier();                              // ... and in every lane
                        }
                        if constexpr (I > BAR && more) {
                            read_one(rt_c, std::integral_constant<int, 2 * (I - BAR - 1)>{}, nslot, 0, x0, y0);
                            read_one(rt_c, std::integral_constant<int, 2 * (I - BAR - 1) + 1>{}, nslot, 0, x0, y0);
                        }
                    });
                    slot = nslot;
                };
                for (int kt = 0; kt + 1 < KT; ++kt) stage(kt, std::true_type{});
                stage(KT - 1, std::false_type{});
            } else {
                // per stage: step 0 issues step 1's activation reads and the next
                // stage's packed words; the next stage's weights are decoded in 16
                // pieces over the MFMA slots of step 0 and of step 1 up to the
                // barrier; at the barrier this stage's slot is free and the stage
                // after next has landed
                constexpr int DW = S >= 8 ? 3 : (S >= 4 ? 1 : 0);    // step-0 slot of the words' wait
                constexpr int AV0 = S > DW + 1 ? S - DW - 1 : 0;     // decode slots in step 0
                constexpr int AV = AV0 + BAR;                        // ... and in step 1
                // stage kt computes with bc and decodes stage kt+1 into bn
                auto stage = [&](int kt, auto more_c, u32x4 (&bc)[2][2], u32x4 (&bn)[2][2]) {
                    constexpr bool more = decltype(more_c)::value;
                    const int nslot = slot + 1 == NS ? 0 : slot + 1;
                    Q3Raw rw;
                    uint32_t bits[4];
                    float sf[2], m4[2];
                    auto pieces_at = [&](auto step_c, auto slot_c) {
                        constexpr int STEP = decltype(step_c)::value, I = decltype(slot_c)::value;
                        static_for<16>([&](auto p_c) {
                            constexpr int P = decltype(p_c)::value;
                            constexpr int G = AV > 0 ? P * AV / 16 : 0;
                            constexpr int ST = (AV == 0 || G < AV0) ? 0 : 1;
                            constexpr int SL = AV == 0 ? DW + 1 : (G < AV0 ? DW + 1 + G : G - AV0);
                            if constexpr (more && ST == STEP && SL == I) piece(p_c, kt + 1, rw, bits, sf, m4, bn);
                        });
                    };
                    using St0 = std::integral_constant<int, 0>;
                    using St1 = std::integral_constant<int, 1>;
                    lds_wait_frag<0>(x0, y0);
                    __builtin_amdgcn_sched_barrier(0);
                    step_slots<PHASE, RT>(acc, x0, bc[0], [&](auto i) {
                        constexpr int I = decltype(i)::value;
                        if constexpr (I == 0) {
                            reads(rt_c, slot, 1, x1, y1);
                            if constexpr (more) rreads(nslot, kt + 1, rw);
                        }
                        if constexpr (I == DW && more) rwait(rw);
                        pieces_at(St0{}, i);
                    });
                    lds_wait_frag<0>(x1, y1);
                    __builtin_amdgcn_sched_barrier(0);
                    step_slots<PHASE, RT>(acc, x1, bc[1], [&](auto i) {
                        constexpr int I = decltype(i)::value;
                        pieces_at(St1{}, i);
                        if constexpr (I == BAR && more) {
                            vm_wait_stages<LOADS>(max(0, min(NS - 3, KT - 3 - kt)));
                            __builtin_amdgcn_s_barrier();
                        }
                        if constexpr (I > BAR && I <= BAR + LOADS) {
                            if (kt + NS < KT) issue_i(kt + NS, slot, I - BAR - 1);     // one load per MFMA slot
                        }
                        if constexpr (I == BAR + 2 && more) reads(rt_c, nslot, 0, x0, y0);
                    });
                    slot = nslot;
                };
                for (int kt = 0; kt + 2 < KT; kt += 2) {
                    stage(kt, std::true_type{}, B0, B1);
                    stage(kt + 1, std::true_type{}, B1, B0);
                }
                stage(KT - 2, std::true_type{}, B0, B1);
                stage(KT - 1, std::false_type{}, B1, B0);
            }
            __syncthreads();
            fat_epilogue<PHASE, RT>(a, acc, t, nt, smem);
        };
        switch (rt) {
            case 8: kloop(std::integral_constant<int, 8>{}); break;
            case 7: kloop(std::integral_constant<int, 7>{}); break;
            case 6: kloop(std::integral_constant<int, 6>{}); break;
            case 5: kloop(std::integral_constant<int, 5>{}); break;
            case 4: kloop(std::integral_constant<int, 4>{}); break;
            case 3: kloop(std::integral_constant<int, 3>{}); break;
            case 2: kloop(std::integral_constant<int, 2>{}); break;
            default: kloop(std::integral_constant<int, 1>{}); break;
        }
        item += gridDim.x;                                   // static rounds; the tail refetches
    }
    // the last block out re-zeroes the counters for the next launch: every
    // block's claims precede its exit count
    if (PHASE == 1 && threadIdx.x == 0) {
        __threadfence();
        if (atomicAdd(&hdr->tail_done[PHASE - 1], 1) == (int)gridDim.x - 1) {
            atomicExch(&hdr->tail_next[PHASE - 1], 0);
            atomicExch(&hdr->tail_done[PHASE - 1], 0);
        }
    }
}

typedef __attribute__((ext_vector_type(4), aligned(4))) uint32_t u32x4a4;   // 4-byte aligned 16-byte load

// For every token of a thin tile of at most 16 rows: its x row in pair-slot
// order per 128-group (xq) and each group sum of x, summed in fp64 and stored
// as bf16 hi + lo (xs).  A token in several thin tiles is written with the
// same values each time.
__global__ __launch_bounds__(256)
void q3_xprep_kernel(FfnArgs a) {
    const int NG = a.H >> 7;
    const int per_tile = 16 * NG;
    const int n_tasks = a.hdr->n_thin * per_tile;
    for (int task = blockIdx.x * 256 + threadIdx.x; task < n_tasks; task += gridDim.x * 256) {
        const int mt = task / per_tile, rem = task - mt * per_tile;
        const int m = rem / NG, G = rem - m * NG;
        const MTile t = a.thin[mt];
        if (t.rows > 16 || m >= t.rows) continue;
        const size_t tok = (size_t)(a.sorted_pair[t.row0 + m] / a.k);
        q3_prep_group(a.x + tok * a.H + (size_t)G * 128, a.xq + tok * a.H + (size_t)G * 128, a.xs + tok * NG + G);
    }
}

// ------------------------------------------------------------ thin kernels

// CW: 16-byte pieces per lane and row per chunk; lane half g covers 8*CW
// consecutive k of a 16*CW-wide chunk.  D: chunks in the register ring (D - 1
// in flight).  Used with CW = 2 (any K that is a multiple of 128); K a
// multiple of 256 goes to the streaming kernel of stream.hip instead.
template <int PHASE, int CW>
__global__ __launch_bounds__(THIN_THREADS)
void ffn_thin_kernel(FfnArgs a) {
    constexpr int D = CW == 4 ? 2 : 4;
    __shared__ float red[4][16][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
    const int m = lane & 31, g = lane >> 5;
    const int K = PHASE == 1 ? a.H : a.I;
    const int NT = PHASE == 1 ? a.I / 16 : a.H / 32;
    const int n_mt = a.hdr->n_thin;
    const int n_items = n_mt * NT;
    const int Kw = K / 4;                   // reduction slice of this wave
    const int nch = Kw / (16 * CW);         // chunks: lane half g covers 8 CW k of each
    const int kbase = wave * Kw + g * 8 * CW;

    // an item's operand rows: the activation row of lane m (null past the
    // tile) and the weight row (phase 1: gate rows nt*16.. for m < 16 and the
    // matching up rows, phase 2: down rows nt*32 + m)
    auto rows_of = [&](const MTile& t, int nt, int src, const uint16_t*& arow, const uint16_t*& brow) {
        arow = nullptr;
        if (m < t.rows) arow = PHASE == 1 ? a.x + (size_t)src * a.H : a.act + (size_t)(t.row0 + m) * a.I;
        if (PHASE == 1) {
            const size_t n = (size_t)t.e * a.I + nt * 16 + (m & 15);
            brow = reinterpret_cast<const uint16_t*>(m < 16 ? a.wg : a.wu) + n * (size_t)K;
        } else {
            brow = reinterpret_cast<const uint16_t*>(a.wd) + ((size_t)t.e * a.H + nt * 32 + m) * (size_t)K;
        }
    };
    // phase 1: the token of lane m's row (loaded one item ahead)
    auto token_of = [&](const MTile& t) { return PHASE == 1 && m < t.rows ? a.sorted_pair[t.row0 + m] / a.k : 0; };

    u32x4 ra[D][CW], rw[D][CW];
    const uint16_t* arow;
    const uint16_t* brow;
    auto load = [&](int ch, u32x4 (&xa)[CW], u32x4 (&xw)[CW]) {
        const int k0 = kbase + ch * 16 * CW;
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            xa[c] = u32x4{0, 0, 0, 0};
            if (arow) xa[c] = ldg16(arow + k0 + 8 * c);
        }
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const u32x4 v = ldg16(brow + k0 + 8 * c);
            xw[c] = PHASE == 2 ? bf16x8_to_f16x8(v) : v;       // fp16 MFMA for the down projection
        }
    };
    // the first D - 1 chunks of an item go out before the previous item's
    // reduction, so a block's loads do not drain between items
    auto prologue = [&]() {
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (d < nch) load(d, ra[d], rw[d]);
    };

    int item = blockIdx.x;
    MTile t{};
    int nt = 0;
    if (item < n_items) {
        nt = item / n_mt;
        t = a.thin[item % n_mt];
        rows_of(t, nt, token_of(t), arow, brow);
        prologue();
    }
    while (item < n_items) {
        const int next = item + (int)gridDim.x;
        MTile tn{};
        int ntn = 0, srcn = 0;
        if (next < n_items) {
            ntn = next / n_mt;
            tn = a.thin[next % n_mt];
            srcn = token_of(tn);
        }
        f32x16 acc = f32x16{};
        for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int ch = c0 + d;
                if (ch + D - 1 < nch) load(ch + D - 1, ra[(d + D - 1) % D], rw[(d + D - 1) % D]);
                if (ch < nch) {
#pragma unroll
                    for (int c = 0; c < CW; ++c) acc = mma<PHASE>(ra[d][c], rw[d][c], acc);
                }
            }
        }
        if (next < n_items) {
            rows_of(tn, ntn, srcn, arow, brow);
            prologue();
        }
        thin_reduce_store<PHASE>(a, acc, t, nt, red, wave, lane);
        item = next;
        t = tn;
        nt = ntn;
    }
}

// One gate/up item of the 3-bit thin kernel for a tile of at most 16 rows,
// on the pair-slot operands (see q3_xprep_kernel): lanes m < 16 carry the
// activations of group 2p in k-half 0 and lanes m >= 16 those of group 2p + 1
// in k-half 1, so accumulator rows 0..15 collect the first group's sums and
// rows 16..31 the second's for the same tokens; each pair ends with the
// 132 x group-sum step, and the two groups' fp16 scales are applied in fp32.
__device__ __forceinline__ void thin_q3_pairs(const FfnArgs& a, const MTile& t, int nt,
                                              __amdgpu_buffer_rsrc_t xqsrc, __amdgpu_buffer_rsrc_t xssrc,
                                              float (&red)[4][16][64], int wave, int lane) {
    constexpr uint32_t NOWHERE = 0xFFFFFF00u;
    const int m = lane & 31, g = lane >> 5, mm = m & 15;
    const int NG = a.H >> 7, NP = (NG + 1) >> 1;
    const size_t mat_words = (size_t)a.I * NG * Q3_WORDS;
    const bool act_lane = (m >> 4) == g && mm < t.rows;
    uint32_t xo = 0, so = 0;
    if (act_lane) {
        const uint32_t tok = (uint32_t)(a.sorted_pair[t.row0 + mm] / a.k);
        xo = tok * (uint32_t)a.H * 2u;
        so = tok * (uint32_t)NG * 4u;
    }
    // this lane's weight row: gate rows nt*16.. (m < 16), then the matching up
    // rows; plain global loads (the two matrices would make a buffer resource
    // lane-dependent)
    const int row = nt * 16 + mm;
    const uint32_t* wrow = reinterpret_cast<const uint32_t*>(m < 16 ? a.wg : a.wu) + (size_t)t.e * mat_words +
                           (size_t)row * NG * Q3_WORDS;
    const uint16_t* srow = (m < 16 ? a.sg : a.su) + ((size_t)t.e * a.I + row) * NG;
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic));

    // the 13 words of group 2p+g of this lane's row, and the row's scales of groups 2p and 2p+1
    struct Pair {
        uint32_t w[Q3_WORDS];
        uint16_t s0, s1;
    };
    auto load_pair = [&](int p, Pair& q) {
        const int G = min(2 * p + g, NG - 1);     // past an odd count: a real group whose sums are zero
        const uint32_t* gw = wrow + G * Q3_WORDS;
        const u32x4a4 q0 = *reinterpret_cast<const u32x4a4*>(gw);
        const u32x4a4 q1 = *reinterpret_cast<const u32x4a4*>(gw + 4);
        const u32x4a4 q2 = *reinterpret_cast<const u32x4a4*>(gw + 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q.w[i] = q0[i];
            q.w[4 + i] = q1[i];
            q.w[8 + i] = q2[i];
        }
        q.w[12] = gw[12];
        q.s0 = srow[2 * p];
        q.s1 = srow[min(2 * p + 1, NG - 1)];
    };

    // offsets of the activation slots and of the group sum of pair p for this
    // lane (past the buffers -- zeros -- off its half, past the groups or p)
    auto act_off = [&](int p) { return act_lane && 2 * p + g < NG ? xo + (uint32_t)(2 * p + g) * 256u : NOWHERE; };
    auto sum_off = [&](int p) { return act_lane && 2 * p + g < NG ? so + (uint32_t)(2 * p + g) * 4u : NOWHERE; };

    float fin[8] = {};
    Pair cur, nxt;
    u32x4 av[16];
    uint32_t xsum = 0;
    if (wave < NP) {
        load_pair(wave, cur);
        const uint32_t ao = act_off(wave);
#pragma unroll
        for (int j = 0; j < 16; ++j) av[j] = __builtin_amdgcn_raw_buffer_load_b128(xqsrc, ao, 16 * j, 0);
        xsum = __builtin_amdgcn_raw_buffer_load_b32(xssrc, sum_off(wave), 0, 0);
    }
    for (int p = wave; p < NP; p += 4) {
        const bool more = p + 4 < NP;
        if (more) load_pair(p + 4, nxt);         // next pair's words in flight during this one
        // each activation register is refilled with the next pair's slots
        // right after its MFMA has read it
        const uint32_t aon = more ? act_off(p + 4) : NOWHERE;
        f32x16 c = f32x16{};
        static_for<16>([&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            u32x4 bv;
            static_for<4>([&](auto q_c) {
                constexpr int Q = decltype(q_c)::value;
                bv[Q] = magic_pair<4 * J + Q>(cur.w, magic);
            });
            c = mfma_bf16(av[J], bv, c);
            av[J] = __builtin_amdgcn_raw_buffer_load_b128(xqsrc, aon, 16 * J, 0);
        });
        // minus 132 x (group sum, as bf16 hi + lo): exact bf16 weights -132 in k-slots 0 and 1 of each half
        c = mfma_bf16(u32x4{xsum, 0u, 0u, 0u}, u32x4{0xC304C304u, 0u, 0u, 0u}, c);
        xsum = __builtin_amdgcn_raw_buffer_load_b32(xssrc, more ? sum_off(p + 4) : NOWHERE, 0, 0);
        const float s0 = (float)__builtin_bit_cast(_Float16, cur.s0);
        const float s1 = 2 * p + 1 < NG ? (float)__builtin_bit_cast(_Float16, cur.s1) : 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) fin[r] = fmaf(s1, c[r + 8], fmaf(s0, c[r], fin[r]));
        cur = nxt;
    }
    f32x16 acc = f32x16{};
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = fin[r];
    thin_reduce_store<1>(a, acc, t, nt, red, wave, lane);
}

// One lane's 13 packed words of a 52-byte group: three 16-byte loads and one
// 4-byte load (groups are 4-byte aligned)
__device__ __forceinline__ void load_q3_group(const uint32_t* gw, uint32_t (&w)[Q3_WORDS]) {
    const u32x4a4 q0 = *reinterpret_cast<const u32x4a4*>(gw);
    const u32x4a4 q1 = *reinterpret_cast<const u32x4a4*>(gw + 4);
    const u32x4a4 q2 = *reinterpret_cast<const u32x4a4*>(gw + 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[i] = q0[i];
        w[4 + i] = q1[i];
        w[8 + i] = q2[i];
    }
    w[12] = gw[12];
}

// What one lane of thin_q3_pairs_down reads of expert e's W_down for one
// group pair p: row nt*32 + L % 32, group 2 p + L / 32 and the pair's two
// scales (indexes clamped to the row's last group: a pair past the end loads
// real words, which the item does not use or scales by 0)
struct PairW {
    uint32_t w[Q3_WORDS];
    uint16_t s0, s1;
};

__device__ __forceinline__ void pair_load(const FfnArgs& a, int e, int nt, int p, int lane, PairW& o) {
    const int m = lane & 31, g = lane >> 5;
    const int NG = a.I >> 7;
    const size_t row = (size_t)e * a.H + nt * 32 + m;
    load_q3_group(reinterpret_cast<const uint32_t*>(a.wd) + (row * NG + min(2 * p + g, NG - 1)) * Q3_WORDS, o.w);
    const uint16_t* srow = a.sd + row * NG;
    o.s0 = srow[min(2 * p, NG - 1)];
    o.s1 = srow[min(2 * p + 1, NG - 1)];
}

// One down item of a decode batch (a tile of at most 16 rows) on pair-slot
// operands, as thin_q3_pairs: the tile's activation rows are in LDS in slot
// order (xl: XR + 1 rows of K halves, the last all zeros; xsl: their group
// sums, an fp16 hi, lo pair per row and group), the codes enter the fp16
// products as 1024 + u and each pair ends with the -1028 x group-sum step.
// The 32 output columns are the W_down rows nt*32 + n.  The wave's first
// pair comes in `pf`, loaded ahead by the caller; with the item's last
// products issued, `pf` is loaded with the first pair of the next item
// (expert next_e, column tile next_nt; none if next_e < 0), in flight over
// this item's reduction.
template <int XR>
__device__ __forceinline__ void thin_q3_pairs_down(const FfnArgs& a, const MTile& t, int nt, const uint16_t* xl,
                                                   const uint32_t* xsl, float (&red)[4][16][64], int wave,
                                                   int lane, PairW& pf, int next_e, int next_nt) {
    const int m = lane & 31, g = lane >> 5, mm = m & 15;
    const int K = a.I, NG = K >> 7, NP = (NG + 1) >> 1;
    const bool act_lane = (m >> 4) == g && mm < t.rows;
    const int xr = act_lane ? mm : XR;                  // LDS row of this lane's activations
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

    float fin[8] = {};
    PairW cur = pf, nxt;
    for (int p = wave; p < NP; p += 4) {
        if (p + 4 < NP) pair_load(a, t.e, nt, p + 4, lane, nxt);   // next pair's words in flight during this one
        const int G = 2 * p + g;
        const u32x4* xa = reinterpret_cast<const u32x4*>(xl + (size_t)(G < NG ? xr : XR) * K) + 16 * min(G, NG - 1);
        const uint32_t xsum = G < NG ? xsl[xr * NG + G] : 0u;     // (row XR: zeros)
        f32x16 c = f32x16{};
        static_for<16>([&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            u32x4 bv;
            static_for<4>([&](auto q_c) {
                constexpr int Q = decltype(q_c)::value;
                bv[Q] = magic_pair<4 * J + Q>(cur.w, magic);
            });
            c = mfma_f16(xa[J], bv, c);
        });
        // minus 1028 x (group sum, as fp16 hi + lo): exact fp16 weights -1028 in k-slots 0 and 1 of each half
        c = mfma_f16(u32x4{xsum, 0u, 0u, 0u}, u32x4{0xE404E404u, 0u, 0u, 0u}, c);
        const float s0 = (float)__builtin_bit_cast(_Float16, cur.s0);
        const float s1 = 2 * p + 1 < NG ? (float)__builtin_bit_cast(_Float16, cur.s1) : 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) fin[r] = fmaf(s1, c[r + 8], fmaf(s0, c[r], fin[r]));
        cur = nxt;
    }
    // (not above the products: the next pair's words would need registers of
    // their own while this one's are still read)
    __builtin_amdgcn_sched_barrier(0);
    if (next_e >= 0 && wave < NP) pair_load(a, next_e, next_nt, wave, lane, pf);
    // the four waves' partials meet in LDS: lane (m, g) holds column m of
    // rows 4 g + r and 8 + 4 g + r (r < 4); the barriers wait for LDS traffic
    // only, so the loads issued above stay in flight; wave 0 stores
#pragma unroll
    for (int r = 0; r < 8; ++r) red[wave][r][lane] = fin[r];
    lds_barrier();
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float v = red[0][r][lane] + red[1][r][lane] + red[2][r][lane] + red[3][r][lane];
            const int row = 8 * (r >> 2) + 4 * g + (r & 3);
            if (row < t.rows) a.y[(size_t)(t.row0 + row) * a.H + nt * 32 + m] = f32_to_f16_bits(v);
        }
    }
    lds_barrier();
}

// What one lane of thin_q3_quads_down reads of expert e's W_down for one quad
// p of groups: rows nt*32 + n and nt*32 + 16 + n (n = L % 16), group 4 p + q
// (q = L / 16; past the last group, the last group, which the item scales by 0)
struct QuadW {
    uint32_t w0[Q3_WORDS], w1[Q3_WORDS];
    uint16_t s0, s1;
};

__device__ __forceinline__ void quad_load(const FfnArgs& a, int e, int nt, int p, int lane, QuadW& o) {
    const int n = lane & 15, q = lane >> 4;
    const int NG = a.I >> 7;
    const int Gc = min(4 * p + q, NG - 1);
    const size_t row0 = (size_t)e * a.H + nt * 32 + n;
    const uint32_t* wr0 = reinterpret_cast<const uint32_t*>(a.wd) + (row0 * NG + Gc) * Q3_WORDS;
    load_q3_group(wr0, o.w0);
    load_q3_group(wr0 + (size_t)16 * NG * Q3_WORDS, o.w1);
    const uint16_t* sr0 = a.sd + row0 * NG + Gc;
    o.s0 = sr0[0];
    o.s1 = sr0[(size_t)16 * NG];
}

// The same item for a tile of at most 4 rows on 16x16x32 products: lane
// quarter q (L / 16) holds group 4 p + q of its weight row in k-quarter q,
// and the activation lanes of row 4 q + i hold token i of that group there,
// so the 16 result rows are 4 groups x 4 tokens (no padding rows: half the
// MFMA work of the 32-row tiles per weight).  Each group's scale is applied
// on its own result rows; the four groups of a token are then summed across
// the lane quarters.  Columns: W_down rows nt*32 + n and nt*32 + 16 + n.
// The wave's first quad comes in `pf`, loaded ahead by the caller; once the
// item's products are issued, `pf` is loaded with the first quad of the next
// item (expert next_e, column tile next_nt; none if next_e < 0), so those
// loads are in flight over this item's reduction.
__device__ __forceinline__ void thin_q3_quads_down(const FfnArgs& a, const MTile& t, int nt, const uint16_t* xl,
                                                   const uint32_t* xsl, float (&red)[4][16][64], int wave,
                                                   int lane, QuadW& pf, int next_e, int next_nt) {
    constexpr int XR = 4;
    const int n = lane & 15, q = lane >> 4;
    const int K = a.I, NG = K >> 7, NQ = (NG + 3) >> 2;
    const bool act_lane = (n >> 2) == q && (n & 3) < t.rows;    // A row n = 4 q + token
    const int xr = act_lane ? (n & 3) : XR;
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

    float f0[4] = {}, f1[4] = {};
    auto run = [&](const QuadW& w, int p) {
        const int G = 4 * p + q;
        const int Gc = min(G, NG - 1);
        const u32x4* xa = reinterpret_cast<const u32x4*>(xl + (size_t)(G < NG ? xr : XR) * K) + 16 * Gc;
        const uint32_t xsum = G < NG ? xsl[xr * NG + G] : 0u;     // (row XR: zeros)
        f32x4 c0 = f32x4{}, c1 = f32x4{};
        static_for<16>([&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            u32x4 b0, b1;
            static_for<4>([&](auto q_c) {
                constexpr int Q = decltype(q_c)::value;
                b0[Q] = magic_pair<4 * J + Q>(w.w0, magic);
                b1[Q] = magic_pair<4 * J + Q>(w.w1, magic);
            });
            const u32x4 av = xa[J];
            c0 = mfma16_f16(av, b0, c0);
            c1 = mfma16_f16(av, b1, c1);
        });
        // minus 1028 x (group sum, as fp16 hi + lo) in k-slots 0 and 1 of each quarter
        const u32x4 sa = u32x4{xsum, 0u, 0u, 0u}, sb = u32x4{0xE404E404u, 0u, 0u, 0u};
        c0 = mfma16_f16(sa, sb, c0);
        c1 = mfma16_f16(sa, sb, c1);
        // this lane's result rows 4 q + i: token i of group 4 p + q
        const float s0 = G < NG ? (float)__builtin_bit_cast(_Float16, w.s0) : 0.0f;
        const float s1 = G < NG ? (float)__builtin_bit_cast(_Float16, w.s1) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f0[i] = fmaf(s0, c0[i], f0[i]);
            f1[i] = fmaf(s1, c1[i], f1[i]);
        }
    };
    if (wave < NQ) run(pf, wave);
    for (int p = wave + 4; p < NQ; p += 4) {
        QuadW w;
        quad_load(a, t.e, nt, p, lane, w);
        run(w, p);
    }
    // (not above the products: the next quad's words would need registers
    // of their own while this one's are still read)
    __builtin_amdgcn_sched_barrier(0);
    if (next_e >= 0 && wave < NQ) quad_load(a, next_e, next_nt, wave, lane, pf);
    // sum the four groups of each token across the lane quarters; lane L < 32
    // then holds column L (W_down row nt*32 + L) of the tile's rows 0..3, and
    // the four waves' 4 x 32 partials meet in LDS (the barriers wait for LDS
    // traffic only: the loads issued above stay in flight); wave 0 stores
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f0[i] += __shfl_xor(f0[i], 16, 64);
        f0[i] += __shfl_xor(f0[i], 32, 64);
        f1[i] += __shfl_xor(f1[i], 16, 64);
        f1[i] += __shfl_xor(f1[i], 32, 64);
    }
    if (lane < 32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][i][lane] = lane < 16 ? f0[i] : f1[i];
    }
    lds_barrier();
    if (wave == 0 && lane < 32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = red[0][i][lane] + red[1][i][lane] + red[2][i][lane] + red[3][i][lane];
            if (i < t.rows) a.y[(size_t)(t.row0 + i) * a.H + nt * 32 + lane] = f32_to_f16_bits(v);
        }
    }
    lds_barrier();
}

// 3-bit thin kernel: the same items, waves and reduction as the bf16 thin
// kernel, with the reduction index walked a group pair at a time.  For MFMA
// step j (0..15) of pair p, lane half g holds fields 8j..8j+7 of group 2p+g
// of its weight row, and the activation lanes hold the matching 8 k of their
// row (the MFMA sums over k in any order, so both operands only have to agree
// on which k each lane holds).  Every field then sits at a compile-time word
// and bit: one v_bfe_u32, one convert and one fma per weight, no index
// arithmetic.  Each lane loads its group's 13 words with three 16-byte loads
// and one 4-byte load (52-byte groups are 4-byte aligned; a buffer load needs
// no more), instead of re-reading words per 8 fields.
//
// XR > 0 (the down phase of a decode batch, every tile at most XR <= 16
// rows): a block takes a contiguous run of items in tile-major order and
// keeps the activation rows of its current tile in LDS in pair-slot order
// with their group sums (XR rows, then a row of zeros that lanes without a
// row read), and runs each item on the pair-slot operands
// (thin_q3_pairs_down): no per-weight arithmetic, and the activation operand
// of each MFMA step is one LDS read.
// (XR > 0: four blocks per CU, one per SIMD each, as the launch assumes)
template <int PHASE, int XR>
__global__ __launch_bounds__(THIN_THREADS, XR > 0 ? 4 : 1)
void ffn_thin_q3_kernel(FfnArgs a) {
    static_assert(XR == 0 || PHASE == 2, "activation rows in LDS: down phase only");
    __shared__ float red[4][16][64];
    extern __shared__ u32x4 xst[];                   // XR > 0: [XR + 1][K] fp16 in slot order, then [XR + 1][K / 128] sums
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
    const int m = lane & 31, g = lane >> 5;
    const int K = PHASE == 1 ? a.H : a.I;
    const int N = PHASE == 1 ? a.I : a.H;            // rows of one expert matrix
    const int NT = PHASE == 1 ? a.I / 16 : a.H / 32;
    const int NG = K >> 7;                           // groups of 128 per row
    const int NP = (NG + 1) >> 1;                    // group pairs
    const int n_mt = a.hdr->n_thin;
    const int n_items = n_mt * NT;
    const size_t mat_words = (size_t)N * NG * Q3_WORDS;
    const size_t mat_scales = (size_t)N * NG;
    // activation rows through a bounded buffer: a lane without a row (or past
    // an odd group count) gets an offset beyond the buffer, which loads zeros
    const __amdgpu_buffer_rsrc_t asrc = PHASE == 1
        ? make_rsrc(a.x, (uint32_t)((size_t)a.T * a.H * 2))
        : make_rsrc(a.act, (uint32_t)((size_t)a.T * a.k * a.I * 2));
    constexpr uint32_t NOWHERE = 0xFFFFFF00u;
    const __amdgpu_buffer_rsrc_t xqsrc = make_rsrc(a.xq, PHASE == 1 ? (uint32_t)((size_t)a.T * a.H * 2) : 0u);
    const __amdgpu_buffer_rsrc_t xssrc = make_rsrc(a.xs, PHASE == 1 ? (uint32_t)((size_t)a.T * NG * 4) : 0u);

    const int chunk = XR > 0 ? (n_items + (int)gridDim.x - 1) / (int)gridDim.x : 1;
    const int i_first = XR > 0 ? (int)blockIdx.x * chunk : (int)blockIdx.x;
    const int i_end = XR > 0 ? min(n_items, i_first + chunk) : n_items;
    const int i_step = XR > 0 ? 1 : (int)gridDim.x;
    int staged = -1;                                 // XR > 0: the tile whose rows are in LDS
    [[maybe_unused]] QuadW pf;                       // XR == 4: the wave's first quad of its current item
    [[maybe_unused]] PairW pp;                       // other XR > 0: its first group pair
    for (int item = i_first; item < i_end; item += i_step) {
        const int nt = XR > 0 ? item % NT : item / n_mt;
        const int mt = XR > 0 ? item / NT : item % n_mt;
        const MTile t = a.thin[mt];
        if constexpr (XR > 0) {
            // the tile's activation rows in pair-slot order with their group
            // sums (rows past the tile, and row XR, all zeros), then the item
            uint16_t* xl = reinterpret_cast<uint16_t*>(xst);
            uint32_t* xsl = reinterpret_cast<uint32_t*>(xl + (size_t)(XR + 1) * K);
            if (mt != staged) {
                __syncthreads();                     // every wave done with the previous rows
                for (int i = threadIdx.x; i < (XR + 1) * NG; i += THIN_THREADS) {
                    const int r = i / NG, G = i - r * NG;
                    uint16_t* dst = xl + (size_t)r * K + G * 128;
                    if (r < t.rows) {
                        q3_prep_group_f16(a.act + (size_t)(t.row0 + r) * K + G * 128, dst, xsl + i);
                    } else {
#pragma unroll
                        for (int j = 0; j < 16; ++j) reinterpret_cast<u32x4*>(dst)[j] = u32x4{0, 0, 0, 0};
                        xsl[i] = 0u;
                    }
                }
                __syncthreads();
                staged = mt;
                // a tile's first item loads its own weights (for every wave: a
                // wave past the last quad or pair reads the last group; this keeps the
                // words of an earlier item dead over the staging)
                if constexpr (XR == 4) quad_load(a, t.e, nt, wave, lane, pf);
                else pair_load(a, t.e, nt, wave, lane, pp);
            }
            if constexpr (XR == 4) {
                // the next item's words are loaded ahead only within the tile
                const int nx = item + 1;
                const bool ahead = nx < i_end && nx / NT == mt;
                thin_q3_quads_down(a, t, nt, xl, xsl, red, wave, lane, pf, ahead ? t.e : -1, nx % NT);
            } else {
                const int nx = item + 1;
                const bool ahead = nx < i_end && nx / NT == mt;
                thin_q3_pairs_down<XR>(a, t, nt, xl, xsl, red, wave, lane, pp, ahead ? t.e : -1, nx % NT);
            }
            continue;
        }
        if constexpr (PHASE == 1) {
            if (t.rows <= 16) {
                thin_q3_pairs(a, t, nt, xqsrc, xssrc, red, wave, lane);
                continue;
            }
        }
        const bool has_row = m < t.rows;
        uint32_t aoff = 0;
        if (has_row) {
            const uint32_t r = PHASE == 1 ? (uint32_t)(a.sorted_pair[t.row0 + m] / a.k) : (uint32_t)(t.row0 + m);
            aoff = r * (uint32_t)K * 2u;
        }
        // this lane's weight row: phase 1 gate rows nt*16.. (m < 16) and the
        // matching up rows (m >= 16); phase 2 down rows nt*32 + m
        const void* wm = PHASE == 1 ? (m < 16 ? a.wg : a.wu) : a.wd;
        const uint16_t* sm = PHASE == 1 ? (m < 16 ? a.sg : a.su) : a.sd;
        const int row = PHASE == 1 ? nt * 16 + (m & 15) : nt * 32 + m;
        const __amdgpu_buffer_rsrc_t wsrc =
            make_rsrc(reinterpret_cast<const uint32_t*>(wm) + (size_t)t.e * mat_words, (uint32_t)(mat_words * 4));
        const uint16_t* srow = sm + (size_t)t.e * mat_scales + (size_t)row * NG;

        // the 13 words and the scale of group 2p+g of this lane's row
        struct Group {
            uint32_t w[Q3_WORDS];
            uint16_t s;
        };
        auto load_group = [&](int p, Group& q) {
            const int G = min(2 * p + g, NG - 1);     // past an odd count: a real group, scaled by 0 below
            const uint32_t off = (uint32_t)(row * NG + G) * (uint32_t)(Q3_WORDS * 4);
            const u32x4 q0 = __builtin_amdgcn_raw_buffer_load_b128(wsrc, off, 0, 0);
            const u32x4 q1 = __builtin_amdgcn_raw_buffer_load_b128(wsrc, off + 16, 0, 0);
            const u32x4 q2 = __builtin_amdgcn_raw_buffer_load_b128(wsrc, off + 32, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                q.w[i] = q0[i];
                q.w[4 + i] = q1[i];
                q.w[8 + i] = q2[i];
            }
            q.w[12] = __builtin_amdgcn_raw_buffer_load_b32(wsrc, off + 48, 0, 0);
            q.s = srow[G];
        };

        f32x16 acc = f32x16{};
        Group cur, nxt;
        if (wave < NP) load_group(wave, cur);
        for (int p = wave; p < NP; p += 4) {
            if (p + 4 < NP) load_group(p + 4, nxt);  // next pair of this wave in flight during the decode
            const int G = 2 * p + g;
            const bool valid = G < NG;
            const float sc = valid ? (float)__builtin_bit_cast(_Float16, cur.s) : 0.0f;
            const float m4 = -4.0f * sc;
            const uint32_t ao = (has_row && valid) ? aoff + (uint32_t)G * 256u : NOWHERE;
            static_for<16>([&](auto j_c) {
                constexpr int J = decltype(j_c)::value;
                const u32x4 av = __builtin_amdgcn_raw_buffer_load_b128(asrc, ao, 16 * J, 0);
                u32x4 bv;
                static_for<4>([&](auto q_c) {
                    constexpr int Q = decltype(q_c)::value;
                    constexpr int F0 = 8 * J + 2 * Q, F1 = F0 + 1;
                    const float v0 = fmaf((float)field3<3 * (F0 % 10)>(cur.w[F0 / 10]), sc, m4);
                    const float v1 = fmaf((float)field3<3 * (F1 % 10)>(cur.w[F1 / 10]), sc, m4);
                    if constexpr (PHASE == 2) {
                        const f16x2 h = {(_Float16)v0, (_Float16)v1};
                        bv[Q] = __builtin_bit_cast(uint32_t, h);
                    } else {
                        const bf16x2 h = {(__bf16)v0, (__bf16)v1};
                        bv[Q] = __builtin_bit_cast(uint32_t, h);
                    }
                });
                acc = mma<PHASE>(av, bv, acc);
            });
            cur = nxt;
        }
        thin_reduce_store<PHASE>(a, acc, t, nt, red, wave, lane);
    }
}

// ------------------------------------------------------------ host side

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct FfnLayout {
    size_t hdr, fat, thin, act, xq, xs, total;
    size_t max_fat, max_thin;
};

FfnLayout ffn_layout(int T, int E, int k, int H, int I, int wfmt) {
    const size_t P = (size_t)T * k;
    const size_t nz = P < (size_t)E ? P : (size_t)E;        // experts that can be non-empty
    FfnLayout L;
    L.max_fat = P / FAT_BM + nz + 1;
    L.max_thin = P / THIN_BM + nz + 1;
    L.hdr = 0;
    L.fat = align256(sizeof(FfnHeader));
    L.thin = L.fat + align256(L.max_fat * sizeof(MTile));
    L.act = L.thin + align256(L.max_thin * sizeof(MTile));
    L.xq = L.act + align256(P * (size_t)I * sizeof(uint16_t));
    // 3-bit weights: reordered x rows and group sums for the thin gate/up path
    const size_t xq_bytes = wfmt == 1 ? align256((size_t)T * H * sizeof(uint16_t)) : 0;
    L.xs = L.xq + xq_bytes;
    L.total = L.xs + (wfmt == 1 ? align256((size_t)T * (H / 128) * sizeof(uint32_t)) : 0);
    return L;
}

// dynamic LDS cap of the 3-bit down kernels with activation rows in LDS
// (the kernel's own 16 KB partial-tile buffer comes on top)
constexpr size_t Q3X_LDS_MAX = 140 * 1024;

struct DevInfo {
    int cus = 0;
    int q3ring = 5;                             // ... of the 3-bit fat kernels (5 or 6)
    bool q3x_ok = false;                        // the LDS cap above could be set
    int thin_blocks[2][2][2] = {};              // [wfmt][phase-1][chunk width 2 / 4]
};

std::mutex g_dev_mu;
DevInfo g_dev[64];

int occupancy_of(const void* f) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, THIN_THREADS, 0) != hipSuccess || n < 1) n = 1;
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
        // the 3-bit fat kernels use up to 126 KB of dynamic LDS (above the
        // default cap): a sixth 21 KB stage where a block may hold that much
        int lds_max = 0;
        err = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (err != hipSuccess) return err;
        const struct {
            const void* f;
            size_t bytes;
        } fats[4] = {{(const void*)ffn_fat_kernel<1, 1, 5>, fat_lds_bytes<1, 5>()},
                     {(const void*)ffn_fat_kernel<2, 1, 5>, fat_lds_bytes<1, 5>()},
                     {(const void*)ffn_fat_kernel<1, 1, 6>, fat_lds_bytes<1, 6>()},
                     {(const void*)ffn_fat_kernel<2, 1, 6>, fat_lds_bytes<1, 6>()}};
        d.q3ring = (size_t)lds_max >= fat_lds_bytes<1, 6>() ? 6 : 5;
        for (const auto& f : fats) {
            if (f.bytes > (size_t)lds_max) continue;
            err = hipFuncSetAttribute(f.f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)f.bytes);
            if (err != hipSuccess) return err;
        }
        d.thin_blocks[0][0][0] = occupancy_of((const void*)ffn_thin_kernel<1, 2>);
        d.thin_blocks[0][0][1] = stream_occupancy(1);
        d.thin_blocks[0][1][0] = occupancy_of((const void*)ffn_thin_kernel<2, 2>);
        d.thin_blocks[0][1][1] = stream_occupancy(2);
        d.thin_blocks[1][0][0] = d.thin_blocks[1][0][1] = occupancy_of((const void*)ffn_thin_q3_kernel<1, 0>);
        d.thin_blocks[1][1][0] = d.thin_blocks[1][1][1] = occupancy_of((const void*)ffn_thin_q3_kernel<2, 0>);
        // the down kernels with activation rows in LDS take up to 139 KB of it
        const void* staged[3] = {(const void*)ffn_thin_q3_kernel<2, 4>, (const void*)ffn_thin_q3_kernel<2, 8>,
                                 (const void*)ffn_thin_q3_kernel<2, 16>};
        for (const void* f : staged) {
            if ((size_t)lds_max < Q3X_LDS_MAX) break;
            err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Q3X_LDS_MAX);
            if (err != hipSuccess) return err;
        }
        d.q3x_ok = (size_t)lds_max >= Q3X_LDS_MAX;
        d.cus = cus;
    }
    out = d;
    return hipSuccess;
}

FfnArgs make_args(const FfnLaunch& a) {
    const FfnLayout L = ffn_layout(a.T, a.E, a.k, a.H, a.I, a.wfmt);
    char* ws = reinterpret_cast<char*>(a.ws);
    FfnArgs fa;
    fa.x = a.x;
    fa.wg = a.wg; fa.wu = a.wu; fa.wd = a.wd;
    fa.sg = a.sg; fa.su = a.su; fa.sd = a.sd;
    fa.sorted_pair = a.sorted_pair;
    fa.T = a.T; fa.k = a.k; fa.H = a.H; fa.I = a.I; fa.E = a.E;
    fa.pairs = a.wfmt == 2;
    fa.act = reinterpret_cast<uint16_t*>(ws + L.act);
    fa.xq = a.wfmt == 1 ? reinterpret_cast<uint16_t*>(ws + L.xq) : nullptr;
    fa.xs = a.wfmt == 1 ? reinterpret_cast<uint32_t*>(ws + L.xs) : nullptr;
    fa.y = a.y;
    fa.hdr = reinterpret_cast<FfnHeader*>(ws + L.hdr);
    fa.fat = reinterpret_cast<MTile*>(ws + L.fat);
    fa.thin = reinterpret_cast<MTile*>(ws + L.thin);
    return fa;
}

// Fat tiles need a route list of at least fat_threshold rows, and a token
// selects an expert at most once, so with T < fat_threshold (decode) there is
// no fat work and that launch is skipped.
template <int PHASE, int WFMT>
hipError_t launch_phase_t(const FfnArgs& fa, const DevInfo& d, bool fat_possible, hipStream_t s) {
    if (fat_possible) {
        if constexpr (WFMT != 0) {
            if (d.q3ring == 6)
                ffn_fat_kernel<PHASE, 1, 6><<<d.cus, FAT_THREADS, fat_lds_bytes<1, 6>(), s>>>(fa);
            else
                ffn_fat_kernel<PHASE, 1, 5><<<d.cus, FAT_THREADS, fat_lds_bytes<1, 5>(), s>>>(fa);
        } else {
            // bf16 weights: eight waves per CU, two per SIMD (fat8.hip)
            const hipError_t err = launch_fat8_phase(fa, PHASE, d.cus, s);
            if (err != hipSuccess) return err;
        }
    }
    if constexpr (WFMT != 0) {
        if constexpr (PHASE == 1) {
            // decode batches: every tile thin and every token's x row in LDS (q3dec.hip)
            if (q3dec_fits(fa.T, fa.E, fa.k, fa.H)) return launch_q3dec_gate_up(fa, d.cus, s);
            q3_xprep_kernel<<<d.cus, 256, 0, s>>>(fa);
        }
        if constexpr (PHASE == 2) {
            // decode batches: every tile has at most T rows; its activation
            // rows (and a zero row) in LDS when they fit
            const int xr = fa.T <= 4 ? 4 : (fa.T <= 8 ? 8 : (fa.T <= 16 ? 16 : 0));
            const size_t xb = (size_t)(xr + 1) * fa.I * 2 + ((size_t)(xr + 1) * (fa.I / 128) * 4 + 15) / 16 * 16;
            if (xr > 0 && d.q3x_ok && xb <= Q3X_LDS_MAX) {
                // blocks per CU as the LDS allows (the 16 KB partial tiles included), at most 4
                const int per_cu = (int)std::min<size_t>(4, (160 * 1024) / (xb + 16 * 1024 + 1024));
                const unsigned grid = (unsigned)(d.cus * std::max(per_cu, 1));
                if (xr == 4) ffn_thin_q3_kernel<2, 4><<<grid, THIN_THREADS, xb, s>>>(fa);
                else if (xr == 8) ffn_thin_q3_kernel<2, 8><<<grid, THIN_THREADS, xb, s>>>(fa);
                else ffn_thin_q3_kernel<2, 16><<<grid, THIN_THREADS, xb, s>>>(fa);
                return hipGetLastError();
            }
        }
        ffn_thin_q3_kernel<PHASE, 0><<<d.cus * d.thin_blocks[1][PHASE - 1][0], THIN_THREADS, 0, s>>>(fa);
    } else {
        // weights through LDS in whole lines (stream.hip) when each wave's
        // quarter of K is a multiple of 64; else straight into registers
        if (stream_fits(PHASE, fa.T, fa.k, fa.H, fa.I))
            return launch_stream_phase(fa, PHASE, d.cus * d.thin_blocks[0][PHASE - 1][1], s);
        if (fa.pairs) return hipErrorInvalidValue;           // the row-pair layout is read by the streaming kernel only
        ffn_thin_kernel<PHASE, 2><<<d.cus * d.thin_blocks[0][PHASE - 1][0], THIN_THREADS, 0, s>>>(fa);
    }
    return hipGetLastError();
}

}  // namespace

size_t ffn_ws_bytes(int T, int E, int k, int H, int I, int wfmt) { return ffn_layout(T, E, k, H, I, wfmt).total; }

FfnPlanPtrs ffn_plan_ptrs(int T, int E, int k, int H, int I, int wfmt, void* ffn_ws) {
    const FfnLayout L = ffn_layout(T, E, k, H, I, wfmt);
    char* ws = reinterpret_cast<char*>(ffn_ws);
    return {reinterpret_cast<FfnHeader*>(ws + L.hdr), reinterpret_cast<MTile*>(ws + L.fat),
            reinterpret_cast<MTile*>(ws + L.thin)};
}

hipError_t launch_ffn_plan(const FfnLaunch& a, hipStream_t s) {
    const FfnLayout L = ffn_layout(a.T, a.E, a.k, a.H, a.I, a.wfmt);
    char* ws = reinterpret_cast<char*>(a.ws);
    build_tiles_kernel<<<1, 1024, 0, s>>>(a.offsets, a.E, a.fat_threshold,
                                          reinterpret_cast<FfnHeader*>(ws + L.hdr),
                                          reinterpret_cast<MTile*>(ws + L.fat),
                                          reinterpret_cast<MTile*>(ws + L.thin), a.counts);
    return hipGetLastError();
}

hipError_t launch_ffn_phase(const FfnLaunch& a, int phase, hipStream_t s) {
    DevInfo d;
    hipError_t err = dev_info(d);
    if (err != hipSuccess) return err;
    const FfnArgs fa = make_args(a);
    const bool fat = a.T >= a.fat_threshold;
    // formats 0 and 2 (bf16, plain or row-pair layout) share the kernels
    if (phase == 1) return a.wfmt != 1 ? launch_phase_t<1, 0>(fa, d, fat, s) : launch_phase_t<1, 1>(fa, d, fat, s);
    return a.wfmt != 1 ? launch_phase_t<2, 0>(fa, d, fat, s) : launch_phase_t<2, 1>(fa, d, fat, s);
}

}  // namespace moe
