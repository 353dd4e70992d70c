// MFMA-tile grouped FFN for bf16 expert weights with two waves per SIMD.
//
// Same work as the bf16 MFMA-tile ("fat") kernels of ffn.hip: busy experts'
// route lists cut into M-tiles of up to 256 rows (dsv41-flash-offload wiki,
// opening paragraph and file table: busy experts as GEMMs; segment patch
// entry: batches sharing one read of the expert's weights), each M-tile
// multiplied with 256 weight rows at a time (phase 1: 128 gate rows and the
// matching 128 up rows, SwiGLU applied in registers; phase 2: 256 rows of
// W_down, converted bf16 -> fp16 for the fp16 products unless stored fp16), operands staged
// through an LDS ring of five 32-k stages by direct-to-LDS buffer loads.
//
// Eight waves per block, one block per CU, so two waves share each SIMD's
// MFMA pipe.  Waves 0-3 (group 0) and 4-7 (group 1) take turns: while the
// waves of one group issue a cluster of MFMAs for a stage, the waves of the
// other group read their operand fragments for the next stage from LDS and
// issue their share of the direct-to-LDS loads; a barrier ends each half.
// A wave that only waits (LDS latency, load issue, the stage barrier) then
// always has a partner on its SIMD with MFMAs ready, where a single wave per
// SIMD leaves the pipe idle.
//
// Wave (G, q): weight rows of column tiles c = 0, 1 (phase 1: gate rows
// 32 q + n and up rows 128 + 32 q + n of the tile; phase 2: rows 64 q + 32 c
// + n), row tiles G, G + 2, G + 4, G + 6 of the M-tile (those below its row
// count), so the two groups share the MFMA work of any M-tile to within one
// row tile.
//
// Weight rows in the row-pair layout (weight format 2: rows 2p and 2p + 1
// alternate every 32 k) make each weight load instruction cover 8 whole
// 128-byte lines instead of 16 half lines; the per-CU load path moves about
// one line per clock either way, so the weight loads cost half as much of it.
// The LDS layout and everything after the loads are the same for both.  That
// format also stores W_down already converted to fp16 (the same conversion
// as below, done once when the weights are packed), which takes the 16
// conversions per stage off the waves that feed the other group's MFMAs.
//
// Per round kt (one 32-k stage):
//   half A: group 0 computes stage kt; group 1 reads its fragments of stage
//           kt and issues its loads of stage kt + 4; barrier.
//   half B: group 1 computes stage kt; group 0 reads its fragments of stage
//           kt + 1 and issues its loads of stage kt + 4; barrier.
// Stage kt + 4 goes into the ring slot of stage kt - 1, which both groups
// finished reading before the previous round's second barrier.  Before the
// first barrier of round kt every wave has waited for its own loads of stage
// kt + 1, which group 0 reads right after it.
#include "common.h"
#include "ffn_shared.h"
#include "lds_dma.h"

#include <mutex>

namespace moe {
namespace {

constexpr int F8_THREADS = 512;
constexpr int F8_NS = 5;                                   // ring stages
constexpr uint32_t F8_STAGE = 2 * DMA_OPER;                // 32 KB: activations + weight rows
constexpr uint32_t F8_LDS = F8_NS * F8_STAGE;              // 160 KB

template <int PHASE>
__device__ __forceinline__ f32x16 mma8(u32x4 a, u32x4 b, f32x16 c) {
    return PHASE == 1 ? mfma_bf16(a, b, c) : mfma_f16(a, b, c);
}

// Epilogue staging rows (halves): output columns per tile plus 8 of padding.
template <int PHASE>
constexpr int f8_ld() {
    return (PHASE == 1 ? 128 : 256) + 8;
}
static_assert(256 * f8_ld<2>() * 2 <= F8_LDS, "the epilogue staging tile exceeds the ring");

template <int PHASE>
__global__ __launch_bounds__(F8_THREADS, 1)
void ffn_fat8_kernel(FfnArgs a) {
    extern __shared__ u32x4 smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..7, wave-uniform
    const int G = wave >> 2, q = wave & 3;
    const int n = lane & 31, g = lane >> 5;
    const int K = PHASE == 1 ? a.H : a.I;
    const int N = PHASE == 1 ? a.I : a.H;
    constexpr int BN = PHASE == 1 ? 128 : 256;
    const int NT = N / BN;
    const int n_items = a.hdr->n_fat * NT;
    const int KT = K / DMA_BK;
    const __amdgpu_buffer_rsrc_t asrc = PHASE == 1
        ? make_rsrc(a.x, (uint32_t)((size_t)a.T * a.H * 2))
        : make_rsrc(a.act, (uint32_t)((size_t)a.T * a.k * a.I * 2));
    const size_t wbytes = (size_t)a.I * a.H * 2;
    // weight bytes between consecutive stages of one row: 64, or 128 in the
    // row-pair layout (rows 2p and 2p + 1 alternate every 32 k)
    const uint32_t wstage = a.pairs ? 2 * DMA_ROW : DMA_ROW;
    // 16 rows x 64 B per load instruction, 4 lanes per row; the chunk landing
    // at position L % 4 of row r is (L % 4) ^ ((r >> 2) & 3)
    const uint32_t lch16 = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
    const uint32_t sbase = lds_addr(smem);
    // fragment reads: chunk 2 s + g of row r at position (2 s + g) ^ ((r >> 2) & 3)
    uint32_t aoffs[2], boffs[2][2];
    const int brow[2] = {PHASE == 1 ? 32 * q + n : 64 * q + n, PHASE == 1 ? 128 + 32 * q + n : 64 * q + 32 + n};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t ch = (uint32_t)(((2 * s + g) ^ ((n >> 2) & 3)) * 16);
        aoffs[s] = (uint32_t)(32 * G + n) * DMA_ROW + ch;
#pragma unroll
        for (int c = 0; c < 2; ++c) boffs[s][c] = DMA_OPER + (uint32_t)brow[c] * DMA_ROW + ch;
    }

    const int n_static = PHASE == 1 ? max(0, n_items / (int)gridDim.x - FAT_TAIL_ROUNDS) * (int)gridDim.x : n_items;
    FfnHeader* const hdr = const_cast<FfnHeader*>(a.hdr);
    volatile int* const bcast = reinterpret_cast<volatile int*>(smem);
    int item = logical_block();
    for (;;) {
        if (PHASE == 1 && item >= n_static) {
            // tail round: the next unclaimed item, the same for the whole block
            __syncthreads();
            if (tid == 0) bcast[0] = n_static + atomicAdd(&hdr->tail_next[PHASE - 1], 1);
            __syncthreads();
            item = __builtin_amdgcn_readfirstlane(bcast[0]);
            __syncthreads();
        }
        if (item >= n_items) break;
        MTile t;
        int nt;
        fat_item(a.fat, item, NT, t, nt);
        const int rt = (t.rows + 31) >> 5;

        // weight rows: waves 0-3 load B rows 0..127, waves 4-7 rows 128..255
        // (phase 1: the gate rows, then the matching up rows)
        const char* wmatp = reinterpret_cast<const char*>(PHASE == 1 ? (wave < 4 ? a.wg : a.wu) : a.wd);
        const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(wmatp + t.e * wbytes, (uint32_t)wbytes);
        // activation instruction j covers tile rows 128 j + 16 wave + L / 4
        // (rows past the M-tile repeat its last row; never stored), weight
        // instruction j rows 32 wave + 16 j + L / 4
        uint32_t aoff[2], boff[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = min(128 * j + 16 * wave + (lane >> 2), t.rows - 1);
            const uint32_t src = PHASE == 1 ? (uint32_t)(a.sorted_pair[t.row0 + r] / a.k) : (uint32_t)(t.row0 + r);
            aoff[j] = src * (uint32_t)K * 2u + lch16;
            const int b = 32 * wave + 16 * j + (lane >> 2);
            const uint32_t wrow = PHASE == 1 ? (uint32_t)(nt * 128 + (b & 127)) : (uint32_t)(nt * 256 + b);
            boff[j] = a.pairs ? (wrow & ~1u) * (uint32_t)K * 2u + (wrow & 1u) * DMA_ROW + lch16
                              : wrow * (uint32_t)K * 2u + lch16;
        }

        auto kloop = [&](auto rt_c) {
            constexpr int RT = decltype(rt_c)::value;
            constexpr int LA = RT > 4 ? 2 : 1;                   // activation loads per wave per stage
            constexpr int L = LA + 2;                            // loads per wave per stage
            // this wave's loads of stage kt into ring slot `slot`
            auto issue_stage = [&](int kt, int slot) {
                char* st = reinterpret_cast<char*>(smem) + slot * F8_STAGE;
#pragma unroll
                for (int j = 0; j < LA; ++j)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(asrc, (lds_ptr_t)(st + (8 * j + wave) * 1024), 16,
                                                             aoff[j], kt * DMA_ROW, 0, 0);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc, (lds_ptr_t)(st + DMA_OPER + (2 * wave + j) * 1024),
                                                             16, boff[j], kt * wstage, 0, 0);
            };
            auto run = [&](auto rg_c, auto g0_c) {
                constexpr int RG = decltype(rg_c)::value;            // row tiles of this wave
                constexpr bool G0 = decltype(g0_c)::value;
                constexpr int RA = RG > 0 ? RG : 1;
                f32x16 acc[RA][2];
#pragma unroll
                for (int i = 0; i < RA; ++i)
#pragma unroll
                    for (int c = 0; c < 2; ++c) acc[i][c] = f32x16{};
                u32x4 fa[2][RA], fb[2][2];
                // fragments of both 16-k steps of the stage in `slot`
                auto read_stage = [&](int slot) {
                    const uint32_t st = sbase + slot * F8_STAGE;
                    static_for<2>([&](auto s_c) {
                        constexpr int S = decltype(s_c)::value;
                        static_for<RG>([&](auto i_c) {
                            constexpr int I = decltype(i_c)::value;
                            fa[S][I] = ds_read16<I * 64 * (int)DMA_ROW>(st + aoffs[S]);
                        });
                        if constexpr (RG > 0) {
                            fb[S][0] = ds_read16<0>(st + boffs[S][0]);
                            fb[S][1] = ds_read16<0>(st + boffs[S][1]);
                        }
                    });
                };
                // wait for the reads; phase 2 converts the W_down fragments to fp16
                auto wait_frags = [&]() {
                    if constexpr (RG > 0) {
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                        static_for<2>([&](auto s_c) {
                            constexpr int S = decltype(s_c)::value;
                            static_for<RG>([&](auto i_c) { tie_after_wait(fa[S][decltype(i_c)::value]); });
                            tie_after_wait(fb[S][0]);
                            tie_after_wait(fb[S][1]);
                            if constexpr (PHASE == 2) {
                                if (!a.pairs) {                  // (weight format 2 stores W_down as fp16)
                                    fb[S][0] = bf16x8_to_f16x8(fb[S][0]);
                                    fb[S][1] = bf16x8_to_f16x8(fb[S][1]);
                                }
                            }
                        });
                    }
                };
                auto compute = [&]() {
                    if constexpr (RG > 0) {
                        __builtin_amdgcn_sched_barrier(0);
                        __builtin_amdgcn_s_setprio(1);
                        static_for<2>([&](auto s_c) {
                            constexpr int S = decltype(s_c)::value;
                            static_for<RG>([&](auto i_c) {
                                constexpr int I = decltype(i_c)::value;
                                acc[I][0] = mma8<PHASE>(fa[S][I], fb[S][0], acc[I][0]);
                                acc[I][1] = mma8<PHASE>(fa[S][I], fb[S][1], acc[I][1]);
                            });
                        });
                        __builtin_amdgcn_s_setprio(0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                };
                auto barrier = [&]() {
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                };

                // prologue: stages 0 .. NS-2 in flight, stage 0 landed everywhere
                const int pro = min(F8_NS - 1, KT);
                for (int s = 0; s < pro; ++s) issue_stage(s, s);
                vm_wait_stages<L>(pro - 1);
                barrier();
                if constexpr (G0) {
                    read_stage(0);
                    wait_frags();
                }
                int slot = 0;                                    // ring slot of stage kt
                for (int kt = 0; kt < KT; ++kt) {
                    const int nslot = slot + 1 == F8_NS ? 0 : slot + 1;
                    const int fill = kt + F8_NS - 1;             // stage loaded this round
                    const int fslot = slot == 0 ? F8_NS - 1 : slot - 1;
                    // half A
                    if constexpr (G0) {
                        compute();
                        vm_wait_stages<L>(max(0, min(F8_NS - 3, KT - 2 - kt)));
                    } else {
                        read_stage(slot);
                        if (fill < KT) issue_stage(fill, fslot);
                        vm_wait_stages<L>(max(0, min(F8_NS - 2, KT - 2 - kt)));
                        wait_frags();
                    }
                    barrier();
                    // half B
                    if constexpr (G0) {
                        if (kt + 1 < KT) read_stage(nslot);
                        if (fill < KT) issue_stage(fill, fslot);
                        wait_frags();                            // (no reads in the last round)
                    } else {
                        compute();
                    }
                    barrier();
                    slot = nslot;
                }

                // epilogue: every wave's tiles into one LDS staging tile, then
                // 16-byte row stores by the whole block
                constexpr int LD = f8_ld<PHASE>();
                uint16_t* sO = reinterpret_cast<uint16_t*>(smem);
                // this lane's first staged element; opaque per item, so that
                // the compiler derives the 16 x RG addresses here rather than
                // keeping them live (and spilled) across the item loop
                int e0 = (32 * G + 4 * g) * LD + (PHASE == 1 ? 32 : 64) * q + n;
                asm volatile("" : "+v"(e0));
                static_for<RG>([&](auto i_c) {
                    constexpr int I = decltype(i_c)::value;
                    static_for<16>([&](auto r_c) {
                        constexpr int R = decltype(r_c)::value;
                        constexpr int M = 64 * I + 8 * (R >> 2) + (R & 3);
                        if constexpr (PHASE == 1) {
                            sO[e0 + M * LD] = f32_to_f16_bits(silu_mul(acc[I][0][R], acc[I][1][R]));
                        } else {
                            sO[e0 + M * LD] = f32_to_f16_bits(acc[I][0][R]);
                            sO[e0 + M * LD + 32] = f32_to_f16_bits(acc[I][1][R]);
                        }
                    });
                });
            };
            constexpr int RG0 = (RT + 1) / 2, RG1 = RT / 2;
            if (G == 0)
                run(std::integral_constant<int, RG0>{}, std::true_type{});
            else
                run(std::integral_constant<int, RG1>{}, std::false_type{});
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
        __syncthreads();
        {
            constexpr int LD = f8_ld<PHASE>();
            constexpr int CPR = BN / 8;                          // 16-byte chunks per output row
            constexpr int RPP = F8_THREADS / CPR;                // rows per pass
            const uint16_t* sO = reinterpret_cast<const uint16_t*>(smem);
            uint16_t* dst = PHASE == 1 ? a.act : a.y;
            const int ch = tid % CPR;
            for (int r = tid / CPR; r < t.rows; r += RPP)
                stg16(dst + (size_t)(t.row0 + r) * N + nt * BN + ch * 8,
                      *reinterpret_cast<const u32x4*>(sO + r * LD + ch * 8));
        }
        __syncthreads();                                     // staging read before the next item's loads
        item += gridDim.x;
    }
    // the last block out re-zeroes the counters for the next launch
    if (PHASE == 1 && tid == 0) {
        __threadfence();
        if (atomicAdd(&hdr->tail_done[PHASE - 1], 1) == (int)gridDim.x - 1) {
            atomicExch(&hdr->tail_next[PHASE - 1], 0);
            atomicExch(&hdr->tail_done[PHASE - 1], 0);
        }
    }
}

std::mutex g_f8_mu;
bool g_f8_ready[64] = {};

}  // namespace

hipError_t launch_fat8_phase(const FfnArgs& fa, int phase, int cus, hipStream_t s) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    {
        std::lock_guard<std::mutex> lock(g_f8_mu);
        if (!g_f8_ready[dev]) {
            err = hipFuncSetAttribute((const void*)ffn_fat8_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)F8_LDS);
            if (err == hipSuccess)
                err = hipFuncSetAttribute((const void*)ffn_fat8_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)F8_LDS);
            if (err != hipSuccess) return err;
            g_f8_ready[dev] = true;
        }
    }
    if (phase == 1)
        ffn_fat8_kernel<1><<<cus, F8_THREADS, F8_LDS, s>>>(fa);
    else
        ffn_fat8_kernel<2><<<cus, F8_THREADS, F8_LDS, s>>>(fa);
    return hipGetLastError();
}

}  // namespace moe
