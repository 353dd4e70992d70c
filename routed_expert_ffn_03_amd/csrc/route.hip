// Router: per-token top-k over the layer's experts, gate weights and the
// load histogram.
//
// Routing to a few of the layer's routed experts per token: dsv41-flash-offload
// wiki, opening paragraph.  The gate is not written on the pages; this is the
// reading the library implements: the k largest logits (ties -> lower expert
// index, -0 == +0), weights = softmax over the selected logits.
//
// One wavefront per token.  Lane i holds experts i, i+64, ... as 64-bit keys
//   key = (order-preserving bits of the logit) << 32 | ~expert
// so one unsigned max over the wave yields the largest logit and, among equal
// logits, the lowest expert index.  k rounds of (lane-local max, 6-step
// butterfly max, owner clears the winner) give the ordered top-k.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "route_keys.h"

#include <mutex>

namespace moe {
namespace {

constexpr int ROUTE_THREADS = 256;
constexpr int ROUTE_WAVES = ROUTE_THREADS / WAVE;

// tokens_per_block tokens per block; waves take tokens round-robin.
// hist_mode 0: the block histograms merge into counts with integer atomics;
// 1: the grid is one block covering all tokens, so the block histogram is the
// answer (no zeroing pass, no atomics); 2: no histogram (a later step derives
// the counts from the route lists).
template <int NV>                                   // keys per lane (>= E / 64)
__global__ __launch_bounds__(ROUTE_THREADS)
void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k, int tokens_per_block,
                       int hist_mode, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                       int32_t* __restrict__ counts) {
    __shared__ int hist[MAX_EXPERTS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) hist[e] = 0;
    __syncthreads();

    const int t0 = blockIdx.x * tokens_per_block;
    const int t1 = min(T, t0 + tokens_per_block);
    for (int t = t0 + wave; t < t1; t += ROUTE_WAVES) {
        const float* row = logits + (size_t)t * E;
        uint32_t ord[1][NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + WAVE * i;
            ord[0][i] = e < E ? ordered_bits(row[e]) : 0u;
        }
        int my_e[1] = {0};
        float my_v[1] = {0.0f};
        wave_topk<NV, 1>(ord, k, lane, my_e, my_v);
        const float v0 = __shfl(my_v[0], 0, 64);
        const float z = lane < k ? expf(my_v[0] - v0) : 0.0f;
        const float s = wave_sum(z);
        if (lane < k) {
            topk_ids[(size_t)t * k + lane] = my_e[0];
            topk_w[(size_t)t * k + lane] = z / s;
            if (hist_mode != 2) atomicAdd(&hist[my_e[0]], 1);
        }
    }
    if (hist_mode == 2) return;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) {
        if (hist_mode == 1) counts[e] = hist[e];
        else if (hist[e]) atomicAdd(&counts[e], hist[e]);
    }
}

// route_topk with one token per lane (k <= 8, E a multiple of 16 up to 512):
// a block takes RL_TOK tokens and stages their logits in LDS with coalesced
// loads (rows of E + 4 floats: 16 lanes reading 16 B of 16 rows hit distinct
// banks); wave w keeps, per token, the 8 largest of experts [w E/4, (w + 1)
// E/4) (Top8); waves 1-3 hand their lists to wave 0, which merges them in
// wave order.  Choice, order and weights equal route_topk_kernel's bit for
// bit; hist_mode as there.
constexpr int RL_TOK = 64;
__host__ __device__ constexpr uint32_t route_lane_lds_bytes(int E) {
    return (uint32_t)RL_TOK * (E + 4) * 4 + 3 * 8 * RL_TOK * 8;
}

__global__ __launch_bounds__(ROUTE_THREADS)
void route_topk_lane_kernel(const float* __restrict__ logits, int T, int E, int k, int hist_mode,
                            int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                            int32_t* __restrict__ counts) {
    extern __shared__ u32x4 lane_smem[];
    __shared__ int hist[MAX_EXPERTS];
    float* lgs = reinterpret_cast<float*>(lane_smem);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int LD = E + 4;
    const int t0 = blockIdx.x * RL_TOK, rows = min(RL_TOK, T - t0);
    const int c4n = E / 4;                                         // float4 per row
    const float4* src = reinterpret_cast<const float4*>(logits + (size_t)t0 * E);
    for (int i = tid; i < rows * c4n; i += ROUTE_THREADS) {
        const int r = i / c4n;
        *reinterpret_cast<float4*>(lgs + r * LD + 4 * (i - r * c4n)) = src[i];
    }
    if (hist_mode != 2)
        for (int e = tid; e < E; e += ROUTE_THREADS) hist[e] = 0;
    __syncthreads();

    Top8 tl;
    top8_init(tl);
    const int qe = E / 4;                                          // experts per wave
    const float* lrow = lgs + min(lane, rows - 1) * LD + wave * qe;   // lanes past the rows repeat the last
    for (int c = 0; c < qe / 4; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(lrow + 4 * c);
        const int e0 = wave * qe + 4 * c;
        top8_insert(tl, ordered_bits(v.x), e0);
        top8_insert(tl, ordered_bits(v.y), e0 + 1);
        top8_insert(tl, ordered_bits(v.z), e0 + 2);
        top8_insert(tl, ordered_bits(v.w), e0 + 3);
    }
    uint32_t* mv = reinterpret_cast<uint32_t*>(lgs + RL_TOK * LD);   // [3][8][RL_TOK] keys, then experts
    int* mi = reinterpret_cast<int*>(mv + 3 * 8 * RL_TOK);
    if (wave > 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            mv[((wave - 1) * 8 + j) * RL_TOK + lane] = tl.v[j];
            mi[((wave - 1) * 8 + j) * RL_TOK + lane] = tl.e[j];
        }
    }
    __syncthreads();
    if (wave == 0) {
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int j = 0; j < 8; ++j) top8_insert(tl, mv[(w * 8 + j) * RL_TOK + lane], mi[(w * 8 + j) * RL_TOK + lane]);
        if (lane < rows) {
            float wj[8];
            top8_weights(tl, k, wj);
            const size_t t = (size_t)(t0 + lane);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < k) {
                    topk_ids[t * k + j] = tl.e[j];
                    topk_w[t * k + j] = wj[j];
                    if (hist_mode != 2) atomicAdd(&hist[tl.e[j]], 1);
                }
        }
    }
    if (hist_mode == 2) return;
    __syncthreads();
    for (int e = tid; e < E; e += ROUTE_THREADS) {
        if (hist_mode == 1) counts[e] = hist[e];
        else if (hist[e]) atomicAdd(&counts[e], hist[e]);
    }
}

std::mutex g_rl_mu;
bool g_rl_ready[64] = {};

// the per-lane kernel's LDS cap, once per device; false where it cannot be set
bool route_lane_ready() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::lock_guard<std::mutex> lock(g_rl_mu);
    if (!g_rl_ready[dev]) {
        if (hipFuncSetAttribute((const void*)route_topk_lane_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)route_lane_lds_bytes(512)) != hipSuccess)
            return false;
        g_rl_ready[dev] = true;
    }
    return true;
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

template <int NV>
void route_launch(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w, int32_t* counts,
                  hipStream_t s) {
    // Small batches: one block owns every token and writes the histogram
    // directly.  Larger ones: 16 tokens per block (4 per wave) keeps ~1k
    // blocks in flight at 16k tokens; bins merge with integer atomics after a
    // zeroing pass (integer sums are order-independent, so the result is
    // deterministic).
    const int single_max = 64;
    if (T <= single_max) {
        route_topk_kernel<NV><<<1, ROUTE_THREADS, 0, s>>>(logits, T, E, k, T, counts ? 1 : 2, topk_ids, topk_w,
                                                         counts);
        return;
    }
    // (counts == nullptr: no histogram; the global atomics of ~1k blocks on E
    // bins are a third of this launch at 16k tokens)
    if (k <= 8 && E % 16 == 0 && E <= 512 && ((uintptr_t)logits & 15) == 0 && route_lane_ready()) {
        if (counts) zero_i32_kernel<<<(E + 255) / 256, 256, 0, s>>>(counts, E);
        route_topk_lane_kernel<<<(T + RL_TOK - 1) / RL_TOK, ROUTE_THREADS, route_lane_lds_bytes(E), s>>>(
            logits, T, E, k, counts ? 0 : 2, topk_ids, topk_w, counts);
        return;
    }
    const int tpb = 16;
    if (counts) zero_i32_kernel<<<(E + 255) / 256, 256, 0, s>>>(counts, E);
    const int blocks = (T + tpb - 1) / tpb;
    route_topk_kernel<NV><<<blocks, ROUTE_THREADS, 0, s>>>(logits, T, E, k, tpb, counts ? 0 : 2, topk_ids, topk_w,
                                                          counts);
}

// ------------------------------------------------------------ fused router

// Router GEMM + top-k: logits[t, e] = x[t] . W_router[e] (bf16 products, fp32
// accumulate on MFMA) for a block of RB tokens against all E experts, kept in
// registers and then in LDS, followed by the same top-k, softmax and histogram
// as route_topk_kernel (so the choice is exactly route_topk's on these fp32
// logits).  The logits reach HBM only when the caller asks for them.
//
// Tile: RB = 64 tokens x E experts; the four waves side by side, wave w owning
// experts [w E/4, (w+1) E/4) as CT = E/128 column tiles of 32 against both
// 32-token row tiles.  Operands stream through two LDS slots of 64 k each
// (activation rows 64 x 128 B, then router rows E x 128 B): direct-to-LDS
// loads of 8 rows x 128 B, whole lines (the per-CU load path moves about one
// line per clock whether it is used in full or not, so 64-byte pieces of a
// 32-k stage cost twice the time per byte); the 16-byte piece c of LDS row r
// at position c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1).  The next slot
// is in flight while the current one is multiplied.
constexpr int RB = 64;                    // tokens per block
constexpr int R_THREADS = 256;
constexpr uint32_t R_ROW = 128;           // bytes of one row per 64-k slot

__host__ __device__ constexpr uint32_t router_stage_bytes(int E) { return (uint32_t)(RB + E) * R_ROW; }
// staged logits [RB][E + 4] fp32, then the three partial top-8 lists of
// waves 1-3 ([3][8][RB] keys and experts)
__host__ __device__ constexpr uint32_t router_gate_bytes(int E) { return (uint32_t)RB * (E + 4) * 4 + 3 * 8 * RB * 8; }
__host__ __device__ constexpr uint32_t router_lds_bytes(int E) {
    return router_stage_bytes(E) * 2 > router_gate_bytes(E) ? router_stage_bytes(E) * 2 : router_gate_bytes(E);
}

template <int CT>
__global__ __launch_bounds__(R_THREADS, 1)
void router_topk_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int k,
                        int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ counts,
                        float* __restrict__ logits_out) {
    constexpr int E = 128 * CT;
    constexpr int NO = (RB + E) / 8;                     // 8-row octets per slot
    constexpr int LW = (NO + 3) / 4;                     // load instructions per wave per slot (at most)
    constexpr uint32_t SB = router_stage_bytes(E);
    // staged logit row (floats): E + 4 = 4 (mod 64), so 16 lanes reading 16 B
    // of 16 different rows hit distinct banks
    constexpr int LD = E + 4;
    extern __shared__ u32x4 smem[];
    __shared__ int hist[E];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int t0 = blockIdx.x * RB;
    const int KD = (H + 63) / 64;                        // 64-k slots (the last one may hold 32 k)
    for (int e = tid; e < E; e += R_THREADS) hist[e] = 0;

    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(wr, (uint32_t)((size_t)E * H * 2));
    // wave w moves octets w, w + 4, ...: octet o < 8 is activation rows 8 o ..
    // (rows past T repeat the last one), the rest router rows 8 (o - 8) ..;
    // lane L puts row 8 o + L / 8 of the slot at position L % 8, which holds
    // piece (L % 8) ^ (L / 8) ^ (o & 1)
    uint32_t loff[LW];
#pragma unroll
    for (int j = 0; j < LW; ++j) {
        const int o = wave + 4 * j;
        const uint32_t pc = (uint32_t)(((lane & 7) ^ (lane >> 3) ^ (o & 1)) * 16);
        const int r = 8 * o + (lane >> 3);
        loff[j] = o < 8 ? (uint32_t)min(t0 + r, T - 1) * (uint32_t)H * 2u + pc
                        : (uint32_t)(r - RB) * (uint32_t)H * 2u + pc;
    }
    const uint32_t sbase = lds_addr(smem);
    auto issue = [&](int d, int slot) {
        char* st = reinterpret_cast<char*>(smem) + slot * SB;
        const uint32_t soff = (uint32_t)d * R_ROW;
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int o = wave + 4 * j;
            if (o < NO) dma16(o < 8 ? xsrc : wsrc, st + o * 1024, loff[j], soff);
        }
    };

    f32x16 acc[2][CT];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[r][c] = f32x16{};

    // fragment reads: step s (16 k) of a slot, lane (n, g): piece 2 s + g of
    // row n of its tile; every tile's rows are n modulo 16, so one swizzle
    const int swn = (n & 7) ^ ((n >> 3) & 1);
    uint32_t arow[2], brow[CT];
#pragma unroll
    for (int r = 0; r < 2; ++r) arow[r] = (uint32_t)(32 * r + n) * R_ROW;
#pragma unroll
    for (int c = 0; c < CT; ++c) brow[c] = (uint32_t)(RB + wave * (E / 4) + 32 * c + n) * R_ROW;

    issue(0, 0);
    for (int d = 0; d < KD; ++d) {
        const int slot = d & 1;
        vm_wait<0>();                                             // this wave's part of slot d landed ...
        // (LDS-only barrier: __syncthreads() would also wait for the next
        // slot's loads)
        lds_barrier();                                            // ... every wave's, and slot d - 1 is free
        if (d + 1 < KD) issue(d + 1, slot ^ 1);
        const uint32_t st = sbase + slot * SB;
        // 4 steps of 16 k, or 2 in a last slot of 32 k (H % 64 == 32): its
        // steps 2 and 3 read whatever the slot holds and multiply zeros
        // instead
        const bool full = H - 64 * d >= 64;
        // fragments of step s into buffer s & 1; the reads of step s + 1 go
        // out after the wait for step s and before its MFMAs, so their LDS
        // latency passes under the MFMAs (one wave per SIMD: nothing else
        // would hide it).  Every read is waited for on every path.
        u32x4 af[2][2], bf[2][CT];
        auto rd = [&](auto s_c) {
            constexpr int S = decltype(s_c)::value, B = S & 1;
            const uint32_t pc = (uint32_t)(((2 * S + g) ^ swn) * 16);
#pragma unroll
            for (int r = 0; r < 2; ++r) af[B][r] = ds_read16<0>(st + arow[r] + pc);
#pragma unroll
            for (int c = 0; c < CT; ++c) bf[B][c] = ds_read16<0>(st + brow[c] + pc);
        };
        rd(std::integral_constant<int, 0>{});
        static_for<4>([&](auto s_c) {
            constexpr int S = decltype(s_c)::value, B = S & 1;
            lds_wait_all();
#pragma unroll
            for (int r = 0; r < 2; ++r) tie_after_wait(af[B][r]);
#pragma unroll
            for (int c = 0; c < CT; ++c) tie_after_wait(bf[B][c]);
            if constexpr (S >= 2) {
                if (!full) {                                      // (zeros on both sides: no 0 x NaN)
#pragma unroll
                    for (int r = 0; r < 2; ++r) af[B][r] = u32x4{0, 0, 0, 0};
#pragma unroll
                    for (int c = 0; c < CT; ++c) bf[B][c] = u32x4{0, 0, 0, 0};
                }
            }
            if constexpr (S + 1 < 4) rd(std::integral_constant<int, S + 1>{});
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int c = 0; c < CT; ++c) acc[r][c] = mfma_bf16(af[B][r], bf[B][c], acc[r][c]);
        });
    }
    lds_barrier();                                                // every wave done with the last slot

    // logits to LDS: lane holds expert column n of its tile, tokens 8 (i >> 2) + 4 g + (i & 3)
    float* lg = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                lg[(32 * r + 8 * (i >> 2) + 4 * g + (i & 3)) * LD + wave * (E / 4) + 32 * c + n] = acc[r][c][i];
    __syncthreads();
    const int rows = min(RB, T - t0);
    if (logits_out) {
        for (int i = tid; i < rows * (E / 4); i += R_THREADS) {
            const int r = i / (E / 4), c4 = i % (E / 4);
            const float* src = lg + r * LD + 4 * c4;
            *reinterpret_cast<float4*>(logits_out + (size_t)(t0 + r) * E + 4 * c4) =
                make_float4(src[0], src[1], src[2], src[3]);
        }
    }
    if (k <= 8 && rows > 16) {
        // Top-k with one token per lane (lane l: row l of the block): wave w
        // keeps, per token, the 8 largest of experts [w E/4, (w + 1) E/4) as a
        // sorted list (ordered logit bits, expert), each logit entering by a
        // branch-free insertion that puts it after equal ones (experts taken
        // in ascending order, so equal logits stay in ascending expert order);
        // waves 1-3 hand their lists to wave 0 through LDS, which inserts them
        // in wave order and so keeps the same order across the four ranges.
        // The first k entries are route_topk's choice, in its order.  (A block
        // of at most 16 tokens, e.g. a decode batch, takes the per-wave
        // selection below instead: four tokens per wave beat 64 lanes of
        // which a few hold a token.)
        Top8 tl;
        top8_init(tl);
        const int rl = min(lane, rows - 1);                         // lanes past the rows repeat the last
        const float* lrow = lg + rl * LD + wave * (E / 4);
#pragma unroll 4
        for (int c4 = 0; c4 < E / 16; ++c4) {
            const float4 q4 = *reinterpret_cast<const float4*>(lrow + 4 * c4);
            const int e0 = wave * (E / 4) + 4 * c4;
            top8_insert(tl, ordered_bits(q4.x), e0);
            top8_insert(tl, ordered_bits(q4.y), e0 + 1);
            top8_insert(tl, ordered_bits(q4.z), e0 + 2);
            top8_insert(tl, ordered_bits(q4.w), e0 + 3);
        }
        uint32_t* mv = reinterpret_cast<uint32_t*>(lg + RB * LD);  // [3][8][RB] keys, then experts
        int* mi = reinterpret_cast<int*>(mv + 3 * 8 * RB);
        if (wave > 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                mv[((wave - 1) * 8 + j) * RB + lane] = tl.v[j];
                mi[((wave - 1) * 8 + j) * RB + lane] = tl.e[j];
            }
        }
        __syncthreads();
        if (wave == 0) {
            for (int w = 0; w < 3; ++w)
#pragma unroll
                for (int j = 0; j < 8; ++j) top8_insert(tl, mv[(w * 8 + j) * RB + lane], mi[(w * 8 + j) * RB + lane]);
            if (lane < rows) {
                float wj[8];
                top8_weights(tl, k, wj);
                const size_t t = (size_t)(t0 + lane);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (j < k) {
                        topk_ids[t * k + j] = tl.e[j];
                        topk_w[t * k + j] = wj[j];
                        atomicAdd(&hist[tl.e[j]], 1);
                    }
            }
        }
    } else {
        // top-k per token, one wave per token: the selection of route_topk_kernel,
        // four tokens at a time (r, r + 4, r + 8, r + 12) so that their chains of
        // k dependent wave reductions interleave (one wave per SIMD here: nothing
        // else hides their latency); a slot past the block's rows repeats the
        // last row and stores nothing
        constexpr int NV = E / 64;
        constexpr int TS = R_THREADS / 64;
        constexpr int RQ = 4;
        for (int r = wave; r < rows; r += RQ * TS) {
            int rr[RQ];
    #pragma unroll
            for (int q = 0; q < RQ; ++q) rr[q] = min(r + q * TS, rows - 1);
            uint32_t ord[RQ][NV];
    #pragma unroll
            for (int q = 0; q < RQ; ++q)
    #pragma unroll
                for (int i = 0; i < NV; ++i) ord[q][i] = ordered_bits(lg[rr[q] * LD + lane + 64 * i]);
            int my_e[RQ];
            float my_v[RQ];
    #pragma unroll
            for (int q = 0; q < RQ; ++q) {
                my_e[q] = 0;
                my_v[q] = 0.0f;
            }
            wave_topk<NV, RQ>(ord, k, lane, my_e, my_v);
    #pragma unroll
            for (int q = 0; q < RQ; ++q) {
                const float v0 = __shfl(my_v[q], 0, 64);
                const float z = lane < k ? expf(my_v[q] - v0) : 0.0f;
                const float sum = wave_sum(z);
                if (lane < k && r + q * TS < rows) {
                    const size_t t = (size_t)(t0 + rr[q]);
                    topk_ids[t * k + lane] = my_e[q];
                    topk_w[t * k + lane] = z / sum;
                    atomicAdd(&hist[my_e[q]], 1);
                }
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += R_THREADS)
        if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// Router logits for a few tokens (T <= 32), split over the experts: block j
// computes logits[t, 32 j .. 32 j + 31] for every token and writes them out.
// The fused kernel has one block stream the whole router matrix; here E / 32
// blocks each stream their 32 rows.  Every logit goes through exactly the MFMA
// chain of router_topk_kernel (bf16 32x32x16, acc starting at zero, the 16-k
// steps of the reduction in ascending order, lane half g holding k 8 g .. 8 g
// + 7 of a step), so both kernels produce the same logits bit for bit, and
// the gate applied to them afterwards makes the same choice.
//
// The four waves fill an LDS ring of 512-k batches by direct-to-LDS loads
// (one 1 KB row per instruction: rows 0..31 the block's router rows, then XR
// token rows, zeros past T read from past the buffer end); wave 0 runs the
// MFMAs of one batch while the later ones land.  XR = 16 token rows (T <= 16)
// leave room for three slots, so 96 KB of router rows are in flight per CU
// instead of 64 KB; A-operand lanes past XR repeat a row (their results are
// never stored).  Position p of a row holds its 16-byte chunk p ^ (r & 15),
// so each 16-lane fragment read covers 16 distinct bank groups.
constexpr int RS_BK = 512;                           // k per batch
constexpr uint32_t RS_ROW = RS_BK * 2;               // bytes of one row per batch
constexpr int RS_TMAX = 32;
template <int XR>
struct SplitRing {
    static constexpr int ROWS = 32 + XR;             // router rows + token rows per slot
    static constexpr int LPW = ROWS / 4;             // load instructions per wave per batch
    static constexpr int NSL = XR == 16 ? 3 : 2;     // slots
    static constexpr uint32_t SLOT = ROWS * RS_ROW;
    static constexpr uint32_t LDS = NSL * SLOT;
    static_assert(LDS <= 160 * 1024, "the ring exceeds the LDS");
    static_assert(NSL * LPW <= 63 && NSL <= 3, "loads in flight beyond the wait counter or the wait table");
};

// wait until at most N of this wave's LDS reads are outstanding, the four
// operand registers of one two-step group tied to the wait
template <int N>
__device__ __forceinline__ void lds_wait_group(u32x4 (&a)[2], u32x4 (&w)[2]) {
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a[0]), "+v"(a[1]), "+v"(w[0]), "+v"(w[1]) : "n"(N) : "memory");
}

template <int XR>
__global__ __launch_bounds__(R_THREADS, 1)
void router_logits_split_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int E,
                                int H, float* __restrict__ logits) {
    using R = SplitRing<XR>;
    extern __shared__ u32x4 smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int e0 = blockIdx.x * 32;
    const int NB = (H + RS_BK - 1) / RS_BK;
    const uint32_t xbytes = (uint32_t)((size_t)T * H * 2);
    const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(wr, (uint32_t)((size_t)E * H * 2));
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x, xbytes);
    // load instruction i of wave w fills row r = LPW w + i of a slot
    uint32_t voff[R::LPW];
#pragma unroll
    for (int i = 0; i < R::LPW; ++i) {
        const int r = R::LPW * wave + i;
        const uint32_t ch = (uint32_t)((lane ^ (r & 15)) * 16);
        if (r < 32) voff[i] = (uint32_t)(e0 + r) * (uint32_t)H * 2u + ch;
        else voff[i] = r - 32 < T ? (uint32_t)(r - 32) * (uint32_t)H * 2u + ch : xbytes;
    }
    auto issue = [&](int b, int slot) {
        char* st = reinterpret_cast<char*>(smem) + slot * R::SLOT;
#pragma unroll
        for (int i = 0; i < R::LPW; ++i) {
            const int r = R::LPW * wave + i;                // wave-uniform: the resource stays scalar
            dma16(r < 32 ? wsrc : xsrc, st + r * RS_ROW, voff[i], (uint32_t)b * RS_ROW);
        }
    };

    f32x16 acc = f32x16{};
    for (int b = 0; b < min(R::NSL, NB); ++b) issue(b, b);
    int slot = 0;
    for (int b = 0; b < NB; ++b) {
        switch (min(R::NSL - 1, NB - 1 - b)) {              // batch b landed (this wave's rows) ...
            case 0: vm_wait<0>(); break;
            case 1: vm_wait<R::LPW>(); break;
            default: vm_wait<2 * R::LPW>(); break;
        }
        lds_barrier();                                      // ... and every wave's
        if (wave == 0) {
            const uint32_t st = lds_addr(smem) + slot * R::SLOT;
            const uint32_t wb = st + (uint32_t)n * RS_ROW, xb = st + (uint32_t)(32 + (n & (XR - 1))) * RS_ROW;
            const uint32_t sw = (uint32_t)(n & 15);
            const int nq = min(RS_BK, H - b * RS_BK) / 32;  // groups of two 16-k steps (H % 32 == 0)
            auto rd = [&](int q, u32x4 (&a)[2], u32x4 (&w)[2]) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint32_t off = ((uint32_t)(4 * q + 2 * s + g) ^ sw) * 16u;
                    a[s] = ds_read16<0>(xb + off);
                    w[s] = ds_read16<0>(wb + off);
                }
            };
            auto mfma2 = [&](const u32x4 (&a)[2], const u32x4 (&w)[2]) {
                acc = mfma_bf16(a[0], w[0], acc);
                acc = mfma_bf16(a[1], w[1], acc);
            };
            if (nq == RS_BK / 32) {
                // a full batch, unrolled: the next group's reads are in flight
                // during this group's MFMAs (no register set carried round a
                // loop, which would let the compiler copy a read's destination
                // before its wait)
                u32x4 a0[2], w0[2], a1[2], w1[2];
                rd(0, a0, w0);
                static_for<RS_BK / 64>([&](auto h_c) {
                    constexpr int Q = 2 * decltype(h_c)::value;
                    rd(Q + 1, a1, w1);
                    lds_wait_group<4>(a0, w0);
                    mfma2(a0, w0);
                    if constexpr (Q + 2 < RS_BK / 32) {
                        rd(Q + 2, a0, w0);
                        lds_wait_group<4>(a1, w1);
                    } else {
                        lds_wait_group<0>(a1, w1);
                    }
                    mfma2(a1, w1);
                });
            } else {
                for (int q = 0; q < nq; ++q) {                // the last, partial batch
                    u32x4 a[2], w[2];
                    rd(q, a, w);
                    lds_wait_group<0>(a, w);
                    mfma2(a, w);
                }
            }
        }
        lds_barrier();                                      // slot free
        if (b + R::NSL < NB) issue(b + R::NSL, slot);
        slot = slot + 1 == R::NSL ? 0 : slot + 1;
    }
    // lane holds expert e0 + n, tokens 8 (i >> 2) + 4 g + (i & 3)
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * g + (i & 3);
            if (m < T) logits[(size_t)m * E + e0 + n] = acc[i];
        }
    }
}

// the router kernels use more dynamic LDS than the default cap: raised once
// per device (and kernel) before its first launch there
std::mutex g_router_mu;
bool g_router_lds_set[64][4] = {};
bool g_split_lds_set[64][2] = {};

template <int XR>
hipError_t router_split_launch(const uint16_t* x, const uint16_t* wr, int T, int E, int H, int k, int32_t* ids,
                               float* w, int32_t* counts, float* logits, hipStream_t s) {
    using R = SplitRing<XR>;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    {
        std::lock_guard<std::mutex> lock(g_router_mu);
        if (!g_split_lds_set[dev][XR / 16 - 1]) {
            err = hipFuncSetAttribute((const void*)router_logits_split_kernel<XR>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)R::LDS);
            if (err != hipSuccess) return err;
            g_split_lds_set[dev][XR / 16 - 1] = true;
        }
    }
    router_logits_split_kernel<XR><<<E / 32, R_THREADS, R::LDS, s>>>(x, wr, T, E, H, logits);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_route_topk(logits, T, E, k, ids, w, counts, s);
}

template <int CT>
hipError_t router_launch(const uint16_t* x, const uint16_t* wr, int T, int H, int k, int32_t* ids, float* w,
                         int32_t* counts, float* logits, hipStream_t s) {
    constexpr int E = 128 * CT;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    {
        std::lock_guard<std::mutex> lock(g_router_mu);
        if (!g_router_lds_set[dev][CT - 1]) {
            err = hipFuncSetAttribute((const void*)router_topk_kernel<CT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)router_lds_bytes(E));
            if (err != hipSuccess) return err;
            g_router_lds_set[dev][CT - 1] = true;
        }
    }
    zero_i32_kernel<<<(E + 255) / 256, 256, 0, s>>>(counts, E);
    router_topk_kernel<CT><<<(T + RB - 1) / RB, R_THREADS, router_lds_bytes(E), s>>>(x, wr, T, H, k, ids, w,
                                                                                      counts, logits);
    return hipGetLastError();
}

}  // namespace

bool router_shape_ok(int T, int E, int H) {
    return E % 128 == 0 && E >= 128 && E <= 512 && H % 32 == 0 && H >= 32 && (size_t)T * H * 2 < (1ull << 32) &&
           (size_t)E * H * 2 < (1ull << 32);
}

hipError_t launch_router_topk(const uint16_t* x, const uint16_t* w_router, int T, int E, int H, int k,
                              int32_t* topk_ids, float* topk_w, int32_t* counts, float* logits, float* scratch_logits,
                              hipStream_t s) {
    // a few tokens with somewhere to put the logits (the caller's buffer, or
    // else the caller's workspace): the GEMM over E / 32 blocks, then the
    // gate on the stored logits (the same logits and choice as on chip)
    if (!logits && T <= RS_TMAX) logits = scratch_logits;
    if (logits && T <= 16) return router_split_launch<16>(x, w_router, T, E, H, k, topk_ids, topk_w, counts, logits, s);
    if (logits && T <= RS_TMAX)
        return router_split_launch<32>(x, w_router, T, E, H, k, topk_ids, topk_w, counts, logits, s);
    switch (E / 128) {
        case 1: return router_launch<1>(x, w_router, T, H, k, topk_ids, topk_w, counts, logits, s);
        case 2: return router_launch<2>(x, w_router, T, H, k, topk_ids, topk_w, counts, logits, s);
        case 3: return router_launch<3>(x, w_router, T, H, k, topk_ids, topk_w, counts, logits, s);
        default: return router_launch<4>(x, w_router, T, H, k, topk_ids, topk_w, counts, logits, s);
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, hipStream_t s) {
    const int nv = (E + WAVE - 1) / WAVE;
    if (nv <= 1) route_launch<1>(logits, T, E, k, topk_ids, topk_w, counts, s);
    else if (nv <= 2) route_launch<2>(logits, T, E, k, topk_ids, topk_w, counts, s);
    else if (nv <= 4) route_launch<4>(logits, T, E, k, topk_ids, topk_w, counts, s);
    else if (nv <= 6) route_launch<6>(logits, T, E, k, topk_ids, topk_w, counts, s);    // E = 384
    else if (nv <= 8) route_launch<8>(logits, T, E, k, topk_ids, topk_w, counts, s);
    else route_launch<16>(logits, T, E, k, topk_ids, topk_w, counts, s);
    return hipGetLastError();
}

}  // namespace moe
