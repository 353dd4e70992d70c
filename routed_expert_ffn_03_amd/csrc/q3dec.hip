// 3-bit gate/up for decode batches: a = silu(x W_gate^T) * (x W_up^T) for
// every (token, expert) pair when the batch has only a few tokens, so that
// every route list is a streaming ("thin") tile of at most Q3DEC_MAX_T rows.
//
// Same arithmetic as the pair-slot path of the 3-bit streaming kernel in
// ffn.hip (3-bit codes fed to the MFMA as the exact bf16 numbers 128 + u,
// activations in the matching pair-slot order, minus 132 x the group sum of
// x, fp16 group scales applied in fp32), reorganised around the two facts of
// a decode step: all tokens' x rows fit in LDS, and the weights are streamed
// once.  Sources: the 3-bit experts served by the pages (dsv41-flash-offload
// wiki, opening paragraph: 3.0 bpw experts); the format is this library's
// reading (groups of 128, 13 words, fp16 scale).
//
// One block of 16 waves per CU:
//   1. the block stages every token's x row in pair-slot order and its group
//      sums in LDS (row T is zeros, for lanes without a token);
//   2. wave p owns group pair p (groups 2p, 2p+1) of the reduction index for
//      the whole launch and streams, item after item, the 13 words of its
//      groups of the item's 16 gate and 16 up rows, two items ahead of the
//      one it computes (the loads of a wave never wait on an item boundary);
//   3. per item the 16 waves' partial 32 x 32 tiles are summed through LDS
//      and SwiGLU is applied across the gate and up halves by a lane shuffle.
// Items are (thin tile, 16-row N-tile) pairs in the order of the streaming
// kernel, handed out to blocks in static rounds.
#include "common.h"
#include "ffn_shared.h"

#include <mutex>

namespace moe {
namespace {

constexpr int QD_WAVES = 16;
constexpr int QD_THREADS = QD_WAVES * WAVE;
constexpr uint32_t QD_RED = QD_WAVES * 8 * 64 * 4;      // partial tiles: [wave][8 rows][64 lanes] fp32

__host__ __device__ constexpr uint32_t qd_sums_bytes(int T, int H) { return (uint32_t)(T * (H / 128) * 4 + 15) / 16 * 16; }
// NRED partial-tile buffers: with two, an item's partials go to one while the
// previous item's are summed from the other, so one barrier per item suffices
// the thin tile list (expert, first row << 6 | rows): with at most 14 tokens
// an expert's route list is one tile, so there are at most min(E, T k) tiles
__host__ __device__ constexpr uint32_t qd_tiles_bytes(int T, int E, int k) {
    return (uint32_t)((T * k < E ? T * k : E) * 8 + 15) / 16 * 16;
}
__host__ __device__ constexpr uint32_t qd_lds_bytes(int T, int H, int E, int k, int NRED) {
    return (uint32_t)((T + 1) * H * 2) + qd_sums_bytes(T, H) + qd_tiles_bytes(T, E, k) + NRED * QD_RED;
}

typedef __attribute__((ext_vector_type(4), aligned(4))) uint32_t u32x4w;   // 4-byte aligned 16-byte load

// One item's operands of one lane, as loaded: nothing is computed from a
// loaded value until the item is run (two items later), so no wait for the
// loads is placed where they are issued.
struct QdItem {
    uint32_t w[Q3_WORDS];           // the 13 words of its group of its weight row
    uint32_t s;                     // fp16 scales of groups 2p (low half) and 2p + 1 (high half)
    int pr;                         // the pair of the tile row of this lane (of its last row past the rows)
    int rr;                         // the tile's first sorted row << 6 | its row count
};

// QUAD (at most 4 tokens): 16x16x32 products instead.  Waves 0-7 take the
// item's 16 gate rows, waves 8-15 its 16 up rows, wave w & 7 a quad of
// groups (4 (w & 7) ..); lane quarter q (L / 16) holds group 4 (w & 7) + q of
// its weight row (column L % 16) in k-quarter q, and the activation lanes of
// row 4 q + i hold token i of that group there, so the 16 result rows are 4
// groups x 4 tokens with no padding rows (half the MFMA work of the 32-row
// tiles); each group's scale is applied on its own rows, the four groups are
// summed across the lane quarters, and 64 threads sum the 8 waves of each half
// and apply SwiGLU.
template <int NRED, bool QUAD>
__global__ __launch_bounds__(QD_THREADS, 1)
void ffn_q3_decode_kernel(FfnArgs a) {
    extern __shared__ u32x4 smem[];
    const int T = a.T, H = a.H, I = a.I, k = a.k;
    const int NG = H >> 7, NP = (NG + 1) >> 1;
    uint16_t* xl = reinterpret_cast<uint16_t*>(smem);
    uint32_t* xsl = reinterpret_cast<uint32_t*>(xl + (size_t)(T + 1) * H);
    int2* const tl = reinterpret_cast<int2*>(reinterpret_cast<char*>(smem) + (T + 1) * H * 2 + qd_sums_bytes(T, H));
    float* const red0 = reinterpret_cast<float*>(reinterpret_cast<char*>(tl) + qd_tiles_bytes(T, a.E, k));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 31, g = lane >> 5, mm = m & 15;

    // 1. x rows in pair-slot order and group sums; row T all zeros.  QUAD:
    //    the rows first go as they are into the first reduction buffer
    //    (unused until the first item; T <= 4 and H <= 16 x 256 bound them
    //    to its 32 KB), in whole 16-byte pieces, and
    //    are reordered from there by eight threads per token and group (two
    //    of its 16 slot chunks each; their partial sums meet by xor shuffles
    //    in a fixed order)
    if constexpr (QUAD) {
        uint16_t* xraw = reinterpret_cast<uint16_t*>(red0);
        for (int i = tid; i < T * H / 8; i += QD_THREADS)
            reinterpret_cast<u32x4*>(xraw)[i] = ldg16(a.x + 8 * (size_t)i);
        __syncthreads();
        for (int u = tid; u < T * NG * 8; u += QD_THREADS) {
            const int task = u >> 3, part = u & 7;
            const int tok = task / NG, G = task - tok * NG;
            double sum = q3_prep_part_lds(xraw + (size_t)tok * H + G * 128, xl + (size_t)tok * H + G * 128, part, 8);
            sum += __shfl_xor(sum, 1, 64);
            sum += __shfl_xor(sum, 2, 64);
            sum += __shfl_xor(sum, 4, 64);
            if (part == 0) xsl[tok * NG + G] = q3_sum_pair_bf16(sum);
        }
    } else {
        for (int task = tid; task < T * NG; task += QD_THREADS) {
            const int tok = task / NG, G = task - tok * NG;
            q3_prep_group(a.x + (size_t)tok * H + G * 128, xl + (size_t)tok * H + G * 128, xsl + tok * NG + G);
        }
    }
    for (int i = tid; i < H / 8; i += QD_THREADS) reinterpret_cast<u32x4*>(xl + (size_t)T * H)[i] = u32x4{0, 0, 0, 0};
    const int n_mt = a.hdr->n_thin, NT = I / 16;
    if (n_mt == 0) return;                                 // every route list ran as MFMA tiles
    for (int i = tid; i < n_mt; i += QD_THREADS) {
        const MTile t = a.thin[i];
        tl[i] = make_int2(t.e, (t.row0 << 6) | t.rows);
    }
    __syncthreads();

    const int n_items = n_mt * NT;
    // QUAD: this wave's half (gate / up) and quad, this lane's column and quarter
    const int NQ = (NG + 3) >> 2;
    const int half = wave >> 3, pq = wave & 7, qn = lane & 15, qq = lane >> 4;
    const int p = wave;                                    // this wave's group pair
    const bool active = QUAD ? pq < NQ : p < NP;
    const int Gl = QUAD ? 4 * pq + qq : 2 * p + g;         // this lane's group
    const int Gw = min(Gl, NG - 1);
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic));

    // operands of `item` for this lane.  Every call issues the same seven
    // loads at valid addresses (past the last item: the last item again;
    // waves past the group pairs: the last pair; the token of the tile's last
    // row for lanes without a row), so the wait counts the compiler places
    // before an item's first use are exact and never drain the loads of the
    // items after it.
    const int pl = min(p, NP - 1);
    const int Gld = QUAD ? min(4 * min(pq, NQ - 1) + qq, NG - 1) : min(2 * pl + g, NG - 1);
    auto load_item = [&](int item, QdItem& q) {
        const int ic = min(item, n_items - 1);
        const int nt = ic / n_mt, mt = ic - nt * n_mt;
        const int2 t = tl[mt];
        q.rr = t.y;
        const int rows = t.y & 63, row0 = t.y >> 6;
        if constexpr (QUAD) {
            const size_t row = (size_t)t.x * I + nt * 16 + qn;   // gate (waves 0-7) or up (8-15) row of column qn
            const uint32_t* gw = reinterpret_cast<const uint32_t*>(half ? a.wu : a.wg) + (row * NG + Gld) * Q3_WORDS;
            const u32x4w q0 = *reinterpret_cast<const u32x4w*>(gw);
            const u32x4w q1 = *reinterpret_cast<const u32x4w*>(gw + 4);
            const u32x4w q2 = *reinterpret_cast<const u32x4w*>(gw + 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                q.w[i] = q0[i];
                q.w[4 + i] = q1[i];
                q.w[8 + i] = q2[i];
            }
            q.w[12] = gw[12];
            q.s = (half ? a.su : a.sg)[row * NG + Gld];
            q.pr = a.sorted_pair[row0 + min(qn & 3, rows - 1)];   // the token of activation row qn
            return;
        }
        const size_t row = (size_t)t.x * I + nt * 16 + mm;   // gate rows (m < 16), then the matching up rows
        const uint32_t* gw = reinterpret_cast<const uint32_t*>(m < 16 ? a.wg : a.wu) + (row * NG + Gld) * Q3_WORDS;
        const u32x4w q0 = *reinterpret_cast<const u32x4w*>(gw);
        const u32x4w q1 = *reinterpret_cast<const u32x4w*>(gw + 4);
        const u32x4w q2 = *reinterpret_cast<const u32x4w*>(gw + 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q.w[i] = q0[i];
            q.w[4 + i] = q1[i];
            q.w[8 + i] = q2[i];
        }
        q.w[12] = gw[12];
        const uint16_t* srow = (m < 16 ? a.sg : a.su) + row * NG;
        q.s = *reinterpret_cast<const uint32_t*>(srow + 2 * pl);   // NG even: both scales, one aligned dword
        q.pr = a.sorted_pair[row0 + min(mm, rows - 1)];
    };

    auto run_item = [&](int item, const QdItem& q, int buf) {
        const int nt = item / n_mt;
        float* red = red0 + buf * (QD_RED / 4);
        if constexpr (QUAD) {
            if (active) {
                const bool act = (qn >> 2) == qq && (qn & 3) < (q.rr & 63) && Gl < NG;
                const int xr = act ? q.pr / k : T;             // LDS row of the token (T: zeros)
                const uint16_t* xa = xl + (size_t)xr * H + Gw * 128;
                f32x4 c = f32x4{};
                static_for<16>([&](auto j_c) {
                    constexpr int J = decltype(j_c)::value;
                    const u32x4 av = *reinterpret_cast<const u32x4*>(xa + 8 * J);
                    u32x4 bv;
                    static_for<4>([&](auto q_c) {
                        constexpr int Q = decltype(q_c)::value;
                        bv[Q] = magic_pair<4 * J + Q>(q.w, magic);
                    });
                    c = mfma16_bf16(av, bv, c);
                });
                // minus 132 x (group sum, bf16 hi + lo) in k-slots 0 and 1 of each quarter
                const uint32_t xs = xr < T ? xsl[xr * NG + Gl] : 0u;
                c = mfma16_bf16(u32x4{xs, 0u, 0u, 0u}, u32x4{0xC304C304u, 0u, 0u, 0u}, c);
                // result rows 4 qq + i: token i of group Gl; scaled, then the quad's four groups summed
                const uint16_t sh = (uint16_t)q.s;
                const float sc = Gl < NG ? (float)__builtin_bit_cast(_Float16, sh) : 0.0f;
                float f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f[i] = sc * c[i];
                    f[i] += __shfl_xor(f[i], 16, 64);
                    f[i] += __shfl_xor(f[i], 32, 64);
                }
                if (qq == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * 16 + qn] = f[i];
                }
            }
            __syncthreads();
            // token i, column n: the 8 gate waves' and the 8 up waves' partials
            if (tid < 64) {
                const int i = tid >> 4, n = tid & 15;
                float gs = 0.0f, us = 0.0f;
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    if (w < NQ) {
                        gs += red[(w * 4 + i) * 16 + n];
                        us += red[((8 + w) * 4 + i) * 16 + n];
                    }
                }
                const int rows = q.rr & 63, row0 = q.rr >> 6;
                if (i < rows) a.act[(size_t)(row0 + i) * I + nt * 16 + n] = f32_to_f16_bits(silu_mul(gs, us));
            }
            if (NRED == 1) __syncthreads();
            return;
        }
        if (active) {
            const bool act = (m >> 4) == g && mm < (q.rr & 63) && Gl < NG;
            const int xr = act ? q.pr / k : T;                 // LDS row of the token (T: zeros)
            const uint16_t* xa = xl + (size_t)xr * H + Gw * 128;
            f32x16 c = f32x16{};
            static_for<16>([&](auto j_c) {
                constexpr int J = decltype(j_c)::value;
                const u32x4 av = *reinterpret_cast<const u32x4*>(xa + 8 * J);
                u32x4 bv;
                static_for<4>([&](auto q_c) {
                    constexpr int Q = decltype(q_c)::value;
                    bv[Q] = magic_pair<4 * J + Q>(q.w, magic);
                });
                c = mfma_bf16(av, bv, c);
            });
            // minus 132 x (group sum, bf16 hi + lo): bf16 weights -132 in k-slots 0 and 1 of each half
            const uint32_t xs = xr < T ? xsl[xr * NG + Gl] : 0u;
            c = mfma_bf16(u32x4{xs, 0u, 0u, 0u}, u32x4{0xC304C304u, 0u, 0u, 0u}, c);
            const float s0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(q.s & 0xFFFFu));
            const float s1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(q.s >> 16));
#pragma unroll
            for (int r = 0; r < 8; ++r) red[(wave * 8 + r) * 64 + lane] = fmaf(s1, c[r + 8], s0 * c[r]);
        }
        __syncthreads();
        // the 16 partial tiles summed (all reads issued at once; waves past
        // the group pairs wrote nothing and are skipped); lane n < 16 of a
        // half holds gate column n, lane n + 16 the matching up column; output
        // row 8 (r >> 2) + 4 g + (r & 3)
        if (tid < 8 * 64) {
            const int r = tid >> 6, ln = tid & 63;
            float part[QD_WAVES];
#pragma unroll
            for (int w = 0; w < QD_WAVES; ++w) part[w] = w < NP ? red[(w * 8 + r) * 64 + ln] : 0.0f;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < QD_WAVES; ++w) v += part[w];
            const float u = __shfl(v, (ln + 16) & 63, 64);
            const int rows = q.rr & 63, row0 = q.rr >> 6;
            const int n = ln & 31, row = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
            if (n < 16 && row < rows)
                a.act[(size_t)(row0 + row) * I + nt * 16 + n] = f32_to_f16_bits(silu_mul(v, u));
        }
        if (NRED == 1) __syncthreads();
    };

    // 2.-3. items b, b + G, ... with the weights of the next two in flight
    const int G = gridDim.x;
    QdItem ring[3];
    int it = blockIdx.x;
    int par = 0;                                          // the partial buffer of ring slot 0 this round
    load_item(it, ring[0]);
    load_item(it + G, ring[1]);
    for (;;) {
        bool done = false;
        static_for<3>([&](auto s_c) {
            constexpr int S = decltype(s_c)::value;
            if (done) return;
            if (it >= n_items) {
                done = true;
                return;
            }
            load_item(it + 2 * G, ring[(S + 2) % 3]);
            run_item(it, ring[S], NRED == 2 ? (S & 1) ^ par : 0);
            it += G;
        });
        if (done) break;
        par ^= 1;                                         // three items per round: the parity flips
    }
}

std::mutex g_qd_mu;
bool g_qd_ready[64] = {};

}  // namespace

bool q3dec_fits(int T, int E, int k, int H) {
    return T >= 1 && T <= Q3DEC_MAX_T && H % 256 == 0 && H / 256 <= QD_WAVES && qd_lds_bytes(T, H, E, k, 1) <= 160u * 1024u;
}

hipError_t launch_q3dec_gate_up(const FfnArgs& fa, int cus, hipStream_t s) {
    if (!q3dec_fits(fa.T, fa.E, fa.k, fa.H)) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    {
        std::lock_guard<std::mutex> lock(g_qd_mu);
        if (!g_qd_ready[dev]) {
            const void* kern[4] = {(const void*)ffn_q3_decode_kernel<1, false>, (const void*)ffn_q3_decode_kernel<2, false>,
                                   (const void*)ffn_q3_decode_kernel<1, true>, (const void*)ffn_q3_decode_kernel<2, true>};
            for (int i = 0; i < 4 && err == hipSuccess; ++i)
                err = hipFuncSetAttribute(kern[i], hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (err != hipSuccess) return err;
            g_qd_ready[dev] = true;
        }
    }
    // at most 4 tokens (so every tile at most 4 rows): the 16x16x32 form
    const bool quad = fa.T <= 4;
    const bool two = qd_lds_bytes(fa.T, fa.H, fa.E, fa.k, 2) <= 160u * 1024u;
    const uint32_t lds = qd_lds_bytes(fa.T, fa.H, fa.E, fa.k, two ? 2 : 1);
    if (quad) {
        if (two) ffn_q3_decode_kernel<2, true><<<cus, QD_THREADS, lds, s>>>(fa);
        else ffn_q3_decode_kernel<1, true><<<cus, QD_THREADS, lds, s>>>(fa);
    } else {
        if (two) ffn_q3_decode_kernel<2, false><<<cus, QD_THREADS, lds, s>>>(fa);
        else ffn_q3_decode_kernel<1, false><<<cus, QD_THREADS, lds, s>>>(fa);
    }
    return hipGetLastError();
}

}  // namespace moe
