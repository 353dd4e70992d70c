// HBM-streaming ("thin") grouped FFN kernel for bf16 expert weights: route
// lists of fewer than fat_threshold rows, and every expert of a decode step.
//
// Same work items and results as the thin kernels of ffn.hip (work item = 32
// weight rows x one thin M-tile of up to 32 rows; phase 1: 16 gate rows + the
// 16 matching up rows with SwiGLU in the epilogue, phase 2: 32 rows of
// W_down; the four waves split the reduction index and sum their partial
// tiles through LDS).  Sources: less busy experts on their own streaming path
// (dsv41-flash-offload wiki, opening paragraph and file table, stock
// group-kernel entry); decode reads only the experts its tokens picked
// (wiki, "PCIe is the bottleneck" paragraph).
//
// What differs is how the weights travel.  Each weight element is used once,
// so the kernel is bound by HBM reads, and their rate depends on the shape of
// each load instruction: one that covers whole 128-byte lines with the
// non-temporal hint streams ~18% faster on MI355X than the MFMA operand
// layout read straight from memory, which touches 32 bytes of each of 32
// rows per instruction (6.8 vs 5.7 TB/s over 906 MB of 32-row x 8 KB items).
// So the weights go through LDS: a direct-to-LDS buffer load moves 8 rows x
// 128 bytes (8 lanes per line), and the MFMA fragments are read back with
// ds_read_b128.  Every wave streams its own quarter of the reduction index
// through its own two-slot ring (one 64-k chunk = 32 rows x 128 B in flight
// while the previous one is multiplied), so the waves never wait for each
// other inside an item.  The chunk sequence runs on across items: the first
// chunk of a block's next item is in flight while the current item's four
// partial tiles are reduced.  Activations (a few rows, re-read by every item
// of their M-tile) stay on the ordinary cached path, straight into registers.
//
// LDS layout of a chunk slot: row r (0..31) at r * 128 bytes; its 16-byte
// piece c at position c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1), so the
// eight (or sixteen) lanes of one ds_read_b128 pass hit distinct banks.
#include "common.h"
#include "ffn_shared.h"
#include "kernels.h"
#include "lds_dma.h"

namespace moe {
namespace {

constexpr int ST_K = 64;                             // k per chunk: one line of every weight row
constexpr uint32_t ST_CHUNK = 32 * ST_K * 2;         // 4 KB: the item's 32 weight rows
constexpr int ST_SLOTS = 2;

// phase 2: b already holds fp16 weights (converted after the LDS read, or
// stored fp16 by weight format 2)
template <int PHASE>
__device__ __forceinline__ f32x16 st_mma(u32x4 a, u32x4 b, f32x16 c) {
    return PHASE == 1 ? mfma_bf16(a, b, c) : mfma_f16(a, b, c);
}

// One work item (wave-uniform: scalar registers).
struct StItem {
    MTile t;
    int nt;                              // column block of the expert matrix
    int es;                              // phase 1: its slot of route-list entries in LDS
};

template <int PHASE>
__global__ __launch_bounds__(THIN_THREADS)
void ffn_stream_kernel(FfnArgs a) {
    __shared__ __attribute__((aligned(1024))) char ring[4 * ST_SLOTS * ST_CHUNK];
    __shared__ float red[4][16][64];
    __shared__ int ent[4][3][64];                          // phase 1: route-list entries per wave
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 31, g = lane >> 5;
    const int K = PHASE == 1 ? a.H : a.I;
    const int N = PHASE == 1 ? a.I : a.H;                  // rows of one expert matrix
    const int NT = PHASE == 1 ? a.I / 16 : a.H / 32;
    const int n_mt = a.hdr->n_thin;
    const int n_items = n_mt * NT;
    const int G = gridDim.x;
    int item = blockIdx.x;
    if (item >= n_items) return;                           // the whole block
    const int Kw = K / 4;                                  // this wave's slice of k
    const int nch = Kw / ST_K;
    const uint32_t rowb = (uint32_t)K * 2u;
    const uint32_t kslice = (uint32_t)(wave * Kw) * 2u;
    const bool pairs = a.pairs != 0;                       // row-pair layout (weight format 2)
    // bytes from a row's (pair's) start to this wave's slice, and per chunk
    const uint32_t kofs = pairs ? 2 * kslice : kslice;
    const uint32_t chofs = pairs ? 2 * (ST_K * 2) : ST_K * 2;
    const size_t mbytes = (size_t)N * K * 2;

    // load instruction i moves rows 8 i .. 8 i + 7 of the chunk; lane L puts
    // row 8 i + L / 8, position L % 8, which holds piece (L % 8) ^ swz(row).
    // Piece P of a row's 64-k chunk lies at 16 P bytes from the chunk's start
    // in the plain layout; in the row-pair layout (rows 2p and 2p + 1
    // alternate every 32 k, 64 B each) the pair's chunk is 256 contiguous
    // bytes and the piece lies at 128 (P / 4) + 64 (row & 1) + 16 (P % 4).
    const int lr = lane >> 3;
    auto piece_off = [&](int P) -> uint32_t {
        return pairs ? (uint32_t)((P >> 2) * 128 + (lr & 1) * 64 + (P & 3) * 16) : (uint32_t)(P * 16);
    };
    const uint32_t pofs[2] = {piece_off((lane & 7) ^ lr), piece_off((lane & 7) ^ lr ^ 1)};
    const int lrow = pairs ? (lr & ~1) : lr;               // the row (pair) whose start the lane adds
    uint32_t vconst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r8 = PHASE == 1 ? 8 * (i & 1) : 8 * i;     // phase 1: i < 2 gate rows, i >= 2 up rows
        vconst[i] = (uint32_t)r8 * rowb + pofs[i & 1];
    }
    // fragment reads: MFMA step s (16 k), lane (m, g) takes row m, piece 4 g + s
    const int swn = (m & 7) ^ ((m >> 3) & 1);
    const uint32_t wbase = lds_addr(ring) + (uint32_t)(wave * ST_SLOTS) * ST_CHUNK;
    uint32_t rdo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) rdo[s] = wbase + (uint32_t)m * (ST_K * 2) + (uint32_t)(((4 * g + s) ^ swn) << 4);

    // An item's values come from its M-tile (a scalar load) and, in phase 1,
    // the route-list entries of its rows, which give the tokens.  Both are
    // fetched ahead (M-tiles three items ahead; entries two items ahead,
    // straight into LDS) and used an item later, so that no wait for them
    // drains the weight stream: an item is at least one chunk, and every
    // chunk waits for all loads but its successor's eight.  Only scalar
    // values carry over from one chunk to the next; the per-lane addresses
    // are recomputed at every issue (a vector register that carried over
    // could share its register with a load in flight, and copying it would
    // wait for that load).  Items past the end are clamped to the last one
    // (valid addresses, never multiplied).
    const __amdgpu_buffer_rsrc_t psrc = make_rsrc(a.sorted_pair, (uint32_t)((size_t)a.T * a.k * 4));
    // (the tile list is read-only here: through the constant address space
    // it is fetched with scalar loads)
    typedef const __attribute__((address_space(4))) MTile* ctile_t;
    auto load_item = [&](int it, int es) {
        StItem q;
        const int ic = min(it, n_items - 1);
        q.nt = ic / n_mt;
        const ctile_t tp = (ctile_t)a.thin + __builtin_amdgcn_readfirstlane(ic - q.nt * n_mt);
        q.t = MTile{};
        q.t.e = tp->e;
        q.t.row0 = tp->row0;
        q.t.rows = tp->rows;
        q.es = es;
        return q;
    };
    // the route-list entries of item q's rows (lane L: row min(L % 32, rows - 1)) into its LDS slot
    auto load_entries = [&](const StItem& q) {
        if constexpr (PHASE == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(psrc, (lds_ptr_t)&ent[wave][q.es][0], 4,
                                                     (uint32_t)(q.t.row0 + min(m, q.t.rows - 1)) * 4u, 0, 0, 0);
    };
    // the weights of chunk ch of item q into ring slot sl: four direct-to-LDS
    // loads of 8 rows x 128 B (non-temporal)
    auto issue_w = [&](const StItem& q, int ch, int sl) {
        const size_t eoff = (size_t)q.t.e * mbytes;
        const __amdgpu_buffer_rsrc_t w0 =
            make_rsrc(reinterpret_cast<const char*>(PHASE == 1 ? a.wg : a.wd) + eoff, (uint32_t)mbytes);
        const __amdgpu_buffer_rsrc_t w1 =
            PHASE == 1 ? make_rsrc(reinterpret_cast<const char*>(a.wu) + eoff, (uint32_t)mbytes) : w0;
        const uint32_t vrow = (uint32_t)((PHASE == 1 ? 16 : 32) * q.nt + lrow) * rowb;
        char* st = ring + (wave * ST_SLOTS + sl) * ST_CHUNK;
        const uint32_t soff = kofs + (uint32_t)ch * chofs;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(i < 2 ? w0 : w1, (lds_ptr_t)(st + i * 1024), 16,
                                                     vrow + vconst[i], soff, 0, 2);
    };
    // the activation fragments of chunk ch of item q (lanes past the tile's
    // rows repeat its last row: their output rows are never stored)
    auto issue_a = [&](const StItem& q, int ch, u32x4 (&ra)[4]) {
        const uint16_t* row;
        if constexpr (PHASE == 1) {
            uint32_t entry = ds_read4(lds_addr(&ent[wave][q.es][m]));
            lds_wait_all();
            tie_after_wait(entry);                         // no use of it before the wait
            row = a.x + (size_t)((int)entry / a.k) * a.H;
        } else {
            row = a.act + (size_t)(q.t.row0 + min(m, q.t.rows - 1)) * a.I;
        }
        const uint16_t* arow = row + wave * Kw + 32 * g + ch * ST_K;
#pragma unroll
        for (int s = 0; s < 4; ++s) ra[s] = ldg16(arow + 8 * s);
    };

    // entry slots rotate over three items: current, next, the one after
    StItem cur = load_item(item, 0), nxt = load_item(item + G, 1);
    load_entries(cur);
    load_entries(nxt);
    StItem i2 = load_item(item + 2 * G, 2);
    load_entries(i2);
    StItem i3 = load_item(item + 3 * G, 0);
    vm_wait<0>();
    bool has_next = item + G < n_items;
    int ch = 0, sl = 0;
    f32x16 acc = f32x16{};
    u32x4 ra[4];
    issue_w(cur, 0, 0);
    issue_a(cur, 0, ra);

    // Per chunk: issue the weights of the chunk after it (past the block's
    // last chunk, a repeat of the clamped next item's first one, never read);
    // wait for all loads but those four; multiply; at an item's last chunk
    // reduce and move on; then issue the activation fragments of the chunk
    // after it.  The fragments are issued after the MFMAs that consume the
    // previous ones, so a single set of registers carries them and no
    // register holding a load in flight ever needs to be copied.
    for (;;) {
        const bool last = ch + 1 == nch;
        issue_w(last ? nxt : cur, last ? 0 : ch + 1, sl ^ 1);
        vm_wait<4>();
        u32x4 b[4];
        const uint32_t so = (uint32_t)sl * ST_CHUNK;
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s] = ds_read16<0>(rdo[s] + so);
        lds_wait_all();
#pragma unroll
        for (int s = 0; s < 4; ++s) tie_after_wait(b[s]);
        if constexpr (PHASE == 2) {
            if (!pairs) {                                  // W_down bf16 -> fp16 (format 2 stores fp16)
#pragma unroll
                for (int s = 0; s < 4; ++s) b[s] = bf16x8_to_f16x8(b[s]);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = st_mma<PHASE>(ra[s], b[s], acc);
        sl ^= 1;
        if (last) {
            thin_reduce_store<PHASE>(a, acc, cur.t, cur.nt, red, wave, lane);
            acc = f32x16{};
            if (!has_next) break;
            item += G;
            has_next = item + G < n_items;
            const int free_slot = cur.es;
            cur = nxt;
            nxt = i2;
            i2 = i3;
            i2.es = free_slot;
            load_entries(i2);
            i3 = load_item(item + 3 * G, 0);
            ch = 0;
        } else {
            ++ch;
        }
        issue_a(cur, ch, ra);
    }
    vm_wait<0>();                                          // the unused last chunk has landed
}

}  // namespace

// each wave's quarter of the reduction index a whole number of chunks, and
// every buffer the kernel addresses with 32-bit offsets below 4 GB
bool stream_fits(int phase, int T, int k, int H, int I) {
    const size_t K = phase == 1 ? H : I;
    return K % (4 * ST_K) == 0 && (size_t)H * I * 2 < (1ull << 32) && (size_t)T * k * 4 < (1ull << 32);
}

hipError_t launch_stream_phase(const FfnArgs& fa, int phase, int blocks, hipStream_t s) {
    if (phase == 1) ffn_stream_kernel<1><<<blocks, THIN_THREADS, 0, s>>>(fa);
    else ffn_stream_kernel<2><<<blocks, THIN_THREADS, 0, s>>>(fa);
    return hipGetLastError();
}

int stream_occupancy(int phase) {
    int n = 0;
    const void* f = phase == 1 ? (const void*)ffn_stream_kernel<1> : (const void*)ffn_stream_kernel<2>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, THIN_THREADS, 0) != hipSuccess || n < 1) n = 1;
    return n;
}

}  // namespace moe
