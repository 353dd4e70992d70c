/*
 * moe_mi355x.h -- C ABI of the MI355X routed-expert (MoE) layer library.
 *
 * One MoE layer call is four entry points enqueued on one HIP stream:
 *
 *   moe_route_topk   router logits -> top-k expert ids, gate weights, load histogram
 *   moe_permute      ids -> per-expert route lists (offsets, sorted pairs, inverse)
 *   moe_grouped_ffn  every expert's SwiGLU FFN over its route list
 *   moe_combine      per-token gate-weighted sum of its k expert outputs
 *
 * What is computed, and where the pages say so:
 *   - routed experts per MoE layer (384 in the served model) and per-token
 *     routing: dsv41-flash-offload wiki, opening paragraph;
 *   - per-expert route lists with positive counts, and splitting large lists
 *     into batches that share one read of the expert's weights: wiki,
 *     repository file table, entries for the staged cold-expert prefill and
 *     segment patches;
 *   - busy experts (at least the "fat threshold" of 32 tokens) as GEMMs on
 *     reconstructed weights: wiki opening paragraph and file table (busy-expert
 *     GEMM entry); threshold value 32: recipe page "DeepSeek-V4.1-Flash /
 *     RTX 3090", step 3 environment block;
 *   - split of routed work and combine of the results on the GPU: wiki file
 *     table, CPU-tier entry;
 *   - failing loudly instead of falling back silently, and keeping host work
 *     out of graph-captured regions: "dsv41-flash-engram-disk-prestage",
 *     section "The prestage, per decode step", point 4.
 * The pages do not write down the gate function, the expert's form or the
 * 3-bit format; the readings implemented are stated at each function.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless stated; the caller owns every
 *     buffer (inputs, outputs and the workspace).  The library allocates no
 *     device or host memory; its one static array (the workspace of
 *     moe_grouped_ffn_noalloc, MOE_NOALLOC_SCRATCH_BYTES per GPU) comes with
 *     the code object.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued on it; no call synchronises the host with the
 *     device, so every call may be captured into a HIP graph.
 *   - Outputs are overwritten, never accumulated into.
 *   - The return value reports only what the host can check: argument
 *     validity (MOE_ERR_INVALID_ARG), shapes the kernels do not support
 *     (MOE_ERR_UNSUPPORTED -- there is no slower fallback), a workspace that
 *     is too small (MOE_ERR_WORKSPACE) and launch failures (MOE_ERR_HIP).  On
 *     any error nothing has been enqueued except, for MOE_ERR_HIP, the
 *     launches before the failing one.
 *   - Calls that share a workspace must be ordered on one stream.
 *   - Sizes: 1 <= T, 1 <= k <= min(E, 32), E <= 1024, T*k < 2^31.
 *   - bf16 and fp16 values are passed as their 16-bit patterns (uint16_t).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG  1
#define MOE_ERR_UNSUPPORTED  2
#define MOE_ERR_WORKSPACE    3
#define MOE_ERR_HIP          4

/* Expert weight storage formats accepted by moe_grouped_ffn. */
#define MOE_WFMT_BF16   0   /* bf16 matrices [E, out, in]                       */
#define MOE_WFMT_Q3G128 1   /* 3-bit codes, groups of 128 along `in`, fp16 scale */
#define MOE_WFMT_BF16_PAIRS 2 /* row-pair layout (moe_pack_bf16_pairs): gate/up bf16, down fp16 */

#define MOE_MAX_TOPK    32
#define MOE_MAX_EXPERTS 1024

/* Bytes of the per-GPU array that moe_grouped_ffn_noalloc uses as its
 * workspace (64 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status s);

/* Library version as "major.minor.patch" (static string). */
const char* moe_version(void);

/*
 * Bytes of workspace needed by moe_permute and moe_grouped_ffn for a layer
 * of T tokens, E experts, top-k, hidden H, expert intermediate I and the
 * weight format `wfmt`.  One buffer of this size serves both calls (they
 * use it in stream order).  MOE_WFMT_Q3G128 needs T*H*2 + T*(H/128)*4 more
 * bytes (rounded up to 256 each) than MOE_WFMT_BF16: a reordered copy of the
 * thin experts' activation rows and their 128-group sums.  Returns 0 for
 * arguments that are invalid or unsupported.  Alignment: 256 bytes (any
 * hipMalloc pointer).
 */
size_t moe_workspace_size(int T, int E, int k, int H, int I, int wfmt);

/*
 * moe_route_topk -- top-k gate over the layer's experts.
 *
 * For each token t (row of `logits`, fp32 [T, E], row-major):
 *   topk_ids[t, 0..k-1]  int32  the k experts with the largest logits, in
 *                        descending logit order; equal logits are ordered
 *                        by expert index ascending and -0.0 equals +0.0;
 *   topk_w[t, j]         fp32   softmax over the k selected logits,
 *                        exp(l_j - l_0) / sum_i exp(l_i - l_0);
 *   expert_counts[e]     int32  number of (token, slot) pairs routed to e
 *                        (the router's load histogram, E entries).
 * Reading of the pages (the gate is not written there): softmax over the
 * selected logits, no scaling factor, no shared expert.  Logits must be
 * finite; NaN/Inf give unspecified ids.  Errors: NULL pointers, T < 1,
 * E < 1 or E > 1024, k outside [1, min(E, 32)], T*k >= 2^31 ->
 * MOE_ERR_INVALID_ARG.
 */
moe_status moe_route_topk(const float* logits, int T, int E, int k,
                          int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                          void* stream);

/*
 * moe_router_topk -- the router GEMM fused with moe_route_topk.
 *
 * logits[t, e] = x[t, :] . w_router[e, :] (bf16 products, fp32 accumulation
 * on MFMA), then for every token exactly the selection, gate weights and
 * histogram of moe_route_topk applied to these fp32 logits.  The logits stay
 * on chip unless `logits` is non-NULL, in which case they are also written
 * there (fp32 [T, E], row-major).  For T <= 32 with somewhere to put the
 * logits -- `logits`, or else `workspace` -- the GEMM is spread over E / 32
 * blocks that write them, and the gate then runs on them (at 4 tokens and
 * 384 experts about 17 us instead of 77 us on the single block that keeps
 * them on chip); every logit goes through the same MFMA accumulation chain
 * as on chip, so ids, weights and histogram are bit-identical either way.
 * `workspace` (device, may be NULL) is used only then; when non-NULL it
 * must hold T * E * 4 bytes, else MOE_ERR_WORKSPACE.  Reading of the pages (routing over the
 * layer's routed experts: dsv41-flash-offload wiki, opening paragraph; the
 * router itself is not written there): a bias-free linear router over the
 * hidden state, the expert's rows stored [E, H] like the expert matrices.
 *
 * x          bf16 [T, H];   w_router  bf16 [E, H]
 * topk_ids int32 [T, k], topk_w fp32 [T, k], expert_counts int32 [E]: as
 *            moe_route_topk.
 * Shapes: E a multiple of 128 with 128 <= E <= 512, H a multiple of 32, and
 * T*H*2 and E*H*2 below 4 GiB, else MOE_ERR_UNSUPPORTED (moe_route_topk takes
 * any E <= 1024 from given logits).  Errors: NULL x, w_router, topk_ids,
 * topk_w or expert_counts, T < 1, k outside [1, min(E, 32)], T*k >= 2^31 ->
 * MOE_ERR_INVALID_ARG.
 */
moe_status moe_router_topk(const uint16_t* x, const uint16_t* w_router, int T, int E, int H, int k,
                           int32_t* topk_ids, float* topk_w, int32_t* expert_counts, float* logits,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_permute -- per-expert route lists (a stable counting sort of the
 * T*k pairs p = t*k + j by expert id).
 *
 * Inputs:  topk_ids int32 [T, k], every id in [0, E) and distinct within a
 *          token (ids outside [0, E) are undefined behaviour).
 * Outputs: expert_offsets int32 [E+1]  exclusive prefix sum of the per-expert
 *                                      counts; expert_offsets[E] = T*k;
 *          sorted_pair    int32 [T*k]  pair stored at sorted row i: rows
 *                                      [offsets[e], offsets[e+1]) hold the
 *                                      pairs routed to e, ascending pair index;
 *          pair_to_sorted int32 [T*k]  inverse of sorted_pair.
 * The result is unique and bit-exact (no order depends on scheduling).
 * Workspace: >= moe_workspace_size(T, E, k, ...) bytes (only the permute
 * part is used here), else MOE_ERR_WORKSPACE.
 */
moe_status moe_permute(const int32_t* topk_ids, int T, int E, int k,
                       int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_to_sorted,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_grouped_ffn -- run each expert's SwiGLU FFN over its route list.
 *
 * For every sorted row i in [offsets[e], offsets[e+1]), token t =
 * sorted_pair[i] / k:
 *     g = x[t] . W_gate[e]^T,  u = x[t] . W_up[e]^T        (length I)
 *     a = silu(g) * u,         silu(g) = g / (1 + exp(-g))
 *     y_sorted[i] = a . W_down[e]^T                        (length H)
 * Reading of the pages (the expert's form is not written there): the SwiGLU
 * expert; matrices stored [out, in] with the reduction index contiguous.
 *
 * x          bf16 [T, H]
 * w_gate     MOE_WFMT_BF16: bf16 [E, I, H];   MOE_WFMT_Q3G128: uint32 [E, I, H/128, 13];
 *            MOE_WFMT_BF16_PAIRS: the bf16 [E, I, H] values in the row-pair
 *            layout (moe_pack_bf16_pairs with to_fp16 = 0; same size)
 * w_up       same as w_gate
 * w_down     MOE_WFMT_BF16: bf16 [E, H, I];   MOE_WFMT_Q3G128: uint32 [E, H, I/128, 13];
 *            MOE_WFMT_BF16_PAIRS: the bf16 [E, H, I] values converted to fp16
 *            as the down projection converts them (below), in the row-pair
 *            layout (moe_pack_bf16_pairs with to_fp16 = 1)
 * s_gate, s_up, s_down   fp16 scales [E, I, H/128] / [E, H, I/128] for
 *            MOE_WFMT_Q3G128 (must be NULL for the bf16 formats).  3-bit group
 *            layout: 13 words per 128 weights; field j of a word at bits
 *            [3j, 3j+3), 10 fields in words 0..11, 8 in word 12; weight =
 *            scale * (field - 4).
 * expert_offsets, sorted_pair   as produced by moe_permute.
 * fat_threshold  experts with at least this many rows run as MFMA tiles of
 *            up to 256 rows (the list split evenly into 32-row multiples)
 *            with weight tiles staged in LDS; smaller experts stream their
 *            weights once through a 32-row tile.  Both paths compute the same
 *            function (rounding differs only in summation order).
 *            Must be >= 1.
 * y_sorted   fp16 [T*k, H] output in sorted-row order.
 * Precision: products accumulate in fp32; a is stored as fp16 and the down
 * projection multiplies fp16 a by W_down converted to fp16 (exact for
 * |w| in [2^-14, 65504]; smaller magnitudes lose at most 2^-24 absolute).
 * Shapes: H % 256 == 0 and I % 128 == 0, and each of x (T*H*2 bytes), the
 * activation a (T*k*I*2 bytes) and one expert's bf16 matrix (I*H*2 bytes)
 * below 4 GiB (the kernels address them with 32-bit buffer offsets), else
 * MOE_ERR_UNSUPPORTED.  MOE_WFMT_BF16_PAIRS also needs I % 256 == 0 and
 * T*k < 2^30.  The two bf16 formats give the same results bit for bit.
 * Workspace: >= moe_workspace_size(T, E, k, H, I, wfmt) bytes.
 */
moe_status moe_grouped_ffn(const uint16_t* x, int wfmt,
                           const void* w_gate, const void* w_up, const void* w_down,
                           const uint16_t* s_gate, const uint16_t* s_up, const uint16_t* s_down,
                           const int32_t* expert_offsets, const int32_t* sorted_pair,
                           int T, int E, int k, int H, int I, int fat_threshold,
                           uint16_t* y_sorted, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * The three steps of moe_grouped_ffn, callable one by one (same arguments,
 * same workspace; moe_grouped_ffn == plan + gate_up + down on one stream).
 * They communicate through the workspace: the plan writes the batch lists,
 * gate_up writes the activation a (fp16 [T*k, I]) that down reads.
 *
 * moe_ffn_plan -- cut every non-empty route list into batches that share one
 * read of the expert's weights (wiki file table, segment patch entry): lists
 * of at least fat_threshold rows into MFMA batches of up to 256 rows (equal
 * multiples of 32 rows, the last one ragged), shorter lists
 * into 32-row streaming batches.  Reads expert_offsets only.
 */
moe_status moe_ffn_plan(const int32_t* expert_offsets, int T, int E, int k, int H, int I, int wfmt,
                        int fat_threshold, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_permute_plan -- moe_route_topk, moe_permute and moe_ffn_plan in
 * one call, with the same arguments (H, I, wfmt and fat_threshold as for the
 * plan) and the same results bit for bit.  For T <= 64 tokens (decode
 * batches) the three run in a single launch on one block, with the route
 * lists kept on chip between them; larger batches run the gate, the permute
 * and the plan in order, the plan writing expert_counts from the route lists.
 * Follow it with moe_ffn_gate_up, moe_ffn_down and moe_combine.
 * Errors: those of the three calls (NULL outputs, shapes, workspace size).
 */
moe_status moe_route_permute_plan(const float* logits, int T, int E, int k, int H, int I, int wfmt,
                                  int fat_threshold, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                                  int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_to_sorted,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* moe_ffn_gate_up -- a = silu(x W_gate^T) * (x W_up^T) for every planned batch,
 * stored fp16 in the workspace (row i of a belongs to sorted row i).
 * fat_threshold must equal the value given to moe_ffn_plan; with
 * T < fat_threshold no route list can be fat, so the MFMA-tile kernel is not
 * launched at all.  The MFMA-tile kernel hands out its last batches through
 * a counter in the workspace: moe_ffn_plan zeroes it and each launch leaves
 * it zeroed, so gate_up may run any number of times on one plan, in stream
 * order (two launches on one workspace must not overlap).  The 3-bit format
 * also writes the reordered activation rows of the short lists into the
 * workspace before its streaming kernel. */
moe_status moe_ffn_gate_up(const uint16_t* x, int wfmt, const void* w_gate, const void* w_up,
                           const uint16_t* s_gate, const uint16_t* s_up, const int32_t* sorted_pair,
                           int T, int E, int k, int H, int I, int fat_threshold, void* workspace,
                           size_t workspace_bytes, void* stream);

/* moe_ffn_down -- y_sorted = a W_down^T for every planned batch (same
 * fat_threshold rule as moe_ffn_gate_up). */
moe_status moe_ffn_down(int wfmt, const void* w_down, const uint16_t* s_down, int T, int E, int k, int H, int I,
                        int fat_threshold, uint16_t* y_sorted, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * moe_grouped_ffn_noalloc -- moe_grouped_ffn without a caller workspace and
 * without any allocation, for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, kernels and results as moe_grouped_ffn (bit for bit), minus
 * `workspace` / `workspace_bytes`: the batch lists and the activation a live
 * in one array of MOE_NOALLOC_SCRATCH_BYTES per GPU inside the library (it
 * stays allocated until the process ends).  The FFN part of the workspace,
 * moe_workspace_size(T, E, k, H, I, wfmt) minus the permute part (ceil(T /
 * 256) * E * 4 bytes, rounded up to 256), must fit in it, else
 * MOE_ERR_WORKSPACE and nothing is enqueued: about T * k * I * 2 bytes plus a
 * few KB of lists, so up to 2,048 tokens at k = 8, I = 2048 (the 3-bit format
 * needs T * H * 2 + T * H / 32 bytes more).  Every call writes its lists
 * before reading them, so nothing carries over between calls.
 *
 * Every call on one GPU shares that GPU's array: two calls that overlap on
 * one GPU (on different streams, or from different threads without stream
 * ordering) race and give undefined results.  Calls ordered on one stream are
 * safe.
 */
moe_status moe_grouped_ffn_noalloc(const uint16_t* x, int wfmt, const void* w_gate, const void* w_up,
                                   const void* w_down, const uint16_t* s_gate, const uint16_t* s_up,
                                   const uint16_t* s_down, const int32_t* expert_offsets, const int32_t* sorted_pair,
                                   int T, int E, int k, int H, int I, int fat_threshold, uint16_t* y_sorted,
                                   void* stream);

/*
 * moe_pack_bf16_pairs -- copy bf16 matrices into the row-pair layout of
 * MOE_WFMT_BF16_PAIRS (a storage layout of the same values; the pages fix
 * none for the bf16 experts), optionally converted to fp16.
 *
 * src   bf16 [mats, rows, cols], plain row-major (e.g. W_gate with mats = E,
 *       rows = I, cols = H; W_down with rows = H, cols = I).
 * dst   bf16, same size: element (r, c) of matrix m at
 *       m*rows*cols + ((r/2)*(cols/32) + c/32)*64 + (r%2)*32 + c%32,
 *       i.e. rows 2p and 2p+1 alternate every 32 columns, so that 32 columns
 *       of a row pair fill one 128-byte line.
 * to_fp16  0: dst holds the bf16 values.  1: each value converted to fp16
 *       toward zero (exact for |w| in [2^-14, 65504], smaller magnitudes
 *       truncated, larger ones saturated) -- bit for bit what the down
 *       projection of MOE_WFMT_BF16 computes from bf16 W_down; use it for
 *       w_down of MOE_WFMT_BF16_PAIRS and 0 for w_gate and w_up.
 * rows even and >= 2, cols a multiple of 32, both pointers 16-byte aligned,
 * the two buffers not overlapping (no in-place packing), to_fp16 0 or 1,
 * else MOE_ERR_INVALID_ARG.  One launch on `stream`; done once when weights
 * are loaded, not per layer call.
 */
moe_status moe_pack_bf16_pairs(const uint16_t* src, uint16_t* dst, int64_t mats, int rows, int cols, int to_fp16,
                               void* stream);

/*
 * moe_combine -- out[t, :] = sum_{j=0..k-1} topk_w[t, j] * y_sorted[pair_to_sorted[t*k+j], :]
 *
 * fp32 accumulation in ascending j, no atomics: bit-identical across runs.
 * y_sorted fp16 [T*k, H], topk_w fp32 [T, k], pair_to_sorted int32 [T*k],
 * out fp32 [T, H].  H % 8 == 0 else MOE_ERR_UNSUPPORTED.
 */
moe_status moe_combine(const uint16_t* y_sorted, const float* topk_w, const int32_t* pair_to_sorted,
                       int T, int k, int H, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
