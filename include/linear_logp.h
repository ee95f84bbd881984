/* Fused LM-head + selected-token log-probability (linear_logp), for MI355X (gfx950).
 *
 * Source: PR #495 "zero-workspace backward for generic CUDA fused logp" lists linear_logp,
 * the fused LM-head plus logp op, beside the generic fused logp (Summary); issue #241 "[WS2]
 * TP-aware deterministic logprob …" fixes what the logp path computes and how vocab-parallel
 * partials merge (sections PR 3 and PR6).  The pages give linear_logp no more than its name;
 * the reading here: the logits z = h W^T of BF16 hidden states h [n, H] and the BF16 LM-head
 * weight W [V, H] (one row per vocabulary entry) are formed tile by tile on the matrix cores
 * with FP32 accumulation and reduced at once to the per-tile partials of logp.h, so the
 * [n, V] logits never exist in memory.  logp_merge over those partials then gives logp, LSE
 * and (M, S) exactly as for materialised logits, and a vocab-parallel rank that holds the
 * rows [col_begin, col_end) of W produces its slice of the same partials.
 *
 * Numerical contract (deterministic, independent of n, of a row's position in the batch and
 * of the shard split):
 *   z[t, v]  = sum over k of h[t, k] W[v, k]: products exact, added in FP32 by a fixed
 *              sequence of v_mfma_f32_32x32x16_bf16 steps, k = 0, 16, 32, ... (hidden sizes
 *              that are not a multiple of 32 are padded with zeros);
 *   each 4096-column global tile is reduced in 16 sub-blocks of 256 columns; a sub-block
 *   gives (m_b, s_b) with m_b its max and s_b = sum exp(z - m_b): 4 partial sums over the
 *   sub-block's columns 4p + 16q + e (p = 0..3; q = 0..15 then e = 0..3, in that order, from
 *   +0) combined by a pairwise tree (p xor 1, 2); the tile's (m_l, s_l) folds the sub-blocks
 *   in order, b = 0 .. 15:
 *   m <- max(m, m_b), s <- s exp(m_old - m) + s_b exp(m_b - m) (terms of -inf maxima are 0);
 *   sel_l = z[t, y_t] in the owner tile of a valid row, 0 elsewhere.  exp is the logp
 *   forward's (2^(t log2 e) on the hardware exp2).
 *
 * All pointers are device memory on one device, owned by the caller; arguments are checked
 * on the host before any launch (codes of logp.h).  Nothing is allocated; nothing
 * synchronizes. */
#ifndef LINEAR_LOGP_H
#define LINEAR_LOGP_H

#include <stdint.h>

#include "logp.h"

#ifdef __cplusplus
extern "C" {
#endif

#define LINEAR_LOGP_MAX_HIDDEN 65536  /* largest hidden size H */
#define LINEAR_LOGP_MAX_LD 262144      /* largest row stride of hidden and weight (elements) */
#define LINEAR_LOGP_BWD_MAX_ROWS 8388608    /* largest n of the backward (2^23) */
#define LINEAR_LOGP_BWD_MAX_CHUNK 1048576   /* largest chunk_cols of the backward (2^20) */
#define LINEAR_LOGP_MAX_SAVED_LD 2147483648ll  /* largest row stride of kept logits (2^31) */

/* Per-tile partials of the logits h W^T over the vocabulary columns [col_begin, col_end).
 *   hidden        [n, ld_h] BF16 bits; row t at hidden + t*ld_h; H = hidden_size columns used.
 *   weight        BF16 bits pointing at row col_begin of W: row v of the view at
 *                 weight + (v - col_begin)*ld_w, H columns used.  Rows at or beyond vocab_real
 *                 are never read (they count as -inf logits, like padding columns); for a
 *                 view with no real row (all padding) weight may be NULL.
 *   hidden_size   H, 1 <= H <= LINEAR_LOGP_MAX_HIDDEN, a multiple of 8.
 *   ld_h, ld_w    row strides in elements, >= H, multiples of 8 and at most
 *                 LINEAR_LOGP_MAX_LD; hidden and weight must be 16-byte aligned (else
 *                 LOGP_ERR_SHAPE).
 *   vocab_real, vocab_padded, col_begin, col_end, targets, active, ignore_index, partials,
 *   ldp           exactly as in logp_partials: col_begin a multiple of LOGP_TILE_COLS, col_end
 *                 one too or vocab_padded; partials points at the slot of tile
 *                 col_begin / LOGP_TILE_COLS of row 0 of an [n, ldp] array.
 * logp_merge over all tiles completes the forward (logp, LSE, stats for logp_backward_ex on
 * the same logits). */
LOGP_API logp_status_t linear_logp_partials(const uint16_t* hidden, int64_t ld_h, int64_t n,
                                            int64_t hidden_size, const uint16_t* weight,
                                            int64_t ld_w, int64_t vocab_real,
                                            int64_t vocab_padded, int64_t col_begin,
                                            int64_t col_end, const int64_t* targets,
                                            const uint8_t* active, int64_t ignore_index,
                                            logp_partial_t* partials, int64_t ldp,
                                            hipStream_t stream);

/* linear_logp_partials with temperature-scaled scoring (PR #314 "[WS2][Logp] Deterministic
 * config option", Numerical contract: rollout and trainer score the same logits at
 * temperatures such as 1.0 and 0.7).  Each logit of the FP32 accumulation above is scored
 * once, z = fl32(acc * inv_temperature), before any reduction; m_l, s_l and sel_l are those of
 * the scored logits.  inv_temperature = 1/tau must be finite and > 0 (else LOGP_ERR_ARG).
 * With inv_temperature = 1 the partials are bitwise those of linear_logp_partials, which calls
 * this.  logp_merge then gives logp, LSE and (M, S) of the scored logits; logp_backward_ex
 * with the same inv_temperature on materialised logits h W^T takes those stats. */
LOGP_API logp_status_t linear_logp_partials_ex(float inv_temperature, const uint16_t* hidden,
                                               int64_t ld_h, int64_t n, int64_t hidden_size,
                                               const uint16_t* weight, int64_t ld_w,
                                               int64_t vocab_real, int64_t vocab_padded,
                                               int64_t col_begin, int64_t col_end,
                                               const int64_t* targets, const uint8_t* active,
                                               int64_t ignore_index, logp_partial_t* partials,
                                               int64_t ldp, hipStream_t stream);

/* linear_logp_partials_ex with a caller workspace that lets the launch balance its last rounds
 * (same source passages as linear_logp_partials).  One workgroup per (256-row block, tile)
 * leaves a launch whose workgroup count is not a multiple of the device's compute-unit count
 * with a final round that still lasts a whole tile; with the workspace, the call runs the
 * whole rounds that way and spreads the 256-column sub-blocks of the remaining tiles over
 * every compute unit, each writing its rows' (m_b, s_b) and target logit to the workspace, then
 * folds each tile's sub-blocks in the contract's order b = 0, 1, ... (sub-blocks with no real
 * column leave the fold unchanged bit for bit and are skipped).  The partials are bitwise those
 * of linear_logp_partials_ex at every shape; the call decides from the device's compute-unit
 * count whether the split shortens the schedule and otherwise launches as
 * linear_logp_partials_ex does.
 *   workspace        device memory, 256-byte aligned, owned by the caller, contents irrelevant
 *                    on entry, not overlapping any other argument (LOGP_ERR_OVERLAP); NULL or
 *                    fewer bytes than the split needs means no split.
 *   workspace_bytes  its size; linear_logp_partials_workspace(n, vocab_real, col_begin,
 *                    col_end) bytes always suffice (3072 bytes per 256-row block and
 *                    256-column sub-block of the view's real columns).
 * Every other argument and error as in linear_logp_partials_ex; a misaligned workspace or
 * negative workspace_bytes is LOGP_ERR_SHAPE. */
LOGP_API int64_t linear_logp_partials_workspace(int64_t n, int64_t vocab_real, int64_t col_begin,
                                                int64_t col_end);  /* -1 when out of range */
LOGP_API logp_status_t linear_logp_partials_ws(float inv_temperature, const uint16_t* hidden,
                                               int64_t ld_h, int64_t n, int64_t hidden_size,
                                               const uint16_t* weight, int64_t ld_w,
                                               int64_t vocab_real, int64_t vocab_padded,
                                               int64_t col_begin, int64_t col_end,
                                               const int64_t* targets, const uint8_t* active,
                                               int64_t ignore_index, logp_partial_t* partials,
                                               int64_t ldp, void* workspace,
                                               int64_t workspace_bytes, hipStream_t stream);

/* linear_logp_partials_ws (same source passages as linear_logp_partials: PR #495's Summary
 * names the fused LM-head logp) that also keeps the scored logits it forms, so that
 * linear_logp_backward_saved can read them instead of forming h W^T again: memory for time
 * (4 bytes per logit, 5.0 GB for 8192 rows of a 151936-column vocabulary).  The same kernels
 * run, each also writing the scored logits as the forward's reduction reads them, so the
 * partials are bitwise those of linear_logp_partials_ws.
 *   logits       [n, ld_logits] FP32, device memory owned by the caller, 16-byte aligned:
 *                column c of row t receives z = fl32(acc * inv_temperature) of view column c
 *                for c < vocab_real - col_begin (the view's real columns); no other element
 *                is written.
 *   ld_logits    row stride in elements: >= col_end - col_begin, a multiple of 4, at most
 *                LINEAR_LOGP_MAX_SAVED_LD, and n * ld_logits <= 2^40 (else LOGP_ERR_SHAPE).
 *   workspace    as in linear_logp_partials_ws; NULL gives the one-kernel launch.
 * logits must not overlap any other argument (LOGP_ERR_OVERLAP); NULL logits is
 * LOGP_ERR_NULL.  Every other argument and error as in linear_logp_partials_ws. */
LOGP_API logp_status_t linear_logp_partials_save(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, logp_partial_t* partials, int64_t ldp, float* logits,
    int64_t ld_logits, void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* Backward of linear_logp: the gradients of sum over valid rows t of g_t logp_t (logp of the
 * scored logits z = fl32(acc(h W^T) * inv_temperature) of linear_logp_partials_ex) with respect
 * to h and to the shard's rows of W.  The derivative through logp is the logp path's backward
 * (PR #495 "zero-workspace backward for generic CUDA fused logp", Summary: dlogits =
 * g (onehot - softmax), rounded straight to BF16), times inv_temperature through the scoring
 * multiply (PR #314's temperature):
 *   dz[t, v] = RNE_bf16( g' (1[v == y_t] - exp(z[t, v] - M_t) / S_t) ),  g' = fl32(g_t inv_t),
 *     with z recomputed bit for bit as the forward formed it, (M, S) the forward's stats
 *     (logp_merge), and dz = 0 for rows that are not valid, for M_t = -inf and for padding
 *     columns (v >= vocab_real);
 *   dhidden[t, :] = sum over this shard's columns v of dz[t, v] W[v, :]   (FP32, overwritten);
 *   dweight[v - col_begin, :] = sum over rows t of dz[t, v] h[t, :]      (FP32, overwritten;
 *     rows of padding columns are 0).
 * Both sums run on the matrix cores with FP32 accumulation in a fixed order: dhidden's
 * accumulator runs through the chunks of chunk_cols columns in column order, each chunk's
 * products added onto it in column order, so a row's dhidden does not depend on the other rows
 * of the batch; dweight sums the rows in index order.  Vocab-parallel ranks each produce their shard's dhidden; the caller adds them
 * in a fixed rank order.  Run to run the results are bitwise identical.
 *   hidden, weight, targets, active, ignore_index, vocab_real, vocab_padded, col_begin,
 *   col_end, inv_temperature   as in linear_logp_partials_ex (weight points at row col_begin).
 *   grad_logp     [n] FP32 upstream gradient of logp.   stats  [n] (M, S) of the forward.
 *   dhidden       [n, ld_dh] FP32, ld_dh >= H.   dweight  [col_end - col_begin, ld_dw] FP32.
 *   workspace     device memory of at least linear_logp_backward_workspace(n, H, chunk_cols)
 *                 bytes, 256-byte aligned, owned by the caller, contents irrelevant on entry.
 *   chunk_cols    vocabulary columns per pass (a multiple of LOGP_TILE_COLS, at most
 *                 LINEAR_LOGP_BWD_MAX_CHUNK); larger chunks take more workspace, not more
 *                 time per column.
 * n <= LINEAR_LOGP_BWD_MAX_ROWS.  col_end == col_begin writes dhidden = 0.  Errors as for
 * linear_logp_partials_ex; outputs and the workspace must not overlap any input or each
 * other (LOGP_ERR_OVERLAP); a short or misaligned workspace is LOGP_ERR_SHAPE. */
LOGP_API int64_t linear_logp_backward_workspace(int64_t n, int64_t hidden_size,
                                                int64_t chunk_cols);  /* -1 when out of range */
LOGP_API logp_status_t linear_logp_backward_ex(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, const float* grad_logp, const logp_stats_t* stats, float* dhidden,
    int64_t ld_dh, float* dweight, int64_t ld_dw, void* workspace, int64_t workspace_bytes,
    int64_t chunk_cols, hipStream_t stream);
/* linear_logp_backward_ex for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Every argument is as in
 * linear_logp_backward_ex; there is no workspace argument.  The staging memory is a static
 * device array of LINEAR_LOGP_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU
 * it runs on, from the first call on that GPU until the process ends; a call whose
 * linear_logp_backward_workspace(n, hidden_size, chunk_cols) exceeds it returns
 * LOGP_ERR_SCRATCH without launching (e.g. n = 4096, H = 4096 fits with chunk_cols = 4096).
 * The call allocates nothing and clears nothing: every staging byte a kernel reads was written
 * earlier in the same call.  All calls on one GPU share that GPU's array, so calls that overlap
 * on one GPU (on different streams, or from several host threads without ordering) race; a
 * caller serialises them, e.g. by issuing them on one stream.  Results are bitwise those of
 * linear_logp_backward_ex with the same chunk_cols. */
#define LINEAR_LOGP_NOALLOC_SCRATCH_BYTES (128ll << 20)
LOGP_API logp_status_t linear_logp_backward_noalloc(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, const float* grad_logp, const logp_stats_t* stats, float* dhidden,
    int64_t ld_dh, float* dweight, int64_t ld_dw, int64_t chunk_cols, hipStream_t stream);
/* linear_logp_backward_ex with the gradients written in BF16, the dtype of hidden and W (PR #495
 * "zero-workspace backward for generic CUDA fused logp", Summary: the gradient is written in
 * the inputs' dtype).  Every argument is as in linear_logp_backward_ex except:
 *   dhidden       [n, ld_dh] BF16 bits: RNE_bf16 of the FP32 dhidden linear_logp_backward_ex
 *                 forms (its sum over the chunks is kept in FP32 in the workspace and rounded
 *                 once, so the bits are those of rounding that entry point's output to nearest
 *                 even);
 *   dweight       [col_end - col_begin, ld_dw] BF16 bits: RNE_bf16 of its FP32 dweight;
 *   workspace     at least linear_logp_backward_bf16_workspace(n, H, chunk_cols) bytes: the
 *                 FP32 entry point's workspace followed by the FP32 dhidden accumulator
 *                 (4 x n x H bytes, each padded to a multiple of 256).
 * A vocab-parallel caller that adds the ranks' dhidden should add FP32 partials (the FP32 entry
 * point) and round the total: rounding each rank's dhidden first is a different result. */
LOGP_API int64_t linear_logp_backward_bf16_workspace(int64_t n, int64_t hidden_size,
                                                     int64_t chunk_cols); /* -1 out of range */
LOGP_API logp_status_t linear_logp_backward_bf16(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, const float* grad_logp, const logp_stats_t* stats, uint16_t* dhidden,
    int64_t ld_dh, uint16_t* dweight, int64_t ld_dw, void* workspace, int64_t workspace_bytes,
    int64_t chunk_cols, hipStream_t stream);
/* The backward of linear_logp_backward_ex (out_dtype LOGP_DTYPE_F32) or of
 * linear_logp_backward_bf16 (LOGP_DTYPE_BF16) -- the same derivative, from the same passages
 * (PR #495 "zero-workspace backward for generic CUDA fused logp", Summary) -- from the scored
 * logits that
 * linear_logp_partials_save kept: dz reads z instead of forming it on the matrix cores again,
 * so the call runs two of the three products (dh = dz W, dW = dz^T h).  Given the logits the
 * forward kept for the same hidden, weight, inv_temperature and view, the outputs are bitwise
 * those of the entry point it stands for, since z is the same value either way.
 *   logits      [n, ld_logits] FP32, 4-byte aligned: column c of row t holds z of view column
 *               c (the view's real columns are read); ld_logits >= col_end - col_begin, at
 *               most LINEAR_LOGP_MAX_SAVED_LD, n * ld_logits <= 2^40 (else LOGP_ERR_SHAPE).
 *   dhidden, dweight   FP32 (out_dtype LOGP_DTYPE_F32) or BF16 bits (LOGP_DTYPE_BF16), with
 *               the strides and meaning of the entry point it stands for; any other out_dtype
 *               is LOGP_ERR_ARG.
 *   workspace   at least linear_logp_backward_workspace (FP32) or
 *               linear_logp_backward_bf16_workspace (BF16) bytes for the same n, H and
 *               chunk_cols.
 * hidden and weight are still read.  NULL logits is LOGP_ERR_NULL; every other argument and
 * error as in linear_logp_backward_ex. */
LOGP_API logp_status_t linear_logp_backward_saved(
    float inv_temperature, const float* logits, int64_t ld_logits, const uint16_t* hidden,
    int64_t ld_h, int64_t n, int64_t hidden_size, const uint16_t* weight, int64_t ld_w,
    int64_t vocab_real, int64_t vocab_padded, int64_t col_begin, int64_t col_end,
    const int64_t* targets, const uint8_t* active, int64_t ignore_index,
    const float* grad_logp, const logp_stats_t* stats, void* dhidden, int64_t ld_dh,
    void* dweight, int64_t ld_dw, int32_t out_dtype, void* workspace, int64_t workspace_bytes,
    int64_t chunk_cols, hipStream_t stream);
/* linear_logp_backward_ex at inv_temperature = 1. */
LOGP_API logp_status_t linear_logp_backward(
    const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, const float* grad_logp, const logp_stats_t* stats, float* dhidden,
    int64_t ld_dh, float* dweight, int64_t ld_dw, void* workspace, int64_t workspace_bytes,
    int64_t chunk_cols, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LINEAR_LOGP_H */
