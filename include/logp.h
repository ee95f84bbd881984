/*
 * logp.h - deterministic, batch-invariant selected-token log-probability on MI355X (gfx950).
 *
 * For BF16 logits x[N, V] and targets y[N] the library computes
 *
 *     logp_t  = x[t, y_t] - LSE_t,   LSE_t = logsumexp_v x[t, v]           (forward)
 *     dlogits = g_t * (onehot(y_t) - softmax(x_t))  written as BF16         (backward)
 *
 * with max, sum-exp, exp and log in FP32 (RL-Kernel issue #241 "[WS2] TP-aware
 * deterministic logprob ...", sections Background and Goal; RL-Kernel PR #495
 * "zero-workspace backward for generic CUDA fused logp", section Summary, item 2).
 *
 * Numerical contract (fixed at compile time; changing any of it changes bits):
 *   - The padded row is cut into global tiles of LOGP_TILE_COLS columns starting at
 *     column 0 (PR #314 "[WS2][Logp] Deterministic config option", Tensor Parallel doc,
 *     step 1).  Inside a tile, lane l (0..63) of one wave64 holds columns
 *     tile_start + 512*k + 8*l + e for k, e in 0..7.
 *   - Per tile: m = max over the tile's real columns (-inf if none); s = sum of
 *     exp(x - m) where each lane adds its 64 terms in (k, e) order starting from +0 and
 *     the 64 lane sums are combined by a pairwise tree over lanes 0..63 (xor 1, 2, 4, 8,
 *     16, 32).  A tile with no real column is the (-inf, 0) identity partial (PR #314
 *     commit notes).
 *   - Merge (issue #241, "PR 3"): M = max_l m_l; w_l = 0 if m_l = -inf, else
 *     s_l * exp(m_l - M); lane i adds w_i, w_{i+64}, ... from +0, lanes combine by the
 *     same tree; LSE = M + log S; logp = (sel - M) - log S for a valid row, 0 otherwise
 *     (PR #314 Tensor Parallel doc, steps 4-6).  The selected logit is copied from the
 *     tile that owns the target, never summed (same doc, step 5).
 *   Nothing in this order depends on N, on the row's position in the batch or on how the
 *   vocabulary is sharded, so results are bitwise batch- and shard-invariant.
 *
 * Row validity: a row is valid iff it is active (active == NULL or active[t] != 0), its
 * target differs from ignore_index, and 0 <= target < vocab_real.  Invalid rows produce
 * logp 0 and an all-zero gradient row, silently (PR #495, Behavior changes); callers that
 * want the loud check call logp_check_targets (PR #314 review, target validation).
 * Columns in [vocab_real, vocab_padded) are padding: masked to -inf by index, whatever
 * memory holds, and their gradient is +0 (issue #241, "PR 1"; PR #314 commit notes).
 *
 * Conventions for every entry point:
 *   - BF16 values are passed as raw uint16_t bit patterns.  Every pointer is DEVICE
 *     memory owned by the caller; the library allocates nothing, keeps no mutable global
 *     state, never synchronizes and never prints.  Calls on different streams are
 *     independent.  Outputs must not overlap inputs (the one exception is noted at
 *     logp_backward).
 *   - Device guard (PR #495, author reply, device guard item): the device is taken from
 *     the logits/partials pointer; every other pointer must live on that device, and a
 *     non-null stream must belong to it.  The library makes that device current for the
 *     launch and restores the caller's current device afterwards.
 *   - Arguments are checked on the host before anything is launched; a non-OK status
 *     means nothing was launched.  n == 0 returns LOGP_OK without touching the device
 *     (PR #495, Tests: "empty input").
 *   - Column indices must satisfy vocab_padded + LOGP_TILE_COLS < 2^31 so that all
 *     in-row arithmetic fits 32 bits; row offsets are 64-bit (PR #495, security review,
 *     and author reply on the INT_MAX loop overflow).
 */
#ifndef LOGP_MI355X_LOGP_H
#define LOGP_MI355X_LOGP_H

#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define LOGP_API __attribute__((visibility("default")))
#else
#define LOGP_API
#endif

/* Width of a global vocabulary tile (a numerical-contract constant). */
#define LOGP_TILE_COLS 4096
/* Largest tile count the fused forward accepts (its per-tile partials stay on chip). */
#define LOGP_FWD_MAX_TILES 4096

/* Per-row statistics of the forward: M = row max, S = sum exp(x - M) (FP32). */
typedef struct {
    float max;
    float sumexp;
} logp_stats_t;

/* Per-row, per-global-tile partial: (m_l, s_l) and the selected logit when the tile owns a
 * valid target (0 otherwise).  Issue #241, "PR6": (max, sumexp, selected_logit) in FP32. */
typedef struct {
    float max;
    float sumexp;
    float sel;
} logp_partial_t;

typedef enum {
    LOGP_OK = 0,
    LOGP_ERR_NULL = 1,    /* a required pointer is NULL */
    LOGP_ERR_SHAPE = 2,   /* sizes, strides or column bounds out of range */
    LOGP_ERR_SHARD = 3,   /* a column range is not tile-aligned or lies outside the row */
    LOGP_ERR_DEVICE = 4,  /* a pointer is not device memory of the logits' device, or the
                             stream belongs to another device */
    LOGP_ERR_RANGE = 5,   /* an array's extent runs past the end of its allocation */
    LOGP_ERR_OVERLAP = 6, /* an output overlaps an input or another output */
    LOGP_ERR_HIP = 7,     /* the HIP runtime reported an error (query or launch) */
    LOGP_ERR_ARG = 8,     /* unknown dtype, or inv_temperature not finite and positive */
    LOGP_ERR_SCRATCH = 9  /* an entry point without a workspace argument needs more staging
                             memory than its static scratch array holds */
} logp_status_t;

/* Element type of logits and dlogits for the _ex entry points (PR #495, Tests: the fused
 * kernel is checked for FP32, BF16 and FP16 logits).  Values are widened exactly to FP32;
 * dlogits is rounded to nearest-even in the same type. */
typedef enum {
    LOGP_DTYPE_BF16 = 0,
    LOGP_DTYPE_F16 = 1,
    LOGP_DTYPE_F32 = 2
} logp_dtype_t;

/* Forward over whole rows (issue #241 Background; PR #495 Summary).
 *   logits        [n, ld] BF16 bits, row t at logits + t*ld; columns [0, vocab_real) read.
 *   vocab_real    number of real columns, >= 1.
 *   vocab_padded  padded width, vocab_real <= vocab_padded <= ld; the padding is ignored.
 *                 ceil(vocab_padded / LOGP_TILE_COLS) must not exceed LOGP_FWD_MAX_TILES
 *                 (larger vocabularies go through logp_partials + logp_merge).
 *   targets       [n] int64;  active: [n] uint8 or NULL (all rows active).
 *   logp          [n] FP32 output (required).  lse: [n] FP32 or NULL.  stats: [n] or NULL;
 *                 stats is the only state logp_backward needs.
 * Results are bitwise equal to logp_partials over any tile-aligned shard split followed by
 * logp_merge.  A row whose real logits are all -inf has LSE -inf, stats (-inf, 0) and
 * logp -inf when valid (0 otherwise). */
LOGP_API logp_status_t logp_forward(const uint16_t* logits, int64_t ld, int64_t n,
                                    int64_t vocab_real, int64_t vocab_padded,
                                    const int64_t* targets, const uint8_t* active,
                                    int64_t ignore_index, float* logp, float* lse,
                                    logp_stats_t* stats, hipStream_t stream);

/* Backward (PR #495, Summary item 2: dlogits = g (onehot - softmax) written directly in the
 * logits dtype, no FP32 [N, V] workspace).
 *   logits     points at column col_begin of row 0; row t at logits + t*ld.
 *   col_begin, col_end  the global column range this call covers, 0 <= col_begin <= col_end
 *              <= vocab_padded (0, vocab_padded = whole rows; any sub-range is allowed,
 *              e.g. one vocab shard's slice).
 *   grad_logp  [n] FP32 upstream dL/dlogp (ignored for invalid rows).
 *   stats      [n] from logp_forward or logp_merge for the same rows.
 *   dlogits    [n, ld_out] BF16 bits, pointing at column col_begin; columns
 *              [0, col_end - col_begin) of every row are written: round-to-nearest-even of
 *              g*(onehot - exp(x - M)/S) for real columns of a valid row, +0 elsewhere.
 *              An invalid row (or one whose stats are (-inf, 0)) is written as zeros and
 *              its logits are not read.  dlogits may be exactly the logits buffer (same
 *              pointer and ld_out == ld): each element is read before it is overwritten.
 */
LOGP_API logp_status_t logp_backward(const uint16_t* logits, int64_t ld, int64_t n,
                                     int64_t vocab_real, int64_t vocab_padded, int64_t col_begin,
                                     int64_t col_end, const int64_t* targets,
                                     const uint8_t* active, int64_t ignore_index,
                                     const float* grad_logp, const logp_stats_t* stats,
                                     uint16_t* dlogits, int64_t ld_out, hipStream_t stream);

/* Vocab-tile partials of one shard (issue #241, "PR6": rank-local (max, sumexp,
 * selected_logit) partials; PR #314 Tensor Parallel doc, steps 1-2).
 *   logits     points at column col_begin of row 0 (the shard's local [n, ld] view).
 *   col_begin  multiple of LOGP_TILE_COLS; col_end a multiple of it or equal to
 *              vocab_padded; col_begin < col_end <= vocab_padded.  Otherwise LOGP_ERR_SHARD
 *              (fail loudly on undeclared or uneven shard bounds, issue #241 "PR 1"/"PR6").
 *   partials   points at the entry of global tile col_begin / LOGP_TILE_COLS of row 0;
 *              row t's entries start at partials + t*ldp.  Entries j in
 *              [0, ceil((col_end - col_begin) / LOGP_TILE_COLS)) are written.
 * A shard made only of padding yields (-inf, 0, 0) identity entries. */
LOGP_API logp_status_t logp_partials(const uint16_t* logits, int64_t ld, int64_t n,
                                     int64_t vocab_real, int64_t vocab_padded, int64_t col_begin,
                                     int64_t col_end, const int64_t* targets,
                                     const uint8_t* active, int64_t ignore_index,
                                     logp_partial_t* partials, int64_t ldp, hipStream_t stream);

/* Fixed-order merge of per-tile partials (issue #241, "PR 3"; PR #314 Tensor Parallel
 * doc, steps 4-6).
 *   partials   [n, ldp]; entries [0, num_tiles) of each row are merged in tile order.
 *              num_tiles >= ceil(vocab_real / LOGP_TILE_COLS); extra tiles must be
 *              identity partials or real tiles of the padded row.
 *   logp       [n] FP32 (required); lse [n] FP32 or NULL; stats [n] or NULL.
 * Uses the same device code as the merge inside logp_forward, so the outputs are bitwise
 * equal to logp_forward's for the same logits. */
LOGP_API logp_status_t logp_merge(const logp_partial_t* partials, int64_t ldp, int64_t n,
                                  int64_t num_tiles, int64_t vocab_real, const int64_t* targets,
                                  const uint8_t* active, int64_t ignore_index, float* logp,
                                  float* lse, logp_stats_t* stats, hipStream_t stream);

/* Extended forms: any logits dtype and temperature-scaled scoring.
 *   dtype            element type of logits (and of dlogits in logp_backward_ex): a
 *                    logp_dtype_t value, passed as int32_t (other values: LOGP_ERR_ARG).
 *   inv_temperature  1/tau, finite and > 0.  The scored logits are z = fl32(x * inv_temperature),
 *                    one FP32 product per logit, so training and rollout code that use the same
 *                    inv_temperature see the same z (temperatures 1.0 and 0.7 in the provider
 *                    experiment of PR #495's author reply).  logp, LSE, stats and partials are
 *                    those of z; dlogits = inv_temperature * g * (onehot - softmax(z)), with
 *                    g * inv_temperature rounded once to FP32 per row.  With
 *                    inv_temperature = 1 the results are bitwise those of the plain entry points.
 * Every other argument is as in logp_forward / logp_backward / logp_partials; pointers to logits
 * and dlogits are `void*` of the given dtype, and ld / ld_out count elements.  A view takes the
 * 16-byte vector path when its start is 16-byte aligned and ld * element size is a multiple of
 * 16; the results do not depend on which path runs. */
LOGP_API logp_status_t logp_forward_ex(int32_t dtype, float inv_temperature,
                                       const void* logits, int64_t ld, int64_t n,
                                       int64_t vocab_real, int64_t vocab_padded,
                                       const int64_t* targets, const uint8_t* active,
                                       int64_t ignore_index, float* logp, float* lse,
                                       logp_stats_t* stats, hipStream_t stream);
LOGP_API logp_status_t logp_backward_ex(int32_t dtype, float inv_temperature,
                                        const void* logits, int64_t ld, int64_t n,
                                        int64_t vocab_real, int64_t vocab_padded,
                                        int64_t col_begin, int64_t col_end,
                                        const int64_t* targets, const uint8_t* active,
                                        int64_t ignore_index, const float* grad_logp,
                                        const logp_stats_t* stats, void* dlogits, int64_t ld_out,
                                        hipStream_t stream);
LOGP_API logp_status_t logp_partials_ex(int32_t dtype, float inv_temperature,
                                        const void* logits, int64_t ld, int64_t n,
                                        int64_t vocab_real, int64_t vocab_padded,
                                        int64_t col_begin, int64_t col_end,
                                        const int64_t* targets, const uint8_t* active,
                                        int64_t ignore_index, logp_partial_t* partials,
                                        int64_t ldp, hipStream_t stream);

/* ceil(vocab_padded / LOGP_TILE_COLS); 0 when vocab_padded < 1. */
LOGP_API int64_t logp_num_tiles(int64_t vocab_padded);

/* Loud target validation (PR #314 review: active targets must lie in the real vocab when
 * validation is on).  Writes to *bad_count (one device int64) the number of active rows
 * whose target is neither ignore_index nor in [0, vocab_real).  Unlike the other entry
 * points it also launches for n == 0 (writing 0).  Asynchronous: the caller synchronizes
 * the stream before reading the count. */
LOGP_API logp_status_t logp_check_targets(const int64_t* targets, const uint8_t* active,
                                          int64_t n, int64_t vocab_real, int64_t ignore_index,
                                          int64_t* bad_count, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
LOGP_API const char* logp_status_string(int32_t status);  /* a logp_status_t value */

#ifdef __cplusplus
}
#endif

#endif /* LOGP_MI355X_LOGP_H */
