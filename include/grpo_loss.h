/* Deterministic GRPO loss on selected-token log-probabilities, for MI355X (gfx950).
 *
 * Source: RL-Kernel issue #241 "[WS2] TP-aware deterministic logprob for cross-config
 * alignment", planned PR5 "Deterministic GRPO loss on the TP-aware logprob path": the GRPO
 * objective (ratio, clip, KL, advantage normalization) bound to a declared reduction so that
 * the loss and its gradient are reproducible; normalizers token_mean / seq_mean /
 * seq_sum_token_mean; n_non_ignore global or local; a fixed summation order from tokens to
 * sequences to context-parallel and data-parallel ranks, merged in fixed order rather than
 * by a collective sum; acceptance by the KL=0 identity.
 *
 * Per active token t of sequence i (all float32; the library's reading of the terms the
 * issue names):
 *   r      = exp(logp - old_logp)                      (ratio)
 *   lo, hi = fl32(1 - eps_low), fl32(1 + eps_high)      (clip bounds)
 *   clipped = (A_i > 0 and r > hi) or (A_i < 0 and r < lo)
 *   pg     = -A_i * (clipped ? (A_i > 0 ? hi : lo) : r)  = max(-A r, -A clip(r, lo, hi))
 *   kl     = exp(d) - d - 1, d = ref - logp: for |d| < 1 as d^2 times the Taylor series
 *            of (e^d - 1 - d) / d^2 through d^11 / 13! (no cancellation), else expm1(d) - d
 *   d pg / d logp = clipped ? 0 : -A_i r ;  d kl / d logp = -expm1(ref - logp)
 * Inactive tokens (mask == 0) and A_i == 0 tokens add nothing to pg; inactive tokens get a
 * zero gradient.  Reductions:
 *   token_mean          pg_loss = sum_t pg / D, D = norm_tokens if > 0 else the active-token
 *                       count; d loss / d logp_t = dl_t * fl32(1 / D)
 *   seq_mean            pg_loss = sum_i (P_i / n_i) / D over sequences with n_i > 0,
 *                       D = norm_seqs if > 0 else the number of non-empty sequences;
 *                       d loss / d logp_t = dl_t * fl32(1 / (n_i D))
 *   seq_sum_token_mean  pg_loss = sum_i P_i / n_i ; d loss / d logp_t = dl_t * fl32(1 / n_i)
 * with P_i = sum of pg over sequence i, n_i its active-token count, dl = d pg + beta d kl,
 * the same for kl_loss, and loss = pg_loss + beta kl_loss.
 *
 * Fixed summation order (this is what makes results bitwise reproducible and layout
 * invariant): a sequence's tokens form tiles of GRPO_TOKEN_TILE from token 0; inside a
 * tile, lane l (0..63) adds tokens l, l+64, l+128, l+192 in that order from +0, then lanes
 * combine by the pairwise tree over lane index (xor 1, 2, ..., 32); a sequence's tiles and
 * a batch's sequences are merged the same way (lane l adds items l, l+64, ... in order,
 * then the tree).  Splitting a sequence at tile boundaries (context parallelism) or a
 * batch into groups of whole sequences (data parallelism) therefore changes no bit, given
 * the same normalizers.
 *
 * All pointers are device memory on one device, owned by the caller; every entry point
 * validates its arguments on the host and returns a logp_status_t without launching when
 * one is invalid (LOGP_ERR_NULL, LOGP_ERR_SHAPE, LOGP_ERR_DEVICE, LOGP_ERR_RANGE,
 * LOGP_ERR_OVERLAP, LOGP_ERR_ARG as in logp.h).  Work is queued on `stream`; nothing is
 * allocated and nothing synchronizes.  With n_seqs == 0 (or n == 0) the per-sequence and
 * per-token pointers may be NULL; grpo_loss and grpo_loss_reduce still write the empty
 * reduction (all zeros) to `loss`, the other calls return LOGP_OK without launching.
 */
#ifndef GRPO_LOSS_H
#define GRPO_LOSS_H

#include <stdint.h>

#include "logp.h"

#ifdef __cplusplus
extern "C" {
#endif

#define GRPO_TOKEN_TILE 256  /* tokens per tile of the fixed summation order */
#define GRPO_MAX_SEQ_LEN (GRPO_TOKEN_TILE * 4096)  /* longest sequence (tile slots in LDS) */

typedef enum {
    GRPO_TOKEN_MEAN = 0,
    GRPO_SEQ_MEAN = 1,
    GRPO_SEQ_SUM_TOKEN_MEAN = 2
} grpo_mode_t;

/* Objective and reduction contract (host memory, read during the call). */
typedef struct {
    float eps_low;        /* lower clip width, finite, 0 <= eps_low <= 1            */
    float eps_high;       /* upper clip width, finite, >= 0                          */
    float beta;           /* KL weight, finite, >= 0; no KL when ref_logp is NULL    */
    int32_t mode;         /* grpo_mode_t                                              */
    int64_t norm_tokens;  /* token_mean: global n_non_ignore if > 0, else local count */
    int64_t norm_seqs;    /* seq_mean: global sequence count if > 0, else local count */
} grpo_params_t;

/* Sums over one token tile, or over one whole sequence. */
typedef struct {
    float pg_sum;     /* sum of pg over active tokens   */
    float kl_sum;     /* sum of kl over active tokens   */
    int32_t clipped;  /* active tokens on the clipped branch */
    int32_t tokens;   /* active tokens                  */
} grpo_partial_t;

/* Reduced loss (device memory, written by the library). */
typedef struct {
    float loss;       /* pg_loss + beta * kl_loss                          */
    float pg_loss;
    float kl_loss;
    float clip_frac;  /* clipped / tokens (0 when there are no tokens)     */
    int64_t tokens;   /* active tokens of the batch                        */
    int64_t sequences;/* sequences with at least one active token          */
    int64_t clipped;  /* active tokens on the clipped branch               */
    int64_t norm;     /* the normalizer D that was used (1 for seq_sum_token_mean) */
} grpo_loss_t;

/* Group advantage normalization (issue #241 PR5, "advantage normalization"): for each group
 * of `group_size` consecutive rewards, A = (r - mean) / (std + eps) with the unbiased std
 * (scale_by_std != 0), or A = r - mean (scale_by_std == 0); a group of one gives 0.  Sums
 * follow the fixed lane order above.  rewards, adv: float32 [n], n a multiple of group_size
 * (else LOGP_ERR_SHAPE); adv may alias rewards exactly. */
LOGP_API logp_status_t grpo_advantages(const float* rewards, int64_t n, int64_t group_size,
                                       float eps, int32_t scale_by_std, float* adv,
                                       hipStream_t stream);

/* Active tokens per sequence in token range [t_begin, t_end): counts[i] = number of nonzero
 * mask[i, t] (t_end - t_begin when mask is NULL).  mask: uint8 [n_seqs, ld] (the full
 * rows; only the range is read); counts: int32 [n_seqs].  Counts of the ranges of a
 * context-parallel split add up to the whole-sequence counts. */
LOGP_API logp_status_t grpo_token_counts(const uint8_t* mask, int64_t n_seqs, int64_t seq_len,
                                         int64_t ld, int64_t t_begin, int64_t t_end,
                                         int32_t* counts, hipStream_t stream);

/* The loss over whole sequences, in one call.
 *   logp, old_logp        float32 [n_seqs, ld], row i = sequence i, tokens 0..seq_len-1
 *   ref_logp              float32 [n_seqs, ld] or NULL (no KL term)
 *   adv                   float32 [n_seqs], one advantage per sequence
 *   mask                  uint8 [n_seqs, ld] or NULL (every token active)
 *   seq_stats             out: grpo_partial_t [n_seqs], each sequence's sums
 *   loss                  out: one grpo_loss_t
 *   dlogp                 out: float32 [n_seqs, ld], d loss / d logp (columns >= seq_len are
 *                         not written), or NULL
 * seq_len <= GRPO_MAX_SEQ_LEN, ld >= seq_len.  Outputs may not overlap inputs. */
LOGP_API logp_status_t grpo_loss(const float* logp, const float* old_logp,
                                 const float* ref_logp, const float* adv, const uint8_t* mask,
                                 int64_t n_seqs, int64_t seq_len, int64_t ld,
                                 const grpo_params_t* params, grpo_partial_t* seq_stats,
                                 grpo_loss_t* loss, float* dlogp, hipStream_t stream);

/* Context-parallel shard path: the tokens [t_begin, t_end) of every sequence (t_begin a
 * multiple of GRPO_TOKEN_TILE; t_end a multiple of it or seq_len).  The per-token arrays
 * point at token t_begin of row 0 (a column view with stride ld), as do mask and dlogp.
 * Writes one grpo_partial_t per (sequence, tile): partials points at the slot of tile
 * t_begin / GRPO_TOKEN_TILE of row 0 of a [n_seqs, ldp] array.  The gradient needs the
 * whole-sequence normalizers up front: seq_tokens (int32 [n_seqs], whole-sequence active
 * counts, e.g. the sum of grpo_token_counts over the shards) is required for the seq modes,
 * params->norm_tokens > 0 for token_mean and params->norm_seqs > 0 for seq_mean; missing
 * metadata is LOGP_ERR_ARG (no silent local fallback).  dlogp may be NULL. */
LOGP_API logp_status_t grpo_loss_partials(const float* logp, const float* old_logp,
                                          const float* ref_logp, const float* adv,
                                          const uint8_t* mask, int64_t n_seqs, int64_t seq_len,
                                          int64_t ld, int64_t t_begin, int64_t t_end,
                                          const int32_t* seq_tokens, const grpo_params_t* params,
                                          grpo_partial_t* partials, int64_t ldp, float* dlogp,
                                          hipStream_t stream);

/* Merge of per-tile partials [n_seqs, ldp] (num_tiles = ceil(seq_len / GRPO_TOKEN_TILE)
 * slots per row) into per-sequence sums, in the fixed order: bitwise equal to the
 * seq_stats of grpo_loss over the same tokens. */
LOGP_API logp_status_t grpo_loss_merge(const grpo_partial_t* partials, int64_t ldp,
                                       int64_t n_seqs, int64_t num_tiles,
                                       grpo_partial_t* seq_stats, hipStream_t stream);

/* Data-parallel merge: the loss from per-sequence sums [n_seqs] (e.g. the concatenated
 * seq_stats of several grpo_loss calls over groups of whole sequences, in global sequence
 * order), reduced in the fixed order with params' normalizers.  Bitwise equal to the loss
 * of one grpo_loss call over all the sequences. */
LOGP_API logp_status_t grpo_loss_reduce(const grpo_partial_t* seq_stats, int64_t n_seqs,
                                        const grpo_params_t* params, grpo_loss_t* loss,
                                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GRPO_LOSS_H */
