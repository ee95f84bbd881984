/*
 * FP64 oracle for the selected-token log-probability, its gradient and the vocab-tile
 * partial merge.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
 * file; only the tests, the smoke check and the bench's CPU-baseline leg use it.  It
 * shares no code, header, table or constant with the HIP kernels.
 *
 * Everything here is the plain definition, written out in double precision with
 * straightforward loops over columns in index order:
 *
 *   logp_t  = x[t, y_t] - logsumexp_v x[t, v]
 *     (RL-Kernel issue #241 "TP-aware deterministic logprob", section Background)
 *   dlogits = g_t * (onehot(y_t) - softmax(x_t))
 *     (RL-Kernel PR #495 "zero-workspace backward for generic CUDA fused logp",
 *      section Summary, item 2, and the original_vjp of its Benchmark script)
 *   per-tile (m_l, s_l) and the merge M = max m_l, S = sum s_l exp(m_l - M),
 *   LSE = M + log S (issue #241, section "PR 3"; PR #314 "Deterministic config option",
 *   Tensor Parallel doc excerpt, steps 1-6).
 *
 * Readings of points the pages leave open (each is also listed in the design notes):
 *   - A row is valid iff it is active (or no mask is given), its target differs from
 *     ignore_index and 0 <= target < vocab_real.  An invalid row has logp 0 and an
 *     all-zero gradient row (PR #495, Behavior changes; PR #314 doc step 6).
 *   - Columns in [vocab_real, vocab_padded) are padding: never read, gradient 0
 *     (issue #241 PR 1; PR #314 commit notes on padded columns masked to -inf).
 *   - logp is evaluated as (x_y - M) - log S, which is the same real number as
 *     x_y - LSE; LSE itself is M + log S.
 *   - A row whose real logits are all -inf has M = -inf, S = 0, LSE = -inf,
 *     logp = -inf when valid (0 otherwise) and a zero gradient row.
 *   - The softmax in the gradient is exp(x_c - M) / S.
 *   - BF16 outputs are the round-to-nearest-even of the FP64 value, taken directly from
 *     FP64 (no FP32 intermediate, so no double rounding).
 *   - Logits may also be FP16 or FP32 (the pull request's tests cover FP32/BF16/FP16,
 *     section Tests); the gradient is returned in the logits' own dtype, rounded to
 *     nearest-even straight from FP64.
 *   - Temperature-scaled scoring scores z = fl32(x * inv_temperature), one FP32 product
 *     per logit (the rounding of x / tau is frozen this way so that every consumer gets the
 *     same z); logp and LSE are exact functions of z, and dlogits is
 *     inv_temperature * g * (onehot - softmax(z)).  inv_temperature = 1 leaves x unchanged.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ scalar helpers */

/* A BF16 value is the upper half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* An IEEE binary16 value from its bits: sign, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_bits_to_double(uint16_t h) {
    int sign = (h >> 15) & 1, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m == 0 ? INFINITY : NAN;
    else
        v = ldexp(1024.0 + m, e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

enum { DT_BF16 = 0, DT_F16 = 1, DT_F32 = 2, DT_F64 = 3 };

/* Logit number `index` of a buffer of the given dtype, scaled: fl32(x * inv_temperature).
 * FP64 logits (exact logits of a linear layer, computed in double) are used as they are,
 * times inv_temperature in double. */
static double logit_at(const void* logits, int dtype, int64_t index, float inv_temperature) {
    if (dtype == DT_F64) return ((const double*)logits)[index] * (double)inv_temperature;
    float x;
    if (dtype == DT_BF16)
        x = (float)bf16_bits_to_double(((const uint16_t*)logits)[index]);
    else if (dtype == DT_F16)
        x = (float)f16_bits_to_double(((const uint16_t*)logits)[index]);
    else
        x = ((const float*)logits)[index];
    float z = x * inv_temperature; /* one correctly rounded FP32 product */
    return (double)z;
}

/* Round a double to the nearest BF16 value, ties to even, straight from FP64.
 * BF16: 1 sign bit, 8 exponent bits (bias 127), 7 stored significand bits. */
ORACLE_API uint16_t oracle_rne_bf16(double d) {
    if (isnan(d)) return (uint16_t)0x7FC0;
    uint16_t sign = signbit(d) ? 0x8000 : 0x0000;
    double a = fabs(d);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);               /* a = f * 2^e, 0.5 <= f < 1 */
    int q_exp = e - 8;                /* spacing of BF16 numbers in this binade */
    if (q_exp < -133) q_exp = -133;   /* subnormal spacing 2^-133 below 2^-126 */
    double q = ldexp(a, -q_exp);      /* exact: scaling by a power of two */
    double r = nearbyint(q);          /* default rounding mode: nearest, ties to even */
    double v = ldexp(r, q_exp);       /* exact; now representable in BF16 (or 2^128) */
    if (v >= ldexp(1.0, 128)) return sign | 0x7F80;
    float vf = (float)v;              /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &vf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

ORACLE_API void oracle_rne_bf16_array(const double* in, uint16_t* out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_rne_bf16(in[i]);
}

/* Round a double to the nearest binary16 value, ties to even, straight from FP64.
 * 11 significant bits; normal range from 2^-14; subnormal spacing 2^-24; largest finite
 * 65504, and everything from 65520 (the tie with 2^16) up rounds to infinity. */
ORACLE_API uint16_t oracle_rne_f16(double d) {
    if (isnan(d)) return (uint16_t)0x7E00;
    uint16_t sign = signbit(d) ? 0x8000 : 0x0000;
    double a = fabs(d);
    if (isinf(a)) return sign | 0x7C00;
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);              /* a = f * 2^e, 0.5 <= f < 1 */
    int q_exp = e - 11;              /* spacing of binary16 numbers in this binade */
    if (q_exp < -24) q_exp = -24;    /* subnormal spacing below 2^-14 */
    double v = ldexp(nearbyint(ldexp(a, -q_exp)), q_exp);
    if (v > 65504.0) return sign | 0x7C00;
    if (v < ldexp(1.0, -14)) return sign | (uint16_t)ldexp(v, 24); /* subnormal or zero */
    int ev;
    double f = frexp(v, &ev);        /* v = f * 2^ev, f in [0.5, 1) */
    uint16_t mant = (uint16_t)(ldexp(f, 11) - 1024.0);
    return sign | (uint16_t)((ev - 1 + 15) << 10) | mant;
}

ORACLE_API void oracle_rne_f16_array(const double* in, uint16_t* out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_rne_f16(in[i]);
}

static int row_is_valid(const int64_t* targets, const uint8_t* active, int64_t ignore_index,
                        int64_t vocab_real, int64_t t) {
    int64_t y = targets[t];
    if (active != NULL && active[t] == 0) return 0;
    if (y == ignore_index) return 0;
    return y >= 0 && y < vocab_real;
}

/* ------------------------------------------------------------------ thread plumbing */

typedef void (*row_fn)(void* ctx, int64_t row);

typedef struct {
    row_fn fn;
    void* ctx;
    int64_t begin, end;
} span_t;

static void* run_span(void* p) {
    span_t* s = (span_t*)p;
    for (int64_t t = s->begin; t < s->end; ++t) s->fn(s->ctx, t);
    return NULL;
}

/* Rows are independent; split [0, n) into contiguous blocks, one per thread. */
static int for_each_row(int64_t n, int nthreads, row_fn fn, void* ctx) {
    if (n <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)n;
    pthread_t tid[256];
    span_t span[256];
    int created[256] = {0};
    int64_t per = (n + nthreads - 1) / nthreads;
    for (int i = 0; i < nthreads; ++i) {
        span[i].fn = fn;
        span[i].ctx = ctx;
        span[i].begin = (int64_t)i * per < n ? (int64_t)i * per : n;
        span[i].end = span[i].begin + per < n ? span[i].begin + per : n;
    }
    /* the calling thread takes block 0; a block whose thread cannot start runs here */
    for (int i = 1; i < nthreads; ++i) {
        if (span[i].begin >= span[i].end) continue;
        if (pthread_create(&tid[i], NULL, run_span, &span[i]) == 0)
            created[i] = 1;
        else
            run_span(&span[i]);
    }
    run_span(&span[0]);
    for (int i = 1; i < nthreads; ++i)
        if (created[i]) pthread_join(tid[i], NULL);
    return 0;
}

/* ------------------------------------------------------------------ row statistics */

/* A row of logits: element c is logit_at(base, dtype, offset + c, inv_t). */
typedef struct {
    const void* base;
    int dtype;
    int64_t offset;
    float inv_t;
} row_t;

static double row_x(const row_t* r, int64_t c) {
    return logit_at(r->base, r->dtype, r->offset + c, r->inv_t);
}

/* M = max over real columns, S = sum exp(x_c - M) in column order (S = 0 if M = -inf). */
static void row_max_sumexp(const row_t* row, int64_t vocab_real, double* M_out, double* S_out) {
    double M = -INFINITY;
    for (int64_t c = 0; c < vocab_real; ++c) {
        double x = row_x(row, c);
        if (x > M) M = x;
    }
    double S = 0.0;
    if (M != -INFINITY)
        for (int64_t c = 0; c < vocab_real; ++c) S += exp(row_x(row, c) - M);
    *M_out = M;
    *S_out = S;
}

/* ------------------------------------------------------------------------- forward */

typedef struct {
    const void* logits;
    int dtype;
    float inv_t;
    int64_t ld, vocab_real;
    const int64_t* targets;
    const uint8_t* active;
    int64_t ignore_index;
    double *logp, *lse, *row_max, *row_sumexp;
} fwd_ctx;

static void fwd_row(void* p, int64_t t) {
    fwd_ctx* c = (fwd_ctx*)p;
    row_t row = {c->logits, c->dtype, t * c->ld, c->inv_t};
    double M, S;
    row_max_sumexp(&row, c->vocab_real, &M, &S);
    int valid = row_is_valid(c->targets, c->active, c->ignore_index, c->vocab_real, t);
    double lse, logp;
    if (M == -INFINITY) {
        lse = -INFINITY;
        logp = valid ? -INFINITY : 0.0;
    } else {
        double log_s = log(S);
        lse = M + log_s;
        logp = valid ? (row_x(&row, c->targets[t]) - M) - log_s : 0.0;
    }
    if (c->logp) c->logp[t] = logp;
    if (c->lse) c->lse[t] = lse;
    if (c->row_max) c->row_max[t] = M;
    if (c->row_sumexp) c->row_sumexp[t] = S;
}

/* logits: [n, ld] of the given dtype (0 BF16, 1 FP16, 2 FP32); outputs [n] doubles (each
 * nullable).  The scored logits are fl32(x * inv_temperature). */
ORACLE_API int oracle_forward_ex(int dtype, float inv_temperature, const void* logits, int64_t ld,
                                 int64_t n, int64_t vocab_real, const int64_t* targets,
                                 const uint8_t* active, int64_t ignore_index, double* logp,
                                 double* lse, double* row_max, double* row_sumexp, int nthreads) {
    if (n < 0 || vocab_real < 1 || ld < vocab_real || dtype < 0 || dtype > 3) return 1;
    if (n > 0 && (logits == NULL || targets == NULL)) return 1;
    fwd_ctx c = {logits, dtype, inv_temperature, ld, vocab_real, targets, active, ignore_index,
                 logp, lse, row_max, row_sumexp};
    return for_each_row(n, nthreads, fwd_row, &c);
}

ORACLE_API int oracle_forward(const uint16_t* logits, int64_t ld, int64_t n, int64_t vocab_real,
                              const int64_t* targets, const uint8_t* active,
                              int64_t ignore_index, double* logp, double* lse, double* row_max,
                              double* row_sumexp, int nthreads) {
    return oracle_forward_ex(DT_BF16, 1.0f, logits, ld, n, vocab_real, targets, active,
                             ignore_index, logp, lse, row_max, row_sumexp, nthreads);
}

/* ------------------------------------------------------------------------ backward */

typedef struct {
    const void* logits;
    int dtype;
    float inv_t;
    int64_t ld, vocab_real, vocab_padded;
    const int64_t* targets;
    const uint8_t* active;
    int64_t ignore_index;
    const float* grad;
    double* d64;
    int64_t ld_d64;
    void* d_out; /* rounded to the logits' dtype */
    int64_t ld_out;
} bwd_ctx;

static void store_rounded(void* out, int dtype, int64_t index, double v) {
    if (dtype == DT_BF16)
        ((uint16_t*)out)[index] = oracle_rne_bf16(v);
    else if (dtype == DT_F16)
        ((uint16_t*)out)[index] = oracle_rne_f16(v);
    else
        ((float*)out)[index] = (float)v; /* C's double -> float conversion rounds to nearest */
}

static void bwd_row(void* p, int64_t t) {
    bwd_ctx* c = (bwd_ctx*)p;
    row_t row = {c->logits, c->dtype, t * c->ld, c->inv_t};
    double* d = c->d64 ? c->d64 + t * c->ld_d64 : NULL;
    int valid = row_is_valid(c->targets, c->active, c->ignore_index, c->vocab_real, t);
    double M = -INFINITY, S = 0.0;
    if (valid) row_max_sumexp(&row, c->vocab_real, &M, &S);
    if (!valid || M == -INFINITY) {
        for (int64_t col = 0; col < c->vocab_padded; ++col) {
            if (d) d[col] = 0.0;
            if (c->d_out) store_rounded(c->d_out, c->dtype, t * c->ld_out + col, 0.0);
        }
        return;
    }
    /* d logits = d z / d x * d logp / d z = inv_temperature * g * (onehot - softmax(z)) */
    double g = (double)c->grad[t] * (double)c->inv_t;
    int64_t y = c->targets[t];
    for (int64_t col = 0; col < c->vocab_padded; ++col) {
        double v = 0.0;
        if (col < c->vocab_real) {
            double softmax = exp(row_x(&row, col) - M) / S;
            double onehot = (col == y) ? 1.0 : 0.0;
            v = g * (onehot - softmax);
        }
        if (d) d[col] = v;
        if (c->d_out) store_rounded(c->d_out, c->dtype, t * c->ld_out + col, v);
    }
}

/* d64: [n, ld_d64] doubles, d_out: [n, ld_out] in the logits' dtype (each nullable); columns
 * [0, vocab_padded) of each row are written. */
ORACLE_API int oracle_backward_ex(int dtype, float inv_temperature, const void* logits,
                                  int64_t ld, int64_t n, int64_t vocab_real, int64_t vocab_padded,
                                  const int64_t* targets, const uint8_t* active,
                                  int64_t ignore_index, const float* grad, double* d64,
                                  int64_t ld_d64, void* d_out, int64_t ld_out, int nthreads) {
    if (n < 0 || vocab_real < 1 || vocab_padded < vocab_real || ld < vocab_real) return 1;
    if (dtype < 0 || dtype > 2) return 1;
    if (d64 && ld_d64 < vocab_padded) return 1;
    if (d_out && ld_out < vocab_padded) return 1;
    if (n > 0 && (logits == NULL || targets == NULL || grad == NULL)) return 1;
    bwd_ctx c = {logits, dtype, inv_temperature, ld, vocab_real, vocab_padded, targets, active,
                 ignore_index, grad, d64, ld_d64, d_out, ld_out};
    return for_each_row(n, nthreads, bwd_row, &c);
}

ORACLE_API int oracle_backward(const uint16_t* logits, int64_t ld, int64_t n, int64_t vocab_real,
                               int64_t vocab_padded, const int64_t* targets,
                               const uint8_t* active, int64_t ignore_index, const float* grad,
                               double* d64, int64_t ld_d64, uint16_t* d_bf16, int64_t ld_bf16,
                               int nthreads) {
    return oracle_backward_ex(DT_BF16, 1.0f, logits, ld, n, vocab_real, vocab_padded, targets,
                              active, ignore_index, grad, d64, ld_d64, d_bf16, ld_bf16, nthreads);
}

/* ---------------------------------------------------------------- tile partials */

typedef struct {
    const void* logits;
    int dtype;
    float inv_t;
    int64_t ld, vocab_real, vocab_padded, tile, num_tiles;
    const int64_t* targets;
    const uint8_t* active;
    int64_t ignore_index;
    double *m, *s, *sel;
} part_ctx;

static void part_row(void* p, int64_t t) {
    part_ctx* c = (part_ctx*)p;
    row_t row = {c->logits, c->dtype, t * c->ld, c->inv_t};
    int valid = row_is_valid(c->targets, c->active, c->ignore_index, c->vocab_real, t);
    int64_t y = c->targets[t];
    for (int64_t l = 0; l < c->num_tiles; ++l) {
        int64_t lo = l * c->tile;
        int64_t hi = lo + c->tile;
        if (hi > c->vocab_real) hi = c->vocab_real; /* padded columns are not part of it */
        double m = -INFINITY, s = 0.0;
        for (int64_t col = lo; col < hi; ++col) {
            double x = row_x(&row, col);
            if (x > m) m = x;
        }
        if (m != -INFINITY)
            for (int64_t col = lo; col < hi; ++col) s += exp(row_x(&row, col) - m);
        double sel = 0.0;
        if (valid && y >= lo && y < lo + c->tile) sel = row_x(&row, y);
        c->m[t * c->num_tiles + l] = m;
        c->s[t * c->num_tiles + l] = s;
        c->sel[t * c->num_tiles + l] = sel;
    }
}

/* Per global tile l = [l*tile, (l+1)*tile) of the padded row: m_l = max over the real
 * columns of the tile (-inf when there are none), s_l = sum exp(x - m_l) (0 when
 * m_l = -inf), sel_l = x_y when the row is valid and y lies in the tile, else 0.
 * Outputs are [n, num_tiles] doubles, num_tiles = ceil(vocab_padded / tile). */
ORACLE_API int oracle_tile_partials_ex(int dtype, float inv_temperature, const void* logits,
                                       int64_t ld, int64_t n, int64_t vocab_real,
                                       int64_t vocab_padded, int64_t tile,
                                       const int64_t* targets, const uint8_t* active,
                                       int64_t ignore_index, double* m, double* s, double* sel,
                                       int nthreads) {
    if (n < 0 || vocab_real < 1 || vocab_padded < vocab_real || ld < vocab_real || tile < 1)
        return 1;
    if (dtype < 0 || dtype > 3) return 1;
    if (n > 0 && (logits == NULL || targets == NULL || !m || !s || !sel)) return 1;
    part_ctx c = {logits, dtype, inv_temperature, ld, vocab_real, vocab_padded, tile,
                  (vocab_padded + tile - 1) / tile, targets, active, ignore_index, m, s, sel};
    return for_each_row(n, nthreads, part_row, &c);
}

ORACLE_API int oracle_tile_partials(const uint16_t* logits, int64_t ld, int64_t n,
                                    int64_t vocab_real, int64_t vocab_padded, int64_t tile,
                                    const int64_t* targets, const uint8_t* active,
                                    int64_t ignore_index, double* m, double* s, double* sel,
                                    int nthreads) {
    return oracle_tile_partials_ex(DT_BF16, 1.0f, logits, ld, n, vocab_real, vocab_padded, tile,
                                   targets, active, ignore_index, m, s, sel, nthreads);
}

/* Merge per-tile partials in tile order: M = max m_l, S = sum over tiles with
 * m_l != -inf of s_l * exp(m_l - M), LSE = M + log S, logp = (sel_owner - M) - log S
 * for a valid row, where the owner tile is floor(y / tile) (copied, never summed).
 * A tile with m_l = -inf is the (-inf, 0) identity and contributes nothing. */
ORACLE_API int oracle_merge(const double* m, const double* s, const double* sel, int64_t n,
                            int64_t num_tiles, int64_t tile, int64_t vocab_real,
                            const int64_t* targets, const uint8_t* active,
                            int64_t ignore_index, double* logp, double* lse) {
    if (n < 0 || num_tiles < 1 || tile < 1) return 1;
    for (int64_t t = 0; t < n; ++t) {
        const double* mt = m + t * num_tiles;
        const double* st = s + t * num_tiles;
        double M = -INFINITY;
        for (int64_t l = 0; l < num_tiles; ++l)
            if (mt[l] > M) M = mt[l];
        double S = 0.0;
        if (M != -INFINITY)
            for (int64_t l = 0; l < num_tiles; ++l)
                if (mt[l] != -INFINITY) S += st[l] * exp(mt[l] - M);
        int valid = row_is_valid(targets, active, ignore_index, vocab_real, t);
        double out_lse, out_logp;
        if (M == -INFINITY) {
            out_lse = -INFINITY;
            out_logp = valid ? -INFINITY : 0.0;
        } else {
            double log_s = log(S);
            out_lse = M + log_s;
            out_logp = valid ? (sel[t * num_tiles + targets[t] / tile] - M) - log_s : 0.0;
        }
        if (logp) logp[t] = out_logp;
        if (lse) lse[t] = out_lse;
    }
    return 0;
}

/* ------------------------------------------------------------------ target check */

/* Number of active rows (mask set or absent) whose target is neither ignore_index nor
 * inside [0, vocab_real). */
ORACLE_API int64_t oracle_count_bad_targets(const int64_t* targets, const uint8_t* active,
                                            int64_t n, int64_t vocab_real,
                                            int64_t ignore_index) {
    int64_t bad = 0;
    for (int64_t t = 0; t < n; ++t) {
        if (active != NULL && active[t] == 0) continue;
        int64_t y = targets[t];
        if (y == ignore_index) continue;
        if (y < 0 || y >= vocab_real) ++bad;
    }
    return bad;
}
