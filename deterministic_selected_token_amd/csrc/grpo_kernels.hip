// gfx950 kernels and C entry points of the deterministic GRPO loss (include/grpo_loss.h).
//
// Source: RL-Kernel issue #241 "[WS2] TP-aware deterministic logprob …", planned PR5: the GRPO
// objective (ratio, clip, KL, advantage normalization) under a declared reduction
// (token_mean / seq_mean / seq_sum_token_mean, global or local n_non_ignore) with a fixed
// summation order over tokens, then sequences, then ranks, merged in fixed order instead of
// by a collective sum.
//
//   seq kernel      one workgroup per sequence (one wave per tile, up to 16): its waves take
//                   the sequence's 256-token tiles
//                   round-robin, compute every token's terms and gradient in registers,
//                   reduce each tile with the lane tree, park the tile sums in LDS; wave 0
//                   merges them in the fixed order.  One pass over the per-token inputs.
//   partials kernel one wave per (sequence, tile) of a token range: the same tile code,
//                   written out (context-parallel shards).
//   merge kernel    one wave per sequence over its tile partials: the same merge code.
//   count / norm    active tokens per sequence, then the batch normalizer, each launched only
//                   when a mask makes them unknown on the host and the reduction needs them
//                   before the pass (n_i for seq_mean and seq_sum_token_mean, the sums for a
//                   local normalizer).
//   reduce kernel   one workgroup over the batch's sequences: the same merge order again.
//   advantages      one wave per reward group.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "grpo_loss.h"
#include "host_common.hpp"
#include "logp_device.hpp"

using namespace logp;
using namespace logp_host;

namespace {

constexpr int kTokTile = GRPO_TOKEN_TILE;       // tokens per tile
constexpr int kTokPerLane = kTokTile / kWave;  // 4
constexpr int kSeqMaxWaves = 16;                // most waves per sequence workgroup
constexpr int kMaxTokTiles = GRPO_MAX_SEQ_LEN / kTokTile;
constexpr int kItemWaves = 4;                   // waves per workgroup of per-wave kernels
constexpr int kCountThreads = 256;

static_assert(kTokTile % kWave == 0, "a token tile is whole lanes");

// Per-call constants of the per-token arithmetic.
struct Objective {
    float lo, hi;     // clip bounds fl32(1 - eps_low), fl32(1 + eps_high)
    float beta;       // KL weight (0 without a reference)
    int32_t mode;     // grpo_mode_t
};

// Per-token inputs of one call; row pointers are formed per sequence (stride ld).
struct Tokens {
    const float* logp;
    const float* old_logp;
    const float* ref_logp;  // nullptr: no KL term
    const float* adv;
    const uint8_t* mask;    // nullptr: every token active
    int64_t ld;
    int width;              // tokens in the view (a token range of every sequence)
};

struct TokenTerms {
    float pg, kl, dl;
    bool clipped;
};

// The KL estimator exp(d) - d - 1.  expm1(d) - d cancels when |d| is small (the result is
// about d^2 / 2 while expm1(d) carries an error of about 2^-23 |d|), so for |d| < 1 it is
// formed as d^2 times the Taylor series of (e^d - 1 - d) / d^2 = sum_k d^(k-2) / k!,
// k = 2..13 (the first omitted term is below 2^-31 of the sum there), by Horner's rule with
// fused multiply-adds; for |d| >= 1, as expm1(d) - d, which then loses under 2 bits.
__device__ __forceinline__ float kl_estimator(float d, float em) {
    if (!(fabsf(d) < 1.0f)) return em - d;
    float p = 1.0f / 6227020800.0f;                // 1/13!
    p = __builtin_fmaf(p, d, 1.0f / 479001600.0f);  // 1/12!
    p = __builtin_fmaf(p, d, 1.0f / 39916800.0f);   // 1/11!
    p = __builtin_fmaf(p, d, 1.0f / 3628800.0f);    // 1/10!
    p = __builtin_fmaf(p, d, 1.0f / 362880.0f);     // 1/9!
    p = __builtin_fmaf(p, d, 1.0f / 40320.0f);      // 1/8!
    p = __builtin_fmaf(p, d, 1.0f / 5040.0f);       // 1/7!
    p = __builtin_fmaf(p, d, 1.0f / 720.0f);        // 1/6!
    p = __builtin_fmaf(p, d, 1.0f / 120.0f);        // 1/5!
    p = __builtin_fmaf(p, d, 1.0f / 24.0f);         // 1/4!
    p = __builtin_fmaf(p, d, 1.0f / 6.0f);          // 1/3!
    p = __builtin_fmaf(p, d, 0.5f);                 // 1/2!
    return (d * d) * p;
}

// The GRPO terms of one active token (see include/grpo_loss.h for the definitions).
__device__ __forceinline__ TokenTerms grpo_token(float lp, float old, float ref, bool has_ref,
                                                 float A, const Objective& o) {
    TokenTerms t;
    const float r = expf(lp - old);
    t.clipped = (A > 0.0f && r > o.hi) || (A < 0.0f && r < o.lo);
    const float arg = t.clipped ? (A > 0.0f ? o.hi : o.lo) : r;
    t.pg = A == 0.0f ? 0.0f : -A * arg;
    const float dpg = (t.clipped || A == 0.0f) ? 0.0f : -A * r;
    if (has_ref) {
        const float e = ref - lp;
        const float em = expm1f(e);
        t.kl = kl_estimator(e, em);
        t.dl = dpg + o.beta * (-em);
    } else {
        t.kl = 0.0f;
        t.dl = dpg;
    }
    return t;
}

__device__ __forceinline__ int wave_isum(int v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Sums of tokens [c0, c0 + kTokTile) of view row `row`: lane l holds tokens c0 + l + 64 e,
// adds them in e order from +0, then the lane tree.  Writes each token's gradient times
// `scale` to dlogp (when given); inactive tokens get +0.
__device__ __forceinline__ grpo_partial_t grpo_tile(const Tokens& tk, const Objective& o,
                                                    int64_t row, int c0, float A, float scale,
                                                    float* dlogp, int64_t ld_out, int lane) {
    const int64_t base = row * tk.ld;
    float lp[kTokPerLane], od[kTokPerLane], rf[kTokPerLane];
    bool act[kTokPerLane];
#pragma unroll
    for (int e = 0; e < kTokPerLane; ++e) {
        const int c = c0 + lane + kWave * e;
        const bool in = c < tk.width;
        act[e] = in && (tk.mask == nullptr || tk.mask[base + c] != 0);
        lp[e] = in ? tk.logp[base + c] : 0.0f;
        od[e] = in ? tk.old_logp[base + c] : 0.0f;
        rf[e] = (in && tk.ref_logp != nullptr) ? tk.ref_logp[base + c] : 0.0f;
    }
    float pg = 0.0f, kl = 0.0f;
    int clipped = 0, tokens = 0;
#pragma unroll
    for (int e = 0; e < kTokPerLane; ++e) {
        const int c = c0 + lane + kWave * e;
        float g = 0.0f;
        if (act[e]) {
            const TokenTerms t = grpo_token(lp[e], od[e], rf[e], tk.ref_logp != nullptr, A, o);
            pg = pg + t.pg;
            kl = kl + t.kl;
            clipped += t.clipped ? 1 : 0;
            tokens += 1;
            g = t.dl * scale;
        }
        if (dlogp != nullptr && c < tk.width) dlogp[row * ld_out + c] = g;
    }
    grpo_partial_t s;
    s.pg_sum = wave_sum(pg);
    s.kl_sum = wave_sum(kl);
    s.clipped = wave_isum(clipped);
    s.tokens = wave_isum(tokens);
    return s;
}

// Fixed-order merge of items [0, count) read through src(i): lane l adds items l, l+64, ...
// in order from +0, then the lane tree.  Every lane returns the same sums.  Items are
// fetched kMergeBatch at a time ahead of the additions, which keep their order.
constexpr int kMergeBatch = 8;

template <class Src>
__device__ __forceinline__ grpo_partial_t grpo_merge(const Src& src, int64_t count, int lane) {
    float pg = 0.0f, kl = 0.0f;
    int clipped = 0, tokens = 0;
    for (int64_t i0 = lane; i0 < count; i0 += int64_t(kWave) * kMergeBatch) {
        grpo_partial_t p[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const int64_t i = i0 + int64_t(j) * kWave;
            if (i < count) p[j] = src(i);
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            if (i0 + int64_t(j) * kWave >= count) break;
            pg = pg + p[j].pg_sum;
            kl = kl + p[j].kl_sum;
            clipped += p[j].clipped;
            tokens += p[j].tokens;
        }
    }
    grpo_partial_t s;
    s.pg_sum = wave_sum(pg);
    s.kl_sum = wave_sum(kl);
    s.clipped = wave_isum(clipped);
    s.tokens = wave_isum(tokens);
    return s;
}

// Normalizer D of the reduction from the batch counts (see include/grpo_loss.h).
__host__ __device__ __forceinline__ int64_t grpo_norm(int32_t mode, int64_t norm_tokens,
                                                      int64_t norm_seqs, int64_t tokens,
                                                      int64_t nonempty) {
    if (mode == GRPO_TOKEN_MEAN) return norm_tokens > 0 ? norm_tokens : tokens;
    if (mode == GRPO_SEQ_MEAN) return norm_seqs > 0 ? norm_seqs : nonempty;
    return 1;
}

// Gradient scale of sequence i: 1/D (token_mean), 1/(n_i D) (seq_mean), 1/n_i
// (seq_sum_token_mean), each as the float32 rounding of a double quotient; 0 when the
// denominator is 0.
__device__ __forceinline__ float grpo_scale(int32_t mode, int64_t n_i, int64_t D) {
    double den;
    if (mode == GRPO_TOKEN_MEAN) den = static_cast<double>(D);
    else if (mode == GRPO_SEQ_MEAN) den = static_cast<double>(n_i) * static_cast<double>(D);
    else den = static_cast<double>(n_i);
    return den > 0.0 ? static_cast<float>(1.0 / den) : 0.0f;
}

struct LdsPartials {
    const grpo_partial_t* p;
    __device__ grpo_partial_t operator()(int64_t i) const { return p[i]; }
};

struct RowPartials {
    const grpo_partial_t* p;
    __device__ grpo_partial_t operator()(int64_t i) const { return p[i]; }
};

// ----------------------------------------------------------------------------- kernels

// One workgroup per sequence.  With `counted`, seq_stats[].tokens holds each sequence's
// active-token count n_i (the count kernel's); otherwise every sequence has tk.width active
// tokens, or the reduction does not use n_i.  The normalizer D is `norm_dev[0]` when given
// (formed on the device from the counts), else `norm_host`.
__global__ __launch_bounds__(kSeqMaxWaves* kWave) void grpo_seq_kernel(
    Tokens tk, Objective o, int counted, const int64_t* norm_dev, int64_t norm_host,
    grpo_partial_t* __restrict__ seq_stats, float* dlogp) {
    extern __shared__ grpo_partial_t slots[];  // one slot per tile of the sequence
    const int64_t row = blockIdx.x;
    const int lane = lane_id(), wave = wave_id();
    const int waves = static_cast<int>(blockDim.x) / kWave;
    const float A = tk.adv[row];
    const int64_t n_i = counted ? seq_stats[row].tokens : tk.width;
    const int64_t D = norm_dev != nullptr ? norm_dev[0] : norm_host;
    const float scale = grpo_scale(o.mode, n_i, D);
    const int tiles = (tk.width + kTokTile - 1) / kTokTile;
    for (int t = wave; t < tiles; t += waves) {
        const grpo_partial_t s = grpo_tile(tk, o, row, t * kTokTile, A, scale, dlogp, tk.ld, lane);
        if (lane == 0) slots[t] = s;
    }
    __syncthreads();  // every thread has read seq_stats[row] above, before it is rewritten
    if (wave == 0) {
        const grpo_partial_t s = grpo_merge(LdsPartials{slots}, tiles, lane);
        if (lane == 0) seq_stats[row] = s;
    }
}

// One wave per (sequence, tile of the view).  scale from `seq_tokens` / D as in the seq
// kernel.
__global__ __launch_bounds__(kItemWaves* kWave) void grpo_partials_kernel(
    Tokens tk, Objective o, const int32_t* __restrict__ seq_tokens, int64_t D, int64_t n_seqs,
    int view_tiles, grpo_partial_t* partials, int64_t ldp, float* dlogp) {
    const int64_t item = int64_t(blockIdx.x) * kItemWaves + wave_id();
    if (item >= n_seqs * view_tiles) return;  // whole wave leaves; no barrier follows
    const int lane = lane_id();
    const int64_t row = item / view_tiles;
    const int t = static_cast<int>(item - row * view_tiles);
    const int64_t n_i = seq_tokens != nullptr ? seq_tokens[row] : 0;
    const float scale = grpo_scale(o.mode, n_i, D);
    const grpo_partial_t s = grpo_tile(tk, o, row, t * kTokTile, tk.adv[row], scale, dlogp,
                                       tk.ld, lane);
    if (lane == 0) partials[row * ldp + t] = s;
}

// One wave per sequence over its [num_tiles] partials.
__global__ __launch_bounds__(kItemWaves* kWave) void grpo_merge_kernel(
    const grpo_partial_t* __restrict__ partials, int64_t ldp, int64_t n_seqs, int64_t num_tiles,
    grpo_partial_t* __restrict__ seq_stats) {
    const int64_t row = int64_t(blockIdx.x) * kItemWaves + wave_id();
    if (row >= n_seqs) return;
    const grpo_partial_t s = grpo_merge(RowPartials{partials + row * ldp}, num_tiles, lane_id());
    if (lane_id() == 0) seq_stats[row] = s;
}

// Nonzero bytes of a 32-bit word: bit 7 of each byte of y is set iff that byte of x is not 0.
__device__ __forceinline__ int nonzero_bytes(uint32_t x) {
    const uint32_t y = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
    return __popc(y);
}

// Active tokens of view row blockIdx.x, written to counts[row * stride].  VEC: the row starts
// are 16-byte aligned and the mask is read 16 bytes at a time.
template <bool VEC>
__global__ __launch_bounds__(kCountThreads) void grpo_count_kernel(
    const uint8_t* __restrict__ mask, int64_t ld, int width, int32_t* counts, int64_t stride) {
    __shared__ int wave_counts[kCountThreads / kWave];
    const int64_t row = blockIdx.x;
    int c = 0;
    if (mask == nullptr) {
        c = threadIdx.x == 0 ? width : 0;
    } else {
        const uint8_t* m = mask + row * ld;
        int t0 = 0;
        if (VEC) {
            const int nv = width / 16;
            for (int q = threadIdx.x; q < nv; q += kCountThreads) {
                const uint4 v = reinterpret_cast<const uint4*>(m)[q];
                c += nonzero_bytes(v.x) + nonzero_bytes(v.y) + nonzero_bytes(v.z) +
                     nonzero_bytes(v.w);
            }
            t0 = nv * 16;
        }
        for (int t = t0 + threadIdx.x; t < width; t += kCountThreads) c += m[t] != 0;
    }
    c = wave_isum(c);
    if (lane_id() == 0) wave_counts[wave_id()] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        int total = 0;
        for (int w = 0; w < kCountThreads / kWave; ++w) total += wave_counts[w];
        counts[row * stride] = total;
    }
}

const void* count_kernel(const uint8_t* mask, int64_t ld) {
    const bool vec = mask != nullptr && aligned16(mask) && ld % 16 == 0;
    return vec ? reinterpret_cast<const void*>(&grpo_count_kernel<true>)
               : reinterpret_cast<const void*>(&grpo_count_kernel<false>);
}

// Batch counts and the normalizer from seq_stats[].tokens, into loss->tokens / sequences /
// norm.  One workgroup; integer sums, so any order gives the same result.
__global__ __launch_bounds__(kCountThreads) void grpo_norm_kernel(
    const grpo_partial_t* __restrict__ seq_stats, int64_t n_seqs, int32_t mode,
    int64_t norm_tokens, int64_t norm_seqs, grpo_loss_t* loss) {
    __shared__ long long part[2][kCountThreads / kWave];
    long long tokens = 0, nonempty = 0;
    for (int64_t i = threadIdx.x; i < n_seqs; i += kCountThreads) {
        const int32_t n = seq_stats[i].tokens;
        tokens += n;
        nonempty += n > 0 ? 1 : 0;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        tokens += __shfl_xor(tokens, o, kWave);
        nonempty += __shfl_xor(nonempty, o, kWave);
    }
    if (lane_id() == 0) {
        part[0][wave_id()] = tokens;
        part[1][wave_id()] = nonempty;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        tokens = nonempty = 0;
        for (int w = 0; w < kCountThreads / kWave; ++w) {
            tokens += part[0][w];
            nonempty += part[1][w];
        }
        loss->tokens = tokens;
        loss->sequences = nonempty;
        loss->norm = grpo_norm(mode, norm_tokens, norm_seqs, tokens, nonempty);
    }
}

// Contribution of one sequence to the batch sums: its sums (token_mean) or its token means.
struct SeqContribution {
    const grpo_partial_t* p;
    int32_t mode;
    __device__ grpo_partial_t operator()(int64_t i) const {
        grpo_partial_t s = p[i];
        if (mode != GRPO_TOKEN_MEAN) {
            const float n = static_cast<float>(s.tokens);
            s.pg_sum = s.tokens > 0 ? s.pg_sum / n : 0.0f;
            s.kl_sum = s.tokens > 0 ? s.kl_sum / n : 0.0f;
        }
        return s;
    }
};

// The loss from per-sequence sums: wave 0 merges the float sums in the fixed order while
// every wave adds up the integer counts (order-free).
__global__ __launch_bounds__(kCountThreads) void grpo_reduce_kernel(
    const grpo_partial_t* __restrict__ seq_stats, int64_t n_seqs, int32_t mode, float beta,
    int64_t norm_tokens, int64_t norm_seqs, grpo_loss_t* loss) {
    __shared__ long long part[3][kCountThreads / kWave];
    const int lane = lane_id(), wave = wave_id();
    long long tokens = 0, nonempty = 0, clipped = 0;
    for (int64_t i = threadIdx.x; i < n_seqs; i += kCountThreads) {
        const grpo_partial_t p = seq_stats[i];
        tokens += p.tokens;
        nonempty += p.tokens > 0 ? 1 : 0;
        clipped += p.clipped;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        tokens += __shfl_xor(tokens, o, kWave);
        nonempty += __shfl_xor(nonempty, o, kWave);
        clipped += __shfl_xor(clipped, o, kWave);
    }
    if (lane == 0) {
        part[0][wave] = tokens;
        part[1][wave] = nonempty;
        part[2][wave] = clipped;
    }
    grpo_partial_t s{};
    if (wave == 0) s = grpo_merge(SeqContribution{seq_stats, mode}, n_seqs, lane);
    __syncthreads();
    if (threadIdx.x == 0) {
        tokens = nonempty = clipped = 0;
        for (int w = 0; w < kCountThreads / kWave; ++w) {
            tokens += part[0][w];
            nonempty += part[1][w];
            clipped += part[2][w];
        }
        const int64_t D = grpo_norm(mode, norm_tokens, norm_seqs, tokens, nonempty);
        const double d = static_cast<double>(D);
        const float pg = D > 0 ? static_cast<float>(static_cast<double>(s.pg_sum) / d) : 0.0f;
        const float kl = D > 0 ? static_cast<float>(static_cast<double>(s.kl_sum) / d) : 0.0f;
        loss->pg_loss = pg;
        loss->kl_loss = kl;
        loss->loss = pg + beta * kl;
        loss->clip_frac = tokens > 0 ? static_cast<float>(static_cast<double>(clipped) /
                                                          static_cast<double>(tokens))
                                     : 0.0f;
        loss->tokens = tokens;
        loss->sequences = nonempty;
        loss->clipped = clipped;
        loss->norm = D;
    }
}

// One wave per group of `group` rewards: mean and unbiased std by the fixed lane order.
__global__ __launch_bounds__(kItemWaves* kWave) void grpo_adv_kernel(
    const float* rewards, int64_t n_groups, int64_t group, float eps, int scale_by_std,
    float* adv) {
    const int64_t g = int64_t(blockIdx.x) * kItemWaves + wave_id();
    if (g >= n_groups) return;
    const int lane = lane_id();
    const float* r = rewards + g * group;
    float* a = adv + g * group;
    if (group == 1) {
        if (lane == 0) a[0] = 0.0f;
        return;
    }
    float sum = 0.0f;
    for (int64_t j = lane; j < group; j += kWave) sum = sum + r[j];
    const float mean = wave_sum(sum) / static_cast<float>(group);
    float den = 1.0f;
    if (scale_by_std) {
        float sq = 0.0f;
        for (int64_t j = lane; j < group; j += kWave) {
            const float dv = r[j] - mean;
            sq = sq + dv * dv;
        }
        const float var = wave_sum(sq) / static_cast<float>(group - 1);
        den = sqrtf(var) + eps;
    }
    // adv may alias rewards: each element is read and then written by the same lane, after
    // the group's mean and std are known
    for (int64_t j = lane; j < group; j += kWave) {
        const float dv = r[j] - mean;
        a[j] = scale_by_std ? dv / den : dv;
    }
}

// ------------------------------------------------------------------------------ host

logp_status_t check_params(const grpo_params_t* p) {
    if (p == nullptr) return LOGP_ERR_NULL;
    if (!std::isfinite(p->eps_low) || p->eps_low < 0.0f || p->eps_low > 1.0f ||
        !std::isfinite(p->eps_high) || p->eps_high < 0.0f || !std::isfinite(p->beta) ||
        p->beta < 0.0f || p->mode < GRPO_TOKEN_MEAN || p->mode > GRPO_SEQ_SUM_TOKEN_MEAN ||
        p->norm_tokens < 0 || p->norm_seqs < 0)
        return LOGP_ERR_ARG;
    return LOGP_OK;
}

Objective objective(const grpo_params_t* p, bool has_ref) {
    Objective o;
    o.lo = 1.0f - p->eps_low;
    o.hi = 1.0f + p->eps_high;
    o.beta = has_ref ? p->beta : 0.0f;
    o.mode = p->mode;
    return o;
}

// Workgroups for one wave per (sequence, tile) item, or 0 if it does not fit a 1-D launch.
uint32_t item_blocks(int64_t n_seqs, int64_t tiles) {
    const int64_t blocks = ceil_div(n_seqs * tiles, kItemWaves);
    return blocks > 0x7FFFFFFF ? 0 : static_cast<uint32_t>(blocks);
}

// Shape rules of the per-token arrays: n_seqs rows of `width` tokens at stride ld.
logp_status_t check_tokens(int64_t n_seqs, int64_t seq_len, int64_t ld) {
    if (n_seqs < 0 || seq_len < 0 || seq_len > GRPO_MAX_SEQ_LEN || ld < seq_len ||
        n_seqs > 0x7FFFFFFF)
        return LOGP_ERR_SHAPE;
    if (n_seqs > 0 && ld > 0 && n_seqs > (int64_t(1) << 60) / ld) return LOGP_ERR_SHAPE;
    return LOGP_OK;
}

}  // namespace

extern "C" {

logp_status_t grpo_advantages(const float* rewards, int64_t n, int64_t group_size, float eps,
                              int32_t scale_by_std, float* adv, hipStream_t stream) {
    if (n < 0 || group_size < 1 || n % group_size != 0 || n > (int64_t(1) << 40))
        return LOGP_ERR_SHAPE;
    if (!std::isfinite(eps) || eps < 0.0f) return LOGP_ERR_ARG;
    if (n == 0) return LOGP_OK;
    if (rewards == nullptr || adv == nullptr) return LOGP_ERR_NULL;
    const Span in[] = {{rewards, uint64_t(n) * 4}};
    const Span out[] = {{adv, uint64_t(n) * 4}};
    int dev = -1;
    logp_status_t st = check_buffers(in, 1, out, 1, stream, &dev, in[0]);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;
    int64_t groups = n / group_size;
    const int64_t blocks = ceil_div(groups, kItemWaves);
    if (blocks > 0x7FFFFFFF) return LOGP_ERR_SHAPE;
    int sbs = scale_by_std != 0;
    void* args[] = {&rewards, &groups, &group_size, &eps, &sbs, &adv};
    return launch(reinterpret_cast<const void*>(&grpo_adv_kernel),
                  dim3(static_cast<uint32_t>(blocks)), dim3(kItemWaves * kWave), args, 0, stream);
}

logp_status_t grpo_token_counts(const uint8_t* mask, int64_t n_seqs, int64_t seq_len, int64_t ld,
                                int64_t t_begin, int64_t t_end, int32_t* counts,
                                hipStream_t stream) {
    logp_status_t st = check_tokens(n_seqs, seq_len, ld);
    if (st != LOGP_OK) return st;
    if (t_begin < 0 || t_end < t_begin || t_end > seq_len) return LOGP_ERR_SHAPE;
    if (n_seqs == 0) return LOGP_OK;
    if (counts == nullptr) return LOGP_ERR_NULL;
    int width = static_cast<int>(t_end - t_begin);
    const uint8_t* m = mask != nullptr ? mask + t_begin : nullptr;
    const Span in[] = {{m, m != nullptr ? span_bytes(n_seqs, ld, width, 1) : 0}};
    const Span out[] = {{counts, uint64_t(n_seqs) * 4}};
    int dev = -1;
    st = check_buffers(in, 1, out, 1, stream, &dev);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;
    int64_t stride = 1;
    void* args[] = {&m, &ld, &width, &counts, &stride};
    return launch(count_kernel(m, ld), dim3(static_cast<uint32_t>(n_seqs)), dim3(kCountThreads),
                  args, 0, stream);
}

logp_status_t grpo_loss(const float* logp, const float* old_logp, const float* ref_logp,
                        const float* adv, const uint8_t* mask, int64_t n_seqs, int64_t seq_len,
                        int64_t ld, const grpo_params_t* params, grpo_partial_t* seq_stats,
                        grpo_loss_t* loss, float* dlogp, hipStream_t stream) {
    if (loss == nullptr || (n_seqs > 0 && (logp == nullptr || old_logp == nullptr ||
                                            adv == nullptr || seq_stats == nullptr)))
        return LOGP_ERR_NULL;
    logp_status_t st = check_params(params);
    if (st != LOGP_OK) return st;
    st = check_tokens(n_seqs, seq_len, ld);
    if (st != LOGP_OK) return st;
    const uint64_t tok = span_bytes(n_seqs, ld, seq_len, 4);
    const Span in[] = {{logp, tok}, {old_logp, tok}, {ref_logp, ref_logp ? tok : 0},
                       {adv, uint64_t(n_seqs) * 4},
                       {mask, mask ? span_bytes(n_seqs, ld, seq_len, 1) : 0}};
    const Span out[] = {{seq_stats, uint64_t(n_seqs) * sizeof(grpo_partial_t)},
                        {loss, sizeof(grpo_loss_t)}, {dlogp, dlogp ? tok : 0}};
    int dev = -1;
    st = check_buffers(in, 5, out, 3, stream, &dev);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;

    Tokens tk{logp, old_logp, ref_logp, adv, mask, ld, static_cast<int>(seq_len)};
    Objective o = objective(params, ref_logp != nullptr);
    int64_t nt = params->norm_tokens, ns = params->norm_seqs;
    int32_t mode = params->mode;
    float beta = o.beta;
    if (n_seqs > 0) {
        // Launched only as the reduction needs them before the pass: the counts (a mask makes
        // them unknown on the host) for n_i (seq_mean, seq_sum_token_mean) or a local
        // normalizer; the normalizer kernel only for a local normalizer.  token_mean with a
        // given normalizer needs neither: its counts come out of the pass itself.
        const bool local_norm = (mode == GRPO_TOKEN_MEAN && nt <= 0) ||
                                (mode == GRPO_SEQ_MEAN && ns <= 0);
        int counted = mask != nullptr && (mode != GRPO_TOKEN_MEAN || nt <= 0) ? 1 : 0;
        const int64_t* norm_dev = nullptr;
        int64_t norm_host = grpo_norm(mode, nt, ns, n_seqs * seq_len, seq_len > 0 ? n_seqs : 0);
        if (counted) {
            const uint8_t* m = mask;
            int width = static_cast<int>(seq_len);
            int32_t* counts = &seq_stats[0].tokens;
            int64_t stride = sizeof(grpo_partial_t) / sizeof(int32_t);
            void* ca[] = {&m, &ld, &width, &counts, &stride};
            st = launch(count_kernel(m, ld), dim3(static_cast<uint32_t>(n_seqs)),
                        dim3(kCountThreads), ca, 0, stream);
            if (st != LOGP_OK) return st;
            if (local_norm) {
                void* na[] = {&seq_stats, &n_seqs, &mode, &nt, &ns, &loss};
                st = launch(reinterpret_cast<const void*>(&grpo_norm_kernel), dim3(1),
                            dim3(kCountThreads), na, 0, stream);
                if (st != LOGP_OK) return st;
                norm_dev = &loss->norm;
            }
        }
        void* sa[] = {&tk, &o, &counted, &norm_dev, &norm_host, &seq_stats, &dlogp};
        const int64_t tiles = ceil_div(seq_len, kTokTile);
        const size_t lds = static_cast<size_t>(tiles) * sizeof(grpo_partial_t);
        const int waves = static_cast<int>(std::min<int64_t>(kSeqMaxWaves, std::max<int64_t>(1,
                                                                                     tiles)));
        st = launch(reinterpret_cast<const void*>(&grpo_seq_kernel),
                    dim3(static_cast<uint32_t>(n_seqs)), dim3(waves * kWave), sa, lds, stream);
        if (st != LOGP_OK) return st;
    }
    void* ra[] = {&seq_stats, &n_seqs, &mode, &beta, &nt, &ns, &loss};
    return launch(reinterpret_cast<const void*>(&grpo_reduce_kernel), dim3(1),
                  dim3(kCountThreads), ra, 0, stream);
}

logp_status_t grpo_loss_partials(const float* logp, const float* old_logp, const float* ref_logp,
                                 const float* adv, const uint8_t* mask, int64_t n_seqs,
                                 int64_t seq_len, int64_t ld, int64_t t_begin, int64_t t_end,
                                 const int32_t* seq_tokens, const grpo_params_t* params,
                                 grpo_partial_t* partials, int64_t ldp, float* dlogp,
                                 hipStream_t stream) {
    if (n_seqs > 0 && (logp == nullptr || old_logp == nullptr || adv == nullptr ||
                       partials == nullptr))
        return LOGP_ERR_NULL;
    logp_status_t st = check_params(params);
    if (st != LOGP_OK) return st;
    st = check_tokens(n_seqs, seq_len, ld);
    if (st != LOGP_OK) return st;
    if (t_begin < 0 || t_end < t_begin || t_end > seq_len || t_begin % kTokTile != 0 ||
        (t_end % kTokTile != 0 && t_end != seq_len))
        return LOGP_ERR_SHARD;
    const int64_t num_tiles = ceil_div(seq_len, kTokTile);
    const int64_t tile0 = t_begin / kTokTile;
    const int view_tiles = static_cast<int>(ceil_div(t_end - t_begin, kTokTile));
    if (ldp < num_tiles - tile0) return LOGP_ERR_SHAPE;
    // the gradient's normalizers must be declared: no silent local fallback
    const int32_t mode = params->mode;
    if (dlogp != nullptr) {
        if (mode == GRPO_TOKEN_MEAN && params->norm_tokens <= 0) return LOGP_ERR_ARG;
        if (mode == GRPO_SEQ_MEAN && (params->norm_seqs <= 0 || seq_tokens == nullptr))
            return LOGP_ERR_ARG;
        if (mode == GRPO_SEQ_SUM_TOKEN_MEAN && seq_tokens == nullptr) return LOGP_ERR_ARG;
    }
    if (n_seqs == 0 || view_tiles == 0) return LOGP_OK;
    const int64_t width = t_end - t_begin;
    const uint64_t tok = span_bytes(n_seqs, ld, width, 4);
    const Span in[] = {{logp, tok}, {old_logp, tok}, {ref_logp, ref_logp ? tok : 0},
                       {adv, uint64_t(n_seqs) * 4},
                       {mask, mask ? span_bytes(n_seqs, ld, width, 1) : 0},
                       {seq_tokens, seq_tokens ? uint64_t(n_seqs) * 4 : 0}};
    const Span out[] = {{partials, span_bytes(n_seqs, ldp, view_tiles, sizeof(grpo_partial_t))},
                        {dlogp, dlogp ? tok : 0}};
    int dev = -1;
    st = check_buffers(in, 6, out, 2, stream, &dev);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;
    const uint32_t grid = item_blocks(n_seqs, view_tiles);
    if (grid == 0) return LOGP_ERR_SHAPE;
    Tokens tk{logp, old_logp, ref_logp, adv, mask, ld, static_cast<int>(width)};
    Objective o = objective(params, ref_logp != nullptr);
    int64_t D = grpo_norm(mode, params->norm_tokens, params->norm_seqs, 0, 0);
    int vt = view_tiles;
    void* args[] = {&tk, &o, &seq_tokens, &D, &n_seqs, &vt, &partials, &ldp, &dlogp};
    return launch(reinterpret_cast<const void*>(&grpo_partials_kernel), dim3(grid),
                  dim3(kItemWaves * kWave), args, 0, stream);
}

logp_status_t grpo_loss_merge(const grpo_partial_t* partials, int64_t ldp, int64_t n_seqs,
                              int64_t num_tiles, grpo_partial_t* seq_stats, hipStream_t stream) {
    if (n_seqs < 0 || num_tiles < 0 || num_tiles > kMaxTokTiles || ldp < num_tiles ||
        n_seqs > 0x7FFFFFFF)
        return LOGP_ERR_SHAPE;
    if (n_seqs == 0) return LOGP_OK;
    if (partials == nullptr || seq_stats == nullptr) return LOGP_ERR_NULL;
    const Span in[] = {{partials, span_bytes(n_seqs, ldp, num_tiles, sizeof(grpo_partial_t))}};
    const Span out[] = {{seq_stats, uint64_t(n_seqs) * sizeof(grpo_partial_t)}};
    int dev = -1;
    logp_status_t st = check_buffers(in, 1, out, 1, stream, &dev);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;
    const uint32_t grid = static_cast<uint32_t>(ceil_div(n_seqs, kItemWaves));
    void* args[] = {&partials, &ldp, &n_seqs, &num_tiles, &seq_stats};
    return launch(reinterpret_cast<const void*>(&grpo_merge_kernel), dim3(grid),
                  dim3(kItemWaves * kWave), args, 0, stream);
}

logp_status_t grpo_loss_reduce(const grpo_partial_t* seq_stats, int64_t n_seqs,
                               const grpo_params_t* params, grpo_loss_t* loss,
                               hipStream_t stream) {
    if (loss == nullptr || (n_seqs > 0 && seq_stats == nullptr)) return LOGP_ERR_NULL;
    logp_status_t st = check_params(params);
    if (st != LOGP_OK) return st;
    if (n_seqs < 0 || n_seqs > 0x7FFFFFFF) return LOGP_ERR_SHAPE;
    const Span in[] = {{seq_stats, uint64_t(n_seqs) * sizeof(grpo_partial_t)}};
    const Span out[] = {{loss, sizeof(grpo_loss_t)}};
    int dev = -1;
    st = check_buffers(in, 1, out, 1, stream, &dev);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;
    int32_t mode = params->mode;
    float beta = params->beta;
    int64_t nt = params->norm_tokens, ns = params->norm_seqs;
    void* args[] = {&seq_stats, &n_seqs, &mode, &beta, &nt, &ns, &loss};
    return launch(reinterpret_cast<const void*>(&grpo_reduce_kernel), dim3(1),
                  dim3(kCountThreads), args, 0, stream);
}

}  // extern "C"
