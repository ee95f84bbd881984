// Device building blocks shared by every kernel of the selected-token log-probability
// library, for gfx950 (CDNA4, wave64).
//
// This file IS the numerical contract: the tile shape and lane mapping, the per-tile
// (max, sum-exp) reduction, the fixed lane tree, the canonical merge and the exp/log used
// by them.  The fused forward, the shard-partials kernel and the merge kernel all call the
// same functions below, so their results are bitwise identical.
//
// Sources: per-tile (m, s) partials and the merge M = max m_l, S = sum s_l exp(m_l - M),
// LSE = M + log S follow RL-Kernel issue #241 ("[WS2] TP-aware deterministic logprob",
// section "PR 3") and PR #314 ("[WS2][Logp] Deterministic config option", Tensor Parallel
// doc, steps 1-6: fixed global tiles, identical tile shape on any rank, fixed merge order,
// owner-copied target logit).  FP32 arithmetic for max / sum-exp / exp / log follows issue
// #241, section Goal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace logp {

constexpr int kTile = 4096;    // global tile width in columns
constexpr int kWave = 64;      // lanes per wavefront
constexpr int kLoads = 8;      // 16-byte loads per lane per tile
constexpr int kVec = 8;        // BF16 values per 16-byte load
constexpr int kPerLane = kLoads * kVec;  // 64 values per lane per tile
static_assert(kWave * kPerLane == kTile, "a tile is exactly one wave's load footprint");
constexpr int kLoadStride = kWave * kVec;  // 512 columns between a lane's consecutive loads

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.44269504088896340736f;       // 0x3FB8AA3B = fl32(log2 e)
constexpr float kLn2Hi = 0.693147182464599609375f;     // 0x3F317218 = fl32(ln 2)
constexpr float kLn2Lo = -1.9046542e-09f;               // fl32(ln 2 - kLn2Hi)

// ------------------------------------------------------------------ BF16 unpacking

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte load or store

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// The tile held by one wave: v[8*k + e] is column tile_start + 512*k + 8*lane + e.
struct TileRegs {
    float v[kPerLane];
};

__device__ __forceinline__ void unpack8(const u32x4& w, float* out) {
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
    out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z);
    out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
}

constexpr uint32_t kNegInfBits = 0xFF80u;  // BF16 -inf

// Raw BF16 bits of row[c], or -inf when c is at or past `lim` (never touched in memory).
__device__ __forceinline__ uint32_t masked_bits(const uint16_t* __restrict__ row, int c, int lim) {
    return c < lim ? static_cast<uint32_t>(row[c]) : kNegInfBits;
}

// Loads one tile of a row as raw BF16 bits: w[k] holds view columns
// start + 512k + 8*lane + [0, 8).  `lim` is the number of real columns in the view: columns at
// or past it read as -inf and are never touched in memory.  VEC allows 16-byte loads (it needs
// a 16-byte aligned row start and is used for every 8 columns that are all real); otherwise
// each value is a 2-byte load.  Both fill w[] with the same bits.  All loads of the tile are
// issued before any of them is used.
template <bool VEC>
__device__ __forceinline__ void load_tile_bits(const uint16_t* __restrict__ row, int start,
                                               int lim, int lane, u32x4* w) {
    const int base = start + kVec * lane;
    if (VEC && start + kTile <= lim) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + base);
#pragma unroll
        for (int k = 0; k < kLoads; ++k)
            w[k] = __builtin_nontemporal_load(p + k * (kLoadStride / kVec));
        return;
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const int c = base + k * kLoadStride;
        if (VEC && c + kVec <= lim) {
            w[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + c));
        } else {
            w[k].x = masked_bits(row, c + 0, lim) | (masked_bits(row, c + 1, lim) << 16);
            w[k].y = masked_bits(row, c + 2, lim) | (masked_bits(row, c + 3, lim) << 16);
            w[k].z = masked_bits(row, c + 4, lim) | (masked_bits(row, c + 5, lim) << 16);
            w[k].w = masked_bits(row, c + 6, lim) | (masked_bits(row, c + 7, lim) << 16);
        }
    }
}

// The same tile as FP32 values (exact BF16 promotion; masked columns are -inf).
template <bool VEC>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ row, int start, int lim,
                                          int lane, TileRegs& t) {
    u32x4 w[kLoads];
    load_tile_bits<VEC>(row, start, lim, lane, w);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) unpack8(w[k], &t.v[k * kVec]);
}

// ------------------------------------------------------------------ lane tree

// Pairwise tree over lanes 0..63 in index order: partners at xor 1, 2, 4, 8, 16, 32.
// After each step both partners hold the same value (max and + are commutative), so every
// lane ends with identical bits.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v = v + __shfl_xor(v, o, kWave);
    return v;
}

// ------------------------------------------------------------------ exp / log

// exp(t) for the forward's sum-exp terms and merge weights: 2^(fl(t * log2 e)) on the
// hardware exp2.  t <= 0 always; exp(-inf) = 0.
__device__ __forceinline__ float fwd_exp(float t) { return __builtin_amdgcn_exp2f(t * kLog2e); }

// Natural log used by the merge (accurate library logf).
__device__ __forceinline__ float canon_log(float s) { return logf(s); }

// exp(t) for the backward's softmax, returned as (2^u, delta) with exp(t) ~= 2^u (1 + delta):
// u = fl(t * log2 e) and delta = t - u ln 2, formed with two FMAs (the first one is exact up
// to a rounding far below 2^-24 of delta, since t - u*hi(ln 2) needs about 24 bits).  |delta|
// stays below |t| 2^-24, so the dropped delta^2/2 term is under 2^-40 relative: the result
// is within about one FP32 ulp of exp(t), where exp2(fl(t * log2 e)) alone is off by up to
// |t| 2^-24 relative (tens of ulps near t = -40).
struct ExpSplit {
    float u, delta;
};

__device__ __forceinline__ ExpSplit bwd_exp_split(float t) {
    ExpSplit r;
    r.u = t * kLog2e;
    const float d_hi = __builtin_fmaf(-r.u, kLn2Hi, t);
    r.delta = __builtin_fmaf(-r.u, kLn2Lo, d_hi);
    return r;
}

// -g/S * exp(x - M) for a tile in which every x - M >= -87 (so every exp is a normal float and
// the single product rounds correctly even when it lands in the subnormal range).
__device__ __forceinline__ float bwd_term(float x, float M, float neg_c) {
    const ExpSplit s = bwd_exp_split(x - M);
    const float e0 = __builtin_amdgcn_exp2f(s.u);
    return __builtin_fmaf(e0, s.delta, e0) * neg_c;
}

// Same value for any x - M (including -inf).  Where 2^u would be subnormal (u < -126), where
// the hardware exp2 returns zero, it is computed as 2^(u+64) (u + 64 is exact there) and
// multiplied by neg_c_lo = neg_c * 2^-64, which rounds the product exactly as neg_c * e would.
// For u >= -126 it performs the same operations as bwd_term, so both give identical bits.
__device__ __forceinline__ float bwd_term_deep(float x, float M, float neg_c, float neg_c_lo) {
    const ExpSplit s = bwd_exp_split(fmaxf(x - M, -150.0f));
    const bool tiny = s.u < -126.0f;
    const float e0 = __builtin_amdgcn_exp2f(tiny ? s.u + 64.0f : s.u);
    return __builtin_fmaf(e0, s.delta, e0) * (tiny ? neg_c_lo : neg_c);
}

// ------------------------------------------------------------------ tile statistics

// (m, s) of one tile held in registers: m = max over the tile (exact), s = sum of
// exp(x - m) with each lane adding its 64 values in index order from +0, then the lane tree.
// A tile with no real column gives the (-inf, 0) identity.
__device__ __forceinline__ void tile_stats(const TileRegs& t, float& m, float& s) {
    float lm = t.v[0];
#pragma unroll
    for (int i = 1; i < kPerLane; ++i) lm = fmaxf(lm, t.v[i]);
    m = wave_max(lm);
    float ls = 0.0f;
    if (m != kNegInf) {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) ls = ls + fwd_exp(t.v[i] - m);
    }
    s = wave_sum(ls);
}

// ------------------------------------------------------------------ canonical merge

// Merge of per-tile (m_l, s_l), l in [0, L), read through `src.m(l)` / `src.s(l)` by one
// wave: M = max m_l; w_l = 0 for an identity tile (m_l = -inf), else s_l * exp(m_l - M);
// lane i adds w_i, w_{i+64}, ... in order from +0; the lane tree gives S.  Trailing
// identity tiles add +0 to a lane's running sum and leave M unchanged, so S and M do not
// depend on how many of them there are.
template <class Src>
__device__ __forceinline__ void canonical_merge(const Src& src, int L, int lane, float& M,
                                                float& S) {
    float lm = kNegInf;
    for (int l = lane; l < L; l += kWave) lm = fmaxf(lm, src.m(l));
    M = wave_max(lm);
    float ls = 0.0f;
    if (M != kNegInf) {
        for (int l = lane; l < L; l += kWave) {
            const float ml = src.m(l);
            const float w = (ml == kNegInf) ? 0.0f : src.s(l) * fwd_exp(ml - M);
            ls = ls + w;
        }
    }
    S = wave_sum(ls);
}

struct RowResult {
    float logp, lse, max, sumexp;
};

// LSE = M + log S; logp = (sel - M) - log S for a valid row, 0 for an invalid one.
// M = -inf (no finite real logit) gives LSE = -inf and logp = -inf for a valid row.
__device__ __forceinline__ RowResult finalize_row(float M, float S, bool valid, float sel) {
    RowResult r;
    r.max = M;
    r.sumexp = S;
    if (M == kNegInf) {
        r.lse = kNegInf;
        r.logp = valid ? kNegInf : 0.0f;
    } else {
        const float log_s = canon_log(S);
        r.lse = M + log_s;
        r.logp = valid ? (sel - M) - log_s : 0.0f;
    }
    return r;
}

// Row validity: active (or no mask), target != ignore_index and 0 <= target < vocab_real.
__device__ __forceinline__ bool row_valid(const int64_t* __restrict__ targets,
                                          const uint8_t* __restrict__ active,
                                          int64_t ignore_index, int64_t vocab_real, int64_t row,
                                          int64_t& y) {
    y = targets[row];
    if (active != nullptr && active[row] == 0) return false;
    if (y == ignore_index) return false;
    return y >= 0 && y < vocab_real;
}

}  // namespace logp
