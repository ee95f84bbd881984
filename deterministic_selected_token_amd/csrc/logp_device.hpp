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

// ------------------------------------------------------------------ logits dtypes

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte load or store
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Logits (and dlogits) element types: BF16, FP16, FP32 (values match logp_dtype_t).
enum class Dt : int { BF16 = 0, F16 = 1, F32 = 2 };

template <Dt D>
struct DtInfo;
template <>
struct DtInfo<Dt::BF16> {
    using Storage = uint16_t;
    static constexpr uint32_t kNegInfBits = 0xFF80u;
};
template <>
struct DtInfo<Dt::F16> {
    using Storage = uint16_t;
    static constexpr uint32_t kNegInfBits = 0xFC00u;
};
template <>
struct DtInfo<Dt::F32> {
    using Storage = uint32_t;  // raw FP32 bits
    static constexpr uint32_t kNegInfBits = 0xFF800000u;
};

// Eight consecutive logits as raw bits: one 16-byte vector for 2-byte types, two for FP32.
template <Dt D>
struct Raw8 {
    u32x4 w;
};
template <>
struct Raw8<Dt::F32> {
    u32x4 w, w2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Exact widening of one element's raw bits to FP32.
template <Dt D>
__device__ __forceinline__ float elem_to_f32(uint32_t bits) {
    if constexpr (D == Dt::BF16) {
        return __uint_as_float(bits << 16);
    } else if constexpr (D == Dt::F16) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
    } else {
        return __uint_as_float(bits);
    }
}

// The 8 values of a Raw8 as FP32 (exact).
template <Dt D>
__device__ __forceinline__ void unpack8(const Raw8<D>& r, float* out) {
    if constexpr (D == Dt::BF16) {
        out[0] = bf16_lo(r.w.x); out[1] = bf16_hi(r.w.x);
        out[2] = bf16_lo(r.w.y); out[3] = bf16_hi(r.w.y);
        out[4] = bf16_lo(r.w.z); out[5] = bf16_hi(r.w.z);
        out[6] = bf16_lo(r.w.w); out[7] = bf16_hi(r.w.w);
    } else if constexpr (D == Dt::F16) {
        const uint32_t q[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2 h = __builtin_bit_cast(f16x2, q[i]);
            out[2 * i] = static_cast<float>(h.x);
            out[2 * i + 1] = static_cast<float>(h.y);
        }
    } else {
        out[0] = __uint_as_float(r.w.x); out[1] = __uint_as_float(r.w.y);
        out[2] = __uint_as_float(r.w.z); out[3] = __uint_as_float(r.w.w);
        out[4] = __uint_as_float(r.w2.x); out[5] = __uint_as_float(r.w2.y);
        out[6] = __uint_as_float(r.w2.z); out[7] = __uint_as_float(r.w2.w);
    }
}

// Scored logit: x, or fl32(x * inv_t) for temperature-scaled scoring.  x * 1 = x exactly, so
// the unscaled instantiations compute the same bits as a scaled call with inv_t = 1.
template <bool SCALED>
__device__ __forceinline__ float scored(float x, float inv_t) {
    return SCALED ? x * inv_t : x;
}

// The tile held by one wave: v[8*k + e] is column tile_start + 512*k + 8*lane + e.
struct TileRegs {
    float v[kPerLane];
};

// Raw bits of row[c], or -inf when c is at or past `lim` (never touched in memory).
template <Dt D>
__device__ __forceinline__ uint32_t masked_bits(const typename DtInfo<D>::Storage* __restrict__ row,
                                                int c, int lim) {
    return c < lim ? static_cast<uint32_t>(row[c]) : DtInfo<D>::kNegInfBits;
}

// The 8 values at view columns [c, c+8) of a row (c a multiple of 8).  Columns at or past
// `lim` (the number of real columns in the view) read as -inf and are never touched in
// memory.  VEC allows 16-byte loads when all 8 are real (it needs 16-byte aligned rows);
// otherwise each value is an element load.  Both fill r identically.
template <Dt D, bool VEC>
__device__ __forceinline__ void load8(const typename DtInfo<D>::Storage* __restrict__ row, int c,
                                      int lim, Raw8<D>& r) {
    if (VEC && c + kVec <= lim) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + c);
        r.w = __builtin_nontemporal_load(p);
        if constexpr (D == Dt::F32) r.w2 = __builtin_nontemporal_load(p + 1);
        return;
    }
    if constexpr (D == Dt::F32) {
        r.w.x = masked_bits<D>(row, c + 0, lim); r.w.y = masked_bits<D>(row, c + 1, lim);
        r.w.z = masked_bits<D>(row, c + 2, lim); r.w.w = masked_bits<D>(row, c + 3, lim);
        r.w2.x = masked_bits<D>(row, c + 4, lim); r.w2.y = masked_bits<D>(row, c + 5, lim);
        r.w2.z = masked_bits<D>(row, c + 6, lim); r.w2.w = masked_bits<D>(row, c + 7, lim);
    } else {
        r.w.x = masked_bits<D>(row, c + 0, lim) | (masked_bits<D>(row, c + 1, lim) << 16);
        r.w.y = masked_bits<D>(row, c + 2, lim) | (masked_bits<D>(row, c + 3, lim) << 16);
        r.w.z = masked_bits<D>(row, c + 4, lim) | (masked_bits<D>(row, c + 5, lim) << 16);
        r.w.w = masked_bits<D>(row, c + 6, lim) | (masked_bits<D>(row, c + 7, lim) << 16);
    }
}

// One tile of a row as raw bits: r[k] holds view columns start + 512k + 8*lane + [0, 8);
// `start` is the tile's first view column.  All loads of the tile are issued before any of
// them is used.
template <Dt D, bool VEC>
__device__ __forceinline__ void load_tile_raw(const typename DtInfo<D>::Storage* __restrict__ row,
                                              int start, int lim, int lane, Raw8<D>* r) {
    const int base = start + kVec * lane;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) load8<D, VEC>(row, base + k * kLoadStride, lim, r[k]);
}

// The same tile as FP32 values (exact widening; masked columns are -inf).  Scoring with a
// temperature is applied later, in tile_stats.
template <Dt D, bool VEC>
__device__ __forceinline__ void load_tile(const typename DtInfo<D>::Storage* __restrict__ row,
                                          int start, int lim, int lane, TileRegs& t) {
    Raw8<D> r[kLoads];
    load_tile_raw<D, VEC>(row, start, lim, lane, r);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) unpack8<D>(r[k], &t.v[k * kVec]);
}

// A 16-byte streaming store of the gradient: non-temporal at device scope (`sc1 nt`).  The
// gradient is written once and not read again by this kernel; with the device-scope bit its
// lines leave L2 for memory as they are written.  Plain copies of 4 GiB move 6.25 TB/s with
// it against 6.11 with the non-temporal bit alone (16 KiB per wave), and the headline
// backward runs 2.4% faster; the stored bits are the same.  A store of more than 8 bytes
// reads its data registers after it issues, and on this family a VALU write to them needs 2
// wait states first: the compiler keeps that distance for the stores it emits but does not
// look inside an asm statement, so the `s_nop 1` (2 wait states) is part of it.  The clobber
// keeps the compiler from moving other memory accesses across it (an in-place backward reads
// each element before this store overwrites it).
__device__ __forceinline__ void store_stream16(u32x4* p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" : : "v"(p), "v"(v)
                 : "memory");
}

// Round 8 gradients to the output dtype (nearest, ties to even) and store them at view
// columns [c, c+8) of an output row: 16-byte stores when VEC and all 8 lie inside `width`,
// element stores for the columns below `width` otherwise.
template <Dt D, bool VEC>
__device__ __forceinline__ void store8(typename DtInfo<D>::Storage* out, int c, int width,
                                       const float* d) {
    uint32_t q[8];
    if constexpr (D == Dt::F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = __float_as_uint(d[e]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (D == Dt::BF16) {
                bf16x2 v;
                v.x = static_cast<__bf16>(d[2 * i]);
                v.y = static_cast<__bf16>(d[2 * i + 1]);
                q[i] = __builtin_bit_cast(uint32_t, v);
            } else {
                f16x2 v;
                v.x = static_cast<_Float16>(d[2 * i]);
                v.y = static_cast<_Float16>(d[2 * i + 1]);
                q[i] = __builtin_bit_cast(uint32_t, v);
            }
        }
    }
    if (VEC && c + kVec <= width) {
        u32x4* p = reinterpret_cast<u32x4*>(out + c);
        store_stream16(p, u32x4{q[0], q[1], q[2], q[3]});
        if constexpr (D == Dt::F32) store_stream16(p + 1, u32x4{q[4], q[5], q[6], q[7]});
        return;
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        if (c + e >= width) continue;
        if constexpr (D == Dt::F32)
            out[c + e] = q[e];
        else
            out[c + e] = static_cast<uint16_t>(e & 1 ? q[e / 2] >> 16 : q[e / 2] & 0xFFFFu);
    }
}

// ------------------------------------------------------------------ lane tree

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}
__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }


// Pairwise tree over lanes 0..63 in index order: level k combines the aligned groups of
// 2^k lanes pairwise (the xor-1, 2, 4, 8, 16, 32 butterfly).  After each level every lane of
// a group holds the group's value (max and + are commutative, so both partners compute the
// same bits), which lets a lane take its partner value from ANY lane of the sibling group:
// DPP quad permutes for levels 1-2, the half-row and row mirrors for levels 3-4, and gfx950's
// permlane16 / permlane32 swaps (which hand every lane the even and odd row of its 32-lane
// half, then the low and high half of the wave) for levels 5-6.  Every lane ends with the
// xor butterfly's bits, without a round trip through the LDS crossbar per level.  Callers run
// it in wave-uniform control flow, all 64 lanes active: the permutes read every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_lanes(float v) {
    return __uint_as_float(
        __builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}

template <typename Op>
__device__ __forceinline__ float wave_tree(float v, Op op) {
    v = op(v, dpp_lanes<0xB1>(v));   // quad_perm [1,0,3,2]: the other lane of the pair
    v = op(v, dpp_lanes<0x4E>(v));   // quad_perm [2,3,0,1]: the other pair of the quad
    v = op(v, dpp_lanes<0x141>(v));  // row_half_mirror: the other quad of the 8
    v = op(v, dpp_lanes<0x140>(v));  // row_mirror: the other 8 of the 16-lane row
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));  // even row, odd row of the 32
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return op(__uint_as_float(h[0]), __uint_as_float(h[1]));  // low half, high half
}

__device__ __forceinline__ float wave_max(float v) {
    return wave_tree(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ float wave_sum(float v) {
    return wave_tree(v, [](float a, float b) { return a + b; });
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

// Rounding error of s = fl(a + b): a + b = s + err exactly (Knuth's two-sum, 6 operations).
__device__ __forceinline__ float two_sum_err(float a, float b, float s) {
    const float bb = s - a;
    return (a - (s - bb)) + (b - bb);
}

// Rounding error of t = fl(z - M) when |z| <= M (Dekker's fast two-sum with the larger
// operand -M first, 2 operations): z - M = t + err exactly.
__device__ __forceinline__ float fast_two_sum_err(float z, float M, float t) {
    return z - (t + M);
}

// -g/S * exp(z - M) for a tile in which every z - M >= -87 (so every exp is a normal float and
// the single product rounds correctly even when it lands in the subnormal range).  When z - M
// is not exact in FP32 (FP32 logits, or scored ones z = fl32(x * inv_t)), TWO_SUM adds its
// rounding error to delta, so the result is exp of the exact difference; such tiles take
// this path only when also |z| <= M, which the fast two-sum needs.
template <bool TWO_SUM>
__device__ __forceinline__ float bwd_term(float z, float M, float neg_c) {
    const float t = z - M;
    ExpSplit s = bwd_exp_split(t);
    if (TWO_SUM) s.delta = s.delta + fast_two_sum_err(z, M, t);
    const float e0 = __builtin_amdgcn_exp2f(s.u);
    return __builtin_fmaf(e0, s.delta, e0) * neg_c;
}

// Same value for any z and M (z - M down to -inf), with the general two-sum.  Where 2^u
// would be subnormal (u < -126), where the hardware exp2 returns zero, it is computed as
// 2^(u+64) (u + 64 is exact there) and multiplied by neg_c_lo = neg_c * 2^-64, which rounds
// the product exactly as neg_c * e would.  For u >= -126 it performs the same operations as
// bwd_term (both two-sums give the exact error where the fast one applies), so both give
// identical bits.
template <bool TWO_SUM>
__device__ __forceinline__ float bwd_term_deep(float z, float M, float neg_c, float neg_c_lo) {
    const float t = z - M;
    const bool finite = t > -150.0f;  // exp(t) underflows to 0 below; -inf lands here too
    ExpSplit s = bwd_exp_split(finite ? t : -150.0f);
    if (TWO_SUM) s.delta = s.delta + (finite ? two_sum_err(z, -M, t) : 0.0f);
    const bool tiny = s.u < -126.0f;
    const float e0 = __builtin_amdgcn_exp2f(tiny ? s.u + 64.0f : s.u);
    return __builtin_fmaf(e0, s.delta, e0) * (tiny ? neg_c_lo : neg_c);
}

// ------------------------------------------------------------------ tile statistics

// (m, s) of one tile of scored logits z = scored(x) held in registers as x: m = max z (exact),
// s = sum of exp(z - m) with each lane adding its 64 values in index order from +0, then the
// lane tree.  Rounding x * inv_t is monotone for inv_t > 0, so max z = scored(max x) exactly
// and the max pass runs on x; z is formed once per value in the sum pass.  A tile with no
// real column gives the (-inf, 0) identity.
template <bool SCALED>
__device__ __forceinline__ void tile_stats(const TileRegs& t, float inv_t, float& m, float& s) {
    float lm = t.v[0];
#pragma unroll
    for (int i = 1; i < kPerLane; ++i) lm = fmaxf(lm, t.v[i]);
    m = scored<SCALED>(wave_max(lm), inv_t);
    float ls = 0.0f;
    if (m != kNegInf) {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) ls = ls + fwd_exp(scored<SCALED>(t.v[i], inv_t) - m);
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
