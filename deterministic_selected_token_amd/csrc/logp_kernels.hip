// gfx950 kernels and the C ABI of the selected-token log-probability library.
//
//   forward   one workgroup per row; its waves take the row's global tiles round-robin,
//             reduce each in registers to (m_l, s_l), park them in LDS, and wave 0 runs
//             the canonical merge (RL-Kernel issue #241, "PR 3"; PR #314 Tensor Parallel
//             doc, steps 1-6).  One HBM pass over the logits, nothing else written but
//             logp / LSE / (M, S).
//   backward  dlogits = g (onehot - exp(x - M) / S) rounded to the logits' dtype straight
//             from registers (PR #495 "zero-workspace backward for generic CUDA fused
//             logp", Summary item 2: no FP32 [N, V] workspace; one read of the logits instead
//             of the three its kernel needs, Results section).  Element-wise, so its work
//             split is free: a flat walk over 16-byte vectors for aligned views, (row, tile)
//             items otherwise.
//   partials  one wave per (row, tile of the shard): the forward's tile reduction, written
//             out as (m_l, s_l, sel_l) (issue #241, "PR6").
//   merge     one wave per row over [L] partials: the forward's merge code.
//
// Every kernel is instantiated for BF16, FP16 and FP32 logits (PR #495, Tests: FP32 / BF16 /
// FP16) and for temperature-scaled scoring, z = fl32(x * inv_temperature) (the rollout
// temperatures of the provider experiment in PR #495's author reply); the unscaled
// instantiations compute exactly what a scaled one computes with inv_temperature = 1.
//
// Host entry points validate every argument before launching and report failures as
// status codes (see include/logp.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "host_common.hpp"
#include "logp.h"
#include "logp_device.hpp"

using namespace logp;
using namespace logp_host;

namespace {

constexpr int kFwdWaves = 4;         // waves per forward workgroup (one row)
constexpr int kItemWaves = 4;        // waves per workgroup of the partials kernel
constexpr int kBwdWaves = 16;        // waves per backward workgroup
constexpr int kBwdTilesPerWave = 2;  // consecutive (row, tile) items per tile-path wave
// FP32 tiles take twice the registers: one item per wave and 512-thread workgroups keep them
// clear of the register cap that 1024-thread workgroups impose (128 per lane).
template <Dt D>
constexpr int bwd_tiles_per_wave() { return D == Dt::F32 ? 1 : kBwdTilesPerWave; }
template <Dt D>
constexpr int bwd_tile_waves() { return D == Dt::F32 ? 8 : kBwdWaves; }
constexpr int kMergeWaves = 4;       // rows per merge workgroup
constexpr int kCheckThreads = 1024;
// Largest padded width: keeps vocab_padded + kTile below 2^31 so in-row column arithmetic
// never overflows a 32-bit int.
constexpr int64_t kMaxCols = (int64_t(1) << 31) - 1 - kTile;

struct LdsTiles {
    const float2* p;
    __device__ float m(int l) const { return p[l].x; }
    __device__ float s(int l) const { return p[l].y; }
};

struct GlobalTiles {
    const logp_partial_t* p;
    __device__ float m(int l) const { return p[l].max; }
    __device__ float s(int l) const { return p[l].sumexp; }
};

__device__ __forceinline__ void write_row(const RowResult& r, int64_t row, float* logp, float* lse,
                                          logp_stats_t* stats) {
    logp[row] = r.logp;
    if (lse != nullptr) lse[row] = r.lse;
    if (stats != nullptr) {
        stats[row].max = r.max;
        stats[row].sumexp = r.sumexp;
    }
}

// ---------------------------------------------------------------------------- forward

template <Dt D, bool VEC, bool SCALED>
__global__ __launch_bounds__(kFwdWaves* kWave) void fwd_kernel(
    const typename DtInfo<D>::Storage* __restrict__ logits, int64_t ld, int vocab_real,
    float inv_t, const int64_t* __restrict__ targets, const uint8_t* __restrict__ active,
    int64_t ignore_index, float* __restrict__ logp, float* __restrict__ lse,
    logp_stats_t* __restrict__ stats) {
    extern __shared__ float2 slots[];  // (m_l, s_l) per real tile
    const int64_t row = blockIdx.x;
    const int wave = wave_id();
    const int lane = lane_id();
    const typename DtInfo<D>::Storage* __restrict__ x = logits + row * ld;
    const int real_tiles = (vocab_real + kTile - 1) / kTile;

    // Wave 0 fetches the target and its logit first so the gather overlaps the streaming.
    int64_t y = 0;
    bool valid = false;
    float sel = 0.0f;
    if (wave == 0) {
        valid = row_valid(targets, active, ignore_index, vocab_real, row, y);
        if (valid) sel = scored<SCALED>(elem_to_f32<D>(x[y]), inv_t);
    }

    for (int l = wave; l < real_tiles; l += kFwdWaves) {
        TileRegs t;
        load_tile<D, VEC>(x, l * kTile, vocab_real, lane, t);
        float m, s;
        tile_stats<SCALED>(t, inv_t, m, s);
        if (lane == 0) slots[l] = make_float2(m, s);
    }
    __syncthreads();
    if (wave == 0) {
        // Tiles past the last real column are identity partials: merging only the real ones
        // gives the same bits as merging the whole padded row.
        float M, S;
        canonical_merge(LdsTiles{slots}, real_tiles, lane, M, S);
        if (lane == 0) write_row(finalize_row(M, S, valid, sel), row, logp, lse, stats);
    }
}

// --------------------------------------------------------------------------- partials

template <Dt D, bool VEC, bool SCALED>
__global__ __launch_bounds__(kItemWaves* kWave) void partials_kernel(
    const typename DtInfo<D>::Storage* __restrict__ logits, int64_t ld, int64_t n,
    int view_tiles, int lim, int64_t col_begin, int64_t col_end, int64_t vocab_real, float inv_t,
    const int64_t* __restrict__ targets, const uint8_t* __restrict__ active, int64_t ignore_index,
    logp_partial_t* __restrict__ partials, int64_t ldp) {
    const int64_t item = int64_t(blockIdx.x) * kItemWaves + wave_id();
    if (item >= n * view_tiles) return;  // whole wave leaves; this kernel has no barrier
    const int lane = lane_id();
    const int64_t row = item / view_tiles;
    const int j = static_cast<int>(item - row * view_tiles);
    const int start = j * kTile;
    const typename DtInfo<D>::Storage* __restrict__ x = logits + row * ld;

    TileRegs t;
    load_tile<D, VEC>(x, start, lim, lane, t);
    float m, s;
    tile_stats<SCALED>(t, inv_t, m, s);
    if (lane == 0) {
        int64_t y;
        const bool valid = row_valid(targets, active, ignore_index, vocab_real, row, y);
        const int64_t g0 = col_begin + start;  // global column of this tile's first entry
        float sel = 0.0f;
        if (valid && y >= g0 && y < g0 + kTile && y < col_end)
            sel = scored<SCALED>(elem_to_f32<D>(x[y - col_begin]), inv_t);
        logp_partial_t* out = partials + row * ldp + j;
        out->max = m;
        out->sumexp = s;
        out->sel = sel;
    }
}

// ------------------------------------------------------------------------------ merge

__global__ __launch_bounds__(kMergeWaves* kWave) void merge_kernel(
    const logp_partial_t* __restrict__ partials, int64_t ldp, int64_t n, int num_tiles,
    int64_t vocab_real, const int64_t* __restrict__ targets, const uint8_t* __restrict__ active,
    int64_t ignore_index, float* __restrict__ logp, float* __restrict__ lse,
    logp_stats_t* __restrict__ stats) {
    const int64_t row = int64_t(blockIdx.x) * kMergeWaves + wave_id();
    if (row >= n) return;
    const int lane = lane_id();
    const logp_partial_t* __restrict__ p = partials + row * ldp;
    float M, S;
    canonical_merge(GlobalTiles{p}, num_tiles, lane, M, S);
    if (lane == 0) {
        int64_t y;
        const bool valid = row_valid(targets, active, ignore_index, vocab_real, row, y);
        const float sel = valid ? p[y / kTile].sel : 0.0f;  // copied from the owner tile
        write_row(finalize_row(M, S, valid, sel), row, logp, lse, stats);
    }
}

// --------------------------------------------------------------------------- backward

// Per-row constants of the backward.
// For unscaled BF16 / FP16 values, z - M is exact in FP32 whenever z = 0 or |z| and |M| lie
// within a factor of about 2^15 (BF16) or 2^12 (FP16) of each other: the exact difference
// then needs at most 24 significant bits.  Outside that (a logit very close to zero in a
// row whose max is far from zero, or far below a small max) the FP32 difference t carries
// up to half an FP32 spacing of t, so exp(t) is off by at most 2^-24 |t| relative (about
// 8 FP32 ulps at |t| = 30): far below the 2^-9 spacing of the BF16 result, though it can
// move a value that lies within that distance of a rounding boundary.  FP32 and scored
// logits carry the rounding error of t into the exponential instead.
template <Dt D, bool SCALED>
__host__ __device__ constexpr bool bwd_two_sum() {
    return SCALED || D == Dt::F32;
}

struct BwdRow {
    bool valid;  // row valid and its stats finite
    float M, g, neg_c, neg_c_lo;  // g is the scored upstream gradient g * inv_t
    int64_t y;   // target in view coordinates
    float thr;   // raw logits below this need the general path (see below)
};

// The stats and g loads do not wait for the validity test (they are in bounds for every
// row), so one memory round trip resolves all of them.
template <Dt D, bool SCALED>
__device__ __forceinline__ BwdRow bwd_row(int64_t row, int64_t col_begin, int64_t vocab_real,
                                          float inv_t, const int64_t* __restrict__ targets,
                                          const uint8_t* __restrict__ active,
                                          int64_t ignore_index, const float* __restrict__ grad,
                                          const logp_stats_t* __restrict__ stats) {
    BwdRow r;
    const float M = stats[row].max, S = stats[row].sumexp;
    int64_t y;
    r.valid = row_valid(targets, active, ignore_index, vocab_real, row, y) && M != kNegInf;
    r.M = M;
    r.g = SCALED ? grad[row] * inv_t : grad[row];  // d z / d x = inv_t
    r.neg_c = -(r.g / S);                          // -g/S, one rounding per row
    r.neg_c_lo = r.neg_c * 0x1p-64f;               // exact unless |g/S| < 2^-62
    r.y = y - col_begin;
    // exp(z - M) may leave the normal range only where z - M < -87, i.e. for raw logits
    // below (M - 87) / inv_t; the margin of one unit absorbs the roundings of z and of this
    // quotient.  False alarms only select the slower path, which gives the same bits.
    r.thr = SCALED ? (M - 86.0f) / inv_t : M - 87.0f;
    if (bwd_two_sum<D, SCALED>()) {
        // The fast two-sum of z - M needs |z| <= M: M >= 0 and z >= -M, which holds for raw
        // logits at or above -(M / inv_t) (1 - 2^-20); the factor covers the roundings of
        // the quotient and of z.  M < 0 sends every tile of the row to the general path.
        const float far = M >= 0.0f ? -(SCALED ? M / inv_t : M) * (1.0f - 0x1p-20f)
                                    : __builtin_inff();
        r.thr = fmaxf(r.thr, far);
    }
    return r;
}

// True when some value of the raw tile words may lie below `thr` (a per-lane threshold).
// Works on raw bits: for a negative threshold, a value below it has larger unsigned
// magnitude bits than the threshold rounded toward zero (RTZ keeps the test conservative).
template <Dt D>
__device__ __forceinline__ bool below_threshold(const Raw8<D>& r, float thr) {
    if (!(thr < 0.0f)) return true;  // non-negative (or NaN) threshold: always the safe path
    if constexpr (D == Dt::F32) {
        const uint32_t t = __float_as_uint(thr);
        const uint32_t m = std::max(std::max(std::max(r.w.x, r.w.y), std::max(r.w.z, r.w.w)),
                                    std::max(std::max(r.w2.x, r.w2.y), std::max(r.w2.z, r.w2.w)));
        return m > t;
    } else {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        unsigned t16;
        if constexpr (D == Dt::BF16) {
            t16 = __float_as_uint(thr) >> 16;  // truncation = rounding toward zero
        } else {
            typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
            const fp16x2 h = __builtin_amdgcn_cvt_pkrtz(thr, thr);  // round toward zero
            t16 = __builtin_bit_cast(uint32_t, h) & 0xFFFFu;
        }
        // The words are copied to plain scalars before the casts: hipcc's front end turns
        // __builtin_bit_cast of a vector component (r.w.y) into a load from the vector's
        // first component, which made this test look at 2 of the 8 values.
        const uint32_t q[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
        u16x2 mx = __builtin_elementwise_max(__builtin_bit_cast(u16x2, q[0]),
                                             __builtin_bit_cast(u16x2, q[1]));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, q[2]));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, q[3]));
        return mx.x > t16 || mx.y > t16;
    }
}

// Gradient of the 8 columns at view column c from their scored logits v[0..7].
template <bool DEEP, bool TWO_SUM>
__device__ __forceinline__ void bwd_vec(const BwdRow& r, const float* v, int c, int lim,
                                        float* d) {
#pragma unroll
    for (int e = 0; e < kVec; ++e)
        d[e] = DEEP ? bwd_term_deep<TWO_SUM>(v[e], r.M, r.neg_c, r.neg_c_lo)
                    : bwd_term<TWO_SUM>(v[e], r.M, r.neg_c);
    const int64_t yo = r.y - c;  // the target's offset from c
    if (yo >= 0 && yo < kVec) {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (e == yo) d[e] = r.g + d[e];  // g * (1 - p)
    }
    if (c + kVec > lim) {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (c + e >= lim) d[e] = 0.0f;  // padding and past-the-vocab columns
    }
}

template <Dt D, bool SCALED>
__device__ __forceinline__ void bwd_compute_store(const BwdRow& r, const Raw8<D>& raw, bool deep,
                                                  float inv_t, int c, int lim, float* d) {
    constexpr bool kTwoSum = bwd_two_sum<D, SCALED>();
    float v[kVec];
    unpack8<D>(raw, v);
#pragma unroll
    for (int e = 0; e < kVec; ++e) v[e] = scored<SCALED>(v[e], inv_t);
    if (!deep) bwd_vec<false, kTwoSum>(r, v, c, lim, d);
    else bwd_vec<true, kTwoSum>(r, v, c, lim, d);
}

// (row, tile) items: any alignment, any width.  Each wave owns kBwdTilesPerWave consecutive
// items and issues all their loads before computing any of them.
template <Dt D, bool VEC_IN, bool VEC_OUT, bool SCALED>
__global__ __launch_bounds__(bwd_tile_waves<D>() * kWave) void bwd_kernel(
    const typename DtInfo<D>::Storage* logits, int64_t ld, int64_t n, int view_tiles, int width,
    int lim, int64_t col_begin, int64_t vocab_real, float inv_t,
    const int64_t* __restrict__ targets, const uint8_t* __restrict__ active, int64_t ignore_index,
    const float* __restrict__ grad, const logp_stats_t* __restrict__ stats,
    typename DtInfo<D>::Storage* dlogits, int64_t ld_out) {
    // logits and dlogits may be the same buffer: every element is loaded into registers
    // before the lane that loaded it stores to it, and no other lane touches it.
    constexpr int TPW = bwd_tiles_per_wave<D>();
    const int64_t first = (int64_t(blockIdx.x) * bwd_tile_waves<D>() + wave_id()) * TPW;
    const int64_t total = n * view_tiles;
    if (first >= total) return;  // whole wave leaves; this kernel has no barrier
    const int lane = lane_id();

    int64_t row[TPW];
    int start[TPW];
    BwdRow r[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        if (first + i >= total) break;
        row[i] = (first + i) / view_tiles;
        start[i] = static_cast<int>(first + i - row[i] * view_tiles) * kTile;
        r[i] = bwd_row<D, SCALED>(row[i], col_begin, vocab_real, inv_t, targets, active,
                                  ignore_index, grad, stats);
    }
    Raw8<D> w[TPW][kLoads];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
        if (first + i < total && r[i].valid)  // invalid rows are not read
            load_tile_raw<D, VEC_IN>(logits + row[i] * ld, start[i], lim, lane, w[i]);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        if (first + i >= total) break;
        typename DtInfo<D>::Storage* out = dlogits + row[i] * ld_out;
        const int base = start[i] + kVec * lane;
        if (!r[i].valid) {
            float z[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) z[e] = 0.0f;
#pragma unroll
            for (int k = 0; k < kLoads; ++k)
                store8<D, VEC_OUT>(out, base + k * kLoadStride, width, z);
            continue;
        }
        bool hit = false;
#pragma unroll
        for (int k = 0; k < kLoads; ++k) hit = hit || below_threshold<D>(w[i][k], r[i].thr);
        const bool deep = __any(hit);  // masked columns (-inf) always count
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            float d[kVec];
            const int c = base + k * kLoadStride;
            bwd_compute_store<D, SCALED>(r[i], w[i][k], deep, inv_t, c, lim, d);
            store8<D, VEC_OUT>(out, c, width, d);
        }
    }
}

// Dense, 16-byte aligned views whose width is a multiple of 8 and at least one tile: the
// view is the flat sequence of its [n, width/8] 8-element vectors and every wave takes
// 64 * NV consecutive vectors (lane l holds vectors 64k + l, so each load instruction covers
// contiguous memory).  NV is chosen so a wave moves 16 KiB each way (16 vectors per lane for
// 2-byte types, 8 for FP32), and the host keeps 64 * NV <= vectors per row, so a wave's
// vectors span at most two rows.  Loads run kLoads deep as a rolling window: the first kLoads
// are issued up front, and the register slot of each computed vector is refilled with the
// load kLoads vectors ahead before that vector is stored, so a wave keeps 8 loads in flight
// over its whole 16 KiB with the registers of 8.  The fast/general exponential path is chosen
// once per group of kLoads vectors (all of them loaded by then).  Same element-wise formulas
// as bwd_kernel, so the same bits; the split only gives every wave the same amount of work
// whatever the row width.
template <Dt D, bool SCALED, int NV>
__global__ __launch_bounds__(kBwdWaves* kWave) void bwd_flat_kernel(
    const typename DtInfo<D>::Storage* logits, int64_t ld, int64_t n, int vpr, int lim,
    int64_t col_begin, int64_t vocab_real, float inv_t, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ active, int64_t ignore_index, const float* __restrict__ grad,
    const logp_stats_t* __restrict__ stats, typename DtInfo<D>::Storage* dlogits,
    int64_t ld_out) {
    // logits and dlogits may be the same buffer: each vector is loaded and stored by the
    // same lane, load first, and no other lane touches it.
    using St = typename DtInfo<D>::Storage;
    static_assert(NV % kLoads == 0, "whole groups of kLoads vectors");
    constexpr int kChunk = kWave * NV;
    const int64_t total = n * vpr;
    // Workgroups take the chunks from the end of the view backwards: after a forward, which
    // streams the rows in order, the first chunks read are the ones the memory-side cache
    // still holds, and the next forward starts on the rows this kernel touched last
    // (about 1% on the backward inside a step at 32768 x 151936).
    const uint32_t blk = gridDim.x - 1 - blockIdx.x;
    const int64_t q0 = (int64_t(blk) * kBwdWaves + wave_id()) * kChunk;
    if (q0 >= total) return;  // whole wave leaves; this kernel has no barrier
    const int lane = lane_id();

    // Wave-uniform geometry: the chunk starts at vector off_a of row_a; its first `split`
    // vectors lie in row_a and the rest in row_a + 1; only the first `live` exist.
    const int64_t row_a = q0 / vpr;
    const int off_a = static_cast<int>(q0 - row_a * vpr);
    const int split = vpr - off_a < kChunk ? vpr - off_a : kChunk;
    const int64_t left = total - q0;
    const int live = left < kChunk ? static_cast<int>(left) : kChunk;
    const BwdRow ra = bwd_row<D, SCALED>(row_a, col_begin, vocab_real, inv_t, targets, active,
                                         ignore_index, grad, stats);
    BwdRow rb = ra;
    if (split < live)  // the chunk reaches row_a + 1, which then exists
        rb = bwd_row<D, SCALED>(row_a + 1, col_begin, vocab_real, inv_t, targets, active,
                                ignore_index, grad, stats);
    // Row bases; the second pair is only dereferenced when the chunk reaches row_a + 1.
    const St* xa = logits + row_a * ld;
    const St* xb = xa + ld;
    St* oa = dlogits + row_a * ld_out;
    St* ob = oa + ld_out;
    const int width = vpr * kVec;

    // Vector k of this lane: index idx = 64k + lane in the chunk, in row b when idx >= split,
    // at view column `col`; it is read only when it exists and its row is valid.
    auto col_of = [&](int idx) { return (off_a + idx - (idx >= split ? vpr : 0)) * kVec; };
    auto fetch = [&](int k, Raw8<D>& dst) {
        const int idx = k * kWave + lane;
        const bool in_b = idx >= split;
        if (idx < live && (in_b ? rb.valid : ra.valid))
            load8<D, true>(in_b ? xb : xa, col_of(idx), lim, dst);
    };

    // the first loads issue at raised wave priority, so a wave that has its row constants
    // gets its window in flight ahead of waves that are computing
    __builtin_amdgcn_s_setprio(1);
    Raw8<D> w[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) fetch(k, w[k]);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int k0 = 0; k0 < NV; k0 += kLoads) {
        bool hit = false;
#pragma unroll
        for (int k = k0; k < k0 + kLoads; ++k) {
            const int idx = k * kWave + lane;
            const bool in_b = idx >= split;
            if (idx < live && (in_b ? rb.valid : ra.valid))
                hit = hit || below_threshold<D>(w[k - k0], in_b ? rb.thr : ra.thr);
        }
        const bool deep = __any(hit);
#pragma unroll
        for (int k = k0; k < k0 + kLoads; ++k) {
            const int idx = k * kWave + lane;
            const bool in_b = idx >= split;
            const BwdRow r = in_b ? rb : ra;
            const int col = col_of(idx);
            float d[kVec];
            if (idx < live && r.valid) {
                bwd_compute_store<D, SCALED>(r, w[k - k0], deep, inv_t, col, lim, d);
            } else {
#pragma unroll
                for (int e = 0; e < kVec; ++e) d[e] = 0.0f;
            }
            if (k + kLoads < NV) fetch(k + kLoads, w[k - k0]);  // refill the freed slot
            if (idx < live) store8<D, true>(in_b ? ob : oa, col, width, d);
        }
    }
}

// Vectors per lane of the flat backward: 16 KiB per wave when the row holds at least one
// full chunk, otherwise kLoads (a chunk must not span more than two rows).
template <Dt D>
constexpr int bwd_flat_nv() { return D == Dt::F32 ? kLoads : 2 * kLoads; }

// --------------------------------------------------------------------- target check

__global__ __launch_bounds__(kCheckThreads) void check_targets_kernel(
    const int64_t* __restrict__ targets, const uint8_t* __restrict__ active, int64_t n,
    int64_t vocab_real, int64_t ignore_index, int64_t* __restrict__ bad_count) {
    __shared__ long long wave_counts[kCheckThreads / kWave];
    long long local = 0;
    for (int64_t i = threadIdx.x; i < n; i += kCheckThreads) {
        if (active != nullptr && active[i] == 0) continue;
        const int64_t y = targets[i];
        if (y == ignore_index) continue;
        if (y < 0 || y >= vocab_real) ++local;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) local += __shfl_xor(local, o, kWave);
    if (lane_id() == 0) wave_counts[threadIdx.x / kWave] = local;
    __syncthreads();
    if (threadIdx.x == 0) {
        long long total = 0;
        for (int w = 0; w < kCheckThreads / kWave; ++w) total += wave_counts[w];
        *bad_count = total;
    }
}

// =============================================================================== host

// Shape rules shared by every entry point that reads logits.
logp_status_t check_vocab(int64_t n, int64_t vocab_real, int64_t vocab_padded) {
    if (n < 0 || vocab_real < 1 || vocab_padded < vocab_real || vocab_padded > kMaxCols)
        return LOGP_ERR_SHAPE;
    return LOGP_OK;
}

// Grid size for `items_per_block` (row, tile) items per workgroup, or 0 if it does not fit a
// 1-D launch.
uint32_t item_grid(int64_t n, int64_t tiles_per_row, int64_t items_per_block) {
    if (n > (int64_t(1) << 62) / tiles_per_row) return 0;
    const int64_t blocks = ceil_div(n * tiles_per_row, items_per_block);
    return blocks > 0x7FFFFFFF ? 0 : static_cast<uint32_t>(blocks);
}

// Kernel selection: one pointer per (dtype, load/store path, scaled) combination.
template <Dt D>
const void* fwd_ptr(bool vec, bool scaled) {
    if (vec) return scaled ? reinterpret_cast<const void*>(&fwd_kernel<D, true, true>)
                           : reinterpret_cast<const void*>(&fwd_kernel<D, true, false>);
    return scaled ? reinterpret_cast<const void*>(&fwd_kernel<D, false, true>)
                  : reinterpret_cast<const void*>(&fwd_kernel<D, false, false>);
}

template <Dt D>
const void* partials_ptr(bool vec, bool scaled) {
    if (vec) return scaled ? reinterpret_cast<const void*>(&partials_kernel<D, true, true>)
                           : reinterpret_cast<const void*>(&partials_kernel<D, true, false>);
    return scaled ? reinterpret_cast<const void*>(&partials_kernel<D, false, true>)
                  : reinterpret_cast<const void*>(&partials_kernel<D, false, false>);
}

template <Dt D, bool SCALED>
const void* bwd_ptr(bool vin, bool vout) {
    if (vin) return vout ? reinterpret_cast<const void*>(&bwd_kernel<D, true, true, SCALED>)
                         : reinterpret_cast<const void*>(&bwd_kernel<D, true, false, SCALED>);
    return vout ? reinterpret_cast<const void*>(&bwd_kernel<D, false, true, SCALED>)
                : reinterpret_cast<const void*>(&bwd_kernel<D, false, false, SCALED>);
}

template <Dt D, bool SCALED>
const void* bwd_flat_ptr(int nv) {
    constexpr int kWide = bwd_flat_nv<D>();
    if (nv == kWide) return reinterpret_cast<const void*>(&bwd_flat_kernel<D, SCALED, kWide>);
    return reinterpret_cast<const void*>(&bwd_flat_kernel<D, SCALED, kLoads>);
}

// flat_nv = 0 selects the (row, tile) kernel, otherwise the flat one with that many vectors
// per lane.
template <Dt D>
const void* bwd_ptr(bool vin, bool vout, bool scaled, int flat_nv) {
    if (flat_nv != 0)
        return scaled ? bwd_flat_ptr<D, true>(flat_nv) : bwd_flat_ptr<D, false>(flat_nv);
    return scaled ? bwd_ptr<D, true>(vin, vout) : bwd_ptr<D, false>(vin, vout);
}

// Element size of a dtype, or 0 when the value is not a logp_dtype_t.
// dtype travels as an int32 (a logp_dtype_t value): any value a caller passes is defined here.
int64_t elem_bytes(int32_t dtype) {
    switch (dtype) {
        case LOGP_DTYPE_BF16: return 2;
        case LOGP_DTYPE_F16: return 2;
        case LOGP_DTYPE_F32: return 4;
    }
    return 0;
}

bool valid_inv_temperature(float inv_t) { return std::isfinite(inv_t) && inv_t > 0.0f; }

// 16-byte loads/stores need an aligned view start and rows that stay aligned.
bool vec_ok(const void* p, int64_t ld, int64_t elem) {
    return aligned16(p) && (ld * elem) % 16 == 0;
}

}  // namespace

// ============================================================================ C ABI

extern "C" {

int64_t logp_num_tiles(int64_t vocab_padded) {
    return vocab_padded < 1 ? 0 : ceil_div(vocab_padded, kTile);
}

const char* logp_status_string(int32_t status) {
    // an int, not the enum: any value a caller passes is defined here
    switch (status) {
        case LOGP_OK: return "ok";
        case LOGP_ERR_NULL: return "a required pointer is NULL";
        case LOGP_ERR_SHAPE: return "sizes, strides or column bounds out of range";
        case LOGP_ERR_SHARD:
            return "column range is not tile-aligned (interior bounds must be multiples of "
                   "LOGP_TILE_COLS) or lies outside [0, vocab_padded]";
        case LOGP_ERR_DEVICE:
            return "a pointer is not device memory of the logits' device, or the stream "
                   "belongs to another device";
        case LOGP_ERR_RANGE: return "an array extends past the end of its allocation";
        case LOGP_ERR_OVERLAP: return "an output overlaps an input or another output";
        case LOGP_ERR_HIP: return "the HIP runtime reported an error";
        case LOGP_ERR_ARG:
            return "unknown dtype, or inv_temperature not a finite positive number";
        case LOGP_ERR_SCRATCH:
            return "the call needs more staging memory than the library's static scratch "
                   "array holds (use the entry point that takes a workspace)";
    }
    return "unknown status";
}

logp_status_t logp_forward_ex(int32_t dtype, float inv_temperature, const void* logits,
                              int64_t ld, int64_t n, int64_t vocab_real, int64_t vocab_padded,
                              const int64_t* targets, const uint8_t* active, int64_t ignore_index,
                              float* logp, float* lse, logp_stats_t* stats, hipStream_t stream) {
    const int64_t eb = elem_bytes(dtype);
    if (eb == 0 || !valid_inv_temperature(inv_temperature)) return LOGP_ERR_ARG;
    logp_status_t st = check_vocab(n, vocab_real, vocab_padded);
    if (st != LOGP_OK) return st;
    if (ld < vocab_padded || logp_num_tiles(vocab_padded) > LOGP_FWD_MAX_TILES)
        return LOGP_ERR_SHAPE;
    if (n > 0x7FFFFFFF) return LOGP_ERR_SHAPE;  // one workgroup per row on a 1-D grid
    if (n == 0) return LOGP_OK;
    if (logits == nullptr || targets == nullptr || logp == nullptr) return LOGP_ERR_NULL;
    const uint64_t lg_bytes = span_bytes(n, ld, vocab_real, eb);
    if (lg_bytes == 0) return LOGP_ERR_SHAPE;
    const Span in[] = {{logits, lg_bytes}, {targets, uint64_t(n) * 8},
                       {active, active ? uint64_t(n) : 0}};
    const Span out[] = {{logp, uint64_t(n) * 4}, {lse, lse ? uint64_t(n) * 4 : 0},
                        {stats, stats ? uint64_t(n) * 8 : 0}};
    int device = -1;
    st = check_buffers(in, 3, out, 3, stream, &device);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(device);
    if (!guard.ok()) return LOGP_ERR_HIP;

    int vr = static_cast<int>(vocab_real);
    float inv_t = inv_temperature;
    void* args[] = {&logits, &ld, &vr, &inv_t, &targets, &active, &ignore_index, &logp, &lse,
                    &stats};
    const bool vec = vec_ok(logits, ld, eb);
    const bool scaled = inv_temperature != 1.0f;
    const void* k = dtype == LOGP_DTYPE_BF16 ? fwd_ptr<Dt::BF16>(vec, scaled)
                    : dtype == LOGP_DTYPE_F16 ? fwd_ptr<Dt::F16>(vec, scaled)
                                              : fwd_ptr<Dt::F32>(vec, scaled);
    const size_t lds = size_t(ceil_div(vocab_real, kTile)) * sizeof(float2);
    return launch(k, dim3(static_cast<uint32_t>(n)), dim3(kFwdWaves * kWave), args, lds, stream);
}

logp_status_t logp_forward(const uint16_t* logits, int64_t ld, int64_t n, int64_t vocab_real,
                           int64_t vocab_padded, const int64_t* targets, const uint8_t* active,
                           int64_t ignore_index, float* logp, float* lse, logp_stats_t* stats,
                           hipStream_t stream) {
    return logp_forward_ex(LOGP_DTYPE_BF16, 1.0f, logits, ld, n, vocab_real, vocab_padded,
                           targets, active, ignore_index, logp, lse, stats, stream);
}

logp_status_t logp_backward_ex(int32_t dtype, float inv_temperature, const void* logits,
                               int64_t ld, int64_t n, int64_t vocab_real, int64_t vocab_padded,
                               int64_t col_begin, int64_t col_end, const int64_t* targets,
                               const uint8_t* active, int64_t ignore_index,
                               const float* grad_logp, const logp_stats_t* stats, void* dlogits,
                               int64_t ld_out, hipStream_t stream) {
    const int64_t eb = elem_bytes(dtype);
    if (eb == 0 || !valid_inv_temperature(inv_temperature)) return LOGP_ERR_ARG;
    logp_status_t st = check_vocab(n, vocab_real, vocab_padded);
    if (st != LOGP_OK) return st;
    if (col_begin < 0 || col_end < col_begin || col_end > vocab_padded) return LOGP_ERR_SHARD;
    const int64_t width = col_end - col_begin;
    if (ld < width || ld_out < width) return LOGP_ERR_SHAPE;
    if (n == 0 || width == 0) return LOGP_OK;
    if (logits == nullptr || targets == nullptr || grad_logp == nullptr || stats == nullptr ||
        dlogits == nullptr)
        return LOGP_ERR_NULL;
    const int64_t lim = std::max<int64_t>(0, std::min(vocab_real, col_end) - col_begin);
    const int64_t view_tiles = ceil_div(width, kTile);
    const bool f32 = dtype == LOGP_DTYPE_F32;
    const int tile_waves = f32 ? bwd_tile_waves<Dt::F32>() : bwd_tile_waves<Dt::BF16>();
    const int tpw = f32 ? bwd_tiles_per_wave<Dt::F32>() : bwd_tiles_per_wave<Dt::BF16>();
    const uint32_t grid = item_grid(n, view_tiles, tile_waves * tpw);
    const uint64_t in_bytes = span_bytes(n, ld, lim, eb);
    const uint64_t out_bytes = span_bytes(n, ld_out, width, eb);
    if (grid == 0 || out_bytes == 0 || (lim > 0 && in_bytes == 0)) return LOGP_ERR_SHAPE;
    // In place is allowed only as an exact alias with the same row stride.
    Span alias = {nullptr, 0};
    if (dlogits == logits && ld_out == ld) alias = {logits, in_bytes};
    const Span in[] = {{logits, in_bytes}, {targets, uint64_t(n) * 8},
                       {active, active ? uint64_t(n) : 0}, {grad_logp, uint64_t(n) * 4},
                       {stats, uint64_t(n) * 8}};
    const Span out[] = {{dlogits, alias.p ? in_bytes : out_bytes}};
    int device = -1;
    st = check_buffers(in, 5, out, 1, stream, &device, alias);
    if (st != LOGP_OK) return st;
    if (alias.p != nullptr && out_bytes != in_bytes) {
        // the written span is larger than the read span: it still must fit the allocation
        int d2 = -1;
        st = locate(dlogits, out_bytes, &d2);
        if (st != LOGP_OK) return st;
    }
    DeviceGuard guard(device);
    if (!guard.ok()) return LOGP_ERR_HIP;

    const bool vin = vec_ok(logits, ld, eb);
    const bool vout = vec_ok(dlogits, ld_out, eb);
    const bool scaled = inv_temperature != 1.0f;
    const bool flat = vin && vout && width % kVec == 0 && width >= kTile;
    // vectors per lane of the flat kernel: its wide form needs a whole chunk in every row
    const int wide = f32 ? bwd_flat_nv<Dt::F32>() : bwd_flat_nv<Dt::BF16>();
    const int flat_nv = !flat ? 0 : width / kVec >= int64_t(kWave) * wide ? wide : kLoads;
    const void* k = dtype == LOGP_DTYPE_BF16 ? bwd_ptr<Dt::BF16>(vin, vout, scaled, flat_nv)
                    : dtype == LOGP_DTYPE_F16 ? bwd_ptr<Dt::F16>(vin, vout, scaled, flat_nv)
                                              : bwd_ptr<Dt::F32>(vin, vout, scaled, flat_nv);
    float inv_t = inv_temperature;
    int li = static_cast<int>(lim);
    if (flat) {
        const int64_t vectors = n * (width / kVec);
        const int64_t blocks = ceil_div(vectors, int64_t(kBwdWaves) * kWave * flat_nv);
        if (blocks > 0x7FFFFFFF) return LOGP_ERR_SHAPE;
        int vpr = static_cast<int>(width / kVec);
        void* args[] = {&logits, &ld, &n, &vpr, &li, &col_begin, &vocab_real, &inv_t, &targets,
                        &active, &ignore_index, &grad_logp, &stats, &dlogits, &ld_out};
        return launch(k, dim3(static_cast<uint32_t>(blocks)), dim3(kBwdWaves * kWave), args, 0,
                      stream);
    }
    int vt = static_cast<int>(view_tiles), w = static_cast<int>(width);
    void* args[] = {&logits, &ld, &n, &vt, &w, &li, &col_begin, &vocab_real, &inv_t, &targets,
                    &active, &ignore_index, &grad_logp, &stats, &dlogits, &ld_out};
    return launch(k, dim3(grid), dim3(tile_waves * kWave), args, 0, stream);
}

logp_status_t logp_backward(const uint16_t* logits, int64_t ld, int64_t n, int64_t vocab_real,
                            int64_t vocab_padded, int64_t col_begin, int64_t col_end,
                            const int64_t* targets, const uint8_t* active, int64_t ignore_index,
                            const float* grad_logp, const logp_stats_t* stats, uint16_t* dlogits,
                            int64_t ld_out, hipStream_t stream) {
    return logp_backward_ex(LOGP_DTYPE_BF16, 1.0f, logits, ld, n, vocab_real, vocab_padded,
                            col_begin, col_end, targets, active, ignore_index, grad_logp, stats,
                            dlogits, ld_out, stream);
}

logp_status_t logp_partials_ex(int32_t dtype, float inv_temperature, const void* logits,
                               int64_t ld, int64_t n, int64_t vocab_real, int64_t vocab_padded,
                               int64_t col_begin, int64_t col_end, const int64_t* targets,
                               const uint8_t* active, int64_t ignore_index,
                               logp_partial_t* partials, int64_t ldp, hipStream_t stream) {
    const int64_t eb = elem_bytes(dtype);
    if (eb == 0 || !valid_inv_temperature(inv_temperature)) return LOGP_ERR_ARG;
    logp_status_t st = check_vocab(n, vocab_real, vocab_padded);
    if (st != LOGP_OK) return st;
    if (col_begin < 0 || col_end <= col_begin || col_end > vocab_padded ||
        col_begin % kTile != 0 || (col_end % kTile != 0 && col_end != vocab_padded))
        return LOGP_ERR_SHARD;
    const int64_t width = col_end - col_begin;
    const int64_t view_tiles = ceil_div(width, kTile);
    if (ld < width || ldp < view_tiles) return LOGP_ERR_SHAPE;
    if (n == 0) return LOGP_OK;
    if (logits == nullptr || targets == nullptr || partials == nullptr) return LOGP_ERR_NULL;
    const int64_t lim = std::max<int64_t>(0, std::min(vocab_real, col_end) - col_begin);
    const uint32_t grid = item_grid(n, view_tiles, kItemWaves);
    const uint64_t in_bytes = span_bytes(n, ld, lim, eb);
    const uint64_t part_bytes = span_bytes(n, ldp, view_tiles, sizeof(logp_partial_t));
    if (grid == 0 || part_bytes == 0 || (lim > 0 && in_bytes == 0)) return LOGP_ERR_SHAPE;
    const Span in[] = {{logits, in_bytes}, {targets, uint64_t(n) * 8},
                       {active, active ? uint64_t(n) : 0}};
    const Span out[] = {{partials, part_bytes}};
    int device = -1;
    st = check_buffers(in, 3, out, 1, stream, &device);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(device);
    if (!guard.ok()) return LOGP_ERR_HIP;

    int vt = static_cast<int>(view_tiles), li = static_cast<int>(lim);
    float inv_t = inv_temperature;
    void* args[] = {&logits, &ld, &n, &vt, &li, &col_begin, &col_end, &vocab_real, &inv_t,
                    &targets, &active, &ignore_index, &partials, &ldp};
    const bool vec = vec_ok(logits, ld, eb);
    const bool scaled = inv_temperature != 1.0f;
    const void* k = dtype == LOGP_DTYPE_BF16 ? partials_ptr<Dt::BF16>(vec, scaled)
                    : dtype == LOGP_DTYPE_F16 ? partials_ptr<Dt::F16>(vec, scaled)
                                              : partials_ptr<Dt::F32>(vec, scaled);
    return launch(k, dim3(grid), dim3(kItemWaves * kWave), args, 0, stream);
}

logp_status_t logp_partials(const uint16_t* logits, int64_t ld, int64_t n, int64_t vocab_real,
                            int64_t vocab_padded, int64_t col_begin, int64_t col_end,
                            const int64_t* targets, const uint8_t* active, int64_t ignore_index,
                            logp_partial_t* partials, int64_t ldp, hipStream_t stream) {
    return logp_partials_ex(LOGP_DTYPE_BF16, 1.0f, logits, ld, n, vocab_real, vocab_padded,
                            col_begin, col_end, targets, active, ignore_index, partials, ldp,
                            stream);
}

logp_status_t logp_merge(const logp_partial_t* partials, int64_t ldp, int64_t n,
                         int64_t num_tiles, int64_t vocab_real, const int64_t* targets,
                         const uint8_t* active, int64_t ignore_index, float* logp, float* lse,
                         logp_stats_t* stats, hipStream_t stream) {
    if (n < 0 || vocab_real < 1 || vocab_real > kMaxCols ||
        num_tiles < ceil_div(vocab_real, kTile) || num_tiles > ceil_div(kMaxCols, kTile) ||
        ldp < num_tiles)
        return LOGP_ERR_SHAPE;
    if (n == 0) return LOGP_OK;
    if (partials == nullptr || targets == nullptr || logp == nullptr) return LOGP_ERR_NULL;
    const uint64_t part_bytes = span_bytes(n, ldp, num_tiles, sizeof(logp_partial_t));
    const int64_t blocks = ceil_div(n, kMergeWaves);
    if (part_bytes == 0 || blocks > 0x7FFFFFFF) return LOGP_ERR_SHAPE;
    const Span in[] = {{partials, part_bytes}, {targets, uint64_t(n) * 8},
                       {active, active ? uint64_t(n) : 0}};
    const Span out[] = {{logp, uint64_t(n) * 4}, {lse, lse ? uint64_t(n) * 4 : 0},
                        {stats, stats ? uint64_t(n) * 8 : 0}};
    int device = -1;
    logp_status_t st = check_buffers(in, 3, out, 3, stream, &device);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(device);
    if (!guard.ok()) return LOGP_ERR_HIP;

    int nt = static_cast<int>(num_tiles);
    void* args[] = {&partials, &ldp, &n, &nt, &vocab_real, &targets, &active, &ignore_index,
                    &logp, &lse, &stats};
    return launch(reinterpret_cast<const void*>(&merge_kernel), dim3(static_cast<uint32_t>(blocks)),
                  dim3(kMergeWaves * kWave), args, 0, stream);
}

logp_status_t logp_check_targets(const int64_t* targets, const uint8_t* active, int64_t n,
                                 int64_t vocab_real, int64_t ignore_index, int64_t* bad_count,
                                 hipStream_t stream) {
    if (n < 0 || vocab_real < 1) return LOGP_ERR_SHAPE;
    if (bad_count == nullptr || (n > 0 && targets == nullptr)) return LOGP_ERR_NULL;
    const Span in[] = {{targets, uint64_t(n) * 8}, {active, active ? uint64_t(n) : 0}};
    const Span out[] = {{bad_count, 8}};
    int device = -1;
    logp_status_t st = check_buffers(in, 2, out, 1, stream, &device);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(device);
    if (!guard.ok()) return LOGP_ERR_HIP;
    void* args[] = {&targets, &active, &n, &vocab_real, &ignore_index, &bad_count};
    return launch(reinterpret_cast<const void*>(&check_targets_kernel), dim3(1),
                  dim3(kCheckThreads), args, 0, stream);
}

}  // extern "C"
