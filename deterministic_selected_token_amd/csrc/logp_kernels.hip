// gfx950 kernels and the C ABI of the selected-token log-probability library.
//
//   forward   one workgroup per row; its waves take the row's global tiles round-robin,
//             reduce each in registers to (m_l, s_l), park them in LDS, and wave 0 runs
//             the canonical merge (RL-Kernel issue #241, "PR 3"; PR #314 Tensor Parallel
//             doc, steps 1-6).  One HBM pass over the logits, nothing else written but
//             logp / LSE / (M, S).
//   backward  one wave per (row, tile): read the tile once, write
//             dlogits = g (onehot - exp(x - M) / S) rounded to BF16 straight from
//             registers (PR #495 "zero-workspace backward for generic CUDA fused logp",
//             Summary item 2: no FP32 [N, V] workspace; a single read instead of the
//             three the pages' kernel needs, Results section).
//   partials  one wave per (row, tile of the shard): the forward's tile reduction, written
//             out as (m_l, s_l, sel_l) (issue #241, "PR6").
//   merge     one wave per row over [L] partials: the forward's merge code.
//
// Host entry points validate every argument before launching and report failures as
// status codes (see include/logp.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "logp.h"
#include "logp_device.hpp"

using namespace logp;

namespace {

constexpr int kFwdWaves = 4;     // waves per forward workgroup (one row)
constexpr int kItemWaves = 4;    // waves per workgroup of the partials kernel
constexpr int kBwdWaves = 16;    // waves per backward workgroup
constexpr int kBwdTilesPerWave = 2;  // consecutive (row, tile) items per backward wave
constexpr int kMergeWaves = 4;   // rows per merge workgroup
constexpr int kCheckThreads = 1024;
// Largest padded width: keeps vocab_padded + kTile below 2^31 so in-row column arithmetic
// never overflows a 32-bit int.
constexpr int64_t kMaxCols = (int64_t(1) << 31) - 1 - kTile;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two floats to BF16 (nearest, ties to even) and pack them, low element first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v.x = static_cast<__bf16>(lo);
    v.y = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}
__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

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

template <bool VEC>
__global__ __launch_bounds__(kFwdWaves* kWave) void fwd_kernel(
    const uint16_t* __restrict__ logits, int64_t ld, int vocab_real,
    const int64_t* __restrict__ targets, const uint8_t* __restrict__ active, int64_t ignore_index,
    float* __restrict__ logp, float* __restrict__ lse, logp_stats_t* __restrict__ stats) {
    extern __shared__ float2 slots[];  // (m_l, s_l) per real tile
    const int64_t row = blockIdx.x;
    const int wave = wave_id();
    const int lane = lane_id();
    const uint16_t* __restrict__ x = logits + row * ld;
    const int real_tiles = (vocab_real + kTile - 1) / kTile;

    // Wave 0 fetches the target and its logit first so the gather overlaps the streaming.
    int64_t y = 0;
    bool valid = false;
    float sel = 0.0f;
    if (wave == 0) {
        valid = row_valid(targets, active, ignore_index, vocab_real, row, y);
        if (valid) sel = bf16_to_f32(x[y]);
    }

    for (int l = wave; l < real_tiles; l += kFwdWaves) {
        TileRegs t;
        load_tile<VEC>(x, l * kTile, vocab_real, lane, t);
        float m, s;
        tile_stats(t, m, s);
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

template <bool VEC>
__global__ __launch_bounds__(kItemWaves* kWave) void partials_kernel(
    const uint16_t* __restrict__ logits, int64_t ld, int64_t n, int view_tiles, int lim,
    int64_t col_begin, int64_t col_end, int64_t vocab_real, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ active, int64_t ignore_index, logp_partial_t* __restrict__ partials,
    int64_t ldp) {
    const int64_t item = int64_t(blockIdx.x) * kItemWaves + wave_id();
    if (item >= n * view_tiles) return;  // whole wave leaves; this kernel has no barrier
    const int lane = lane_id();
    const int64_t row = item / view_tiles;
    const int j = static_cast<int>(item - row * view_tiles);
    const int start = j * kTile;
    const uint16_t* __restrict__ x = logits + row * ld;

    TileRegs t;
    load_tile<VEC>(x, start, lim, lane, t);
    float m, s;
    tile_stats(t, m, s);
    if (lane == 0) {
        int64_t y;
        const bool valid = row_valid(targets, active, ignore_index, vocab_real, row, y);
        const int64_t g0 = col_begin + start;  // global column of this tile's first entry
        float sel = 0.0f;
        if (valid && y >= g0 && y < g0 + kTile && y < col_end) sel = bf16_to_f32(x[y - col_begin]);
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

// Writes 8 consecutive outputs starting at view column c (c is a multiple of 8): one
// 16-byte store when the vector path is allowed and all 8 lie inside the row, else
// element-wise stores for the columns below `width`.
template <bool VEC>
__device__ __forceinline__ void store8(uint16_t* out, int c, int width, const float* d) {
    if (VEC && c + kVec <= width) {
        u32x4 w;
        w.x = pack_bf16x2(d[0], d[1]);
        w.y = pack_bf16x2(d[2], d[3]);
        w.z = pack_bf16x2(d[4], d[5]);
        w.w = pack_bf16x2(d[6], d[7]);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(out + c));
    } else {
#pragma unroll
        for (int e = 0; e < kVec; e += 2) {
            const uint32_t w = pack_bf16x2(d[e], d[e + 1]);
            if (c + e < width) out[c + e] = static_cast<uint16_t>(w & 0xFFFFu);
            if (c + e + 1 < width) out[c + e + 1] = static_cast<uint16_t>(w >> 16);
        }
    }
}

// Per-item (row, tile) state of the backward.
struct BwdItem {
    int64_t row, y;
    int start;      // first view column of the tile
    bool valid;     // row valid and its stats finite
    float M, g, neg_c, neg_c_lo;
};

// Row-side inputs of one item: validity, (M, S), g and the per-row scale -g/S.  The stats and
// g loads do not wait for the validity test (they are in bounds for every row), so one
// memory round trip resolves all of them.
__device__ __forceinline__ BwdItem bwd_item(int64_t item, int view_tiles,
                                            const int64_t* __restrict__ targets,
                                            const uint8_t* __restrict__ active,
                                            int64_t ignore_index, int64_t vocab_real,
                                            const float* __restrict__ grad,
                                            const logp_stats_t* __restrict__ stats) {
    BwdItem it;
    it.row = item / view_tiles;
    it.start = static_cast<int>(item - it.row * view_tiles) * kTile;
    const float M = stats[it.row].max, S = stats[it.row].sumexp, g = grad[it.row];
    it.valid = row_valid(targets, active, ignore_index, vocab_real, it.row, it.y) && M != kNegInf;
    it.M = M;
    it.g = g;
    it.neg_c = -(g / S);                // -g/S, one rounding per row
    it.neg_c_lo = it.neg_c * 0x1p-64f;  // exact unless |g/S| < 2^-62
    return it;
}

// True when some value of the packed tile may lie below M - 87 (so exp(x - M) could fall
// outside the normal range).  Works on raw BF16 bits: a negative value below the threshold
// has larger unsigned bits than the threshold truncated toward zero, and false alarms only
// select the slower path, which gives the same bits.
__device__ __forceinline__ bool bwd_needs_deep(const u32x4* w, float M) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const float thr = M - 87.0f;
    u16x2 mx = {0, 0};
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[k].x));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[k].y));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[k].z));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[k].w));
    }
    const unsigned t16 = 0x8000u | ((__float_as_uint(thr) >> 16) & 0x7FFFu);
    return __any(thr >= 0.0f || mx.x > t16 || mx.y > t16);
}

// Gradient of the 8 columns at view column c of one item, from their logits v[0..7].
template <bool DEEP>
__device__ __forceinline__ void bwd_vec(const BwdItem& it, const float* v, int c, int lim,
                                        bool partial, float* d) {
#pragma unroll
    for (int e = 0; e < kVec; ++e)
        d[e] = DEEP ? bwd_term_deep(v[e], it.M, it.neg_c, it.neg_c_lo)
                    : bwd_term(v[e], it.M, it.neg_c);
    const int64_t yo = it.y - c;  // the target's offset from c (within this view)
    if (yo >= 0 && yo < kVec) {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (e == yo) d[e] = it.g + d[e];  // g * (1 - p)
    }
    if (partial) {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (c + e >= lim) d[e] = 0.0f;  // padding and past-the-vocab columns
    }
}

template <bool VEC_IN, bool VEC_OUT>
__global__ __launch_bounds__(kBwdWaves* kWave) void bwd_kernel(
    const uint16_t* logits, int64_t ld, int64_t n, int view_tiles, int width, int lim,
    int64_t col_begin, int64_t vocab_real, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ active, int64_t ignore_index, const float* __restrict__ grad,
    const logp_stats_t* __restrict__ stats, uint16_t* dlogits, int64_t ld_out) {
    // logits and dlogits may be the same buffer: every element is loaded into registers
    // before the lane that loaded it stores to it, and no other lane touches it.
    const int64_t first = (int64_t(blockIdx.x) * kBwdWaves + wave_id()) * kBwdTilesPerWave;
    const int64_t total = n * view_tiles;
    if (first >= total) return;  // whole wave leaves; this kernel has no barrier
    const int lane = lane_id();

    BwdItem it[kBwdTilesPerWave];
#pragma unroll
    for (int i = 0; i < kBwdTilesPerWave; ++i)
        if (first + i < total)
            it[i] = bwd_item(first + i, view_tiles, targets, active, ignore_index, vocab_real,
                             grad, stats);
    // Issue the loads of every tile this wave owns before computing any of them, so the
    // second tile's bytes are in flight while the first is processed.  Invalid rows are not
    // read.
    u32x4 w[kBwdTilesPerWave][kLoads];
#pragma unroll
    for (int i = 0; i < kBwdTilesPerWave; ++i)
        if (first + i < total && it[i].valid)
            load_tile_bits<VEC_IN>(logits + it[i].row * ld, it[i].start, lim, lane, w[i]);
#pragma unroll
    for (int i = 0; i < kBwdTilesPerWave; ++i) {
        if (first + i >= total) break;
        BwdItem t = it[i];
        uint16_t* out = dlogits + t.row * ld_out;
        const int base = t.start + kVec * lane;
        if (!t.valid) {
            float z[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) z[e] = 0.0f;
#pragma unroll
            for (int k = 0; k < kLoads; ++k) store8<VEC_OUT>(out, base + k * kLoadStride, width, z);
            continue;
        }
        t.y -= col_begin;  // the target in view coordinates
        const bool partial = t.start + kTile > lim;
        const bool deep = bwd_needs_deep(w[i], t.M);  // masked columns (-inf) always count
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            float v[kVec], d[kVec];
            unpack8(w[i][k], v);
            const int c = base + k * kLoadStride;
            if (!deep) bwd_vec<false>(t, v, c, lim, partial, d);
            else bwd_vec<true>(t, v, c, lim, partial, d);
            store8<VEC_OUT>(out, c, width, d);
        }
    }
}

// Backward over a dense, 16-byte aligned view whose width is a multiple of 8 and at least
// one tile: the view is treated as the flat sequence of its [n, width/8] 16-byte vectors and
// every wave takes kBwdTilesPerWave chunks of 512 consecutive vectors (lane l holds vectors
// 64k + l of a chunk, so each load instruction still covers 1 KiB of contiguous memory).
// The element-wise formulas are those of bwd_kernel, so the bits are the same; this split
// just gives every wave the same amount of work whatever the row width.  A chunk spans at
// most two rows (width >= 4096 columns = 512 vectors).
struct FlatRow {
    bool valid;
    float M, g, neg_c, neg_c_lo;
    int y;         // target in view coordinates (any value when invalid)
    unsigned t16;  // raw-bits threshold of the subnormal-safe path test
};

__device__ __forceinline__ FlatRow flat_row(int64_t row, int64_t col_begin, int64_t vocab_real,
                                            const int64_t* __restrict__ targets,
                                            const uint8_t* __restrict__ active,
                                            int64_t ignore_index, const float* __restrict__ grad,
                                            const logp_stats_t* __restrict__ stats) {
    FlatRow r;
    const float M = stats[row].max, S = stats[row].sumexp;
    int64_t y;
    r.valid = row_valid(targets, active, ignore_index, vocab_real, row, y) && M != kNegInf;
    r.M = M;
    r.g = grad[row];
    r.neg_c = -(r.g / S);
    r.neg_c_lo = r.neg_c * 0x1p-64f;
    r.y = static_cast<int>(y - col_begin);
    const float thr = M - 87.0f;
    r.t16 = thr >= 0.0f ? 0u : (0x8000u | ((__float_as_uint(thr) >> 16) & 0x7FFFu));
    return r;
}

template <bool DEEP>
__device__ __forceinline__ void flat_vec(const FlatRow& r, const float* v, int col, int lim,
                                         float* d) {
#pragma unroll
    for (int e = 0; e < kVec; ++e)
        d[e] = DEEP ? bwd_term_deep(v[e], r.M, r.neg_c, r.neg_c_lo)
                    : bwd_term(v[e], r.M, r.neg_c);
    const int yo = r.y - col;
    if (yo >= 0 && yo < kVec) {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (e == yo) d[e] = r.g + d[e];  // g * (1 - p)
    }
    if (col + kVec > lim) {
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (col + e >= lim) d[e] = 0.0f;  // padding columns
    }
}

__global__ __launch_bounds__(kBwdWaves* kWave) void bwd_flat_kernel(
    const uint16_t* logits, int64_t ld, int64_t n, int vpr, int lim, int64_t col_begin,
    int64_t vocab_real, const int64_t* __restrict__ targets, const uint8_t* __restrict__ active,
    int64_t ignore_index, const float* __restrict__ grad, const logp_stats_t* __restrict__ stats,
    uint16_t* dlogits, int64_t ld_out) {
    // logits and dlogits may be the same buffer: each 16-byte vector is loaded and stored by
    // the same lane, load first.
    constexpr int kChunk = kWave * kLoads;  // 512 vectors per wave
    const int64_t total = n * vpr;
    const int64_t q0 = (int64_t(blockIdx.x) * kBwdWaves + wave_id()) * kChunk;
    if (q0 >= total) return;  // whole wave leaves; this kernel has no barrier
    const int lane = lane_id();

    const int64_t row_a = q0 / vpr;
    const int64_t sp = (row_a + 1) * vpr - q0;
    const int split = sp < kChunk ? static_cast<int>(sp) : kChunk;  // vectors in row_a
    const FlatRow ra = flat_row(row_a, col_begin, vocab_real, targets, active, ignore_index,
                                grad, stats);
    FlatRow rb = ra;
    if (split < kChunk && row_a + 1 < n)
        rb = flat_row(row_a + 1, col_begin, vocab_real, targets, active, ignore_index, grad,
                      stats);

    // issue every load of the wave before computing
    u32x4 w[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const int idx = k * kWave + lane;
        const bool in_b = idx >= split;
        const int64_t row = row_a + (in_b ? 1 : 0);
        const int col = static_cast<int>(q0 + idx - row * vpr) * kVec;
        if (q0 + idx < total && (in_b ? rb.valid : ra.valid)) {
            const uint16_t* src = logits + row * ld;
            if (col + kVec <= lim) {
                w[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + col));
            } else {
                w[k].x = masked_bits(src, col + 0, lim) | (masked_bits(src, col + 1, lim) << 16);
                w[k].y = masked_bits(src, col + 2, lim) | (masked_bits(src, col + 3, lim) << 16);
                w[k].z = masked_bits(src, col + 4, lim) | (masked_bits(src, col + 5, lim) << 16);
                w[k].w = masked_bits(src, col + 6, lim) | (masked_bits(src, col + 7, lim) << 16);
            }
        }
    }
    // subnormal-safe path if any valid vector may hold x < M - 87 of its own row
    bool hit = false;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const int idx = k * kWave + lane;
        const bool in_b = idx >= split;
        const bool valid = in_b ? rb.valid : ra.valid;
        const unsigned t16 = in_b ? rb.t16 : ra.t16;
        if (q0 + idx < total && valid) {
            typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
            u16x2 mx = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w[k].x),
                                                 __builtin_bit_cast(u16x2, w[k].y));
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[k].z));
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[k].w));
            hit = hit || t16 == 0u || mx.x > t16 || mx.y > t16;
        }
    }
    const bool deep = __any(hit);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const int idx = k * kWave + lane;
        if (q0 + idx >= total) continue;
        const bool in_b = idx >= split;
        const int64_t row = row_a + (in_b ? 1 : 0);
        const FlatRow r = in_b ? rb : ra;
        const int col = static_cast<int>(q0 + idx - row * vpr) * kVec;
        float d[kVec];
        if (!r.valid) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) d[e] = 0.0f;
        } else {
            float v[kVec];
            unpack8(w[k], v);
            if (!deep) flat_vec<false>(r, v, col, lim, d);
            else flat_vec<true>(r, v, col, lim, d);
        }
        store8<true>(dlogits + row * ld_out, col, vpr * kVec, d);
    }
}

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

struct Span {
    const void* p;
    uint64_t bytes;
};

bool overlaps(Span a, Span b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Bytes spanned by `rows` rows of `width` elements of `elem` bytes at stride `ld` elements,
// or 0 on overflow (callers have already bounded every factor).
uint64_t span_bytes(int64_t rows, int64_t ld, int64_t width, int64_t elem) {
    if (rows <= 0 || width <= 0) return 0;
    const unsigned __int128 b =
        (static_cast<unsigned __int128>(rows - 1) * static_cast<uint64_t>(ld) + width) * elem;
    if (b > (static_cast<unsigned __int128>(1) << 62)) return 0;
    return static_cast<uint64_t>(b);
}

// Device of `p` (device or managed memory), checked to hold `bytes` from `p` on.
logp_status_t locate(const void* p, uint64_t bytes, int* device) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();  // our failed query must not leak into the caller's checks
        return LOGP_ERR_DEVICE;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return LOGP_ERR_DEVICE;
    *device = attr.device;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return LOGP_ERR_DEVICE;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    if (q < b || q - b > size || bytes > size - (q - b)) return LOGP_ERR_RANGE;
    return LOGP_OK;
}

// Checks that every non-null span lives on one device, that no output overlaps another
// span (an exact alias listed in `allowed_alias` excepted), and that the stream belongs to
// that device.  On success *device is the device to launch on.
logp_status_t check_buffers(const Span* in, int n_in, const Span* out, int n_out,
                            hipStream_t stream, int* device, Span allowed_alias = {nullptr, 0}) {
    int dev = -1;
    for (int i = 0; i < n_in + n_out; ++i) {
        const Span s = i < n_in ? in[i] : out[i - n_in];
        if (s.p == nullptr || s.bytes == 0) continue;
        int d = -1;
        const logp_status_t st = locate(s.p, s.bytes, &d);
        if (st != LOGP_OK) return st;
        if (dev < 0) dev = d;
        if (d != dev) return LOGP_ERR_DEVICE;
    }
    for (int o = 0; o < n_out; ++o) {
        for (int i = 0; i < n_in; ++i) {
            if (allowed_alias.p != nullptr && out[o].p == allowed_alias.p &&
                in[i].p == allowed_alias.p && out[o].bytes == in[i].bytes)
                continue;
            if (overlaps(out[o], in[i])) return LOGP_ERR_OVERLAP;
        }
        for (int k = o + 1; k < n_out; ++k)
            if (overlaps(out[o], out[k])) return LOGP_ERR_OVERLAP;
    }
    if (stream != nullptr) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice(stream, &sd) != hipSuccess) {
            (void)hipGetLastError();
            return LOGP_ERR_DEVICE;
        }
        if (dev >= 0 && static_cast<int>(sd) != dev) return LOGP_ERR_DEVICE;
    }
    *device = dev;
    return LOGP_OK;
}

// Makes `device` current for the lifetime of the guard and restores the previous one.
class DeviceGuard {
  public:
    explicit DeviceGuard(int device) {
        if (hipGetDevice(&prev_) != hipSuccess) {
            (void)hipGetLastError();
            ok_ = false;
            return;
        }
        if (device >= 0 && device != prev_) {
            ok_ = hipSetDevice(device) == hipSuccess;
            changed_ = ok_;
            if (!ok_) (void)hipGetLastError();
        }
    }
    ~DeviceGuard() {
        if (changed_) (void)hipSetDevice(prev_);
    }
    bool ok() const { return ok_; }

  private:
    int prev_ = -1;
    bool changed_ = false;
    bool ok_ = true;
};

logp_status_t launch(const void* kernel, dim3 grid, dim3 block, void** args, size_t lds,
                     hipStream_t stream) {
    if (hipLaunchKernel(kernel, grid, block, args, lds, stream) != hipSuccess) {
        (void)hipGetLastError();
        return LOGP_ERR_HIP;
    }
    return LOGP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

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

}  // namespace

// ============================================================================ C ABI

extern "C" {

int64_t logp_num_tiles(int64_t vocab_padded) {
    return vocab_padded < 1 ? 0 : ceil_div(vocab_padded, kTile);
}

const char* logp_status_string(logp_status_t status) {
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
    }
    return "unknown status";
}

logp_status_t logp_forward(const uint16_t* logits, int64_t ld, int64_t n, int64_t vocab_real,
                           int64_t vocab_padded, const int64_t* targets, const uint8_t* active,
                           int64_t ignore_index, float* logp, float* lse, logp_stats_t* stats,
                           hipStream_t stream) {
    logp_status_t st = check_vocab(n, vocab_real, vocab_padded);
    if (st != LOGP_OK) return st;
    if (ld < vocab_padded || logp_num_tiles(vocab_padded) > LOGP_FWD_MAX_TILES)
        return LOGP_ERR_SHAPE;
    if (n > 0x7FFFFFFF) return LOGP_ERR_SHAPE;  // one workgroup per row on a 1-D grid
    if (n == 0) return LOGP_OK;
    if (logits == nullptr || targets == nullptr || logp == nullptr) return LOGP_ERR_NULL;
    const uint64_t lg_bytes = span_bytes(n, ld, vocab_real, 2);
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
    void* args[] = {&logits, &ld, &vr, &targets, &active, &ignore_index, &logp, &lse, &stats};
    const bool vec = aligned16(logits) && (ld % kVec) == 0;
    const void* k = vec ? reinterpret_cast<const void*>(&fwd_kernel<true>)
                        : reinterpret_cast<const void*>(&fwd_kernel<false>);
    const size_t lds = size_t(ceil_div(vocab_real, kTile)) * sizeof(float2);
    return launch(k, dim3(static_cast<uint32_t>(n)), dim3(kFwdWaves * kWave), args, lds, stream);
}

logp_status_t logp_backward(const uint16_t* logits, int64_t ld, int64_t n, int64_t vocab_real,
                            int64_t vocab_padded, int64_t col_begin, int64_t col_end,
                            const int64_t* targets, const uint8_t* active, int64_t ignore_index,
                            const float* grad_logp, const logp_stats_t* stats, uint16_t* dlogits,
                            int64_t ld_out, hipStream_t stream) {
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
    const uint32_t grid = item_grid(n, view_tiles, kBwdWaves * kBwdTilesPerWave);
    const uint64_t in_bytes = span_bytes(n, ld, lim, 2);
    const uint64_t out_bytes = span_bytes(n, ld_out, width, 2);
    if (grid == 0 || out_bytes == 0 || (lim > 0 && in_bytes == 0)) return LOGP_ERR_SHAPE;
    // In place is allowed only as an exact alias with the same row stride.
    Span alias = {nullptr, 0};
    if (static_cast<const void*>(dlogits) == static_cast<const void*>(logits) && ld_out == ld)
        alias = {logits, in_bytes};
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

    int vt = static_cast<int>(view_tiles), w = static_cast<int>(width), li = static_cast<int>(lim);
    void* args[] = {&logits, &ld, &n, &vt, &w, &li, &col_begin, &vocab_real, &targets, &active,
                    &ignore_index, &grad_logp, &stats, &dlogits, &ld_out};
    const bool vin = aligned16(logits) && (ld % kVec) == 0;
    const bool vout = aligned16(dlogits) && (ld_out % kVec) == 0;
    if (vin && vout && width % kVec == 0 && width >= kTile) {
        const int64_t vectors = n * (width / kVec);
        const int64_t per_block = int64_t(kBwdWaves) * kWave * kLoads;  // 512 vectors per wave
        const int64_t blocks = ceil_div(vectors, per_block);
        if (blocks > 0x7FFFFFFF) return LOGP_ERR_SHAPE;
        int vpr = static_cast<int>(width / kVec), li = static_cast<int>(lim);
        void* fargs[] = {&logits, &ld, &n, &vpr, &li, &col_begin, &vocab_real, &targets,
                         &active, &ignore_index, &grad_logp, &stats, &dlogits, &ld_out};
        return launch(reinterpret_cast<const void*>(&bwd_flat_kernel),
                      dim3(static_cast<uint32_t>(blocks)), dim3(kBwdWaves * kWave), fargs, 0,
                      stream);
    }
    const void* k = vin ? (vout ? reinterpret_cast<const void*>(&bwd_kernel<true, true>)
                                : reinterpret_cast<const void*>(&bwd_kernel<true, false>))
                        : (vout ? reinterpret_cast<const void*>(&bwd_kernel<false, true>)
                                : reinterpret_cast<const void*>(&bwd_kernel<false, false>));
    return launch(k, dim3(grid), dim3(kBwdWaves * kWave), args, 0, stream);
}

logp_status_t logp_partials(const uint16_t* logits, int64_t ld, int64_t n, int64_t vocab_real,
                            int64_t vocab_padded, int64_t col_begin, int64_t col_end,
                            const int64_t* targets, const uint8_t* active, int64_t ignore_index,
                            logp_partial_t* partials, int64_t ldp, hipStream_t stream) {
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
    const uint64_t in_bytes = span_bytes(n, ld, lim, 2);
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
    void* args[] = {&logits, &ld, &n, &vt, &li, &col_begin, &col_end, &vocab_real, &targets,
                    &active, &ignore_index, &partials, &ldp};
    const bool vec = aligned16(logits) && (ld % kVec) == 0;
    const void* k = vec ? reinterpret_cast<const void*>(&partials_kernel<true>)
                        : reinterpret_cast<const void*>(&partials_kernel<false>);
    return launch(k, dim3(grid), dim3(kItemWaves * kWave), args, 0, stream);
}

logp_status_t logp_merge(const logp_partial_t* partials, int64_t ldp, int64_t n,
                         int64_t num_tiles, int64_t vocab_real, const int64_t* targets,
                         const uint8_t* active, int64_t ignore_index, float* logp, float* lse,
                         logp_stats_t* stats, hipStream_t stream) {
    if (n < 0 || vocab_real < 1 || vocab_real > kMaxCols || num_tiles < ceil_div(vocab_real, kTile) ||
        num_tiles > ceil_div(kMaxCols, kTile) || ldp < num_tiles)
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
