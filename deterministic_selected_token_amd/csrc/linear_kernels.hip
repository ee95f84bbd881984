// gfx950 kernel and C entry point of the fused LM-head + selected-token log-probability
// (include/linear_logp.h).
//
// One workgroup (8 waves) per (block of 256 rows, global vocab tile of 4096 columns).  It walks
// the tile in 16 sub-blocks of 256 columns; for each it forms the 256 x 256 logits block on the
// matrix cores (v_mfma_f32_32x32x16_bf16, FP32 accumulation over the hidden dimension; each
// wave holds a 64 x 128 block; the hidden states and weight rows are staged through
// double-buffered LDS with the next stage's global loads in flight), reduces the block to a
// per-row (max, sum-exp) through LDS (half the rows at a time, 4 threads per row over 64
// columns each, then a 2-level lane tree), and folds it into the row's running tile state in
// LDS.  After the last sub-block the tile's (m, s, sel) partial is written in logp.h's layout,
// and logp_merge completes the forward.  The logits never leave the chip.
//
// Sources: PR #495 (Summary) names the fused LM-head + logp op; issue #241 ("PR 3", "PR6")
// and PR #314 (Tensor Parallel doc) fix the per-tile partials and their merge.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "host_common.hpp"
#include "linear_logp.h"
#include "logp_device.hpp"

using namespace logp;
using namespace logp_host;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

constexpr int kWM = 4, kWN = 2;               // waves along rows / columns
constexpr int kTM = 2, kTN = 4;               // 32 x 32 MFMA tiles per wave along rows / cols
constexpr int kThreads = kWM * kWN * kWave;   // 512
constexpr int kBM = kWM * kTM * 32;           // rows per workgroup
constexpr int kBN = kWN * kTN * 32;           // columns per sub-block
constexpr int kBK = 64;                       // hidden elements per LDS stage
constexpr int kRow = kBK + 8;                 // LDS row stride in elements (144 bytes)
constexpr int kSubBlocks = kTile / kBN;       // sub-blocks per vocab tile
constexpr int kChunksA = kBM * kBK / 8 / kThreads;  // 16-byte chunks per thread per stage
constexpr int kChunksB = kBN * kBK / 8 / kThreads;
constexpr int kChunksPerRow = kBK / 8;

// Sub-block reduction through LDS: half a row block (kBM / kTM rows) at a time, kRedThreads
// threads per row, each reducing kRedCols columns.
constexpr int kHalfRows = kWM * 32;
constexpr int kRedThreads = kThreads / kHalfRows;     // 4
constexpr int kRedCols = kBN / kRedThreads;           // 64
constexpr int kRedRow = kBN + 32;                     // floats per LDS row (bank spread)

static_assert(kChunksA * kThreads * 8 == kBM * kBK, "A stage is whole chunks per thread");
static_assert(kChunksB * kThreads * 8 == kBN * kBK, "B stage is whole chunks per thread");
static_assert(kTile % kBN == 0, "a vocab tile is whole sub-blocks");
static_assert(kRedCols % 4 == 0 && kHalfRows * kRedThreads == kThreads, "reduction layout");

// The stage arrays are 16-byte aligned so their 16-byte chunks move as single ds_read_b128 /
// ds_write_b128 instructions.
struct alignas(16) Smem {
    alignas(16) uint16_t a[2][kBM * kRow];  // hidden-state stage, [row][k]
    alignas(16) uint16_t b[2][kBN * kRow];  // weight stage, [vocab row][k]
    float m[kBM], s[kBM], sel[kBM];  // running tile state per row
    int y_rel[kBM];             // target column inside this tile, or -1
};

// One stage of this thread's chunks in registers (global loads in flight).
struct Stage {
    u32x4v a[kChunksA];
    u32x4v b[kChunksB];
};

static_assert(sizeof(float) * kHalfRows * kRedRow <= sizeof(Smem::a) + sizeof(Smem::b),
              "the reduction area fits in the stage buffers");

// Loads this thread's 16-byte chunks of one stage: rows [0, kBM) of the hidden-state block at
// `hb` (n_here of them real) and rows [col0, col0 + kBN) of the weight tile at `wb` (lim_here
// real), hidden elements [k0, k0 + kBK); out-of-range chunks are zero.  Offsets from the two
// wave-uniform bases are 32-bit.
__device__ __forceinline__ void load_stage(const uint16_t* __restrict__ hb, uint32_t ld_h,
                                           int n_here, const uint16_t* __restrict__ wb,
                                           uint32_t ld_w, int lim_here, int H, int col0, int k0,
                                           Stage& st) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
        const int q = t + i * kThreads;
        const int r = q / kChunksPerRow, k = k0 + (q % kChunksPerRow) * 8;
        st.a[i] = (r < n_here && k < H)
                      ? *reinterpret_cast<const u32x4v*>(hb + (uint32_t(r) * ld_h + uint32_t(k)))
                      : u32x4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) {
        const int q = t + i * kThreads;
        const int r = q / kChunksPerRow, k = k0 + (q % kChunksPerRow) * 8;
        const int col = col0 + r;
        st.b[i] = (col < lim_here && k < H)
                      ? *reinterpret_cast<const u32x4v*>(wb + (uint32_t(col) * ld_w + uint32_t(k)))
                      : u32x4v{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_stage(Smem& sm, int buf, const Stage& st) {
    const u32x4v (&ra)[kChunksA] = st.a;
    const u32x4v (&rb)[kChunksB] = st.b;
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
        const int q = t + i * kThreads;
        *reinterpret_cast<u32x4v*>(&sm.a[buf][(q / kChunksPerRow) * kRow +
                                              (q % kChunksPerRow) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) {
        const int q = t + i * kThreads;
        *reinterpret_cast<u32x4v*>(&sm.b[buf][(q / kChunksPerRow) * kRow +
                                              (q % kChunksPerRow) * 8]) = rb[i];
    }
}

// The matrix-core steps of one LDS stage: kBK / 16 steps of k, each wave's kTM x kTN tiles.
__device__ __forceinline__ void mma_stage(const Smem& sm, int buf, int wm, int wn, int lane,
                                          f32x16 (&acc)[kTM][kTN]) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
        const int k = ks * 16 + 8 * (lane >> 5);
        bf16x8 fa[kTM], fb[kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
            fa[i] = *reinterpret_cast<const bf16x8*>(
                &sm.a[buf][(wm * kTM * 32 + i * 32 + (lane & 31)) * kRow + k]);
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            fb[j] = *reinterpret_cast<const bf16x8*>(
                &sm.b[buf][(wn * kTN * 32 + j * 32 + (lane & 31)) * kRow + k]);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                acc[i][j] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
}

// 8 waves per workgroup (148 KB of LDS, one workgroup per CU): two waves per SIMD cover each
// other's global-load latency.
// SCALED = false is the unit temperature: the multiply by inv_t (exact at 1) is left out, as
// it lengthens the epilogue, which no matrix-core work overlaps.
template <bool SCALED>
__global__ __launch_bounds__(kThreads) void linear_partials_kernel(
    const uint16_t* __restrict__ h, int64_t ld_h, int64_t n, int H,
    const uint16_t* __restrict__ w, int64_t ld_w, int lim, int row_blocks, int64_t col_begin,
    int64_t vocab_real, float inv_t, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ active, int64_t ignore_index,
    logp_partial_t* __restrict__ partials, int64_t ldp) {
    __shared__ Smem sm;
    const int rb_idx = static_cast<int>(blockIdx.x % static_cast<uint32_t>(row_blocks));
    const int tile = static_cast<int>(blockIdx.x / static_cast<uint32_t>(row_blocks));
    const int64_t row0 = int64_t(rb_idx) * kBM;
    const int tile_col0 = tile * kTile;  // first view column of the tile
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / kWN, wn = wave % kWN;

    if (threadIdx.x < kBM) {
        const int t = threadIdx.x;
        const int64_t row = row0 + t;
        int yr = -1;
        if (row < n) {
            int64_t y;
            if (row_valid(targets, active, ignore_index, vocab_real, row, y)) {
                const int64_t c = y - col_begin - tile_col0;
                if (c >= 0 && c < kTile) yr = static_cast<int>(c);
            }
        }
        sm.y_rel[t] = yr;
        sm.m[t] = kNegInf;
        sm.s[t] = 0.0f;
        sm.sel[t] = 0.0f;
    }

    // wave-uniform bases of the row block and of the tile's weight rows
    const uint16_t* hb = h + row0 * ld_h;
    const uint16_t* wb = w + int64_t(tile_col0) * ld_w;
    const int n_here = static_cast<int>(std::min<int64_t>(kBM, n - row0));
    const int lim_here = lim - tile_col0;  // real weight rows of the tile (may exceed kTile)
    const uint32_t ldh = static_cast<uint32_t>(ld_h), ldw = static_cast<uint32_t>(ld_w);

    const int nk = (H + kBK - 1) / kBK;
    for (int sb = 0; sb < kSubBlocks; ++sb) {
        const int col0 = sb * kBN;  // first column of the sub-block inside the tile
        f32x16 acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // The global loads of stage kt + 1 are issued before the matrix-core work of stage
        // kt and go to the other LDS buffer after it.
        Stage rs;
        load_stage(hb, ldh, n_here, wb, ldw, lim_here, H, col0, 0, rs);
        store_stage(sm, 0, rs);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk)
                load_stage(hb, ldh, n_here, wb, ldw, lim_here, H, col0, (kt + 1) * kBK, rs);
            mma_stage(sm, cur, wm, wn, lane, acc);
            if (kt + 1 < nk) store_stage(sm, cur ^ 1, rs);
            __syncthreads();
        }

        // ---- sub-block reduction through LDS (the stage buffers are free now), one half of
        // the row block at a time: each wave writes its scored accumulators
        // fl32(acc * inv_t) (masked columns as -inf; inv_t = 1 leaves acc unchanged),
        // then 4 threads per row reduce 64 columns each and combine by a 2-level lane tree.
        float* red = reinterpret_cast<float*>(&sm.a[0][0]);
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int col = wn * (kTN * 32) + j * 32 + (lane & 31);  // in the sub-block
                const bool ok = tile_col0 + sb * kBN + col < lim;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int hr = wm * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
                    const float z = SCALED ? acc[i][j][r] * inv_t : acc[i][j][r];
                    red[hr * kRedRow + col] = ok ? z : kNegInf;
                }
            }
            __syncthreads();
            {
                const int t = threadIdx.x;
                const int hr = t / kRedThreads, part = t % kRedThreads;
                const int row = (hr / 32) * (kTM * 32) + i * 32 + (hr % 32);  // in the block
                // two passes over the row's columns in LDS (max, then the sum), so no row
                // values stay in registers beside the accumulators of the other half
                const int yr = sm.y_rel[row] - sb * kBN;  // target column in the sub-block
                const float* src = &red[hr * kRedRow + 4 * part];
                float mb = kNegInf;
#pragma unroll
                for (int q = 0; q < kRedCols / 4; ++q) {
                    const float4 x = *reinterpret_cast<const float4*>(src + kRedThreads * 4 * q);
                    mb = fmaxf(mb, fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w)));
                }
                // the selected logit: the thread whose columns hold the target picks it up
                if (yr >= 0 && yr < kBN && ((yr >> 2) & (kRedThreads - 1)) == part)
                    sm.sel[row] = red[hr * kRedRow + yr];
#pragma unroll
                for (int o = 1; o < kRedThreads; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o, kWave));
                float ls = 0.0f;
                if (mb != kNegInf) {
#pragma unroll
                    for (int q = 0; q < kRedCols / 4; ++q) {
                        const float4 x =
                            *reinterpret_cast<const float4*>(src + kRedThreads * 4 * q);
                        ls = ls + (x.x == kNegInf ? 0.0f : fwd_exp(x.x - mb));
                        ls = ls + (x.y == kNegInf ? 0.0f : fwd_exp(x.y - mb));
                        ls = ls + (x.z == kNegInf ? 0.0f : fwd_exp(x.z - mb));
                        ls = ls + (x.w == kNegInf ? 0.0f : fwd_exp(x.w - mb));
                    }
                }
#pragma unroll
                for (int o = 1; o < kRedThreads; o <<= 1) ls = ls + __shfl_xor(ls, o, kWave);
                if (part == 0) {
                    const float m_old = sm.m[row];
                    const float m_new = fmaxf(m_old, mb);
                    const float a = m_old == kNegInf ? 0.0f : sm.s[row] * fwd_exp(m_old - m_new);
                    const float b = mb == kNegInf ? 0.0f : ls * fwd_exp(mb - m_new);
                    sm.m[row] = m_new;
                    sm.s[row] = a + b;
                }
            }
            __syncthreads();
        }
        // the next sub-block's first barrier orders these LDS updates before any reuse
    }
    __syncthreads();
    if (threadIdx.x < kBM) {
        const int t = threadIdx.x;
        const int64_t row = row0 + t;
        if (row < n) {
            logp_partial_t p;
            p.max = sm.m[t];
            p.sumexp = sm.s[t];
            p.sel = sm.sel[t];
            partials[row * ldp + tile] = p;
        }
    }
}

}  // namespace

extern "C" {

logp_status_t linear_logp_partials_ex(float inv_temperature, const uint16_t* hidden,
                                      int64_t ld_h, int64_t n, int64_t hidden_size,
                                      const uint16_t* weight, int64_t ld_w, int64_t vocab_real,
                                      int64_t vocab_padded, int64_t col_begin, int64_t col_end,
                                      const int64_t* targets, const uint8_t* active,
                                      int64_t ignore_index, logp_partial_t* partials,
                                      int64_t ldp, hipStream_t stream) {
    if (!(inv_temperature > 0.0f) || !std::isfinite(inv_temperature)) return LOGP_ERR_ARG;
    if (n < 0 || vocab_real < 1 || vocab_padded < vocab_real ||
        vocab_padded > (int64_t(1) << 31) - 1 - kTile)
        return LOGP_ERR_SHAPE;
    if (col_begin < 0 || col_end < col_begin || col_end > vocab_padded ||
        col_begin % kTile != 0 || (col_end % kTile != 0 && col_end != vocab_padded))
        return LOGP_ERR_SHARD;
    if (n == 0 || col_end == col_begin) return LOGP_OK;
    if (hidden == nullptr || weight == nullptr || targets == nullptr || partials == nullptr)
        return LOGP_ERR_NULL;
    const int64_t H = hidden_size;
    if (H < 1 || H > LINEAR_LOGP_MAX_HIDDEN || H % 8 != 0 || ld_h < H || ld_w < H ||
        ld_h % 8 != 0 || ld_w % 8 != 0 || ld_h > LINEAR_LOGP_MAX_LD ||
        ld_w > LINEAR_LOGP_MAX_LD || !aligned16(hidden) || !aligned16(weight))
        return LOGP_ERR_SHAPE;
    // in-kernel offsets from a row block's or a tile's first row are 32-bit
    static_assert(uint64_t(kTile) * LINEAR_LOGP_MAX_LD < (uint64_t(1) << 32), "tile offsets");
    static_assert(uint64_t(kBM) * LINEAR_LOGP_MAX_LD < (uint64_t(1) << 32), "block offsets");
    const int64_t width = col_end - col_begin;
    const int64_t view_tiles = ceil_div(width, kTile);
    if (ldp < view_tiles) return LOGP_ERR_SHAPE;
    if (n > (int64_t(1) << 40) / ld_h) return LOGP_ERR_SHAPE;
    // weight rows actually read: the view's real vocabulary rows
    const int64_t lim = std::max<int64_t>(0, std::min(width, vocab_real - col_begin));
    const Span in[] = {{hidden, span_bytes(n, ld_h, H, 2)},
                       {weight, lim > 0 ? span_bytes(lim, ld_w, H, 2) : 0},
                       {targets, uint64_t(n) * 8},
                       {active, active ? uint64_t(n) : 0}};
    const Span out[] = {{partials, span_bytes(n, ldp, view_tiles, sizeof(logp_partial_t))}};
    int dev = -1;
    logp_status_t st = check_buffers(in, 4, out, 1, stream, &dev);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;
    const int64_t row_blocks = ceil_div(n, kBM);
    if (row_blocks * view_tiles > 0x7FFFFFFF) return LOGP_ERR_SHAPE;
    int Hi = static_cast<int>(H), lim_i = static_cast<int>(lim);
    int rbk = static_cast<int>(row_blocks);
    void* args[] = {&hidden,    &ld_h,       &n,     &Hi,     &weight,       &ld_w,
                    &lim_i,     &rbk,        &col_begin,     &vocab_real,   &inv_temperature,
                    &targets,   &active,     &ignore_index,  &partials,     &ldp};
    const void* kernel = inv_temperature == 1.0f
                             ? reinterpret_cast<const void*>(&linear_partials_kernel<false>)
                             : reinterpret_cast<const void*>(&linear_partials_kernel<true>);
    return launch(kernel, dim3(static_cast<uint32_t>(row_blocks * view_tiles)), dim3(kThreads),
                  args, 0, stream);
}

logp_status_t linear_logp_partials(const uint16_t* hidden, int64_t ld_h, int64_t n,
                                   int64_t hidden_size, const uint16_t* weight, int64_t ld_w,
                                   int64_t vocab_real, int64_t vocab_padded, int64_t col_begin,
                                   int64_t col_end, const int64_t* targets, const uint8_t* active,
                                   int64_t ignore_index, logp_partial_t* partials, int64_t ldp,
                                   hipStream_t stream) {
    return linear_logp_partials_ex(1.0f, hidden, ld_h, n, hidden_size, weight, ld_w, vocab_real,
                                   vocab_padded, col_begin, col_end, targets, active,
                                   ignore_index, partials, ldp, stream);
}

}  // extern "C"
