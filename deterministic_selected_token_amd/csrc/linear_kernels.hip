// gfx950 kernel and C entry point of the fused LM-head + selected-token log-probability
// (include/linear_logp.h).
//
// One workgroup (8 waves) per (block of 256 rows, global vocab tile of 4096 columns).  It walks
// the tile in 16 sub-blocks of 256 columns; for each it forms the 256 x 256 logits block on the
// matrix cores (v_mfma_f32_32x32x16_bf16, FP32 accumulation over the hidden dimension; each
// wave holds a 64 x 128 block; the hidden states and weight rows are staged through
// double-buffered LDS by direct-to-LDS buffer loads, and the two groups of four waves
// alternate between reading fragments from LDS and feeding the matrix cores), reduces the
// block to a per-row (max, sum-exp) through LDS (half the rows at a time, 4 threads per row
// over 64 columns each, then a 2-level lane tree), and folds it into the row's running tile
// state in LDS.  After the last sub-block the tile's (m, s, sel) partial is written in logp.h's
// layout, and logp_merge completes the forward.  The logits never leave the chip.  With a
// workspace the launch's last rounds are balanced: the remaining tiles' sub-blocks spread over
// every CU and are folded afterwards in the same order (linear_split_kernel,
// linear_fold_kernel).  The backward recomputes each logits block with the same product and
// forms dh and dW with TN products (linear_dz_kernel, gemm_tn_kernel).
//
// Sources: PR #495 (Summary) names the fused LM-head + logp op; issue #241 ("PR 3", "PR6")
// and PR #314 (Tensor Parallel doc) fix the per-tile partials and their merge.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <mutex>
#include <type_traits>

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
constexpr int kSubBlocks = kTile / kBN;       // sub-blocks per vocab tile
constexpr int kChunksA = kBM * kBK / 8 / kThreads;  // 16-byte chunks per thread per stage
constexpr int kChunksB = kBN * kBK / 8 / kThreads;  // (= load instructions per wave)

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

// Stage layout: [row][64 hidden elements], 128-byte rows with no padding; the 16-byte chunk c of
// row r sits at position c ^ swz(r), so that the 16 consecutive rows a fragment read touches
// fall in distinct banks.  The stages are filled by direct-to-LDS buffer loads (each wave
// instruction writes 64 consecutive 16-byte slots); out-of-range chunks load as zero.
constexpr int kStageA = kBM * kBK, kStageB = kBN * kBK;  // elements
constexpr int kRedBytes = int(sizeof(float)) * kHalfRows * kRedRow;
constexpr int kStageBytes = 2 * 2 * (kStageA + kStageB);
constexpr int kPadElems = kRedBytes > kStageBytes ? (kRedBytes - kStageBytes) / 2 : 0;
struct alignas(16) Smem {
    alignas(16) uint16_t a[2][kStageA];  // hidden-state stage
    alignas(16) uint16_t b[2][kStageB];  // weight stage
    uint16_t pad[kPadElems];             // the reduction area overlays a, b and pad
    float m[kBM], s[kBM], sel[kBM];  // running tile state per row
    int y_rel[kBM];             // target column inside this tile, or -1
};
static_assert(kRedBytes <= kStageBytes + 2 * kPadElems, "the reduction area fits");

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

typedef __attribute__((address_space(3))) void* lds_vptr;
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every range: loads zero

// The stage loads of one operand block (rows [0, rows) of `base`, row stride ld, H valid
// elements per row): each load instruction of a wave covers 8 rows, through a buffer resource
// of its own whose range ends at the last valid element of those rows.  The lane offset is the
// same for every group (a lane whose row lies past the group's valid rows is past the range,
// since ld >= H), so the offsets stay small and out-of-range chunks load as zero.
template <int N>
struct OperandLoads {
    __amdgpu_buffer_rsrc_t rs[N];
    uint32_t off;  // this lane's byte offset inside its 8-row group at k0 = 0
};

template <int N>
__device__ __forceinline__ void plan_operand(const uint16_t* base, uint32_t ld, int rows, int H,
                                             int wave, int lane, int c,
                                             OperandLoads<N>& ol) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int r0 = (i * (kThreads / kWave) + wave) * 8;
        const int here = std::min(8, std::max(0, rows - r0));
        const uint32_t bytes = here > 0 ? (uint32_t(here - 1) * ld + uint32_t(H)) * 2u : 0u;
        ol.rs[i] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(base) + int64_t(r0) * ld, 0, static_cast<int>(bytes),
            0x00020000);
    }
    ol.off = (uint32_t(lane >> 3) * ld + uint32_t(8 * c)) * 2u;
}

template <int N>
__device__ __forceinline__ void issue_operand(uint16_t* stage, const OperandLoads<N>& ol,
                                              bool k_ok, int k0, int wave) {
#pragma unroll
    for (int i = 0; i < N; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ol.rs[i], (lds_vptr)&stage[(i * (kThreads / kWave) + wave) * 512], 16,
            k_ok ? ol.off + 2u * uint32_t(k0) : kOob, 0, 0, 0);
}

// Ping-pong block product.  The 8 waves form two groups of four, one wave of each group per
// SIMD (waves 0-3 and 4-7).  A stage of kBK hidden elements is worked in two phases of
// kBK / 32 MFMA k-steps; each group alternates between reading a phase's fragments from LDS
// into registers and running that phase's MFMAs back to back, the second group one phase
// behind the first, with a workgroup barrier between phases: while one wave of a SIMD feeds
// the matrix core, the other reads LDS.  Stage s + 2's direct-to-LDS loads go into stage s's
// buffer once both groups have read it: the second group issues its half right after its own
// last read of stage s, the first group its half one phase later; each waits for its loads
// just before the barrier that precedes the first read of that stage.
constexpr int kKsPhase = 2;                    // MFMA k-steps per phase
constexpr int kPhases = kBK / 16 / kKsPhase;   // phases per stage
static_assert(kPhases == 2, "two phases per stage");

struct Frags {
    bf16x8 a[kKsPhase][kTM];
    bf16x8 b[kKsPhase][kTN];
};

typedef __attribute__((address_space(3))) const char lds_cchar;
typedef __attribute__((address_space(3))) const bf16x8 lds_frag;

// Byte offsets inside the shared block of this lane's fragment rows for each k-step of a stage
// (buffer 0, tile 0): one register per k-step and operand; the buffer and tile offsets are
// constants small enough for the instructions' offset field.  Loads go through a pointer
// derived from the block itself, so the compiler knows they may alias the direct-to-LDS writes.
struct FragAddr {
    uint32_t a[kKsPhase * kPhases], b[kKsPhase * kPhases];
};

__device__ __forceinline__ FragAddr frag_addr(int wm, int wn, int lane) {
    const int q = (lane >> 5) ^ swz(lane & 31);
    const uint32_t a0 =
        uint32_t(offsetof(Smem, a)) + uint32_t((wm * kTM * 32 + (lane & 31)) * kBK * 2);
    const uint32_t b0 =
        uint32_t(offsetof(Smem, b)) + uint32_t((wn * kTN * 32 + (lane & 31)) * kBK * 2);
    FragAddr fa;
#pragma unroll
    for (int ks = 0; ks < kKsPhase * kPhases; ++ks) {
        fa.a[ks] = a0 + uint32_t(((2 * ks) ^ q) * 16);
        fa.b[ks] = b0 + uint32_t(((2 * ks) ^ q) * 16);
    }
    return fa;
}

template <int BUF, int HALF>
__device__ __forceinline__ void read_frags(const Smem& sm, const FragAddr& fa, Frags& f) {
    lds_cchar* base = (lds_cchar*)(&sm);
#pragma unroll
    for (int kk = 0; kk < kKsPhase; ++kk) {
        const int ks = HALF * kKsPhase + kk;
#pragma unroll
        for (int i = 0; i < kTM; ++i)
            f.a[kk][i] = *(lds_frag*)(base + fa.a[ks] + (BUF * kStageA + i * 32 * kBK) * 2);
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            f.b[kk][j] = *(lds_frag*)(base + fa.b[ks] + (BUF * kStageB + j * 32 * kBK) * 2);
    }
}

__device__ __forceinline__ void mma_frags(const Frags& f, f32x16 (&acc)[kTM][kTN]) {
#pragma unroll
    for (int kk = 0; kk < kKsPhase; ++kk)
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][i], f.b[kk][j],
                                                                   acc[i][j], 0, 0, 0);
}

// A workgroup barrier that also keeps the compiler from moving memory accesses across it (a
// wavefront-scope fence orders them for the compiler and emits no wait).
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// acc += the 256 x 256 block of A B^T for rows [0, n_here) of `hb` and rows
// [col0, col0 + kBN) of `wb` (rows at or past lim_here and hidden elements at or past H read
// as zero), in nk stages of kBK hidden elements: the one fixed accumulation order of every
// logit (k ascending into each accumulator), shared by the forward and the backward's
// recomputation.  Every wave passes the same number of barriers (4 nk + 2); afterwards no
// load is in flight and the stage buffers are free.
__device__ __forceinline__ void block_product(Smem& sm, const uint16_t* __restrict__ hb,
                                              uint32_t ldh, int n_here,
                                              const uint16_t* __restrict__ wb, uint32_t ldw,
                                              int lim_here, int H, int col0, int nk, int wm,
                                              int wn, int lane, f32x16 (&acc)[kTM][kTN]) {
    const int wave = wm * kWN + wn;
    const bool second = wave >= kThreads / kWave / 2;
    // the chunk a lane loads: position lane & 7 of row lane >> 3 of an 8-row group, whose
    // swizzle is (lane >> 3) ^ (wave & 1) (group bases are multiples of 8; odd groups flip)
    const int c = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
    OperandLoads<kChunksA> la;
    OperandLoads<kChunksB> lb;
    plan_operand(hb, ldh, n_here, H, wave, lane, c, la);
    plan_operand(wb + int64_t(col0) * ldw, ldw, std::min(kBN, lim_here - col0), H, wave, lane,
                 c, lb);
    constexpr int kPerStage = kChunksA + kChunksB;  // load instructions per wave per stage
    static_assert(kPerStage == 8, "vmcnt immediates below assume 8 loads per stage");
    issue_operand(sm.a[0], la, 8 * c < H, 0, wave);
    issue_operand(sm.b[0], lb, 8 * c < H, 0, wave);
    if (nk > 1) {
        issue_operand(sm.a[1], la, kBK + 8 * c < H, kBK, wave);
        issue_operand(sm.b[1], lb, kBK + 8 * c < H, kBK, wave);
        __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): this wave's part of stage 0 landed
    } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    const FragAddr fa = frag_addr(wm, wn, lane);
    phase_barrier();
    if (second) phase_barrier();  // the second group runs one phase behind
    Frags f;
    // stage s, phase HALF of buffer BUF: read, issue / wait loads, barrier, MFMAs, barrier
    auto phase = [&](int s, auto buf_c, auto half_c) {
        constexpr int BUF = decltype(buf_c)::value, HALF = decltype(half_c)::value;
        read_frags<BUF, HALF>(sm, fa, f);
        // the second half's reads must be done before the barrier (the buffer is reloaded in
        // the next phase); the first half's may finish while the barrier synchronizes
        if (HALF == 1) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        if (second && HALF == 1) {
            // this group read stage s last: stage s + 2 may go into its buffer; then its part
            // of stage s + 1 must have landed before the next barrier (the first group reads
            // stage s + 1 right after it)
            if (s + 2 < nk) {
                const int k0 = (s + 2) * kBK;
                issue_operand(sm.a[BUF], la, k0 + 8 * c < H, k0, wave);
                issue_operand(sm.b[BUF], lb, k0 + 8 * c < H, k0, wave);
                __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
            } else {
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            }
        }
        if (!second && HALF == 0 && s >= 1 && s + 1 < nk) {
            // the second group finished stage s - 1 one phase ago: stage s + 1 into its buffer
            const int k0 = (s + 1) * kBK;
            issue_operand(sm.a[BUF ^ 1], la, k0 + 8 * c < H, k0, wave);
            issue_operand(sm.b[BUF ^ 1], lb, k0 + 8 * c < H, k0, wave);
        }
        phase_barrier();
        if (HALF == 0) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_setprio(1);
        mma_frags(f, acc);
        __builtin_amdgcn_s_setprio(0);
        if (!second && HALF == 1)
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this group's part of stage s + 1
        phase_barrier();
    };
    int s = 0;
    for (; s + 1 < nk; s += 2) {
        phase(s, std::integral_constant<int, 0>(), std::integral_constant<int, 0>());
        phase(s, std::integral_constant<int, 0>(), std::integral_constant<int, 1>());
        phase(s + 1, std::integral_constant<int, 1>(), std::integral_constant<int, 0>());
        phase(s + 1, std::integral_constant<int, 1>(), std::integral_constant<int, 1>());
    }
    if (s < nk) {
        phase(s, std::integral_constant<int, 0>(), std::integral_constant<int, 0>());
        phase(s, std::integral_constant<int, 0>(), std::integral_constant<int, 1>());
    }
    if (!second) phase_barrier();
}

// One step of the tile's fold over its sub-blocks (the contract's order, b = 0 .. 15):
// (m, s) <- (max(m, mb), s exp(m - m') + ls exp(mb - m')), terms of -inf maxima are 0.
__device__ __forceinline__ void fold_subblock(float& m, float& s, float mb, float ls) {
    const float m_new = fmaxf(m, mb);
    const float a = m == kNegInf ? 0.0f : s * fwd_exp(m - m_new);
    const float b = mb == kNegInf ? 0.0f : ls * fwd_exp(mb - m_new);
    m = m_new;
    s = a + b;
}

// Reduction of one 256 x 256 sub-block of scored logits (this wave's accumulators) through
// LDS (the stage buffers are free when it starts; it ends with a barrier after the last LDS
// read), one half of the row block at a time: each wave writes fl32(acc * inv_t) (masked
// columns as -inf; inv_t = 1 leaves acc unchanged), then 4 threads per row reduce 64 columns
// each and combine by a 2-level lane tree.  For each row r of the block (0..255):
// on_sel(r, z) with the target's scored logit when the row's target column in the tile
// (y_rel[r]) lies in this sub-block, and on_stats(r, mb, ls) with the sub-block's max and
// sum-exp, both from one thread.  col_tile0: the sub-block's first column in the tile;
// lim_tile: the tile's real columns (columns at or past it are masked).  on_z(r, c, x), when
// given, receives every scored logit once, four at a time: columns c .. c + 3 of the sub-block
// in row r (masked columns as -inf).
struct NoZ {
    __device__ void operator()(int, int, const float4&) const {}
};
template <bool SCALED, typename OnSel, typename OnStats, typename OnZ = NoZ>
__device__ __forceinline__ void reduce_subblock(Smem& sm, f32x16 (&acc)[kTM][kTN], int wm,
                                                int wn, int lane, float inv_t, int col_tile0,
                                                int lim_tile, const int* y_rel, OnSel on_sel,
                                                OnStats on_stats, OnZ on_z = OnZ()) {
    float* red = reinterpret_cast<float*>(&sm.a[0][0]);
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int col = wn * (kTN * 32) + j * 32 + (lane & 31);  // in the sub-block
            const bool ok = col_tile0 + col < lim_tile;
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
            // two passes over the row's columns in LDS (max, then the sum), so no row values
            // stay in registers beside the accumulators of the other half
            const int yr = y_rel[row] - col_tile0;  // target column in the sub-block
            const float* src = &red[hr * kRedRow + 4 * part];
            float mb = kNegInf;
#pragma unroll
            for (int q = 0; q < kRedCols / 4; ++q) {
                const float4 x = *reinterpret_cast<const float4*>(src + kRedThreads * 4 * q);
                mb = fmaxf(fmaxf(mb, x.x), fmaxf(x.y, fmaxf(x.z, x.w)));
                on_z(row, kRedThreads * 4 * q + 4 * part, x);
            }
            // the selected logit: the thread whose columns hold the target picks it up
            if (yr >= 0 && yr < kBN && ((yr >> 2) & (kRedThreads - 1)) == part)
                on_sel(row, red[hr * kRedRow + yr]);
#pragma unroll
            for (int o = 1; o < kRedThreads; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o, kWave));
            float ls = 0.0f;
            if (mb != kNegInf) {
#pragma unroll
                for (int q = 0; q < kRedCols / 4; ++q) {
                    const float4 x = *reinterpret_cast<const float4*>(src + kRedThreads * 4 * q);
                    // exp2(-inf) = +0: a masked column adds +0 without a select
                    ls = ls + fwd_exp(x.x - mb);
                    ls = ls + fwd_exp(x.y - mb);
                    ls = ls + fwd_exp(x.z - mb);
                    ls = ls + fwd_exp(x.w - mb);
                }
            }
#pragma unroll
            for (int o = 1; o < kRedThreads; o <<= 1) ls = ls + __shfl_xor(ls, o, kWave);
            if (part == 0) on_stats(row, mb, ls);
        }
        __syncthreads();
    }
}

// Where the forward writes the scored logits when asked to keep them: z (FP32) with row stride
// ld_z, view column 0 first; rows at or past n and columns at or past width are not written.
struct ZOut {
    float* z;
    int64_t ld_z, n;
    int width;
};

// Four scored logits of row `row` at view columns [vc, vc + 4) (vc a multiple of 4; z 16-byte
// aligned and ld_z a multiple of 4, so whole groups go out as one 16-byte store).  They are
// read back by a later launch, not by this one: streaming stores, non-temporal at device
// scope (`sc1 nt`, as the logp backward's gradient stores: the kept-logits forward ran 8.32
// against 8.52 ms with the non-temporal bit alone, same bits), with the 2 wait states a VALU
// needs before it may write the store's data registers (the compiler does not look inside
// asm).
__device__ __forceinline__ void store_z4(const ZOut& o, int64_t row, int vc, const float4& x) {
    if (row >= o.n || vc >= o.width) return;
    float* p = o.z + row * o.ld_z + vc;
    if (vc + 4 <= o.width) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" : : "v"(p),
                     "v"(f32x4{x.x, x.y, x.z, x.w}) : "memory");
        return;
    }
    p[0] = x.x;
    if (vc + 1 < o.width) p[1] = x.y;
    if (vc + 2 < o.width) p[2] = x.z;
}

// Row constants of one (row block, tile): y_rel[t] = the target's column inside the tile for a
// valid row whose target lies in it, else -1.
// Used by the fold kernel only: in a kernel with a block product, calling it (rather than
// writing the same conditions inline) made the compiler move the product's load descriptors
// to vector registers and wrap every load in a loop over their distinct values.
__device__ __forceinline__ int tile_target(int64_t row, int64_t n, const int64_t* targets,
                                           const uint8_t* active, int64_t ignore_index,
                                           int64_t vocab_real, int64_t tile_view_col0) {
    int yr = -1;
    if (row < n) {
        int64_t y;
        if (row_valid(targets, active, ignore_index, vocab_real, row, y)) {
            const int64_t c = y - tile_view_col0;
            if (c >= 0 && c < kTile) yr = static_cast<int>(c);
        }
    }
    return yr;
}

// 8 waves per workgroup (148 KB of LDS, one workgroup per CU): two waves per SIMD cover each
// other's global-load latency.
// SCALED = false is the unit temperature: the multiply by inv_t (exact at 1) is left out, as
// it lengthens the epilogue, which no matrix-core work overlaps.  SAVE: the scored logits are
// also written to zo (zo is not read otherwise).
template <bool SCALED, bool SAVE>
__global__ __launch_bounds__(kThreads) void linear_partials_kernel(
    const uint16_t* __restrict__ h, int64_t ld_h, int64_t n, int H,
    const uint16_t* __restrict__ w, int64_t ld_w, int lim, int row_blocks, int64_t col_begin,
    int64_t vocab_real, float inv_t, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ active, int64_t ignore_index,
    logp_partial_t* __restrict__ partials, int64_t ldp, ZOut zo) {
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

        block_product(sm, hb, ldh, n_here, wb, ldw, lim_here, H, col0, nk, wm, wn, lane, acc);
        reduce_subblock<SCALED>(
            sm, acc, wm, wn, lane, inv_t, col0, lim_here, sm.y_rel,
            [&](int row, float z) { sm.sel[row] = z; },
            [&](int row, float mb, float ls) { fold_subblock(sm.m[row], sm.s[row], mb, ls); },
            [&](int row, int c, const float4& x) {
                if constexpr (SAVE) store_z4(zo, row0 + row, tile_col0 + col0 + c, x);
            });
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

// ------------------------------------------------------------- balanced last rounds
//
// linear_partials_kernel runs one workgroup per (row block, tile), 16 sub-blocks each, so a
// launch whose workgroup count is not a multiple of the CU count ends with a partly empty
// round that still lasts 16 sub-blocks.  linear_logp_partials_ws runs whole rounds with it
// (tiles [0, tile0)) and spreads the sub-blocks of the remaining tiles over every CU: each
// task computes one sub-block's per-row (max, sum-exp) and target logit into the workspace,
// and linear_fold_kernel folds a tile's sub-blocks in order b = 0, 1, ... with the same
// fold_subblock steps, so the partials are bitwise those of the one-kernel launch (fully
// masked sub-blocks, which leave the fold's state unchanged bit for bit, are not computed).

// Task j: row block j % row_blocks of sub-block pair p = j / row_blocks, which is sub-block
// p % kSubBlocks of tile tile0 + p / kSubBlocks (only the last tile with real columns has
// fewer than kSubBlocks, and its pairs come last).  Workgroup g takes tasks g, g + grid, ...
// With row blocks fastest, the tasks in flight share sub-blocks of W the way the workgroups
// of linear_partials_kernel share tiles.
template <bool SCALED, bool SAVE>
__global__ __launch_bounds__(kThreads) void linear_split_kernel(
    const uint16_t* __restrict__ h, int64_t ld_h, int64_t n, int H,
    const uint16_t* __restrict__ w, int64_t ld_w, int lim, int row_blocks, int64_t col_begin,
    int64_t vocab_real, float inv_t, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ active, int64_t ignore_index, int tile0, int tasks,
    float2* __restrict__ ws_stats, float* __restrict__ ws_sel, ZOut zo) {
    __shared__ Smem sm;
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / kWN, wn = wave % kWN;
    const uint32_t ldh = static_cast<uint32_t>(ld_h), ldw = static_cast<uint32_t>(ld_w);
    const int nk = (H + kBK - 1) / kBK;
    for (int j = static_cast<int>(blockIdx.x); j < tasks; j += static_cast<int>(gridDim.x)) {
        const int rb_idx = j % row_blocks, pair = j / row_blocks;
        const int tile = tile0 + pair / kSubBlocks, sb = pair % kSubBlocks;
        const int64_t row0 = int64_t(rb_idx) * kBM;
        const int tile_col0 = tile * kTile, col0 = sb * kBN;
        // the previous task's reduction ended with a barrier after its last read of y_rel;
        // block_product's barriers order these writes before this task's reduction
        if (threadIdx.x < kBM) {
            const int64_t row = row0 + threadIdx.x;
            int yr = -1;
            if (row < n) {
                int64_t y;
                if (row_valid(targets, active, ignore_index, vocab_real, row, y)) {
                    const int64_t c = y - col_begin - tile_col0;
                    if (c >= 0 && c < kTile) yr = static_cast<int>(c);
                }
            }
            sm.y_rel[threadIdx.x] = yr;
        }
        const uint16_t* hb = h + row0 * ld_h;
        const uint16_t* wb = w + int64_t(tile_col0) * ld_w;
        const int n_here = static_cast<int>(std::min<int64_t>(kBM, n - row0));
        const int lim_here = lim - tile_col0;
        f32x16 acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int jj = 0; jj < kTN; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
        block_product(sm, hb, ldh, n_here, wb, ldw, lim_here, H, col0, nk, wm, wn, lane, acc);
        float2* st = ws_stats + int64_t(j) * kBM;
        float* se = ws_sel + int64_t(j) * kBM;
        reduce_subblock<SCALED>(
            sm, acc, wm, wn, lane, inv_t, col0, lim_here, sm.y_rel,
            [&](int row, float z) { se[row] = z; },
            [&](int row, float mb, float ls) { st[row] = make_float2(mb, ls); },
            [&](int row, int c, const float4& x) {
                if constexpr (SAVE) store_z4(zo, row0 + row, tile_col0 + col0 + c, x);
            });
    }
}

// One workgroup per (row block, tile of [tile0, view_tiles)), one thread per row: the tile's
// partial from its sub-blocks' workspace entries.  nsb_last: sub-blocks of tile real_tiles - 1
// (the last with real columns); tiles at or past real_tiles have none.
__global__ __launch_bounds__(kBM) void linear_fold_kernel(
    int64_t n, int row_blocks, int tile0, int real_tiles, int nsb_last,
    const float2* __restrict__ ws_stats, const float* __restrict__ ws_sel,
    const int64_t* __restrict__ targets, const uint8_t* __restrict__ active,
    int64_t ignore_index, int64_t vocab_real, int64_t col_begin,
    logp_partial_t* __restrict__ partials, int64_t ldp) {
    const int rb_idx = static_cast<int>(blockIdx.x % static_cast<uint32_t>(row_blocks));
    const int tile = tile0 + static_cast<int>(blockIdx.x / static_cast<uint32_t>(row_blocks));
    const int r = threadIdx.x;
    const int64_t row = int64_t(rb_idx) * kBM + r;
    if (row >= n) return;
    const int nsb = tile < real_tiles - 1 ? kSubBlocks : (tile == real_tiles - 1 ? nsb_last : 0);
    const int64_t pair0 = int64_t(tile - tile0) * kSubBlocks;
    float m = kNegInf, s = 0.0f;
    for (int b = 0; b < nsb; ++b) {
        const float2 v = ws_stats[((pair0 + b) * row_blocks + rb_idx) * kBM + r];
        fold_subblock(m, s, v.x, v.y);
    }
    float sel = 0.0f;
    const int yr = tile_target(row, n, targets, active, ignore_index, vocab_real,
                               col_begin + int64_t(tile) * kTile);
    if (yr >= 0) sel = ws_sel[((pair0 + yr / kBN) * row_blocks + rb_idx) * kBM + r];
    logp_partial_t p;
    p.max = m;
    p.sumexp = s;
    p.sel = sel;
    partials[row * ldp + tile] = p;
}

// ------------------------------------------------------------------------------ backward
//
// dz = g inv_t (onehot - softmax(z)) of the scored logits, recomputed block by block with the
// forward's block_product (so z is bit for bit the forward's), written to a workspace in BF16
// twice ([row][column] and [column][row]); then dh = dz W and dW = dz^T h as "TN" products
// (both operands with the reduction index contiguous) on the same matrix-core path, W and h
// transposed into the workspace first.  Every operand in the workspace is zero-padded to whole
// 256 x 256 blocks, so the products need no load bounds.

// Row constants of dz, for row t of the block at row0: m = M, s = -g'/S, sel = that times
// 2^-64, gsc = g' = g inv_t, and y_rel = the target's column inside the sub-block at chunk
// column col0, -1 when elsewhere, -2 for a row without gradient (padding, masked, ignored,
// out-of-range target, M = -inf).
template <bool SCALED>
__device__ __forceinline__ void dz_row_constants(
    int t, int64_t row0, int col0, int64_t n, int64_t chunk_col0, int64_t vocab_real,
    float inv_t, const int64_t* __restrict__ targets, const uint8_t* __restrict__ active,
    int64_t ignore_index, const float* __restrict__ grad, const logp_stats_t* __restrict__ stats,
    int* y_rel, float* m, float* s, float* sel, float* gsc) {
    const int64_t row = row0 + t;
    int yr = -2;
    float M = 0.0f, nc = 0.0f, gs = 0.0f;
    if (row < n) {
        int64_t y;
        const logp_stats_t st = stats[row];
        if (row_valid(targets, active, ignore_index, vocab_real, row, y) && st.max != kNegInf) {
            gs = SCALED ? grad[row] * inv_t : grad[row];  // d z / d x = inv_t
            M = st.max;
            nc = -(gs / st.sumexp);
            const int64_t c = y - chunk_col0 - col0;
            yr = (c >= 0 && c < kBN) ? static_cast<int>(c) : -1;
        }
    }
    y_rel[t] = yr;
    m[t] = M;
    s[t] = nc;
    sel[t] = nc * 0x1p-64f;
    gsc[t] = gs;
}

// dz of one 256 x 256 block (rows at row0, chunk columns at col0; lim: the chunk's real
// columns) from the scored logits held in the accumulator layout of block_product: z =
// fl32(acc inv_t) when SCALE, else acc holds z itself.  Written in BF16 to dz [row][column]
// and to dzt [column][row]; rows without gradient and masked columns get 0.
template <bool SCALE>
__device__ __forceinline__ void dz_block_out(
    const f32x16 (&acc)[kTM][kTN], float inv_t, int wm, int wn, int lane, int64_t row0,
    int col0, int lim, const int* y_rel, const float* m, const float* s, const float* sel,
    const float* gsc, uint16_t* __restrict__ dz, int64_t ldz, uint16_t* __restrict__ dzt,
    int64_t ldzt) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int lc = col0 + wn * (kTN * 32) + j * 32 + (lane & 31);  // in the chunk
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int lr0 = wm * (kTM * 32) + i * 32 + 8 * q + 4 * (lane >> 5);
                uint16_t out[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int lr = lr0 + e;
                    const int yr = y_rel[lr];
                    float d = 0.0f;
                    if (yr != -2 && lc < lim) {
                        const float acc_v = acc[i][j][4 * q + e];
                        const float z = SCALE ? acc_v * inv_t : acc_v;
                        d = bwd_term_deep<true>(z, m[lr], s[lr], sel[lr]);
                        if (lc - col0 == yr) d = gsc[lr] + d;  // g' (1 - p)
                    }
                    out[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(d));
                    dz[(row0 + lr) * ldz + lc] = out[e];
                }
                // the 4 rows are consecutive: one 8-byte store into the transposed copy
                *reinterpret_cast<uint2*>(&dzt[int64_t(lc) * ldzt + row0 + lr0]) =
                    make_uint2(uint32_t(out[0]) | (uint32_t(out[1]) << 16),
                               uint32_t(out[2]) | (uint32_t(out[3]) << 16));
            }
        }
    }
}

// dz of one (row block, 256-column sub-block) of the chunk at chunk_col0, the logits
// recomputed by block_product: bit for bit the forward's.
template <bool SCALED>
__global__ __launch_bounds__(kThreads) void linear_dz_kernel(
    const uint16_t* __restrict__ h, int64_t ld_h, int64_t n, int H,
    const uint16_t* __restrict__ w, int64_t ld_w, int lim, int row_blocks, int64_t chunk_col0,
    int64_t vocab_real, float inv_t, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ active, int64_t ignore_index, const float* __restrict__ grad,
    const logp_stats_t* __restrict__ stats, uint16_t* __restrict__ dz, int64_t ldz,
    uint16_t* __restrict__ dzt, int64_t ldzt) {
    __shared__ Smem sm;
    __shared__ float gsc[kBM];
    const int rb_idx = static_cast<int>(blockIdx.x % static_cast<uint32_t>(row_blocks));
    const int sb = static_cast<int>(blockIdx.x / static_cast<uint32_t>(row_blocks));
    const int64_t row0 = int64_t(rb_idx) * kBM;
    const int col0 = sb * kBN;  // first column of the sub-block inside the chunk
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / kWN, wn = wave % kWN;

    // block_product's barriers order these LDS writes before the epilogue reads them
    if (threadIdx.x < kBM)
        dz_row_constants<SCALED>(threadIdx.x, row0, col0, n, chunk_col0, vocab_real, inv_t,
                                 targets, active, ignore_index, grad, stats, sm.y_rel, sm.m,
                                 sm.s, sm.sel, gsc);

    f32x16 acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int n_here = static_cast<int>(std::min<int64_t>(kBM, n - row0));
    block_product(sm, h + row0 * ld_h, static_cast<uint32_t>(ld_h), n_here, w,
                  static_cast<uint32_t>(ld_w), lim, H, col0, (H + kBK - 1) / kBK, wm, wn, lane,
                  acc);
    dz_block_out<SCALED>(acc, inv_t, wm, wn, lane, row0, col0, lim, sm.y_rel, sm.m, sm.s, sm.sel,
                         gsc, dz, ldz, dzt, ldzt);
}

// The same dz from scored logits the forward kept (z [row][chunk column], FP32, row stride
// ld_z, the chunk's column 0 first): each value is read where the accumulator layout holds
// it, so dz_block_out applies the same arithmetic to the same z and the bits are those of
// linear_dz_kernel.  Memory-bound: 4 bytes read and 4 written per logit.
template <bool SCALED>
__global__ __launch_bounds__(kThreads) void linear_dz_saved_kernel(
    const float* __restrict__ z, int64_t ld_z, int64_t n, int lim, int row_blocks,
    int64_t chunk_col0, int64_t vocab_real, float inv_t, const int64_t* __restrict__ targets,
    const uint8_t* __restrict__ active, int64_t ignore_index, const float* __restrict__ grad,
    const logp_stats_t* __restrict__ stats, uint16_t* __restrict__ dz, int64_t ldz,
    uint16_t* __restrict__ dzt, int64_t ldzt) {
    __shared__ int y_rel[kBM];
    __shared__ float m[kBM], s[kBM], sel[kBM], gsc[kBM];
    const int rb_idx = static_cast<int>(blockIdx.x % static_cast<uint32_t>(row_blocks));
    const int sb = static_cast<int>(blockIdx.x / static_cast<uint32_t>(row_blocks));
    const int64_t row0 = int64_t(rb_idx) * kBM;
    const int col0 = sb * kBN;
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / kWN, wn = wave % kWN;
    if (threadIdx.x < kBM)
        dz_row_constants<SCALED>(threadIdx.x, row0, col0, n, chunk_col0, vocab_real, inv_t,
                                 targets, active, ignore_index, grad, stats, y_rel, m, s, sel,
                                 gsc);
    __syncthreads();
    f32x16 acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int lc = col0 + wn * (kTN * 32) + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wm * (kTM * 32) + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
                // only the logits dz_block_out uses: rows with a gradient, real columns
                acc[i][j][r] = (y_rel[lr] != -2 && lc < lim)
                                   ? __builtin_nontemporal_load(&z[(row0 + lr) * ld_z + lc])
                                   : 0.0f;
            }
        }
    }
    dz_block_out<false>(acc, inv_t, wm, wn, lane, row0, col0, lim, y_rel, m, s, sel, gsc, dz,
                        ldz, dzt, ldzt);
}

// Where gemm_tn_kernel's FP32 block results go.  The accumulating forms start the accumulator
// from the stored partial sum, so a chunk's products are added onto it one MFMA k-step at a
// time, in k order.  The BF16 forms round to nearest even once, after the FP32 value is
// complete; kOutAddBf16 forms that value exactly as kOutAddF32 does, so its bits are the
// rounding of what the FP32 forms would have stored.
enum GemmOut : int {
    kOutF32 = 0,     // c32 = a b^T
    kOutAddF32 = 1,  // c32 = (c32 + a b^T), the products added onto c32 in k order
    kOutBf16 = 2,    // c16 = RNE_bf16(a b^T)
    kOutAddBf16 = 3, // c16 = RNE_bf16(c32 + a b^T) as kOutAddF32 forms it; c32 is not written
};

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// c = a b^T (stored per OUT) for one 256 x 256 block: a [m_pad, K] and b [n_pad, K] BF16 with
// K a multiple of kBK and both zero-padded to whole blocks; results stored for rows < m_real
// and columns < n_real.
template <int OUT>
__global__ __launch_bounds__(kThreads) void gemm_tn_kernel(
    const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ b, int64_t ldb,
    int K, int m_real, int n_real, int m_blocks, float* __restrict__ c32, int64_t ld32,
    uint16_t* __restrict__ c16, int64_t ld16) {
    __shared__ Smem sm;
    const int mb = static_cast<int>(blockIdx.x % static_cast<uint32_t>(m_blocks));
    const int nb = static_cast<int>(blockIdx.x / static_cast<uint32_t>(m_blocks));
    const int64_t row0 = int64_t(mb) * kBM, col0 = int64_t(nb) * kBN;
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / kWN, wn = wave % kWN;
    f32x16 acc[kTM][kTN];
    // the accumulating forms start from the stored partial sum (its loads overlap the first
    // stages' loads), the others from zero
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int64_t col = col0 + wn * (kTN * 32) + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row =
                    row0 + wm * (kTM * 32) + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
                float c = 0.0f;
                if constexpr (OUT == kOutAddF32 || OUT == kOutAddBf16)
                    if (row < m_real && col < n_real) c = c32[row * ld32 + col];
                acc[i][j][r] = c;
            }
        }
    block_product(sm, a + row0 * lda, static_cast<uint32_t>(lda), kBM, b + col0 * ldb,
                  static_cast<uint32_t>(ldb), kBN, K, 0, K / kBK, wm, wn, lane, acc);
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int64_t col = col0 + wn * (kTN * 32) + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row =
                    row0 + wm * (kTM * 32) + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
                if (row < m_real && col < n_real) {
                    const float v = acc[i][j][r];
                    if constexpr (OUT == kOutF32) {
                        c32[row * ld32 + col] = v;
                    } else if constexpr (OUT == kOutAddF32) {
                        c32[row * ld32 + col] = v;
                    } else if constexpr (OUT == kOutBf16) {
                        c16[row * ld16 + col] = bf16_bits(v);
                    } else {
                        c16[row * ld16 + col] = bf16_bits(v);
                    }
                }
            }
        }
    }
}

const void* gemm_tn(int out) {
    switch (out) {
        case kOutF32: return reinterpret_cast<const void*>(&gemm_tn_kernel<kOutF32>);
        case kOutAddF32: return reinterpret_cast<const void*>(&gemm_tn_kernel<kOutAddF32>);
        case kOutBf16: return reinterpret_cast<const void*>(&gemm_tn_kernel<kOutBf16>);
        default: return reinterpret_cast<const void*>(&gemm_tn_kernel<kOutAddBf16>);
    }
}

constexpr int kTr = 64;  // transpose tile

// dst[col][row] = src[row][col] for row < rows, col < cols (cols a multiple of 8, rows of src
// 16-byte aligned); zero elsewhere in the [cols_pad, rows_pad] destination (both multiples of
// kTr, covered by the grid).
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src,
                                                       int64_t ld_src, int rows, int cols,
                                                       uint16_t* __restrict__ dst,
                                                       int64_t ld_dst) {
    __shared__ uint32_t tile[kTr][kTr / 2 + 1];  // [row][column pair], padded against conflicts
    const int64_t r0 = int64_t(blockIdx.y) * kTr, c0 = int64_t(blockIdx.x) * kTr;
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = t + 256 * i;
        const int r = q / 8, c8 = (q % 8) * 8;
        u32x4v v = {0u, 0u, 0u, 0u};
        if (r0 + r < rows && c0 + c8 < cols)
            v = *reinterpret_cast<const u32x4v*>(src + (r0 + r) * ld_src + c0 + c8);
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[r][c8 / 2 + e] = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = t + 256 * i;
        const int c = q / 8, r8 = (q % 8) * 8;
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = tile[r8 + 2 * e][c / 2] >> (16 * (c & 1));
            const uint32_t hi = tile[r8 + 2 * e + 1][c / 2] >> (16 * (c & 1));
            o[e] = (lo & 0xFFFFu) | (hi << 16);
        }
        *reinterpret_cast<u32x4v*>(dst + (c0 + c) * ld_dst + r0 + r8) =
            u32x4v{o[0], o[1], o[2], o[3]};
    }
}

template <typename T>
__global__ __launch_bounds__(256) void zero_rows_kernel(T* __restrict__ p, int64_t ld,
                                                       int64_t rows, int cols) {
    const int64_t total = rows * cols;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += int64_t(gridDim.x) * 256)
        p[(i / cols) * ld + i % cols] = T(0);
}

int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace

namespace {

// ------------------------------------------------------------------ no-allocation scratch
//
// Staging memory of linear_logp_backward_noalloc: one static array per GPU, created with the
// code object on that device and held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol); the device
// address is looked up once per device with that device current and kept per device.
constexpr int64_t kNoallocScratchBytes = LINEAR_LOGP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_address[kMaxScratchDevices] = {};

// Device address of `scratch` on `dev`, which must be the current device.
logp_status_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxScratchDevices) return LOGP_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_address[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return LOGP_ERR_HIP;
        }
        g_scratch_address[dev] = p;
    }
    *out = g_scratch_address[dev];
    return LOGP_OK;
}

// Bytes of the FP32 dhidden accumulator that the BF16-output backward keeps after the FP32
// backward's staging: [n_pad, h_pad].
int64_t dh_accumulator_bytes(int64_t n, int64_t hidden_size) {
    return 4 * round_up(std::max<int64_t>(n, 1), kBM) * round_up(hidden_size, kBN);
}

// The backward with its staging either in the caller's workspace (use_scratch false) or in
// this file's static `scratch` array on the launch device (use_scratch true: workspace and
// workspace_bytes are ignored, and a call needing more than kNoallocScratchBytes is
// LOGP_ERR_SCRATCH before anything is checked on the device).  dhidden and dweight are FP32
// (bf16_out false) or BF16 bits (bf16_out true: dhidden is summed over the chunks in an FP32
// accumulator after the staging and rounded once, by the last chunk's product).
logp_status_t backward_impl(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, const float* grad_logp, const logp_stats_t* stats, void* dhidden,
    int64_t ld_dh, void* dweight, int64_t ld_dw, void* workspace, int64_t workspace_bytes,
    int64_t chunk_cols, hipStream_t stream, bool use_scratch, bool bf16_out,
    const float* saved = nullptr, int64_t ld_saved = 0) {
    if (!(inv_temperature > 0.0f) || !std::isfinite(inv_temperature)) return LOGP_ERR_ARG;
    if (n < 0 || vocab_real < 1 || vocab_padded < vocab_real ||
        vocab_padded > (int64_t(1) << 31) - 1 - kTile || n > LINEAR_LOGP_BWD_MAX_ROWS)
        return LOGP_ERR_SHAPE;
    if (col_begin < 0 || col_end < col_begin || col_end > vocab_padded ||
        col_begin % kTile != 0 || (col_end % kTile != 0 && col_end != vocab_padded))
        return LOGP_ERR_SHARD;
    if (chunk_cols < kTile || chunk_cols % kTile != 0 || chunk_cols > LINEAR_LOGP_BWD_MAX_CHUNK)
        return LOGP_ERR_SHAPE;
    // the products' row strides and reduction lengths (padded rows or chunk columns) keep the
    // in-kernel load offsets below the out-of-range marker
    static_assert(uint64_t(16) * 2 * (LINEAR_LOGP_BWD_MAX_ROWS + kBM) < kOob &&
                      LINEAR_LOGP_BWD_MAX_CHUNK <= LINEAR_LOGP_BWD_MAX_ROWS,
                  "product load offsets");
    if (n == 0) return LOGP_OK;
    const int64_t H = hidden_size;
    if (H < 1 || H > LINEAR_LOGP_MAX_HIDDEN || H % 8 != 0 || ld_h < H || ld_w < H ||
        ld_h % 8 != 0 || ld_w % 8 != 0 || ld_h > LINEAR_LOGP_MAX_LD ||
        ld_w > LINEAR_LOGP_MAX_LD || ld_dh < H || ld_dw < H)
        return LOGP_ERR_SHAPE;
    const int64_t width = col_end - col_begin;
    // weight rows actually read: the view's real vocabulary rows (none for an all-padding view,
    // whose weight pointer may then be NULL)
    const int64_t lim = std::max<int64_t>(0, std::min(width, vocab_real - col_begin));
    if (hidden == nullptr || targets == nullptr || grad_logp == nullptr || stats == nullptr ||
        dhidden == nullptr || (lim > 0 && weight == nullptr) ||
        (width > 0 && dweight == nullptr) || (!use_scratch && workspace == nullptr))
        return LOGP_ERR_NULL;
    if (!aligned16(hidden) || (weight != nullptr && !aligned16(weight)) ||
        (!use_scratch && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
        return LOGP_ERR_SHAPE;
    // saved scored logits (optional): [n, ld_saved] FP32, the view's real columns read
    if (saved != nullptr && (ld_saved < width || ld_saved > LINEAR_LOGP_MAX_SAVED_LD ||
                             n > (int64_t(1) << 40) / std::max<int64_t>(ld_saved, 1) ||
                             (reinterpret_cast<uintptr_t>(saved) & 3u) != 0))
        return LOGP_ERR_SHAPE;
    const int64_t staging = linear_logp_backward_workspace(n, H, chunk_cols);
    if (staging < 0) return LOGP_ERR_SHAPE;
    const int64_t need = staging + (bf16_out ? dh_accumulator_bytes(n, H) : 0);
    if (use_scratch ? need > kNoallocScratchBytes : workspace_bytes < need)
        return use_scratch ? LOGP_ERR_SCRATCH : LOGP_ERR_SHAPE;
    if (n > (int64_t(1) << 40) / ld_h) return LOGP_ERR_SHAPE;
    const Span in[] = {{hidden, span_bytes(n, ld_h, H, 2)},
                       {weight, lim > 0 ? span_bytes(lim, ld_w, H, 2) : 0},
                       {targets, uint64_t(n) * 8},
                       {active, active ? uint64_t(n) : 0},
                       {grad_logp, uint64_t(n) * 4},
                       {stats, uint64_t(n) * sizeof(logp_stats_t)},
                       {saved, saved != nullptr && lim > 0 ? span_bytes(n, ld_saved, lim, 4) : 0}};
    // the static scratch array is not a caller buffer: it cannot overlap one, and it is not
    // checked as one
    const int out_size = bf16_out ? 2 : 4;
    const Span out[] = {{dhidden, span_bytes(n, ld_dh, H, out_size)},
                        {dweight, width > 0 ? span_bytes(width, ld_dw, H, out_size) : 0},
                        {use_scratch ? nullptr : workspace, use_scratch ? 0 : uint64_t(need)}};
    int dev = -1;
    logp_status_t st = check_buffers(in, 7, out, 3, stream, &dev);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;
    if (use_scratch) {
        st = scratch_address(dev, &workspace);  // with the launch device current
        if (st != LOGP_OK) return st;
    }

    if (width == 0) {  // no vocabulary columns: this shard contributes dh = 0
        int cols = static_cast<int>(H);
        void* args[] = {&dhidden, &ld_dh, &n, &cols};
        const void* k = bf16_out ? reinterpret_cast<const void*>(&zero_rows_kernel<uint16_t>)
                                 : reinterpret_cast<const void*>(&zero_rows_kernel<float>);
        return launch(k, dim3(1024), dim3(256), args, 0, stream);
    }

    const int64_t n_pad = round_up(n, kBM), h_pad = round_up(H, kBN);
    const int64_t c_pad_max = round_up(chunk_cols, kBN);
    uint16_t* ws = static_cast<uint16_t*>(workspace);
    uint16_t* hT = ws;                      // [h_pad, n_pad]
    uint16_t* wT = hT + h_pad * n_pad;      // [h_pad, c_pad]
    uint16_t* dz = wT + h_pad * c_pad_max;  // [n_pad, c_pad]
    uint16_t* dzT = dz + n_pad * c_pad_max; // [c_pad, n_pad]
    // FP32 dhidden: the caller's output, or (BF16 output) the accumulator after the staging
    float* dh32 = bf16_out ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                                      staging)
                           : static_cast<float*>(dhidden);
    const int64_t ld32 = bf16_out ? h_pad : ld_dh;
    uint16_t* dh16 = bf16_out ? static_cast<uint16_t*>(dhidden) : nullptr;

    int Hi = static_cast<int>(H), ni = static_cast<int>(n);
    {  // h^T, zero-padded
        void* args[] = {&hidden, &ld_h, &ni, &Hi, &hT, const_cast<int64_t*>(&n_pad)};
        st = launch(reinterpret_cast<const void*>(&transpose_kernel),
                    dim3(static_cast<uint32_t>(h_pad / kTr), static_cast<uint32_t>(n_pad / kTr)),
                    dim3(256), args, 0, stream);
        if (st != LOGP_OK) return st;
    }
    const bool scaled = inv_temperature != 1.0f;
    const void* dz_kernel = scaled ? reinterpret_cast<const void*>(&linear_dz_kernel<true>)
                                   : reinterpret_cast<const void*>(&linear_dz_kernel<false>);
    const void* dz_saved_kernel =
        scaled ? reinterpret_cast<const void*>(&linear_dz_saved_kernel<true>)
               : reinterpret_cast<const void*>(&linear_dz_saved_kernel<false>);
    int row_blocks = static_cast<int>(n_pad / kBM);
    for (int64_t off = 0; off < width; off += chunk_cols) {
        const int64_t cw = std::min(chunk_cols, width - off);     // chunk columns
        const int64_t c_pad = round_up(cw, kBN);
        const int64_t chunk_col0 = col_begin + off;              // global column of the chunk
        int lim_c = static_cast<int>(std::max<int64_t>(0, std::min(cw, vocab_real - chunk_col0)));
        const uint16_t* wc = weight + off * ld_w;
        {  // W^T of the chunk's real rows, zero-padded to [h_pad, c_pad]
            void* args[] = {&wc, &ld_w, &lim_c, &Hi, &wT, const_cast<int64_t*>(&c_pad)};
            st = launch(reinterpret_cast<const void*>(&transpose_kernel),
                        dim3(static_cast<uint32_t>(h_pad / kTr),
                             static_cast<uint32_t>(c_pad / kTr)),
                        dim3(256), args, 0, stream);
            if (st != LOGP_OK) return st;
        }
        {  // dz and dz^T: from the saved logits when given, else the logits recomputed
            int64_t ldz = c_pad, ldzt = n_pad;
            int64_t cc0 = chunk_col0;
            float inv_t = inv_temperature;
            const dim3 grid(static_cast<uint32_t>(row_blocks * (c_pad / kBN)));
            if (saved != nullptr) {
                const float* zc = saved + off;
                int64_t ldzc = ld_saved;
                void* args[] = {&zc,      &ldzc,   &n,     &lim_c,        &row_blocks,
                                &cc0,     &vocab_real,     &inv_t,        &targets,
                                &active,  &ignore_index,   &grad_logp,    &stats,
                                &dz,      &ldz,    &dzT,   &ldzt};
                st = launch(dz_saved_kernel, grid, dim3(kThreads), args, 0, stream);
            } else {
                void* args[] = {&hidden, &ld_h, &n,     &Hi,     &wc,          &ld_w,
                                &lim_c,  &row_blocks,   &cc0,    &vocab_real,  &inv_t,
                                &targets, &active,      &ignore_index, &grad_logp, &stats,
                                &dz,     &ldz,          &dzT,    &ldzt};
                st = launch(dz_kernel, grid, dim3(kThreads), args, 0, stream);
            }
            if (st != LOGP_OK) return st;
        }
        {  // dh (= | +=) dz W: a = dz [n_pad, c_pad], b = W^T [h_pad, c_pad]
            const bool first = off == 0, last = off + chunk_cols >= width;
            int out = first ? kOutF32 : kOutAddF32;
            if (bf16_out && last) out = first ? kOutBf16 : kOutAddBf16;
            int64_t lda = c_pad, ldb = c_pad, l32 = ld32, l16 = ld_dh;
            int K = static_cast<int>(c_pad), mr = ni, nr = Hi, mb = row_blocks;
            void* args[] = {&dz, &lda, &wT, &ldb, &K, &mr, &nr, &mb, &dh32, &l32, &dh16, &l16};
            st = launch(gemm_tn(out), dim3(static_cast<uint32_t>(mb * (h_pad / kBN))),
                        dim3(kThreads), args, 0, stream);
            if (st != LOGP_OK) return st;
        }
        {  // dW of the chunk's rows = dz^T h: a = dz^T [c_pad, n_pad], b = h^T [h_pad, n_pad]
            int64_t lda = n_pad, ldb = n_pad, ldc = ld_dw;
            int K = static_cast<int>(n_pad), mr = static_cast<int>(cw), nr = Hi;
            int mb = static_cast<int>(c_pad / kBM);
            float* dw32 = bf16_out ? nullptr : static_cast<float*>(dweight) + off * ld_dw;
            uint16_t* dw16 = bf16_out ? static_cast<uint16_t*>(dweight) + off * ld_dw : nullptr;
            void* args[] = {&dzT, &lda, &hT, &ldb, &K, &mr, &nr, &mb, &dw32, &ldc, &dw16, &ldc};
            st = launch(gemm_tn(bf16_out ? kOutBf16 : kOutF32),
                        dim3(static_cast<uint32_t>(mb * (h_pad / kBN))), dim3(kThreads), args,
                        0, stream);
            if (st != LOGP_OK) return st;
        }
    }
    return LOGP_OK;
}

// Compute units of `dev` (cached; the launch device is current when this is called).
int compute_units(int dev) {
    static std::mutex mu;
    static int cached[kMaxScratchDevices] = {};
    if (dev < 0 || dev >= kMaxScratchDevices) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            cus < 1) {
            (void)hipGetLastError();
            return 0;
        }
        cached[dev] = cus;
    }
    return cached[dev];
}

// Sub-blocks (pairs) of the tiles [t0, view tiles) that hold real columns: every tile before
// the last real one has kSubBlocks, that one ceil(its real columns / kBN).
int64_t split_pairs(int64_t lim, int64_t t0) {
    if (lim <= 0) return 0;
    const int64_t real_tiles = ceil_div(lim, kTile);
    if (t0 >= real_tiles) return 0;
    const int64_t nsb_last = ceil_div(lim - (real_tiles - 1) * kTile, kBN);
    return (real_tiles - 1 - t0) * kSubBlocks + nsb_last;
}

constexpr int64_t kSplitTaskBytes = int64_t(kBM) * (sizeof(float2) + sizeof(float));

logp_status_t partials_impl(float inv_temperature, const uint16_t* hidden, int64_t ld_h,
                            int64_t n, int64_t hidden_size, const uint16_t* weight, int64_t ld_w,
                            int64_t vocab_real, int64_t vocab_padded, int64_t col_begin,
                            int64_t col_end, const int64_t* targets, const uint8_t* active,
                            int64_t ignore_index, logp_partial_t* partials, int64_t ldp,
                            void* workspace, int64_t workspace_bytes, hipStream_t stream,
                            float* saved = nullptr, int64_t ld_saved = 0) {
    if (!(inv_temperature > 0.0f) || !std::isfinite(inv_temperature)) return LOGP_ERR_ARG;
    if (n < 0 || vocab_real < 1 || vocab_padded < vocab_real ||
        vocab_padded > (int64_t(1) << 31) - 1 - kTile)
        return LOGP_ERR_SHAPE;
    if (col_begin < 0 || col_end < col_begin || col_end > vocab_padded ||
        col_begin % kTile != 0 || (col_end % kTile != 0 && col_end != vocab_padded))
        return LOGP_ERR_SHARD;
    if (workspace_bytes < 0 ||
        (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
        return LOGP_ERR_SHAPE;
    if (n == 0 || col_end == col_begin) return LOGP_OK;
    // weight rows actually read: the view's real vocabulary rows (none for an all-padding view,
    // whose weight pointer may then be NULL)
    const int64_t lim =
        std::max<int64_t>(0, std::min(col_end - col_begin, vocab_real - col_begin));
    if (hidden == nullptr || (lim > 0 && weight == nullptr) || targets == nullptr ||
        partials == nullptr)
        return LOGP_ERR_NULL;
    const int64_t H = hidden_size;
    if (H < 1 || H > LINEAR_LOGP_MAX_HIDDEN || H % 8 != 0 || ld_h < H || ld_w < H ||
        ld_h % 8 != 0 || ld_w % 8 != 0 || ld_h > LINEAR_LOGP_MAX_LD ||
        ld_w > LINEAR_LOGP_MAX_LD || !aligned16(hidden) || !aligned16(weight))
        return LOGP_ERR_SHAPE;
    // in-kernel load offsets (bytes from the first row of an 8-row group) stay below the
    // out-of-range marker 2^31
    static_assert(uint64_t(16) * (LINEAR_LOGP_MAX_LD + LINEAR_LOGP_MAX_HIDDEN) < kOob,
                  "load offsets");
    const int64_t width = col_end - col_begin;
    const int64_t view_tiles = ceil_div(width, kTile);
    if (ldp < view_tiles) return LOGP_ERR_SHAPE;
    // saved scored logits (optional): [n, ld_saved] FP32, 16-byte aligned rows
    if (saved != nullptr && (ld_saved < width || ld_saved % 4 != 0 ||
                             ld_saved > LINEAR_LOGP_MAX_SAVED_LD ||
                             n > (int64_t(1) << 40) / std::max<int64_t>(ld_saved, 1) ||
                             !aligned16(saved)))
        return LOGP_ERR_SHAPE;
    if (n > (int64_t(1) << 40) / ld_h) return LOGP_ERR_SHAPE;
    const int64_t row_blocks = ceil_div(n, kBM);
    if (row_blocks * view_tiles > 0x7FFFFFFF) return LOGP_ERR_SHAPE;
    const Span in[] = {{hidden, span_bytes(n, ld_h, H, 2)},
                       {weight, lim > 0 ? span_bytes(lim, ld_w, H, 2) : 0},
                       {targets, uint64_t(n) * 8},
                       {active, active ? uint64_t(n) : 0}};
    const Span out[] = {{partials, span_bytes(n, ldp, view_tiles, sizeof(logp_partial_t))},
                        {workspace, workspace != nullptr ? uint64_t(workspace_bytes) : 0},
                        {saved, saved != nullptr && lim > 0 ? span_bytes(n, ld_saved, lim, 4) : 0}};
    int dev = -1;
    logp_status_t st = check_buffers(in, 4, out, 3, stream, &dev);
    if (st != LOGP_OK) return st;
    DeviceGuard guard(dev);
    if (!guard.ok()) return LOGP_ERR_HIP;

    // Split the work when the workspace allows it and the balanced schedule is shorter: whole
    // rounds of one workgroup per (row block, tile) for the tiles [0, t0), then the sub-blocks
    // of the rest spread over every CU (in units of one sub-block's time per CU, plus two for
    // the fold launch).
    int64_t t0 = view_tiles, tasks = 0;
    const int cus = workspace != nullptr ? compute_units(dev) : 0;
    if (cus > 0) {
        const int64_t items = row_blocks * view_tiles;
        const int64_t c0 = ((items / cus) * cus) / row_blocks;  // whole tiles in whole rounds
        const int64_t t_split = row_blocks * split_pairs(lim, c0);
        const int64_t one = ceil_div(items, cus) * kSubBlocks;
        const int64_t two = ceil_div(row_blocks * c0, cus) * kSubBlocks + ceil_div(t_split, cus) + 2;
        if (two < one && t_split * kSplitTaskBytes <= workspace_bytes && t_split <= 0x7FFFFFFF) {
            t0 = c0;
            tasks = t_split;
        }
    }
    int Hi = static_cast<int>(H), lim_i = static_cast<int>(lim);
    int rbk = static_cast<int>(row_blocks);
    // the view's real columns are written: the others are masked, and the split below skips
    // fully masked sub-blocks
    ZOut zo{saved, ld_saved, n, lim_i};
    const bool unit = inv_temperature == 1.0f, save = saved != nullptr;
    if (t0 > 0) {
        void* args[] = {&hidden,    &ld_h,       &n,     &Hi,     &weight,       &ld_w,
                        &lim_i,     &rbk,        &col_begin,     &vocab_real,   &inv_temperature,
                        &targets,   &active,     &ignore_index,  &partials,     &ldp,
                        &zo};
        const void* kernel =
            unit ? (save ? reinterpret_cast<const void*>(&linear_partials_kernel<false, true>)
                         : reinterpret_cast<const void*>(&linear_partials_kernel<false, false>))
                 : (save ? reinterpret_cast<const void*>(&linear_partials_kernel<true, true>)
                         : reinterpret_cast<const void*>(&linear_partials_kernel<true, false>));
        st = launch(kernel, dim3(static_cast<uint32_t>(row_blocks * t0)), dim3(kThreads), args,
                    0, stream);
        if (st != LOGP_OK) return st;
    }
    if (t0 == view_tiles) return LOGP_OK;
    float2* ws_stats = static_cast<float2*>(workspace);
    float* ws_sel = reinterpret_cast<float*>(ws_stats + tasks * kBM);
    int tile0 = static_cast<int>(t0), ntask = static_cast<int>(tasks);
    if (tasks > 0) {
        void* args[] = {&hidden,  &ld_h,      &n,          &Hi,           &weight,
                        &ld_w,    &lim_i,     &rbk,        &col_begin,    &vocab_real,
                        &inv_temperature, &targets, &active, &ignore_index, &tile0,
                        &ntask,   &ws_stats,  &ws_sel,     &zo};
        const void* kernel =
            unit ? (save ? reinterpret_cast<const void*>(&linear_split_kernel<false, true>)
                         : reinterpret_cast<const void*>(&linear_split_kernel<false, false>))
                 : (save ? reinterpret_cast<const void*>(&linear_split_kernel<true, true>)
                         : reinterpret_cast<const void*>(&linear_split_kernel<true, false>));
        st = launch(kernel, dim3(static_cast<uint32_t>(std::min<int64_t>(cus, tasks))),
                    dim3(kThreads), args, 0, stream);
        if (st != LOGP_OK) return st;
    }
    const int64_t real_tiles = lim > 0 ? ceil_div(lim, kTile) : 0;
    int rt = static_cast<int>(real_tiles);
    int nsb_last = lim > 0 ? static_cast<int>(ceil_div(lim - (real_tiles - 1) * kTile, kBN)) : 0;
    void* fa[] = {&n,       &rbk,          &tile0,  &rt,        &nsb_last,   &ws_stats,
                  &ws_sel,  &targets,      &active, &ignore_index, &vocab_real, &col_begin,
                  &partials, &ldp};
    return launch(reinterpret_cast<const void*>(&linear_fold_kernel),
                  dim3(static_cast<uint32_t>(row_blocks * (view_tiles - t0))), dim3(kBM), fa, 0,
                  stream);
}

}  // namespace

extern "C" {

int64_t linear_logp_partials_workspace(int64_t n, int64_t vocab_real, int64_t col_begin,
                                       int64_t col_end) {
    if (n < 0 || vocab_real < 1 || col_begin < 0 || col_end < col_begin ||
        n > (int64_t(1) << 40) || col_end > (int64_t(1) << 31))
        return -1;
    const int64_t lim = std::max<int64_t>(0, std::min(col_end - col_begin, vocab_real - col_begin));
    return ceil_div(std::max<int64_t>(n, 1), kBM) * split_pairs(lim, 0) * kSplitTaskBytes;
}

logp_status_t linear_logp_partials_ws(float inv_temperature, const uint16_t* hidden,
                                      int64_t ld_h, int64_t n, int64_t hidden_size,
                                      const uint16_t* weight, int64_t ld_w, int64_t vocab_real,
                                      int64_t vocab_padded, int64_t col_begin, int64_t col_end,
                                      const int64_t* targets, const uint8_t* active,
                                      int64_t ignore_index, logp_partial_t* partials,
                                      int64_t ldp, void* workspace, int64_t workspace_bytes,
                                      hipStream_t stream) {
    return partials_impl(inv_temperature, hidden, ld_h, n, hidden_size, weight, ld_w, vocab_real,
                         vocab_padded, col_begin, col_end, targets, active, ignore_index,
                         partials, ldp, workspace, workspace_bytes, stream);
}

logp_status_t linear_logp_partials_save(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, logp_partial_t* partials, int64_t ldp, float* logits,
    int64_t ld_logits, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    if (logits == nullptr) return LOGP_ERR_NULL;
    return partials_impl(inv_temperature, hidden, ld_h, n, hidden_size, weight, ld_w, vocab_real,
                         vocab_padded, col_begin, col_end, targets, active, ignore_index,
                         partials, ldp, workspace, workspace_bytes, stream, logits, ld_logits);
}

logp_status_t linear_logp_partials_ex(float inv_temperature, const uint16_t* hidden,
                                      int64_t ld_h, int64_t n, int64_t hidden_size,
                                      const uint16_t* weight, int64_t ld_w, int64_t vocab_real,
                                      int64_t vocab_padded, int64_t col_begin, int64_t col_end,
                                      const int64_t* targets, const uint8_t* active,
                                      int64_t ignore_index, logp_partial_t* partials,
                                      int64_t ldp, hipStream_t stream) {
    return partials_impl(inv_temperature, hidden, ld_h, n, hidden_size, weight, ld_w, vocab_real,
                         vocab_padded, col_begin, col_end, targets, active, ignore_index,
                         partials, ldp, nullptr, 0, stream);
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

int64_t linear_logp_backward_workspace(int64_t n, int64_t hidden_size, int64_t chunk_cols) {
    if (n < 0 || hidden_size < 1 || chunk_cols < 1 || n > LINEAR_LOGP_BWD_MAX_ROWS ||
        hidden_size > LINEAR_LOGP_MAX_HIDDEN || chunk_cols > LINEAR_LOGP_BWD_MAX_CHUNK)
        return -1;
    const int64_t n_pad = round_up(std::max<int64_t>(n, 1), kBM);
    const int64_t h_pad = round_up(hidden_size, kBN);
    const int64_t c_pad = round_up(chunk_cols, kBN);
    return 2 * (h_pad * n_pad + h_pad * c_pad + 2 * n_pad * c_pad);
}

logp_status_t linear_logp_backward_ex(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, const float* grad_logp, const logp_stats_t* stats, float* dhidden,
    int64_t ld_dh, float* dweight, int64_t ld_dw, void* workspace, int64_t workspace_bytes,
    int64_t chunk_cols, hipStream_t stream) {
    return backward_impl(inv_temperature, hidden, ld_h, n, hidden_size, weight, ld_w, vocab_real,
                         vocab_padded, col_begin, col_end, targets, active, ignore_index,
                         grad_logp, stats, dhidden, ld_dh, dweight, ld_dw, workspace,
                         workspace_bytes, chunk_cols, stream, false, false);
}

int64_t linear_logp_backward_bf16_workspace(int64_t n, int64_t hidden_size,
                                            int64_t chunk_cols) {
    const int64_t staging = linear_logp_backward_workspace(n, hidden_size, chunk_cols);
    return staging < 0 ? -1 : staging + dh_accumulator_bytes(n, hidden_size);
}

logp_status_t linear_logp_backward_bf16(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, const float* grad_logp, const logp_stats_t* stats, uint16_t* dhidden,
    int64_t ld_dh, uint16_t* dweight, int64_t ld_dw, void* workspace, int64_t workspace_bytes,
    int64_t chunk_cols, hipStream_t stream) {
    return backward_impl(inv_temperature, hidden, ld_h, n, hidden_size, weight, ld_w, vocab_real,
                         vocab_padded, col_begin, col_end, targets, active, ignore_index,
                         grad_logp, stats, dhidden, ld_dh, dweight, ld_dw, workspace,
                         workspace_bytes, chunk_cols, stream, false, true);
}

logp_status_t linear_logp_backward_noalloc(
    float inv_temperature, const uint16_t* hidden, int64_t ld_h, int64_t n, int64_t hidden_size,
    const uint16_t* weight, int64_t ld_w, int64_t vocab_real, int64_t vocab_padded,
    int64_t col_begin, int64_t col_end, const int64_t* targets, const uint8_t* active,
    int64_t ignore_index, const float* grad_logp, const logp_stats_t* stats, float* dhidden,
    int64_t ld_dh, float* dweight, int64_t ld_dw, int64_t chunk_cols, hipStream_t stream) {
    return backward_impl(inv_temperature, hidden, ld_h, n, hidden_size, weight, ld_w, vocab_real,
                         vocab_padded, col_begin, col_end, targets, active, ignore_index,
                         grad_logp, stats, dhidden, ld_dh, dweight, ld_dw, nullptr, 0, chunk_cols,
                         stream, true, false);
}

logp_status_t linear_logp_backward_saved(
    float inv_temperature, const float* logits, int64_t ld_logits, const uint16_t* hidden,
    int64_t ld_h, int64_t n, int64_t hidden_size, const uint16_t* weight, int64_t ld_w,
    int64_t vocab_real, int64_t vocab_padded, int64_t col_begin, int64_t col_end,
    const int64_t* targets, const uint8_t* active, int64_t ignore_index,
    const float* grad_logp, const logp_stats_t* stats, void* dhidden, int64_t ld_dh,
    void* dweight, int64_t ld_dw, int32_t out_dtype, void* workspace, int64_t workspace_bytes,
    int64_t chunk_cols, hipStream_t stream) {
    if (out_dtype != LOGP_DTYPE_F32 && out_dtype != LOGP_DTYPE_BF16) return LOGP_ERR_ARG;
    if (logits == nullptr) return LOGP_ERR_NULL;
    return backward_impl(inv_temperature, hidden, ld_h, n, hidden_size, weight, ld_w, vocab_real,
                         vocab_padded, col_begin, col_end, targets, active, ignore_index,
                         grad_logp, stats, dhidden, ld_dh, dweight, ld_dw, workspace,
                         workspace_bytes, chunk_cols, stream, false,
                         out_dtype == LOGP_DTYPE_BF16, logits, ld_logits);
}

logp_status_t linear_logp_backward(const uint16_t* hidden, int64_t ld_h, int64_t n,
                                   int64_t hidden_size, const uint16_t* weight, int64_t ld_w,
                                   int64_t vocab_real, int64_t vocab_padded, int64_t col_begin,
                                   int64_t col_end, const int64_t* targets,
                                   const uint8_t* active, int64_t ignore_index,
                                   const float* grad_logp, const logp_stats_t* stats,
                                   float* dhidden, int64_t ld_dh, float* dweight, int64_t ld_dw,
                                   void* workspace, int64_t workspace_bytes, int64_t chunk_cols,
                                   hipStream_t stream) {
    return linear_logp_backward_ex(1.0f, hidden, ld_h, n, hidden_size, weight, ld_w,
                                   vocab_real, vocab_padded, col_begin, col_end, targets, active,
                                   ignore_index, grad_logp, stats, dhidden, ld_dh, dweight,
                                   ld_dw, workspace, workspace_bytes, chunk_cols, stream);
}

}  // extern "C"
