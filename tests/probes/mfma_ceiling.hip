// Bench probe (not part of the library): the dense BF16 matrix-core rate this part sustains,
// so that the fused LM-head kernels' rates can be stated as a fraction of a measured ceiling
// as well as of the nominal 2.5 PFLOP/s (which assumes the 2.4 GHz peak engine clock).
//
//   mfma_bf16  every wave runs `iters` rounds of TM x TN independent
//              v_mfma_f32_32x32x16_bf16 (a (32 TM) x (32 TN) block of FP32 accumulators) on
//              operands held in registers; with `toggle` set, operand bits flip between rounds
//              so that the data path keeps switching as it does on streamed operands (the
//              switching costs power, and this part's clock follows its power draw).  No
//              memory traffic beyond one store per wave at the end.  Shapes: 4 waves per workgroup with
//              128 x 128 per wave (one wave per SIMD) and 8 waves with 64 x 128 per wave (two
//              per SIMD), the wave blocks of the linear_logp kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

template <int WAVES, int TM, int TN>
__global__ __launch_bounds__(WAVES * kWave) void mfma_kernel(int iters, uint32_t seed,
                                                             uint32_t toggle,
                                                             float* __restrict__ sink) {
    const uint32_t lane = threadIdx.x;
    bf16x8 a[TM], b[TN];
    // operands: bf16 values of magnitude ~1 with varied mantissas (exponent field 0x3F/0x40)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        u32x4 w;
        for (int e = 0; e < 4; ++e) {
            const uint32_t h = (seed ^ (lane * 0x9E3779B9u) ^ uint32_t(i * 4 + e) * 0x85EBCA6Bu);
            w[e] = (h & 0x807F807Fu) | 0x3F803F80u;
        }
        a[i] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        u32x4 w;
        for (int e = 0; e < 4; ++e) {
            const uint32_t h = (seed ^ (lane * 0xC2B2AE35u) ^ uint32_t(j * 4 + e + 64) * 0x27D4EB2Fu);
            w[e] = (h & 0x807F807Fu) | 0x3F803F80u;
        }
        b[j] = __builtin_bit_cast(bf16x8, w);
    }
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    uint32_t flip = toggle ? 0x00010001u : 0u;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        // flip low mantissa bits of the operands (the values stay finite, near 1)
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a[i] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, a[i]) ^ flip);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            b[j] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, b[j]) ^ flip);
        flip = (flip << 1 | flip >> 5) & 0x003F003Fu;
        flip = (flip || !toggle) ? flip : 0x00010001u;
    }
    // each accumulator moved out one at a time (a block copy of all of them would not fit)
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float v;
                asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(acc[i][j][r]));
                s += v;
            }
    sink[blockIdx.x * WAVES * kWave + threadIdx.x] = s;  // keeps every accumulator live
}

template <int WAVES, int TM, int TN>
hipError_t launch(int64_t groups, int iters, uint32_t seed, uint32_t toggle, float* sink,
                  hipStream_t stream) {
    hipLaunchKernelGGL((mfma_kernel<WAVES, TM, TN>), dim3(unsigned(groups)),
                       dim3(WAVES * kWave), 0, stream, iters, seed, toggle, sink);
    return hipGetLastError();
}

}  // namespace

#define CEILING_API extern "C" __attribute__((visibility("default")))

// Dense BF16 flops of one mfma_bf16 launch (-1 for bad arguments).
CEILING_API double mfma_bf16_flops(int waves, int64_t groups, int iters) {
    if ((waves != 4 && waves != 8) || groups < 1 || groups >= (int64_t(1) << 31) || iters < 1)
        return -1.0;
    const int tiles = waves == 4 ? 16 : 8;  // MFMA tiles per wave
    return double(groups) * waves * double(iters) * tiles * (2.0 * 32 * 32 * 16);
}

// waves in {4, 8}; groups workgroups of `waves` waves; toggle 0 keeps the operands fixed, 1
// flips their bits every round; sink holds groups * waves * 64 floats (device memory owned by
// the caller).  Returns 0 on success, 1 for bad arguments (nothing launched), 2 for a launch
// error.
CEILING_API int mfma_bf16(int waves, int64_t groups, int iters, uint32_t seed, int toggle,
                          float* sink, hipStream_t stream) {
    if (sink == nullptr || mfma_bf16_flops(waves, groups, iters) < 0 ||
        (toggle != 0 && toggle != 1))
        return 1;
    const uint32_t t = static_cast<uint32_t>(toggle);
    const hipError_t e = waves == 4 ? launch<4, 4, 4>(groups, iters, seed, t, sink, stream)
                                    : launch<8, 2, 4>(groups, iters, seed, t, sink, stream);
    return e == hipSuccess ? 0 : 2;
}
