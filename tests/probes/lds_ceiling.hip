// Bench probe (not part of the library): the per-CU rates of the two LDS paths the linear_logp
// block product uses, in bytes per core clock, so that its LDS traffic can be set against
// measured limits rather than assumed ones.
//
//   lds_read   every wave of a workgroup (one workgroup per CU: 96 KB of LDS each) runs `iters`
//              rounds of 16 LDS reads of `width` bytes per lane (4, 8 or 16: ds_read_b32 / b64 /
//              b128), lane-contiguous and so free of bank conflicts, then waits for them.
//   lds_dma    every wave runs `iters` rounds of 8 direct-to-LDS buffer loads (16 bytes per
//              lane, 1 KB per instruction, into the wave's own 8 KB of LDS) from a source of
//              `src_bytes` that every workgroup reads (small enough to stay in L2), then waits
//              for them: the L2 -> LDS path of the block product's stage loads.
//
// Wave 0 of each workgroup reads the core clock counter (s_memtime) after the set-up barrier
// and after the closing barrier; the caller gets each workgroup's cycle count.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_vptr;

constexpr int kWave = 64;
constexpr int kLdsBytes = 96 * 1024;    // > half the CU's LDS: one workgroup per CU
constexpr int kReadSpan = 64 * 1024;    // the reads wrap inside this span
constexpr int kDmaPerWave = 8 * 1024;   // each wave's own LDS slots for the loads

template <int WAVES, int WIDTH>
__global__ __launch_bounds__(WAVES * kWave) void read_kernel(int iters, uint32_t* sink,
                                                             int64_t* cycles) {
    __shared__ __attribute__((aligned(16))) unsigned char buf[kLdsBytes];
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    for (int i = t; i < kLdsBytes / 4; i += WAVES * kWave)
        reinterpret_cast<uint32_t*>(buf)[i] = uint32_t(i) * 2654435761u;
    __syncthreads();
    const int64_t c0 = clock64();
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int base = (wave * 4096) & (kReadSpan - 1);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            // in [0, kReadSpan - WIDTH], WIDTH-aligned
            const int off = (base + (j * kWave + lane) * WIDTH) & (kReadSpan - 1);
            if (WIDTH == 16) {
                acc ^= *reinterpret_cast<const u32x4*>(buf + off);
            } else if (WIDTH == 8) {
                const uint64_t v = *reinterpret_cast<const uint64_t*>(buf + off);
                acc.x ^= uint32_t(v);
                acc.y ^= uint32_t(v >> 32);
            } else {
                acc.x ^= *reinterpret_cast<const uint32_t*>(buf + off);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
    __syncthreads();
    const int64_t c1 = clock64();
    sink[int64_t(blockIdx.x) * WAVES * kWave + t] = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (t == 0) cycles[blockIdx.x] = c1 - c0;
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void dma_kernel(const unsigned char* src,
                                                           uint32_t src_bytes, int iters,
                                                           uint32_t* sink, int64_t* cycles) {
    __shared__ __attribute__((aligned(16))) unsigned char buf[kLdsBytes];
    static_assert(WAVES * kDmaPerWave <= kLdsBytes, "each wave's slots fit");
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    // the range is the source itself: any offset past it would load zero, and none is
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(src), 0, static_cast<int>(src_bytes), 0x00020000);
    const uint32_t chunks = src_bytes / 1024u;  // whole 1 KB instruction footprints
    uint32_t pos = (uint32_t(blockIdx.x) * 7u + uint32_t(wave) * 8u) % chunks;
    __syncthreads();
    const int64_t c0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t c = pos + uint32_t(i) < chunks ? pos + uint32_t(i)
                                                          : pos + uint32_t(i) - chunks;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (lds_vptr)&buf[wave * kDmaPerWave + i * 1024], 16,
                c * 1024u + uint32_t(lane) * 16u, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        pos = pos + 8u < chunks ? pos + 8u : pos + 8u - chunks;
    }
    __syncthreads();
    const int64_t c1 = clock64();
    sink[int64_t(blockIdx.x) * WAVES * kWave + t] =
        reinterpret_cast<const uint32_t*>(buf)[t];  // keeps the loads
    if (t == 0) cycles[blockIdx.x] = c1 - c0;
}

template <int WAVES, int WIDTH>
hipError_t launch_read(int64_t groups, int iters, uint32_t* sink, int64_t* cycles,
                       hipStream_t stream) {
    hipLaunchKernelGGL((read_kernel<WAVES, WIDTH>), dim3(unsigned(groups)),
                       dim3(WAVES * kWave), 0, stream, iters, sink, cycles);
    return hipGetLastError();
}

template <int WIDTH>
hipError_t read_by_waves(int waves, int64_t groups, int iters, uint32_t* sink,
                         int64_t* cycles, hipStream_t stream) {
    switch (waves) {
        case 4: return launch_read<4, WIDTH>(groups, iters, sink, cycles, stream);
        case 8: return launch_read<8, WIDTH>(groups, iters, sink, cycles, stream);
        default: return launch_read<16, WIDTH>(groups, iters, sink, cycles, stream);
    }
}

template <int WAVES>
hipError_t launch_dma(const unsigned char* src, uint32_t src_bytes, int64_t groups, int iters,
                      uint32_t* sink, int64_t* cycles, hipStream_t stream) {
    hipLaunchKernelGGL((dma_kernel<WAVES>), dim3(unsigned(groups)), dim3(WAVES * kWave), 0,
                       stream, src, src_bytes, iters, sink, cycles);
    return hipGetLastError();
}

bool bad_shape(int waves, int64_t groups, int iters) {
    return (waves != 4 && waves != 8 && waves != 16) || groups < 1 ||
           groups >= (int64_t(1) << 31) || iters < 1;
}

}  // namespace

#define CEILING_API extern "C" __attribute__((visibility("default")))

// LDS bytes one workgroup reads (lds_read) or loads (lds_dma); -1 for bad arguments.
CEILING_API double lds_read_bytes(int waves, int iters, int width) {
    if (bad_shape(waves, 1, iters) || (width != 4 && width != 8 && width != 16)) return -1.0;
    return double(waves) * iters * 16 * kWave * width;
}
CEILING_API double lds_dma_bytes(int waves, int iters) {
    if (bad_shape(waves, 1, iters) || waves == 16) return -1.0;
    return double(waves) * iters * 8 * 1024;
}

// waves in {4, 8, 16}, width in {4, 8, 16}; sink holds groups * waves * 64 uint32 and cycles
// groups int64 (device memory owned by the caller).  Returns 0 on success, 1 for bad arguments
// (nothing launched), 2 for a launch error.
CEILING_API int lds_read(int waves, int64_t groups, int iters, int width, uint32_t* sink,
                         int64_t* cycles, hipStream_t stream) {
    if (sink == nullptr || cycles == nullptr || bad_shape(waves, groups, iters)) return 1;
    hipError_t e;
    switch (width) {
        case 4: e = read_by_waves<4>(waves, groups, iters, sink, cycles, stream); break;
        case 8: e = read_by_waves<8>(waves, groups, iters, sink, cycles, stream); break;
        case 16: e = read_by_waves<16>(waves, groups, iters, sink, cycles, stream); break;
        default: return 1;
    }
    return e == hipSuccess ? 0 : 2;
}

// waves in {4, 8}; src: src_bytes of device memory (a multiple of 1024, at least 8 KB, below
// 2^31) that every workgroup reads; sink and cycles as for lds_read.
CEILING_API int lds_dma(int waves, int64_t groups, int iters, const void* src,
                        int64_t src_bytes, uint32_t* sink, int64_t* cycles,
                        hipStream_t stream) {
    if (src == nullptr || sink == nullptr || cycles == nullptr ||
        bad_shape(waves, groups, iters) || waves == 16 || src_bytes < 8192 ||
        src_bytes >= (int64_t(1) << 31) || src_bytes % 1024 != 0)
        return 1;
    const auto* s = static_cast<const unsigned char*>(src);
    const uint32_t n = static_cast<uint32_t>(src_bytes);
    const hipError_t e = waves == 4 ? launch_dma<4>(s, n, groups, iters, sink, cycles, stream)
                                    : launch_dma<8>(s, n, groups, iters, sink, cycles, stream);
    return e == hipSuccess ? 0 : 2;
}
