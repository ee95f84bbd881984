// Bench probe (not part of the library): the HBM rates this part reaches on the access
// patterns of the log-probability kernels, so that their measured rates can be stated as a
// fraction of a measured ceiling as well as of the nominal 8 TB/s.
//
//   hbm_read  streams a buffer once: every wave takes one chunk of 64 * NV 16-byte vectors
//             (lane l holds vectors 64 k + l, so each load instruction covers 1 KiB of
//             contiguous memory), non-temporal 16-byte loads, all NV issued before any is
//             used -- the forward's pattern (4 waves per workgroup, 8 KiB per wave per tile).
//   hbm_copy  the same chunks read and written to a second buffer with 16-byte stores,
//             non-temporal at device scope (`sc1 nt`) -- the backward's pattern (one read
//             and one write per element; 16 KiB per wave, 16 waves per workgroup);
//             hbm_copy_nt the same with the non-temporal bit alone on the stores.
//   hbm_write fills the chunks with `sc1 nt` stores and reads nothing.
// Both are plain data movement: no arithmetic beyond an xor that keeps the loads alive.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

template <int NV, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void read_kernel(const u32x4* __restrict__ src,
                                                             int64_t chunks, uint32_t key,
                                                             uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk = int64_t(blockIdx.x) * WAVES + (threadIdx.x / kWave);
    if (chunk >= chunks) return;
    const u32x4* p = src + chunk * (kWave * NV) + lane;
    u32x4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = __builtin_nontemporal_load(p + kWave * k);
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < NV; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    if (acc == key) sink[0] = acc;  // practically never taken; keeps the loads
}

// 16-byte store, non-temporal at device scope; the s_nop gives the 2 wait states a VALU needs
// before it may write the store's data registers (the compiler does not look inside asm).
__device__ __forceinline__ void store_sc1_nt(u32x4* p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" : : "v"(p), "v"(v)
                 : "memory");
}

template <int NV, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void write_kernel(u32x4* __restrict__ dst,
                                                              int64_t chunks, uint32_t key) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk = int64_t(blockIdx.x) * WAVES + (threadIdx.x / kWave);
    if (chunk >= chunks) return;
    const int64_t base = chunk * (kWave * NV) + lane;
    const u32x4 v = {key, uint32_t(base), uint32_t(chunk), key ^ uint32_t(lane)};
#pragma unroll
    for (int k = 0; k < NV; ++k) store_sc1_nt(dst + base + kWave * k, v);
}

template <int NV, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void copy_nt_kernel(const u32x4* __restrict__ src,
                                                                u32x4* __restrict__ dst,
                                                                int64_t chunks) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk = int64_t(blockIdx.x) * WAVES + (threadIdx.x / kWave);
    if (chunk >= chunks) return;
    const int64_t base = chunk * (kWave * NV) + lane;
    u32x4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = __builtin_nontemporal_load(src + base + kWave * k);
#pragma unroll
    for (int k = 0; k < NV; ++k) __builtin_nontemporal_store(v[k], dst + base + kWave * k);
}

template <int NV, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void copy_kernel(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst,
                                                             int64_t chunks) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t chunk = int64_t(blockIdx.x) * WAVES + (threadIdx.x / kWave);
    if (chunk >= chunks) return;
    const int64_t base = chunk * (kWave * NV) + lane;
    u32x4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = __builtin_nontemporal_load(src + base + kWave * k);
#pragma unroll
    for (int k = 0; k < NV; ++k) store_sc1_nt(dst + base + kWave * k, v[k]);
}

template <int NV, int WAVES>
hipError_t launch_read(const void* src, int64_t chunks, uint32_t key, uint32_t* sink,
                       hipStream_t stream) {
    const int64_t groups = (chunks + WAVES - 1) / WAVES;
    hipLaunchKernelGGL((read_kernel<NV, WAVES>), dim3(unsigned(groups)), dim3(WAVES * kWave), 0,
                       stream, static_cast<const u32x4*>(src), chunks, key, sink);
    return hipGetLastError();
}

template <int NV, int WAVES>
hipError_t launch_copy(const void* src, void* dst, int64_t chunks, hipStream_t stream) {
    const int64_t groups = (chunks + WAVES - 1) / WAVES;
    hipLaunchKernelGGL((copy_kernel<NV, WAVES>), dim3(unsigned(groups)), dim3(WAVES * kWave), 0,
                       stream, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), chunks);
    return hipGetLastError();
}

// Chunk count of `bytes` at NV vectors per lane; -1 unless bytes is a positive multiple of
// the chunk and the grid fits.
int64_t chunk_count(int64_t bytes, int nv, int waves) {
    const int64_t chunk = int64_t(kWave) * nv * 16;
    if (bytes <= 0 || bytes % chunk != 0) return -1;
    const int64_t chunks = bytes / chunk;
    if ((chunks + waves - 1) / waves >= (int64_t(1) << 31)) return -1;
    return chunks;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

#define CEILING_API extern "C" __attribute__((visibility("default")))

// Shapes offered: vectors_per_lane in {8, 16, 32} (8, 16, 32 KiB per wave) and waves per
// workgroup in {4, 8, 16} (32 vectors per lane with 4 or 8 waves only: at 16 waves a lane
// has 128 registers, too few for 32 vectors in flight); reads also with 2 vectors per lane
// in 4-wave and 4 vectors in 8-wave workgroups (smaller footprints read about 1% faster).  Returns 0 on success, 1 for bad arguments (nothing launched),
// 2 for a launch error.  The caller owns every buffer; sink is one device uint32.
CEILING_API int hbm_read(const void* src, int64_t bytes, int vectors_per_lane, int waves,
                         uint32_t key, uint32_t* sink, hipStream_t stream) {
    if (src == nullptr || sink == nullptr || !aligned16(src)) return 1;
    const int64_t chunks = chunk_count(bytes, vectors_per_lane, waves);
    if (chunks < 0) return 1;
    hipError_t e = hipErrorInvalidValue;
#define READ_CASE(NV, W) \
    if (vectors_per_lane == NV && waves == W) e = launch_read<NV, W>(src, chunks, key, sink, stream);
    READ_CASE(2, 4) READ_CASE(4, 8)
    READ_CASE(8, 4) READ_CASE(8, 8) READ_CASE(8, 16)
    READ_CASE(16, 4) READ_CASE(16, 8) READ_CASE(16, 16)
    READ_CASE(32, 4) READ_CASE(32, 8)
#undef READ_CASE
    if (e == hipErrorInvalidValue) return 1;
    return e == hipSuccess ? 0 : 2;
}

CEILING_API int hbm_copy(const void* src, void* dst, int64_t bytes, int vectors_per_lane,
                         int waves, hipStream_t stream) {
    if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst)) return 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + uint64_t(bytes) && b < a + uint64_t(bytes)) return 1;  // overlapping buffers
    const int64_t chunks = chunk_count(bytes, vectors_per_lane, waves);
    if (chunks < 0) return 1;
    hipError_t e = hipErrorInvalidValue;
#define COPY_CASE(NV, W) \
    if (vectors_per_lane == NV && waves == W) e = launch_copy<NV, W>(src, dst, chunks, stream);
    COPY_CASE(8, 4) COPY_CASE(8, 8) COPY_CASE(8, 16)
    COPY_CASE(16, 4) COPY_CASE(16, 8) COPY_CASE(16, 16)
    COPY_CASE(32, 4) COPY_CASE(32, 8)
#undef COPY_CASE
    if (e == hipErrorInvalidValue) return 1;
    return e == hipSuccess ? 0 : 2;
}

// The 16 KiB-per-wave, 16-wave shape only; arguments and returns as for hbm_copy.
CEILING_API int hbm_copy_nt(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst)) return 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + uint64_t(bytes) && b < a + uint64_t(bytes)) return 1;  // overlapping buffers
    const int64_t chunks = chunk_count(bytes, 16, 16);
    if (chunks < 0) return 1;
    hipLaunchKernelGGL((copy_nt_kernel<16, 16>), dim3(unsigned((chunks + 15) / 16)),
                       dim3(16 * kWave), 0, stream, static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), chunks);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The 16 KiB-per-wave, 16-wave shape only: dst (bytes, a multiple of 16 KiB) is overwritten
// with values derived from key.  Returns as for hbm_copy.
CEILING_API int hbm_write(void* dst, int64_t bytes, uint32_t key, hipStream_t stream) {
    if (dst == nullptr || !aligned16(dst)) return 1;
    const int64_t chunks = chunk_count(bytes, 16, 16);
    if (chunks < 0) return 1;
    hipLaunchKernelGGL((write_kernel<16, 16>), dim3(unsigned((chunks + 15) / 16)),
                       dim3(16 * kWave), 0, stream, static_cast<u32x4*>(dst), chunks, key);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
