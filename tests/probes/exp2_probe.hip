// Test probe (not part of the library): ulp error of the hardware exp2 (v_exp_f32, through
// __builtin_amdgcn_exp2f) against the float rounding of the double-precision exp2, over a
// contiguous range of float bit patterns.  The logp kernels' softmax terms rest on this
// instruction; the probe measures how far it is from correctly rounded.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

// out[2 b] = largest ulp distance seen by workgroup b, out[2 b + 1] = how many of its values
// were not the correctly rounded result.  Values: bit patterns lo + i, i in [0, count).
__global__ __launch_bounds__(kThreads) void exp2_ulp_kernel(uint32_t lo, uint32_t count,
                                                            uint32_t* __restrict__ out) {
    uint32_t worst = 0, off = 0;
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < count; i += stride) {
        const float x = __uint_as_float(lo + i);
        const uint32_t a = __float_as_uint(__builtin_amdgcn_exp2f(x));
        const uint32_t r = __float_as_uint(static_cast<float>(exp2(static_cast<double>(x))));
        const uint32_t d = a > r ? a - r : r - a;  // both positive: ulp distance
        worst = d > worst ? d : worst;
        off += d != 0 ? 1u : 0u;
    }
    __shared__ uint32_t sw[kThreads], so[kThreads];
    const int t = threadIdx.x;
    sw[t] = worst;
    so[t] = off;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (t < s) {
            sw[t] = sw[t] > sw[t + s] ? sw[t] : sw[t + s];
            so[t] += so[t + s];
        }
        __syncthreads();
    }
    if (t == 0) {
        out[2 * blockIdx.x] = sw[0];
        out[2 * blockIdx.x + 1] = so[0];
    }
}

}  // namespace

// out: 2 * blocks uint32 of device memory.  count < 2^31.  Returns 0, or 1 on a launch error.
extern "C" __attribute__((visibility("default"))) int exp2_probe(uint32_t lo, uint32_t count,
                                                                 uint32_t* out, int blocks,
                                                                 hipStream_t stream) {
    if (out == nullptr || blocks < 1 || count >= (1u << 31)) return 1;
    hipLaunchKernelGGL(exp2_ulp_kernel, dim3(blocks), dim3(kThreads), 0, stream, lo, count,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
