// Host-side argument checks and launch helpers shared by the library's C entry points:
// device location and extent of every buffer, overlap of outputs with inputs, the stream's
// device, a device guard, and launches that report failure as a status code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logp.h"

namespace logp_host {

struct Span {
    const void* p;
    uint64_t bytes;
};

inline bool overlaps(Span a, Span b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Bytes spanned by `rows` rows of `width` elements of `elem` bytes at stride `ld` elements,
// or 0 on overflow (callers have already bounded every factor).
inline uint64_t span_bytes(int64_t rows, int64_t ld, int64_t width, int64_t elem) {
    if (rows <= 0 || width <= 0) return 0;
    const unsigned __int128 b =
        (static_cast<unsigned __int128>(rows - 1) * static_cast<uint64_t>(ld) + width) * elem;
    if (b > (static_cast<unsigned __int128>(1) << 62)) return 0;
    return static_cast<uint64_t>(b);
}

// Device of `p` (device or managed memory), checked to hold `bytes` from `p` on.
inline logp_status_t locate(const void* p, uint64_t bytes, int* device) {
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
inline logp_status_t check_buffers(const Span* in, int n_in, const Span* out, int n_out,
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

inline logp_status_t launch(const void* kernel, dim3 grid, dim3 block, void** args, size_t lds,
                     hipStream_t stream) {
    if (hipLaunchKernel(kernel, grid, block, args, lds, stream) != hipSuccess) {
        (void)hipGetLastError();
        return LOGP_ERR_HIP;
    }
    return LOGP_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace logp_host
