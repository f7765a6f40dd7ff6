// qkrope_host.h -- host-side helpers shared by the C-ABI translation units (qkrope_api.cpp,
// qkrope_api_cam.cpp): the handle, the per-thread error text, argument checks, device guard.
// Not installed.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <string>

#include "qkrope.h"

struct qkrope_ctx {
    int device;
    int num_cus;
    char arch[64];
};

namespace qkrope {
namespace host {

// Record a message for qkrope_last_error() on this thread and return `status`.
int fail(int status, const char *fmt, ...);
// Clear the message and return QKROPE_OK.
int ok();
// The calling thread's last message.
const char *last_error();

inline bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Bytes touched by a strided [tokens, span] tensor: rows of `span` elements every `stride`.
struct Range {
    uintptr_t lo, hi;          // bounding interval [lo, hi)
    int64_t stride_b, span_b;  // row stride and row length in bytes
};

inline Range span_of(const void *p, int64_t tokens, int64_t stride, int64_t span, int64_t esize)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (tokens <= 0 || span <= 0) return {lo, lo, 0, 0};
    return {lo, lo + (uintptr_t)(((tokens - 1) * stride + span) * esize), stride * esize,
            span * esize};
}

// Whether two strided tensors share a byte. Exact when both have the same row stride (rows of
// one sit in a gap of the other's period, as for column slices of one packed buffer);
// otherwise the bounding intervals decide.
inline bool overlap(Range a, Range b)
{
    if (a.lo == a.hi || b.lo == b.hi) return false;
    if (!(a.lo < b.hi && b.lo < a.hi)) return false;
    if (a.stride_b == b.stride_b && a.stride_b > 0 && a.span_b <= a.stride_b &&
        b.span_b <= b.stride_b) {
        const int64_t period = a.stride_b;
        const int64_t diff = (int64_t)(b.lo - a.lo);
        const int64_t d = ((diff % period) + period) % period;  // b's row start in a's period
        if (d >= a.span_b && d + b.span_b <= period) return false;
    }
    return true;
}

inline int next_pow2(int v)
{
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Device guard: make a device current for a launch and restore the caller's device after.
struct DeviceGuard {
    int prev = -1;
    bool switched = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            switched = err == hipSuccess;
        }
    }
    ~DeviceGuard()
    {
        if (switched) (void)hipSetDevice(prev);
    }
};

// Magic pair for n / d, 1 <= d, n < 2^31 (round-up method): with l = ceil(log2 d) and
// m = floor(2^32 * (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l; the sum cannot
// overflow 32 bits because mulhi(n, m) <= n < 2^31.
inline FastDiv make_fast_div(uint32_t d)
{
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l};
}

}  // namespace host
}  // namespace qkrope
