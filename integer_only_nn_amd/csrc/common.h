// Internal helpers shared by the library's translation units: host-side
// argument checking and error state, and the device-side integer primitives
// of the NITI quantiser ("Integer On-Device Training: Overview", section 3,
// steps 1-5).  Device code targets gfx950 only.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/ionn.h"

namespace ionn {

// ---------------------------------------------------------------------------
// Host: error state and checks.
// ---------------------------------------------------------------------------

void set_error(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

#define IONN_REQUIRE(cond, code, ...)      \
    do {                                   \
        if (!(cond)) {                     \
            ::ionn::set_error(__VA_ARGS__); \
            return (code);                 \
        }                                  \
    } while (0)

// Check the launch that was just enqueued.
int check_launch(const char *what);

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned(const void *p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Compute units of the current device (persistent grids), cached per device.
inline int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

// ---------------------------------------------------------------------------
// Device: integer primitives.
// ---------------------------------------------------------------------------

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// |x| as uint32 so |INT32_MIN| = 2^31.
__device__ __forceinline__ uint32_t abs_u32(int32_t x) {
    return x < 0 ? 0u - static_cast<uint32_t>(x) : static_cast<uint32_t>(x);
}

// Number of binary digits: 0 for 0, else floor(log2 m) + 1 == ceil(log2(m+1)).
__device__ __forceinline__ int bitlen_u32(uint32_t m) {
    return m ? 32 - __builtin_clz(m) : 0;
}

// shift = max(0, bitlen(max_val) - target_bits).
__device__ __forceinline__ int niti_shift(uint32_t max_val, int target_bits) {
    int s = bitlen_u32(max_val) - target_bits;
    return s > 0 ? s : 0;
}

// Round-half-up right shift floor((x + 2^(s-1)) / 2^s), computed without the
// overflowing add: floor(x / 2^s) plus bit (s-1) of x.  s in [0, 31].
__device__ __forceinline__ int32_t rhu(int32_t x, int s) {
    if (s == 0) return x;
    return (x >> s) + ((x >> (s - 1)) & 1);
}

__device__ __forceinline__ int32_t sat8(int32_t v) { return v < -128 ? -128 : (v > 127 ? 127 : v); }
__device__ __forceinline__ int32_t sat16(int32_t v) {
    return v < -32768 ? -32768 : (v > 32767 ? 32767 : v);
}

// One element of the static OSS requantisation ("Integer On-Device Training:
// Overview", section 8, PC-side Step 2: Add(offset) -> Mul -> Mul -> Floor ->
// Clip): t = acc + offset modulo 2^32 (the int32 accumulator), t * mult exact
// in 64 bits (|t * mult| <= 2^62), floor division by 2^k as an arithmetic
// shift (k in [0, 62]; & 63 keeps any byte a defined shift), clip to
// [lo, 127].
__device__ __forceinline__ int32_t oss_elem(int32_t acc, int32_t off, int32_t mult, int k, int32_t lo) {
    const int32_t t = int32_t(uint32_t(acc) + uint32_t(off));
    const int64_t y = (int64_t(t) * int64_t(mult)) >> (k & 63);
    return y < lo ? lo : (y > 127 ? 127 : int32_t(y));
}

// Four int8 values (low bytes of a..d) in one dword, a lowest.
__device__ __forceinline__ uint32_t pack4_u8(int32_t a, int32_t b, int32_t c, int32_t d) {
    return (uint32_t(a) & 0xffu) | ((uint32_t(b) & 0xffu) << 8) | ((uint32_t(c) & 0xffu) << 16) |
           (uint32_t(d) << 24);
}

// Max over the 64 lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// Fold a wavefront's value v (already reduced over its lanes) into the
// device-wide max at *absmax.  The atomic is skipped when the current value is
// already at least v: the maximum only grows, so the result is the same, and
// the many wavefronts of a grid do not queue on one address.
__device__ __forceinline__ void publish_max_u32(uint32_t *absmax, uint32_t v) {
    if (v == 0) return;
    if (__hip_atomic_load(absmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= v) return;
    atomicMax(absmax, v);
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace ionn
