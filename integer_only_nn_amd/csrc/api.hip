// Library-wide entry points: status strings, thread-local error message,
// version, and the two small helpers (fill, max-abs).
#include <cstdarg>

#include "common.h"

namespace ionn {

static thread_local char g_last_error[512] = "";

void set_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
}

void clear_error() { g_last_error[0] = 0; }

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
        return IONN_ERR_HIP;
    }
    return IONN_OK;
}

// dst[j] = value.
__global__ void fill_u32_kernel(uint32_t *__restrict__ dst, int64_t n, uint32_t value) {
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (; i < n; i += stride) dst[i] = value;
}

// Max-abs reduction, max-combined into *absmax: 16 elements per thread per
// iteration through 16-byte loads when x is 16-byte aligned, a wavefront
// reduction, then at most one atomicMax per wavefront (order-independent).
template <bool VEC>
__global__ __launch_bounds__(256) void absmax_kernel(const int32_t *__restrict__ x, int64_t n,
                                                     uint32_t *__restrict__ absmax) {
    uint32_t m = 0;
    int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t nthreads = int64_t(gridDim.x) * blockDim.x;
    if (VEC) {
        int64_t nvec = n / 4;
        const v4i *xv = reinterpret_cast<const v4i *>(x);
        for (int64_t i = tid; i < nvec; i += nthreads) {
            v4i v = __builtin_nontemporal_load(xv + i);
            uint32_t a = max(max(abs_u32(v.x), abs_u32(v.y)), max(abs_u32(v.z), abs_u32(v.w)));
            m = a > m ? a : m;
        }
        for (int64_t i = nvec * 4 + tid; i < n; i += nthreads) m = max(m, abs_u32(x[i]));
    } else {
        for (int64_t i = tid; i < n; i += nthreads) m = max(m, abs_u32(x[i]));
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, m);
}

int launch_absmax_i32(const int32_t *x, int64_t n, uint32_t *absmax, hipStream_t st) {
    if (n <= 0) return IONN_OK;
    int64_t blocks = (n + 16 * 256 - 1) / (16 * 256);
    if (blocks > 2048) blocks = 2048;
    if (aligned(x, 16))
        absmax_kernel<true><<<dim3(unsigned(blocks)), dim3(256), 0, st>>>(x, n, absmax);
    else
        absmax_kernel<false><<<dim3(unsigned(blocks)), dim3(256), 0, st>>>(x, n, absmax);
    return check_launch("max-abs");
}

}  // namespace ionn

using namespace ionn;

extern "C" {

const char *ionn_status_str(int status) {
    switch (status) {
        case IONN_OK: return "ok";
        case IONN_ERR_ARG: return "invalid argument";
        case IONN_ERR_SHAPE: return "invalid shape";
        case IONN_ERR_RANGE: return "parameter out of range";
        case IONN_ERR_ALIGN: return "misaligned pointer";
        case IONN_ERR_UNSUPPORTED: return "unsupported configuration";
        case IONN_ERR_HIP: return "HIP runtime error";
        case IONN_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

const char *ionn_last_error(void) { return g_last_error; }

const char *ionn_version(void) { return "ionn 0.1.0 gfx950"; }

int ionn_fill_u32(uint32_t *dst, int64_t n, uint32_t value, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 0, IONN_ERR_SHAPE, "ionn_fill_u32: n = %lld < 0", (long long)n);
    if (n == 0) return IONN_OK;
    IONN_REQUIRE(dst != nullptr, IONN_ERR_ARG, "ionn_fill_u32: dst is NULL");
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    fill_u32_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, as_stream(stream)>>>(dst, n, value);
    return check_launch("ionn_fill_u32");
}

int ionn_absmax_i32(const int32_t *x, int64_t n, uint32_t *absmax, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 0, IONN_ERR_SHAPE, "ionn_absmax_i32: n = %lld < 0", (long long)n);
    IONN_REQUIRE(absmax != nullptr, IONN_ERR_ARG, "ionn_absmax_i32: absmax is NULL");
    if (n == 0) return IONN_OK;
    IONN_REQUIRE(x != nullptr, IONN_ERR_ARG, "ionn_absmax_i32: x is NULL");
    IONN_REQUIRE(aligned(x, 4) && aligned(absmax, 4), IONN_ERR_ALIGN,
                 "ionn_absmax_i32: pointers must be 4-byte aligned");
    return launch_absmax_i32(x, n, absmax, as_stream(stream));
}

}  // extern "C"
