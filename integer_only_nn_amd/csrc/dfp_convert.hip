// Conversions between FP32 and DFP tensors and the FP32 weight update of the
// DFP training pipeline ("Mixed Precision Training of Convolutional Neural
// Networks using Integer Operations": 3 "The Dynamic Fixed Point Format",
// one shared exponent per tensor, or several for Blocked-DFP; 3.1 "DFP
// Tensor Primitives", the shared exponent of a converted tensor comes from
// the exponent of its absolute maximum; 4, FP32 outputs quantised again for
// the next layer, and the operations around the integer kernels in floating
// point).
//
// A P-bit tensor with max |x| = f * 2^q (f in [1, 2)) gets the exponent
// E = q - (P - 2), so max |x| / 2^E lies in [2^(P-2), 2^(P-1)), and every
// value becomes sat_P(round_to_nearest_even(x / 2^E)).  The division is done
// in double, where it is exact for every finite single and every E, so one
// rounding decides each mantissa.
#include "common.h"

namespace ionn {
namespace {

__global__ void zero_u32_kernel(uint32_t *p, int n) {
    if (int(threadIdx.x) < n) p[threadIdx.x] = 0u;
}

__device__ __forceinline__ double pow2(int e) {  // e in [-1022, 1023]
    return __longlong_as_double(int64_t(e + 1023) << 52);
}

// floor(log2 m) of a finite nonzero single given its magnitude bits.
__device__ __forceinline__ int floor_log2_bits(uint32_t u) {
    const int ex = int(u >> 23);
    return ex > 0 ? ex - 127 : -150 + bitlen_u32(u & 0x7fffffu);
}

// The shared exponent for magnitude bits m (0 for an all-zero tensor).
__device__ __forceinline__ int dfp_exponent(uint32_t m, int P) {
    return m ? floor_log2_bits(m) - (P - 2) : 0;
}

__device__ __forceinline__ int32_t dfp_elem(float x, double inv_scale, int32_t lo, int32_t hi) {
    const double r = __builtin_rint(double(x) * inv_scale);  // ties to even
    return r < double(lo) ? lo : (r > double(hi) ? hi : int32_t(r));
}

// Block max of one value per thread, then one publish per workgroup: with
// one per wavefront, the thousands of wavefronts of a large tensor queue on
// the single address (measured: 105 us instead of 15 us for 100 MB).
__device__ __forceinline__ void publish_block_max(uint32_t *m, uint32_t v) {
    __shared__ uint32_t red[4];
    v = wave_max_u32(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) publish_max_u32(m, max(max(red[0], red[1]), max(red[2], red[3])));
}

// Max of the magnitude bits: for non-negative singles the bit patterns order
// as the values, and a NaN or infinity shows as bits >= 0x7f800000.
__global__ __launch_bounds__(256) void absmax_bits_kernel(const float *__restrict__ x, int64_t n,
                                                          uint32_t *__restrict__ m) {
    uint32_t v = 0;
    const int64_t nt = int64_t(gridDim.x) * blockDim.x;
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t n4 = n / 4;
    for (int64_t i = tid; i < n4; i += nt) {
        const v4i q = reinterpret_cast<const v4i *>(x)[i];
        v = max(max(v, max(uint32_t(q.x) & 0x7fffffffu, uint32_t(q.y) & 0x7fffffffu)),
                max(uint32_t(q.z) & 0x7fffffffu, uint32_t(q.w) & 0x7fffffffu));
    }
    for (int64_t i = 4 * n4 + tid; i < n; i += nt) v = max(v, __float_as_uint(x[i]) & 0x7fffffffu);
    publish_block_max(m, v);
}

// Status: 0, 1 (exponent outside the signed 8-bit range), 2 (not finite).
__device__ __forceinline__ int32_t exp_status(uint32_t m, int E) {
    if (m >= 0x7f800000u) return 2;
    return (E < -128 || E > 127) ? 1 : 0;
}

__global__ __launch_bounds__(256) void from_f32_kernel(const float *__restrict__ x, int64_t n, int P,
                                                       const uint32_t *__restrict__ m, int16_t *__restrict__ out,
                                                       int32_t *__restrict__ e_out, int32_t *__restrict__ status) {
    const uint32_t mb = *m;
    const int E = mb >= 0x7f800000u ? 0 : dfp_exponent(mb, P);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nt = int64_t(gridDim.x) * blockDim.x;
    if (tid == 0) {
        *e_out = E;
        if (status) *status = exp_status(mb, E);
    }
    const double inv = pow2(-E);
    const int32_t hi = (int32_t(1) << (P - 1)) - 1, lo = -hi - 1;
    const int64_t n4 = n / 4;
    for (int64_t i = tid; i < n4; i += nt) {
        const float4 q = reinterpret_cast<const float4 *>(x)[i];
        const uint32_t a = uint32_t(dfp_elem(q.x, inv, lo, hi)) & 0xffffu, b = uint32_t(dfp_elem(q.y, inv, lo, hi));
        const uint32_t c = uint32_t(dfp_elem(q.z, inv, lo, hi)) & 0xffffu, d = uint32_t(dfp_elem(q.w, inv, lo, hi));
        reinterpret_cast<uint2 *>(out)[i] = make_uint2(a | (b << 16), c | (d << 16));
    }
    for (int64_t i = 4 * n4 + tid; i < n; i += nt) out[i] = int16_t(dfp_elem(x[i], inv, lo, hi));
}

__global__ __launch_bounds__(256) void to_f32_kernel(const int16_t *__restrict__ I, int64_t n,
                                                     const int32_t *__restrict__ e, float *__restrict__ out) {
    int ev = *e;
    ev = ev < -1022 ? -1022 : (ev > 1023 ? 1023 : ev);
    const double s = pow2(ev);
    const int64_t nt = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += nt)
        out[i] = float(double(I[i]) * s);
}

// Blocked-DFP: one wavefront per block of B values of a row.
__global__ __launch_bounds__(256) void from_f32_blocked_kernel(const float *__restrict__ x, int64_t rows, int64_t K,
                                                               int B, int P, int16_t *__restrict__ out,
                                                               int32_t *__restrict__ e_out,
                                                               int32_t *__restrict__ status) {
    const int64_t nb = (K + B - 1) / B;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    if (wave >= rows * nb) return;
    const int64_t r = wave / nb, b = wave - r * nb;
    const int64_t k0 = b * B, k1 = k0 + B < K ? k0 + B : K;
    const float *xr = x + r * K;
    uint32_t v = 0;
    for (int64_t k = k0 + lane; k < k1; k += 64) v = max(v, __float_as_uint(xr[k]) & 0x7fffffffu);
    v = wave_max_u32(v);
    const int E = v >= 0x7f800000u ? 0 : dfp_exponent(v, P);
    if (lane == 0) {
        e_out[wave] = E;
        const int32_t st = exp_status(v, E);
        if (status && st) atomicMax(status, st);
    }
    const double inv = pow2(-E);
    const int32_t hi = (int32_t(1) << (P - 1)) - 1, lo = -hi - 1;
    for (int64_t k = k0 + lane; k < k1; k += 64) out[r * K + k] = int16_t(dfp_elem(xr[k], inv, lo, hi));
}

// W32 = fl(W32 - fl(lr * G32)) (two roundings: contraction into a fused
// multiply-add is switched off here), with the max of the new magnitudes.
__global__ __launch_bounds__(256) void sgd_kernel(float *__restrict__ W, const float *__restrict__ G, int64_t n,
                                                  float lr, uint32_t *__restrict__ m) {
#pragma clang fp contract(off)
    uint32_t v = 0;
    const int64_t nt = int64_t(gridDim.x) * blockDim.x;
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t n4 = n / 4;
    for (int64_t i = tid; i < n4; i += nt) {
        float4 w = reinterpret_cast<float4 *>(W)[i];
        const float4 g = reinterpret_cast<const float4 *>(G)[i];
        w.x = w.x - lr * g.x;
        w.y = w.y - lr * g.y;
        w.z = w.z - lr * g.z;
        w.w = w.w - lr * g.w;
        reinterpret_cast<float4 *>(W)[i] = w;
        v = max(max(v, max(__float_as_uint(w.x) & 0x7fffffffu, __float_as_uint(w.y) & 0x7fffffffu)),
                max(__float_as_uint(w.z) & 0x7fffffffu, __float_as_uint(w.w) & 0x7fffffffu));
    }
    for (int64_t i = 4 * n4 + tid; i < n; i += nt) {
        W[i] = W[i] - lr * G[i];
        v = max(v, __float_as_uint(W[i]) & 0x7fffffffu);
    }
    publish_block_max(m, v);
}

// Workgroups for a pass over n values, 4 per thread per step, at most 1024
// (four per compute unit; the loops stride over the rest).
unsigned grid_for(int64_t n) {
    int64_t b = (n / 4 + 255) / 256;
    if (b < 1) b = 1;
    if (b > 1024) b = 1024;
    return unsigned(b);
}

// absmax bits of x into ws[0], then the P-bit conversion.
int convert(const float *x, int64_t n, int P, int16_t *out, int32_t *e_out, int32_t *status, uint32_t *m,
            hipStream_t st, const char *who) {
    absmax_bits_kernel<<<dim3(grid_for(n)), dim3(256), 0, st>>>(x, n, m);
    if (int rc = check_launch(who)) return rc;
    from_f32_kernel<<<dim3(grid_for(n)), dim3(256), 0, st>>>(x, n, P, m, out, e_out, status);
    return check_launch(who);
}

}  // namespace
}  // namespace ionn

using namespace ionn;

extern "C" {

size_t dfp_convert_workspace_bytes(void) { return 256; }

int dfp_from_f32(const float *x, int64_t n, int P, int16_t *out, int32_t *e_out, int32_t *status_out,
                 void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 1 && n <= (int64_t(1) << 40), IONN_ERR_SHAPE, "dfp_from_f32: n = %lld", (long long)n);
    IONN_REQUIRE(P >= 2 && P <= 16, IONN_ERR_RANGE, "dfp_from_f32: P = %d outside [2, 16]", P);
    IONN_REQUIRE(x && out && e_out, IONN_ERR_ARG, "dfp_from_f32: NULL argument");
    IONN_REQUIRE(aligned(x, 16) && aligned(out, 8) && aligned(e_out, 4) && aligned(status_out, 4), IONN_ERR_ALIGN,
                 "dfp_from_f32: x needs 16-byte, out 8-byte, e_out/status 4-byte alignment");
    IONN_REQUIRE(workspace && aligned(workspace, 4) && workspace_bytes >= 4, IONN_ERR_WORKSPACE,
                 "dfp_from_f32: needs a 4-byte aligned workspace of dfp_convert_workspace_bytes() bytes");
    hipStream_t st = as_stream(stream);
    uint32_t *m = static_cast<uint32_t *>(workspace);
    zero_u32_kernel<<<dim3(1), dim3(64), 0, st>>>(m, 1);
    if (int rc = check_launch("dfp_from_f32")) return rc;
    return convert(x, n, P, out, e_out, status_out, m, st, "dfp_from_f32");
}

int dfp_to_f32(const int16_t *I, int64_t n, const int32_t *e, float *out, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 1 && n <= (int64_t(1) << 40), IONN_ERR_SHAPE, "dfp_to_f32: n = %lld", (long long)n);
    IONN_REQUIRE(I && e && out, IONN_ERR_ARG, "dfp_to_f32: NULL argument");
    IONN_REQUIRE(aligned(I, 2) && aligned(e, 4) && aligned(out, 4), IONN_ERR_ALIGN, "dfp_to_f32: misaligned");
    to_f32_kernel<<<dim3(grid_for(4 * n)), dim3(256), 0, as_stream(stream)>>>(I, n, e, out);
    return check_launch("dfp_to_f32");
}

int dfp_from_f32_blocked(const float *x, int64_t rows, int64_t K, int B, int P, int16_t *out, int32_t *e_out,
                         int32_t *status_out, void *stream) {
    clear_error();
    IONN_REQUIRE(rows >= 1 && K >= 1 && rows * K <= (int64_t(1) << 40), IONN_ERR_SHAPE,
                 "dfp_from_f32_blocked: rows = %lld, K = %lld", (long long)rows, (long long)K);
    IONN_REQUIRE(B >= 1, IONN_ERR_RANGE, "dfp_from_f32_blocked: B = %d < 1", B);
    IONN_REQUIRE(P >= 2 && P <= 16, IONN_ERR_RANGE, "dfp_from_f32_blocked: P = %d outside [2, 16]", P);
    IONN_REQUIRE(x && out && e_out, IONN_ERR_ARG, "dfp_from_f32_blocked: NULL argument");
    IONN_REQUIRE(aligned(x, 4) && aligned(out, 2) && aligned(e_out, 4) && aligned(status_out, 4), IONN_ERR_ALIGN,
                 "dfp_from_f32_blocked: misaligned pointer");
    const int64_t waves = rows * ((K + B - 1) / B);
    IONN_REQUIRE((waves + 3) / 4 <= 0x7fffffff, IONN_ERR_SHAPE, "dfp_from_f32_blocked: too many blocks");
    hipStream_t st = as_stream(stream);
    if (status_out) {
        zero_u32_kernel<<<dim3(1), dim3(64), 0, st>>>(reinterpret_cast<uint32_t *>(status_out), 1);
        if (int rc = check_launch("dfp_from_f32_blocked")) return rc;
    }
    from_f32_blocked_kernel<<<dim3(unsigned((waves + 3) / 4)), dim3(256), 0, st>>>(x, rows, K, B, P, out, e_out,
                                                                                   status_out);
    return check_launch("dfp_from_f32_blocked");
}

int dfp16_sgd_update(float *W32, const float *G32, int64_t n, float lr, int16_t *W16, int32_t *eW,
                     int32_t *status_out, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 1 && n <= (int64_t(1) << 40), IONN_ERR_SHAPE, "dfp16_sgd_update: n = %lld", (long long)n);
    IONN_REQUIRE(W32 && G32 && W16 && eW, IONN_ERR_ARG, "dfp16_sgd_update: NULL argument");
    IONN_REQUIRE(aligned(W32, 16) && aligned(G32, 16) && aligned(W16, 8) && aligned(eW, 4) &&
                     aligned(status_out, 4),
                 IONN_ERR_ALIGN, "dfp16_sgd_update: W32/G32 need 16-byte, W16 8-byte alignment");
    IONN_REQUIRE(workspace && aligned(workspace, 4) && workspace_bytes >= 4, IONN_ERR_WORKSPACE,
                 "dfp16_sgd_update: needs a 4-byte aligned workspace of dfp_convert_workspace_bytes() bytes");
    hipStream_t st = as_stream(stream);
    uint32_t *m = static_cast<uint32_t *>(workspace);
    zero_u32_kernel<<<dim3(1), dim3(64), 0, st>>>(m, 1);
    if (int rc = check_launch("dfp16_sgd_update")) return rc;
    sgd_kernel<<<dim3(grid_for(n)), dim3(256), 0, st>>>(W32, G32, n, lr, m);
    if (int rc = check_launch("dfp16_sgd_update")) return rc;
    from_f32_kernel<<<dim3(grid_for(n)), dim3(256), 0, st>>>(W32, n, 16, m, W16, eW, status_out);
    return check_launch("dfp16_sgd_update");
}

}  // extern "C"
