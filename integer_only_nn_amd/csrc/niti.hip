// NITI per-tensor dynamic-shift quantiser and weight update ("Integer
// On-Device Training: Overview", section 3 "The NITI Algorithm", steps 1-5),
// and the classifier output error of the device training loop (sections 4
// and 6.2).
//
// All three passes are HBM-bound streams.  A wavefront handles kChunk
// consecutive elements per iteration: instruction c reads int32 elements
// c*256 + 4*lane .. +3 (16 bytes per lane, 1 KiB contiguous per instruction)
// and reads/writes the matching int8 elements as one dword per lane (256
// bytes contiguous per instruction); all loads of an iteration are issued
// before any arithmetic.  This per-instruction contiguity measured 5.0 TB/s
// on the update against 3.2 TB/s for 64 contiguous bytes per lane (where each
// instruction touches a quarter of every cache line of a 4 KiB span).  The
// shift is derived in every thread from the device-resident max-abs scalar,
// so the producer's max and this pass chain on the stream without a host
// round trip.
#include "common.h"

namespace ionn {

__device__ __forceinline__ uint32_t pack4_i8(int32_t a, int32_t b, int32_t c, int32_t d) {
    return (uint32_t(a) & 0xffu) | ((uint32_t(b) & 0xffu) << 8) | ((uint32_t(c) & 0xffu) << 16) |
           (uint32_t(d) << 24);
}

__device__ __forceinline__ int32_t byte_i8(uint32_t w, int k) {
    return int32_t(int8_t(uint8_t(w >> (8 * k))));
}

// Per wavefront and iteration: kInstr load instructions of 1 KiB of int32.
constexpr int kInstr = 8;
constexpr int64_t kChunk = 256 * kInstr;

// out[j] = sat8(rhu(acc[j], s)) (and ReLU), s from *absmax.
template <bool VEC, bool RELU>
__global__ __launch_bounds__(256) void quantize_kernel(const int32_t *__restrict__ acc, int64_t n,
                                                       const uint32_t *__restrict__ absmax,
                                                       int target_bits, int8_t *__restrict__ out,
                                                       int32_t *__restrict__ shift_out) {
    const int s = niti_shift(*absmax, target_bits);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nthreads = int64_t(gridDim.x) * blockDim.x;
    if (tid == 0 && shift_out) *shift_out = s;
    auto q = [&](int32_t v) {
        int32_t r = sat8(rhu(v, s));
        return RELU ? (r > 0 ? r : 0) : r;
    };
    int64_t done = 0;
    if (VEC) {
        const int lane = threadIdx.x & 63;
        const int64_t wave = tid >> 6, nwaves = nthreads >> 6;
        const int64_t nfull = n / kChunk * kChunk;
        // two chunks a wavefront and step, loaded before either is stored
        // (as in update_kernel below)
        for (int64_t base = wave * 2 * kChunk; base < nfull; base += nwaves * 2 * kChunk) {
            const int64_t base2 = base + kChunk < nfull ? base + kChunk : base;
            v4i a[2][kInstr];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < kInstr; ++c)
                    a[h][c] = __builtin_nontemporal_load(
                        reinterpret_cast<const v4i *>(acc + (h ? base2 : base) + c * 256 + 4 * lane));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < kInstr; ++c)
                    *reinterpret_cast<uint32_t *>(out + (h ? base2 : base) + c * 256 + 4 * lane) =
                        pack4_i8(q(a[h][c].x), q(a[h][c].y), q(a[h][c].z), q(a[h][c].w));
        }
        done = nfull;
    }
    for (int64_t i = done + tid; i < n; i += nthreads) out[i] = int8_t(q(acc[i]));
}

// W[j] = sat8(W[j] - rhu(rhu(G[j], s), ws)), s and ws from *absmax.
// clear[0 .. n_clear) = 0 as well (block 0; n_clear <= 256; the host checks
// that clear does not overlap absmax, which every block reads).
template <bool VEC, bool GQ>
__global__ __launch_bounds__(256) void update_kernel(const int32_t *__restrict__ G, int64_t n,
                                                     const uint32_t *__restrict__ absmax,
                                                     int target_bits, int mu_weight,
                                                     int8_t *__restrict__ W,
                                                     int32_t *__restrict__ shifts_out,
                                                     int32_t *__restrict__ gq_out,
                                                     uint32_t *__restrict__ clear = nullptr,
                                                     int n_clear = 0) {
    const int s = niti_shift(*absmax, target_bits);
    const int ws = s - mu_weight > 0 ? s - mu_weight : 0;
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nthreads = int64_t(gridDim.x) * blockDim.x;
    if (tid == 0 && shifts_out) {
        shifts_out[0] = s;
        shifts_out[1] = ws;
    }
    if (tid < n_clear) clear[tid] = 0u;
    int64_t done = 0;
    if (VEC) {
        // Two chunks a wavefront and step, both loaded before the first one's
        // stores: the vector-memory counter retires in order and counts
        // stores, so loads issued after a chunk's stores would wait for them;
        // this way the first chunk's writes overlap the second one's reads.
        // Past the last chunk the second one re-reads the first and writes the
        // same bytes again: no branch, so the compiler neither sinks the
        // second chunk's loads into one nor loses its count of the loads and
        // stores in flight.
        const int lane = threadIdx.x & 63;
        const int64_t wave = tid >> 6, nwaves = nthreads >> 6;
        const int64_t nfull = n / kChunk * kChunk;
        for (int64_t base = wave * 2 * kChunk; base < nfull; base += nwaves * 2 * kChunk) {
            const bool two = base + kChunk < nfull;
            const int64_t base2 = two ? base + kChunk : base;
            v4i g[2][kInstr];
            uint32_t w[2][kInstr];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < kInstr; ++c) {
                    const int64_t e = (h ? base2 : base) + c * 256 + 4 * lane;
                    g[h][c] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(G + e));
                    w[h][c] = *reinterpret_cast<const uint32_t *>(W + e);
                }
            // (kept ahead of every store: the scheduler would otherwise sink
            // the second chunk's loads below the first chunk's stores)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int c = 0; c < kInstr; ++c) {
                    const int64_t e = (h ? base2 : base) + c * 256 + 4 * lane;
                    v4i gq;
                    gq.x = rhu(g[h][c].x, s);
                    gq.y = rhu(g[h][c].y, s);
                    gq.z = rhu(g[h][c].z, s);
                    gq.w = rhu(g[h][c].w, s);
                    if (GQ) *reinterpret_cast<v4i *>(gq_out + e) = gq;
                    *reinterpret_cast<uint32_t *>(W + e) =
                        pack4_i8(sat8(byte_i8(w[h][c], 0) - rhu(gq.x, ws)), sat8(byte_i8(w[h][c], 1) - rhu(gq.y, ws)),
                                 sat8(byte_i8(w[h][c], 2) - rhu(gq.z, ws)), sat8(byte_i8(w[h][c], 3) - rhu(gq.w, ws)));
                }
            }
        }
        done = nfull;
    }
    for (int64_t i = done + tid; i < n; i += nthreads) {
        int32_t gq = rhu(G[i], s);
        if (GQ) gq_out[i] = gq;
        W[i] = int8_t(sat8(int32_t(W[i]) - rhu(gq, ws)));
    }
}

// e[b][c] = (c == labels[b] ? target : 0) - out[b][c], plus max-abs.
__global__ __launch_bounds__(256) void output_error_kernel(const int8_t *__restrict__ out,
                                                           const int32_t *__restrict__ labels,
                                                           int64_t B, int64_t C, int target,
                                                           int32_t *__restrict__ e,
                                                           uint32_t *__restrict__ absmax) {
    uint32_t m = 0;
    const int64_t n = B * C;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        int64_t b = i / C, c = i - b * C;
        int32_t v = (c == int64_t(labels[b]) ? target : 0) - int32_t(out[i]);
        e[i] = v;
        m = max(m, abs_u32(v));
    }
    if (absmax) {
        m = wave_max_u32(m);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, m);
    }
}


// The quantiser's and the update's grid: two chunks per wavefront and step.
static unsigned update_blocks(int64_t n) {
    int64_t b = (n + 8 * kChunk - 1) / (8 * kChunk);
    if (b < 1) b = 1;
    if (b > 2048) b = 2048;
    return unsigned(b);
}

}  // namespace ionn

using namespace ionn;

extern "C" {

int niti_quantize(const int32_t *acc, int64_t n, const uint32_t *absmax, int target_bits, int relu,
                  int8_t *out, int32_t *shift_out, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 0, IONN_ERR_SHAPE, "niti_quantize: n = %lld < 0", (long long)n);
    IONN_REQUIRE(absmax != nullptr, IONN_ERR_ARG, "niti_quantize: absmax is NULL");
    IONN_REQUIRE(n == 0 || (acc != nullptr && out != nullptr), IONN_ERR_ARG,
                 "niti_quantize: acc/out is NULL");
    IONN_REQUIRE(target_bits >= 1 && target_bits <= 31, IONN_ERR_RANGE,
                 "niti_quantize: target_bits = %d outside [1, 31]", target_bits);
    IONN_REQUIRE(relu == 0 || relu == 1, IONN_ERR_ARG, "niti_quantize: relu = %d", relu);
    IONN_REQUIRE(aligned(acc, 4) && aligned(absmax, 4) && aligned(shift_out, 4), IONN_ERR_ALIGN,
                 "niti_quantize: int32 pointers must be 4-byte aligned");
    const bool vec = aligned(acc, 16) && aligned(out, 4);
    dim3 grid(update_blocks(n)), block(256);
    hipStream_t st = as_stream(stream);
    if (vec && relu) quantize_kernel<true, true><<<grid, block, 0, st>>>(acc, n, absmax, target_bits, out, shift_out);
    else if (vec) quantize_kernel<true, false><<<grid, block, 0, st>>>(acc, n, absmax, target_bits, out, shift_out);
    else if (relu) quantize_kernel<false, true><<<grid, block, 0, st>>>(acc, n, absmax, target_bits, out, shift_out);
    else quantize_kernel<false, false><<<grid, block, 0, st>>>(acc, n, absmax, target_bits, out, shift_out);
    return check_launch("niti_quantize");
}

int niti_quantize_update(const int32_t *G, int64_t n, const uint32_t *absmax, int target_bits,
                         int mu_weight, int8_t *W, int32_t *shifts_out, int32_t *gq_out,
                         void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 0, IONN_ERR_SHAPE, "niti_quantize_update: n = %lld < 0", (long long)n);
    IONN_REQUIRE(absmax != nullptr, IONN_ERR_ARG, "niti_quantize_update: absmax is NULL");
    IONN_REQUIRE(n == 0 || (G != nullptr && W != nullptr), IONN_ERR_ARG,
                 "niti_quantize_update: G/W is NULL");
    IONN_REQUIRE(target_bits >= 1 && target_bits <= 31, IONN_ERR_RANGE,
                 "niti_quantize_update: target_bits = %d outside [1, 31]", target_bits);
    IONN_REQUIRE(mu_weight >= 0 && mu_weight <= 31, IONN_ERR_RANGE,
                 "niti_quantize_update: mu_weight = %d outside [0, 31]", mu_weight);
    IONN_REQUIRE(aligned(G, 4) && aligned(absmax, 4) && aligned(shifts_out, 4) &&
                     aligned(gq_out, 4),
                 IONN_ERR_ALIGN, "niti_quantize_update: int32 pointers must be 4-byte aligned");
    const bool vec = aligned(G, 16) && aligned(W, 4) && aligned(gq_out, 16);
    dim3 grid(update_blocks(n)), block(256);
    hipStream_t st = as_stream(stream);
    if (vec && gq_out) update_kernel<true, true><<<grid, block, 0, st>>>(G, n, absmax, target_bits, mu_weight, W, shifts_out, gq_out);
    else if (vec) update_kernel<true, false><<<grid, block, 0, st>>>(G, n, absmax, target_bits, mu_weight, W, shifts_out, gq_out);
    else if (gq_out) update_kernel<false, true><<<grid, block, 0, st>>>(G, n, absmax, target_bits, mu_weight, W, shifts_out, gq_out);
    else update_kernel<false, false><<<grid, block, 0, st>>>(G, n, absmax, target_bits, mu_weight, W, shifts_out, gq_out);
    return check_launch("niti_quantize_update");
}

int niti_quantize_update_clear(const int32_t *G, int64_t n, const uint32_t *absmax, int target_bits,
                               int mu_weight, int8_t *W, int32_t *shifts_out, int32_t *gq_out,
                               uint32_t *clear, int64_t n_clear, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 0, IONN_ERR_SHAPE, "niti_quantize_update_clear: n = %lld < 0", (long long)n);
    IONN_REQUIRE(absmax != nullptr, IONN_ERR_ARG, "niti_quantize_update_clear: absmax is NULL");
    IONN_REQUIRE(n == 0 || (G != nullptr && W != nullptr), IONN_ERR_ARG,
                 "niti_quantize_update_clear: G/W is NULL");
    IONN_REQUIRE(target_bits >= 1 && target_bits <= 31, IONN_ERR_RANGE,
                 "niti_quantize_update_clear: target_bits = %d outside [1, 31]", target_bits);
    IONN_REQUIRE(mu_weight >= 0 && mu_weight <= 31, IONN_ERR_RANGE,
                 "niti_quantize_update_clear: mu_weight = %d outside [0, 31]", mu_weight);
    IONN_REQUIRE(n_clear >= 0 && n_clear <= 256 && (n_clear == 0 || clear != nullptr), IONN_ERR_ARG,
                 "niti_quantize_update_clear: n_clear = %lld (need 0..256 and a clear pointer)",
                 (long long)n_clear);
    const uintptr_t a = uintptr_t(absmax), c0 = uintptr_t(clear), c1 = c0 + uintptr_t(4 * n_clear);
    IONN_REQUIRE(n_clear == 0 || a + 4 <= c0 || a >= c1, IONN_ERR_ARG,
                 "niti_quantize_update_clear: clear overlaps absmax");
    IONN_REQUIRE(aligned(G, 4) && aligned(absmax, 4) && aligned(shifts_out, 4) && aligned(gq_out, 4) &&
                     aligned(clear, 4),
                 IONN_ERR_ALIGN, "niti_quantize_update_clear: int32 pointers must be 4-byte aligned");
    const bool vec = aligned(G, 16) && aligned(W, 4) && aligned(gq_out, 16);
    dim3 grid(update_blocks(n)), block(256);
    hipStream_t st = as_stream(stream);
    const int nc = int(n_clear);
    if (vec && gq_out) update_kernel<true, true><<<grid, block, 0, st>>>(G, n, absmax, target_bits, mu_weight, W, shifts_out, gq_out, clear, nc);
    else if (vec) update_kernel<true, false><<<grid, block, 0, st>>>(G, n, absmax, target_bits, mu_weight, W, shifts_out, gq_out, clear, nc);
    else if (gq_out) update_kernel<false, true><<<grid, block, 0, st>>>(G, n, absmax, target_bits, mu_weight, W, shifts_out, gq_out, clear, nc);
    else update_kernel<false, false><<<grid, block, 0, st>>>(G, n, absmax, target_bits, mu_weight, W, shifts_out, gq_out, clear, nc);
    return check_launch("niti_quantize_update_clear");
}

int int_output_error(const int8_t *out, const int32_t *labels, int64_t B, int64_t C,
                     int target_mag, int32_t *e, uint32_t *absmax_e, void *stream) {
    clear_error();
    IONN_REQUIRE(B >= 0 && C >= 0 && B <= kMaxDim && C <= kMaxDim && B * C <= kMaxDim,
                 IONN_ERR_SHAPE, "int_output_error: bad shape B=%lld C=%lld", (long long)B,
                 (long long)C);
    IONN_REQUIRE(target_mag >= -128 && target_mag <= 127, IONN_ERR_RANGE,
                 "int_output_error: target_mag = %d outside int8", target_mag);
    if (B * C == 0) return IONN_OK;
    IONN_REQUIRE(out && labels && e, IONN_ERR_ARG, "int_output_error: NULL tensor");
    IONN_REQUIRE(aligned(labels, 4) && aligned(e, 4) && aligned(absmax_e, 4), IONN_ERR_ALIGN,
                 "int_output_error: int32 pointers must be 4-byte aligned");
    int64_t blocks = (B * C + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    output_error_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, as_stream(stream)>>>(
        out, labels, B, C, target_mag, e, absmax_e);
    return check_launch("int_output_error");
}

}  // extern "C"
