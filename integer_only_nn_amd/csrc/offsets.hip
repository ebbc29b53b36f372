// Per-channel int32 offsets (bias) and the static OSS forward
// requantisation ("Integer On-Device Training: Overview", section 7: each
// INT_LAYERS entry carries mutable int32 offsets, updated by the backward
// pass, and per-filter right shifts k with multipliers mult; section 8,
// PC-side Step 2: the OSS chain Add(offset) -> Mul(scale1) -> Mul(scale2) ->
// Floor -> Clip), plus the offsets' gradient and their NITI update
// (section 3, steps 1-5).
//
// OSS and the update are HBM-bound streams with the mapping of the NITI
// quantiser: instruction c of a wavefront reads int32 elements
// c*256 + 4*lane .. +3 (1 KiB contiguous per instruction).  The offset
// gradient sums int8 columns: a lane owns 16 columns (16 bytes of a row), a
// workgroup 1 KiB of every row of its row range; the per-range sums go to a
// workspace and a second pass adds them (integer atomics from every
// workgroup queued on the same addresses and ran at a tenth of the
// bandwidth).
#include "common.h"
#include "wgrad_long.h"

#include <algorithm>
#include <mutex>

namespace ionn {
namespace {

constexpr int kInstr = 8;                  // 1 KiB loads per wavefront and iteration
// Size of the allocation-free offset gradient's device scratch (2 MiB: the
// row-range sums of up to 2^19 columns x ranges).
constexpr size_t kBgScratchBytes = size_t(2) << 20;
constexpr size_t kBgScratchInts = kBgScratchBytes / sizeof(int32_t);
constexpr int64_t kChunk = 256 * kInstr;   // int32 elements per wavefront and iteration

// One kChunk per wavefront (4 per block), up to 16384 blocks: a wavefront
// that looped would issue its next chunk's loads after its stores and wait
// for them (the counter retires in order).
unsigned stream_blocks(int64_t n) {
    int64_t b = (n + 4 * kChunk - 1) / (4 * kChunk);
    if (b < 1) b = 1;
    if (b > 16384) b = 16384;
    return unsigned(b);
}

// VEC: C % 4 == 0, acc / offset / mult 16-byte aligned, out / k 4-byte
// aligned, so the four elements of a lane's 16 bytes share one row and
// their parameters are four consecutive entries.
template <bool VEC, bool RELU>
__global__ __launch_bounds__(256) void oss_kernel(const int32_t *__restrict__ acc, int64_t n, int64_t C,
                                                  const int32_t *__restrict__ offset,
                                                  const int32_t *__restrict__ mult,
                                                  const int8_t *__restrict__ k,
                                                  int8_t *__restrict__ out) {
    constexpr int32_t lo = RELU ? 0 : -128;
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nthreads = int64_t(gridDim.x) * blockDim.x;
    int64_t done = 0;
    if (VEC) {
        const int lane = threadIdx.x & 63;
        const int64_t wave = tid >> 6, nwaves = nthreads >> 6;
        const int64_t nfull = n / kChunk * kChunk;
        const uint32_t Cu = uint32_t(C);
        for (int64_t base = wave * kChunk; base < nfull; base += nwaves * kChunk) {
            v4i a[kInstr];
#pragma unroll
            for (int c = 0; c < kInstr; ++c)
                a[c] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(acc + base + c * 256 + 4 * lane));
            // every piece's parameters loaded before the first store (the
            // vector-memory counter retires in order and counts stores, so a
            // load issued after a store would wait for it as well)
            const uint32_t ch0 = uint32_t((base + 4 * lane) % C);
            v4i o[kInstr], m[kInstr];
            uint32_t kk[kInstr];
#pragma unroll
            for (int c = 0; c < kInstr; ++c) {
                const uint32_t ch = (ch0 + uint32_t(c * 256)) % Cu;
                o[c] = *reinterpret_cast<const v4i *>(offset + ch);
                m[c] = *reinterpret_cast<const v4i *>(mult + ch);
                kk[c] = *reinterpret_cast<const uint32_t *>(k + ch);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < kInstr; ++c)
                *reinterpret_cast<uint32_t *>(out + base + c * 256 + 4 * lane) =
                    pack4_u8(oss_elem(a[c].x, o[c].x, m[c].x, int(kk[c] & 0xffu), lo),
                             oss_elem(a[c].y, o[c].y, m[c].y, int((kk[c] >> 8) & 0xffu), lo),
                             oss_elem(a[c].z, o[c].z, m[c].z, int((kk[c] >> 16) & 0xffu), lo),
                             oss_elem(a[c].w, o[c].w, m[c].w, int(kk[c] >> 24), lo));
        }
        done = nfull;
    }
    // n < 2^31: 32-bit element and channel indices
    const uint32_t Cu = uint32_t(C);
    for (uint32_t j = uint32_t(done + tid); j < uint32_t(n); j += uint32_t(nthreads)) {
        const uint32_t ch = j % Cu;
        out[j] = int8_t(oss_elem(acc[j], offset[ch], mult[ch], int(k[ch]), lo));
    }
}

// Column sums of the int8 rows d[M][C] over row range y of the grid.  VEC: a
// lane owns columns 16 cg .. 16 cg + 15 (C % 16 == 0, d 16-byte aligned),
// a workgroup a 1 KiB strip of every row in its range, its eight wavefronts
// every eighth row; otherwise a lane owns one column.  The workgroup's sums
// go to part[y][c] (no atomics: the second pass adds the row ranges).
constexpr int BG_WAVES = 8;
template <bool VEC>
__global__ __launch_bounds__(64 * BG_WAVES) void bias_grad_kernel(const int8_t *__restrict__ d, int64_t M,
                                                                  int64_t C, int64_t rows_per_block,
                                                                  int32_t *__restrict__ part) {
    constexpr int W = VEC ? 16 : 1;  // columns per lane
    __shared__ int32_t red[BG_WAVES][64][W + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t(blockIdx.x) * 64 + lane) * W;
    const int64_t r0 = int64_t(blockIdx.y) * rows_per_block;
    const int64_t r1 = min(M, r0 + rows_per_block);
    int32_t s[W];
#pragma unroll
    for (int e = 0; e < W; ++e) s[e] = 0;
    if (c0 < C) {
        if (VEC) {
            // bytes offset by 128 (x ^ 0x80 = x + 128, in [0, 255]) and added
            // two columns per 32-bit add in 16-bit fields: even bytes of a
            // dword in one word, odd bytes in another; a field holds the sum
            // of up to 257 rows, so the fields go to the int32 sums (less 128
            // per row) every 256 rows of the lane
            constexpr int U = 8, S = BG_WAVES;
            int64_t r = r0 + wave;
            while (r < r1) {
                uint32_t fe[4] = {0, 0, 0, 0}, fo[4] = {0, 0, 0, 0};
                const int64_t rend = min(r1, r + int64_t(256) * S);
                int n = 0;
                auto add = [&](const v4i &w) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t x = uint32_t(w[q]) ^ 0x80808080u;
                        fe[q] += x & 0x00ff00ffu;
                        fo[q] += (x >> 8) & 0x00ff00ffu;
                    }
                };
                for (; r + (U - 1) * S < rend; r += U * S, n += U) {
                    v4i w[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const v4i *>(d + (r + u * S) * C + c0);
#pragma unroll
                    for (int u = 0; u < U; ++u) add(w[u]);
                }
                for (; r < rend; r += S, ++n) add(*reinterpret_cast<const v4i *>(d + r * C + c0));
                const int32_t off = 128 * n;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    s[4 * q] += int32_t(fe[q] & 0xffffu) - off;
                    s[4 * q + 1] += int32_t(fo[q] & 0xffffu) - off;
                    s[4 * q + 2] += int32_t(fe[q] >> 16) - off;
                    s[4 * q + 3] += int32_t(fo[q] >> 16) - off;
                }
            }
        } else {
            for (int64_t r = r0 + wave; r < r1; r += BG_WAVES) s[0] += int32_t(d[r * C + c0]);
        }
    }
#pragma unroll
    for (int e = 0; e < W; ++e) red[wave][lane][e] = s[e];
    __syncthreads();
    if (wave == 0 && c0 < C) {
#pragma unroll
        for (int e = 0; e < W; ++e) {
            uint32_t t = 0;
#pragma unroll
            for (int w = 0; w < BG_WAVES; ++w) t += uint32_t(red[w][lane][e]);
            if (c0 + e < C) part[int64_t(blockIdx.y) * C + c0 + e] = int32_t(t);
        }
    }
}

// Column sums of a narrow d[M][C] (C < 64, d 4-byte aligned): the M*C bytes
// read as one flat array of dwords.  Thread t of the grid takes dwords t,
// t + T, t + 2T, ... (T threads in all, 4T a multiple of C), so byte e of every
// dword it reads lies in the same column (4t + e) mod C.  The thread's four
// sums meet the workgroup's in LDS bins; the workgroup's row goes to
// part[blockIdx.x][c].  Block 0 adds the last n mod 4 bytes.
__global__ __launch_bounds__(256) void bias_grad_narrow(const int8_t *__restrict__ d, int64_t n, int C,
                                                        int32_t *__restrict__ part) {
    __shared__ uint32_t bins[64];
    if (threadIdx.x < 64) bins[threadIdx.x] = 0;
    __syncthreads();
    const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x, T = int64_t(gridDim.x) * blockDim.x;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(d);
    const int64_t nw = n / 4;
    uint32_t s[4] = {0, 0, 0, 0};
    auto add = [&](uint32_t x) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += uint32_t(int32_t(int8_t(uint8_t(x >> (8 * e)))));
    };
    int64_t i = t;
    for (; i + 3 * T < nw; i += 4 * T) {  // four loads in flight
        uint32_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = __builtin_nontemporal_load(w + i + u * T);
#pragma unroll
        for (int u = 0; u < 4; ++u) add(x[u]);
    }
    for (; i < nw; i += T) add(w[i]);
    const int c0 = int((4 * t) % C);
#pragma unroll
    for (int e = 0; e < 4; ++e) atomicAdd(&bins[(c0 + e) % C], s[e]);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        for (int64_t j = 4 * nw; j < n; ++j) atomicAdd(&bins[j % C], uint32_t(int32_t(d[j])));
    __syncthreads();
    if (int(threadIdx.x) < C) part[int64_t(blockIdx.x) * C + threadIdx.x] = int32_t(bins[threadIdx.x]);
}

// Workgroups of bias_grad_narrow: at most `cap` (the rows of partial sums the
// workspace holds) and at most 256, a multiple of C / gcd(C, 1024) so that
// the dword stride 4 * 256 * G is a multiple of C; 0 when no such count fits.
int64_t narrow_blocks(int64_t C, int64_t cap) {
    int64_t a = C, b = 1024;
    while (b) { const int64_t r = a % b; a = b; b = r; }
    const int64_t q = C / a;
    int64_t g = cap < 256 ? cap : 256;
    g -= g % q;
    return g;
}


// Row split of the offset gradient: about 256 workgroups of 1 KiB strips in
// all, each with at least 64 rows; the workspace holds one int32 row of C
// per range.  The split depends on M and C only, so the workspace query
// holds for either layout.
struct BgGrid {
    int64_t gx, gy, rows;
    bool vec;
};
BgGrid bg_grid(int64_t M, int64_t C, bool vec) {
    BgGrid g;
    g.vec = vec;
    const int64_t strips = (C + 1023) / 1024;
    g.gx = vec ? strips : (C + 63) / 64;
    int64_t gy = (256 + strips - 1) / strips;
    int64_t rows = (M + gy - 1) / gy;
    if (rows < 64) rows = 64;
    g.rows = rows;
    g.gy = M > 0 ? (M + rows - 1) / rows : 0;
    return g;
}

__global__ void zero_kernel(int32_t *p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0;
}

// P[j] = sat32(P[j] - rhu(rhu(G[j], s), ws)), s from *absmax.
__global__ __launch_bounds__(256) void update_i32_kernel(const int32_t *__restrict__ G, int64_t n,
                                                         const uint32_t *__restrict__ absmax, int target_bits,
                                                         int mu, int32_t *__restrict__ P,
                                                         int32_t *__restrict__ shifts_out,
                                                         int32_t *__restrict__ gq_out) {
    const int s = niti_shift(*absmax, target_bits);
    const int ws = s > mu ? s - mu : 0;
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (tid == 0 && shifts_out) {
        shifts_out[0] = s;
        shifts_out[1] = ws;
    }
    for (int64_t j = tid; j < n; j += int64_t(gridDim.x) * blockDim.x) {
        const int32_t gq = rhu(G[j], s);
        const int64_t v = int64_t(P[j]) - int64_t(rhu(gq, ws));
        P[j] = v < INT32_MIN ? INT32_MIN : (v > INT32_MAX ? INT32_MAX : int32_t(v));
        if (gq_out) gq_out[j] = gq;
    }
}

}  // namespace
}  // namespace ionn

// Device scratch of ionn_bias_grad_noalloc: the row-range sums of the offset
// gradient, for callers that cannot allocate.  One copy per GPU, held until
// the process ends.  In host code `scratch` only names the symbol; its
// device address comes from hipGetSymbolAddress (bg_scratch) and is what
// the kernels receive.
static __device__ __align__(256) int32_t scratch[ionn::kBgScratchInts];

namespace ionn {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the GPU that owns `st` (the current
// device for the null stream), looked up once per device with that device
// current.
int bg_scratch(hipStream_t st, int32_t **out) {
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    IONN_REQUIRE(e == hipSuccess && dev >= 0 && dev < kMaxDevices, IONN_ERR_HIP,
                 "ionn_bias_grad_noalloc: cannot tell the stream's device (%s)", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        IONN_REQUIRE(hipGetDevice(&cur) == hipSuccess, IONN_ERR_HIP, "ionn_bias_grad_noalloc: hipGetDevice failed");
        if (cur != dev) IONN_REQUIRE(hipSetDevice(dev) == hipSuccess, IONN_ERR_HIP, "ionn_bias_grad_noalloc: hipSetDevice failed");
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        IONN_REQUIRE(e == hipSuccess && p != nullptr, IONN_ERR_HIP,
                     "ionn_bias_grad_noalloc: hipGetSymbolAddress(scratch) failed on device %d (%s)", dev,
                     hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<int32_t *>(p);
    }
    *out = g_scratch_ptr[dev];
    return IONN_OK;
}

// Both offset-gradient entry points: the row-range sums into part (every
// entry part[y][c], y < g.gy, c < C, is written before it is read, so the
// buffer needs no clearing), then their sum into gb.
int bias_grad_launch(const int8_t *d, int64_t M, int64_t C, int32_t *gb, const BgGrid &g, int32_t *part,
                     hipStream_t st, const char *name) {
    IONN_REQUIRE(g.gx <= 0x7fffffff && g.gy <= 65535, IONN_ERR_SHAPE, "%s: grid too large", name);
    if (C < 64 && C % 16 != 0 && aligned(d, 4) && M * C >= (int64_t(1) << 16)) {
        // narrow rows: one lane per column would leave most lanes idle
        const int64_t nb = narrow_blocks(C, g.gy);
        if (nb >= 1) {
            bias_grad_narrow<<<dim3(unsigned(nb)), dim3(256), 0, st>>>(d, M * C, int(C), part);
            if (int rc = check_launch(name)) return rc;
            wl::sum_partials(part, int(nb), C, gb, nullptr, st);
            return check_launch(name);
        }
    }
    const dim3 grid{unsigned(g.gx), unsigned(g.gy), 1u}, block{64u * BG_WAVES, 1u, 1u};
    if (g.vec) bias_grad_kernel<true><<<grid, block, 0, st>>>(d, M, C, g.rows, part);
    else bias_grad_kernel<false><<<grid, block, 0, st>>>(d, M, C, g.rows, part);
    if (int rc = check_launch(name)) return rc;
    wl::sum_partials(part, int(g.gy), C, gb, nullptr, st);
    return check_launch(name);
}

}  // namespace
}  // namespace ionn

using namespace ionn;

extern "C" {

int ionn_oss_requant(const int32_t *acc, const int32_t *offset, const int32_t *mult, const int8_t *k,
                     int64_t M, int64_t C, int relu, int8_t *out, void *stream) {
    clear_error();
    IONN_REQUIRE(M >= 0 && C >= 0 && M <= kMaxDim && C <= kMaxDim && M * C <= kMaxDim, IONN_ERR_SHAPE,
                 "ionn_oss_requant: bad shape M=%lld C=%lld", (long long)M, (long long)C);
    IONN_REQUIRE(relu == 0 || relu == 1, IONN_ERR_ARG, "ionn_oss_requant: relu = %d", relu);
    if (M * C == 0) return IONN_OK;
    IONN_REQUIRE(acc && offset && mult && k && out, IONN_ERR_ARG, "ionn_oss_requant: NULL argument");
    IONN_REQUIRE(aligned(acc, 4) && aligned(offset, 4) && aligned(mult, 4), IONN_ERR_ALIGN,
                 "ionn_oss_requant: int32 pointers must be 4-byte aligned");
    const int64_t n = M * C;
    const bool vec = C % 4 == 0 && aligned(acc, 16) && aligned(offset, 16) && aligned(mult, 16) &&
                     aligned(k, 4) && aligned(out, 4);
    // the element-wise form takes one element per lane (up to 2^21 of them
    // in flight), the vector form 16 bytes per lane and instruction
    const int64_t scalar_blocks = std::min<int64_t>((n + 255) / 256, 8192);
    dim3 grid(vec ? stream_blocks(n) : unsigned(scalar_blocks)), block(256);
    hipStream_t st = as_stream(stream);
    if (vec && relu) oss_kernel<true, true><<<grid, block, 0, st>>>(acc, n, C, offset, mult, k, out);
    else if (vec) oss_kernel<true, false><<<grid, block, 0, st>>>(acc, n, C, offset, mult, k, out);
    else if (relu) oss_kernel<false, true><<<grid, block, 0, st>>>(acc, n, C, offset, mult, k, out);
    else oss_kernel<false, false><<<grid, block, 0, st>>>(acc, n, C, offset, mult, k, out);
    return check_launch("ionn_oss_requant");
}

size_t ionn_bias_grad_workspace_bytes(int64_t M, int64_t C) {
    if (M < 0 || C < 0 || M > kMaxDim || C > kMaxDim || M * C > kMaxDim) return 0;
    const BgGrid g = bg_grid(M, C, C % 16 == 0);
    return size_t(g.gy * C) * sizeof(int32_t);
}

int ionn_bias_grad(const int8_t *d, int64_t M, int64_t C, int32_t *gb, void *workspace, size_t workspace_bytes,
                   void *stream) {
    clear_error();
    IONN_REQUIRE(M >= 0 && C >= 0 && M <= kMaxDim && C <= kMaxDim && M * C <= kMaxDim, IONN_ERR_SHAPE,
                 "ionn_bias_grad: bad shape M=%lld C=%lld", (long long)M, (long long)C);
    if (C == 0) return IONN_OK;
    IONN_REQUIRE(gb != nullptr && (M == 0 || d != nullptr), IONN_ERR_ARG, "ionn_bias_grad: NULL argument");
    IONN_REQUIRE(aligned(gb, 4), IONN_ERR_ALIGN, "ionn_bias_grad: gb must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    if (M == 0) {
        zero_kernel<<<dim3(unsigned((C + 255) / 256 < 1024 ? (C + 255) / 256 : 1024)), dim3(256), 0, st>>>(gb, C);
        return check_launch("ionn_bias_grad");
    }
    const BgGrid g = bg_grid(M, C, C % 16 == 0 && aligned(d, 16));
    const size_t need = size_t(g.gy * C) * sizeof(int32_t);
    IONN_REQUIRE(workspace != nullptr && aligned(workspace, 4) && workspace_bytes >= need, IONN_ERR_WORKSPACE,
                 "ionn_bias_grad: needs a 4-byte aligned workspace of %zu bytes", need);
    return bias_grad_launch(d, M, C, gb, g, static_cast<int32_t *>(workspace), st, "ionn_bias_grad");
}

int ionn_bias_grad_noalloc(const int8_t *d, int64_t M, int64_t C, int32_t *gb, void *stream) {
    clear_error();
    IONN_REQUIRE(M >= 0 && C >= 0 && M <= kMaxDim && C <= kMaxDim && M * C <= kMaxDim, IONN_ERR_SHAPE,
                 "ionn_bias_grad_noalloc: bad shape M=%lld C=%lld", (long long)M, (long long)C);
    if (C == 0) return IONN_OK;
    IONN_REQUIRE(gb != nullptr && (M == 0 || d != nullptr), IONN_ERR_ARG,
                 "ionn_bias_grad_noalloc: NULL argument");
    IONN_REQUIRE(aligned(gb, 4), IONN_ERR_ALIGN, "ionn_bias_grad_noalloc: gb must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    if (M == 0) {
        zero_kernel<<<dim3(unsigned((C + 255) / 256 < 1024 ? (C + 255) / 256 : 1024)), dim3(256), 0, st>>>(gb, C);
        return check_launch("ionn_bias_grad_noalloc");
    }
    const BgGrid g = bg_grid(M, C, C % 16 == 0 && aligned(d, 16));
    const size_t need = size_t(g.gy * C) * sizeof(int32_t);
    IONN_REQUIRE(need <= kBgScratchBytes, IONN_ERR_SHAPE,
                 "ionn_bias_grad_noalloc: M=%lld C=%lld needs %zu bytes of row-range sums, more than the "
                 "%zu-byte device scratch (use ionn_bias_grad with a workspace)",
                 (long long)M, (long long)C, need, kBgScratchBytes);
    int32_t *part = nullptr;
    if (int rc = bg_scratch(st, &part)) return rc;
    return bias_grad_launch(d, M, C, gb, g, part, st, "ionn_bias_grad_noalloc");
}

int niti_quantize_update_i32(const int32_t *G, int64_t n, const uint32_t *absmax, int target_bits, int mu,
                             int32_t *P, int32_t *shifts_out, int32_t *gq_out, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 0, IONN_ERR_SHAPE, "niti_quantize_update_i32: n = %lld < 0", (long long)n);
    IONN_REQUIRE(absmax != nullptr, IONN_ERR_ARG, "niti_quantize_update_i32: absmax is NULL");
    IONN_REQUIRE(n == 0 || (G != nullptr && P != nullptr), IONN_ERR_ARG,
                 "niti_quantize_update_i32: G/P is NULL");
    IONN_REQUIRE(target_bits >= 1 && target_bits <= 31, IONN_ERR_RANGE,
                 "niti_quantize_update_i32: target_bits = %d outside [1, 31]", target_bits);
    IONN_REQUIRE(mu >= 0 && mu <= 31, IONN_ERR_RANGE, "niti_quantize_update_i32: mu = %d outside [0, 31]", mu);
    IONN_REQUIRE(aligned(G, 4) && aligned(P, 4) && aligned(absmax, 4) && aligned(shifts_out, 4) &&
                     aligned(gq_out, 4),
                 IONN_ERR_ALIGN, "niti_quantize_update_i32: int32 pointers must be 4-byte aligned");
    int64_t blocks = (n + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 2048) blocks = 2048;
    update_i32_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, as_stream(stream)>>>(G, n, absmax, target_bits, mu, P,
                                                                                   shifts_out, gq_out);
    return check_launch("niti_quantize_update_i32");
}

}  // extern "C"
