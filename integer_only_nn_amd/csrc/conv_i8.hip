// 3x3 / stride 1 / pad 1 Conv2D contractions (the Conv2D and Conv2D+ReLU
// layers of "Integer On-Device Training: Overview", section 7), NHWC
// activations and OHWI weights (the layouts of the TiGrIS "Compilation
// Pipeline" emission stage), as implicit GEMMs on the shared matrix-core
// mainloop:
//
//   fwd   Y[p][co]  = sum_{tap,ci} X[p + off(tap)][ci] * W[co][tap][ci]
//                     M = pixels, N = Cout, K = 9*Cin; A = im2col(X), B = W (K-major)
//   dgrad dX[p][ci] = sum_{tap,co} dY[p - off(tap)][co] * W[co][tap][ci]
//                     M = pixels, N = Cin,  K = 9*Cout; A = im2col(dY, mirrored), B = W seen [k=(tap,co)][ci]
//   wgrad G[co][tap,ci] = sum_p dY[p][co] * X[p + off(tap)][ci]
//                     M = Cout, N = 9*Cin, K = pixels; split over K, int32 atomics
//
// The im2col matrices are never materialised: the tile loaders gather 16-byte
// channel chunks (Cin, Cout multiples of 16) straight from the image, with
// zeros outside it.  Integer atomics are exact and order-free (sums are
// modulo 2^32), so the split-K weight gradient is bit-identical to any
// other summation order.
//
// Other geometries at stride 1 (any KH x KW, any zero padding P, any
// channel counts; output Ho = H + 2P - KH + 1, Wo = W + 2P - KW + 1), such
// as the 16 x 2 "valid" filter bank of the page's example network, run on
// direct kernels: one thread per output element of fwd and dgrad, one per
// weight element and pixel range of wgrad.  These are small-layer paths.
#include "gemm_core.h"
#include "wgrad_long.h"
#include "conv3x3.h"
#include "conv_pipe.h"

#include <initializer_list>

#include <atomic>

namespace ionn {

int launch_absmax_i32(const int32_t *x, int64_t n, uint32_t *absmax, hipStream_t st);

namespace {

using namespace gemm;

__global__ void zero_i32_kernel(int32_t *C, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        C[i] = 0;
}

int64_t out_h(const ionn_conv_desc *d) { return d->H + 2 * int64_t(d->pad) - d->KH + 1; }
int64_t out_w(const ionn_conv_desc *d) { return d->W + 2 * int64_t(d->pad) - d->KW + 1; }

int check_desc(const ionn_conv_desc *d, const char *name) {
    IONN_REQUIRE(d != nullptr, IONN_ERR_ARG, "%s: desc is NULL", name);
    IONN_REQUIRE(d->N >= 0 && d->H >= 0 && d->W >= 0 && d->Cin >= 0 && d->Cout >= 0,
                 IONN_ERR_SHAPE, "%s: negative size", name);
    IONN_REQUIRE(d->stride == 1 && d->dilation == 1 && d->groups == 1, IONN_ERR_UNSUPPORTED,
                 "%s: only stride 1, dilation 1, groups 1 are implemented (got s%d d%d g%d)", name,
                 d->stride, d->dilation, d->groups);
    IONN_REQUIRE(d->KH >= 1 && d->KW >= 1 && d->KH <= 1024 && d->KW <= 1024 && d->pad >= 0 &&
                     d->pad <= 1024,
                 IONN_ERR_RANGE, "%s: kernel %dx%d with pad %d (need KH, KW in [1, 1024], pad in [0, 1024])",
                 name, d->KH, d->KW, d->pad);
    // Every size on its own first, then each product one factor at a time
    // (a <= kMaxDim / b before a * b), so no intermediate can overflow.
    IONN_REQUIRE(d->N <= kMaxDim && d->H <= kMaxDim && d->W <= kMaxDim && d->Cin <= kMaxDim &&
                     d->Cout <= kMaxDim,
                 IONN_ERR_SHAPE, "%s: every size must be below 2^31", name);
    const int64_t Ho = out_h(d), Wo = out_w(d);
    IONN_REQUIRE(Ho <= kMaxDim && Wo <= kMaxDim, IONN_ERR_SHAPE, "%s: output size out of range", name);
    auto fits = [](std::initializer_list<int64_t> f) {
        int64_t p = 1;
        for (int64_t v : f) {
            if (v <= 0) return true;  // an empty tensor
            if (p > kMaxDim / v) return false;
            p *= v;
        }
        return p <= kMaxDim;
    };
    IONN_REQUIRE(fits({d->N, d->H, d->W, d->Cin}) && fits({d->N, d->H, d->W, d->Cout}) &&
                     fits({d->N, Ho, Wo, d->Cout}) && fits({d->N, Ho, Wo, d->Cin}) &&
                     fits({int64_t(d->KH), int64_t(d->KW), d->Cin, d->Cout}),
                 IONN_ERR_SHAPE, "%s: tensors must hold fewer than 2^31 elements", name);
    return IONN_OK;
}

// The 3 x 3 / pad 1 paths (implicit GEMM, and the 64-channel kernels): 16-byte
// channel chunks, so Cin and Cout are multiples of 16 and tensors 16-byte aligned.
bool geom33(const ionn_conv_desc *d) {
    return d->KH == 3 && d->KW == 3 && d->pad == 1 && d->Cin % 16 == 0 && d->Cout % 16 == 0;
}

// ---- direct kernels for other geometries (stride 1) ----
__global__ __launch_bounds__(256) void conv_direct_fwd(const int8_t *__restrict__ X, const int8_t *__restrict__ Wt,
                                                       int32_t *__restrict__ Y, int H, int W, int Cin, int Cout,
                                                       int KH, int KW, int P, int Ho, int Wo, int64_t n_out,
                                                       uint32_t *__restrict__ absmax) {
    uint32_t amax = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_out;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int co = int(i % Cout);
        int64_t t = i / Cout;
        const int wo = int(t % Wo);
        t /= Wo;
        const int ho = int(t % Ho);
        const int64_t n = t / Ho;
        uint32_t acc = 0;
        for (int kh = 0; kh < KH; ++kh) {
            const int y = ho + kh - P;
            if (y < 0 || y >= H) continue;
            for (int kw = 0; kw < KW; ++kw) {
                const int x = wo + kw - P;
                if (x < 0 || x >= W) continue;
                const int8_t *xp = X + ((n * H + y) * W + x) * Cin;
                const int8_t *wp = Wt + ((int64_t(co) * KH + kh) * KW + kw) * Cin;
                for (int ci = 0; ci < Cin; ++ci) acc += uint32_t(int32_t(xp[ci]) * int32_t(wp[ci]));
            }
        }
        Y[i] = int32_t(acc);
        amax = max(amax, abs_u32(int32_t(acc)));
    }
    if (absmax) {
        amax = wave_max_u32(amax);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, amax);
    }
}

__global__ __launch_bounds__(256) void conv_direct_dgrad(const int8_t *__restrict__ dY,
                                                         const int8_t *__restrict__ Wt, int32_t *__restrict__ dX,
                                                         int H, int W, int Cin, int Cout, int KH, int KW, int P,
                                                         int Ho, int Wo, int64_t n_in,
                                                         uint32_t *__restrict__ absmax) {
    uint32_t amax = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_in;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int ci = int(i % Cin);
        int64_t t = i / Cin;
        const int w = int(t % W);
        t /= W;
        const int h = int(t % H);
        const int64_t n = t / H;
        uint32_t acc = 0;
        for (int kh = 0; kh < KH; ++kh) {
            const int y = h - kh + P;
            if (y < 0 || y >= Ho) continue;
            for (int kw = 0; kw < KW; ++kw) {
                const int x = w - kw + P;
                if (x < 0 || x >= Wo) continue;
                const int8_t *dp = dY + ((n * Ho + y) * Wo + x) * Cout;
                const int8_t *wp = Wt + (int64_t(kh) * KW + kw) * Cin + ci;
                const int64_t wstride = int64_t(KH) * KW * Cin;
                for (int co = 0; co < Cout; ++co) acc += uint32_t(int32_t(dp[co]) * int32_t(wp[co * wstride]));
            }
        }
        dX[i] = int32_t(acc);
        amax = max(amax, abs_u32(int32_t(acc)));
    }
    if (absmax) {
        amax = wave_max_u32(amax);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, amax);
    }
}

// G (zeroed) += this workgroup's share of the sum over output rows, rows
// being (n, ho) pairs.  Every thread of the workgroup works: thread t takes
// weight element w = wc + t % NW (NW = min(n_g - wc, 256) for the weight
// chunk wc) and every S-th row of the workgroup's range from t / NW on
// (S = 256 / NW); the S partial sums of a weight meet in LDS and one atomic
// per weight and workgroup adds them into G.
__global__ __launch_bounds__(256) void conv_direct_wgrad(const int8_t *__restrict__ dY,
                                                         const int8_t *__restrict__ X, int32_t *__restrict__ G,
                                                         int H, int W, int Cin, int Cout, int KH, int KW, int P,
                                                         int Ho, int Wo, int64_t rows, int64_t rows_per,
                                                         int64_t n_g) {
    __shared__ uint32_t red[256];
    const int t = threadIdx.x;
    const int64_t r0 = int64_t(blockIdx.x) * rows_per, r1 = min(rows, r0 + rows_per);
    for (int64_t wc = 0; wc < n_g; wc += 256) {
        const int NW = int(min<int64_t>(n_g - wc, 256));
        const int S = 256 / NW;
        const int wl = t % NW, sub = t / NW;
        uint32_t acc = 0;
        if (sub < S) {
            const int64_t i = wc + wl;
            const int ci = int(i % Cin);
            int64_t q = i / Cin;
            const int kw = int(q % KW);
            q /= KW;
            const int kh = int(q % KH);
            const int co = int(q / KH);
            int64_t n = (r0 + sub) / Ho;
            int ho = int(r0 + sub - n * Ho);
            for (int64_t r = r0 + sub; r < r1; r += S) {
                const int y = ho + kh - P;
                if (y >= 0 && y < H) {
                    const int8_t *dp = dY + ((n * Ho + ho) * Wo) * Cout + co;
                    const int8_t *xp = X + ((n * H + y) * W) * Cin + ci;
                    for (int wo = 0; wo < Wo; ++wo) {
                        const int x = wo + kw - P;
                        if (x >= 0 && x < W) acc += uint32_t(int32_t(dp[int64_t(wo) * Cout]) * int32_t(xp[int64_t(x) * Cin]));
                    }
                }
                ho += S;
                while (ho >= Ho) {
                    ho -= Ho;
                    ++n;
                }
            }
        }
        red[t] = acc;
        __syncthreads();
        if (t < NW) {
            uint32_t v = 0;
            for (int k = 0; k < S; ++k) v += red[t + k * NW];
            if (v) atomicAdd(G + wc + t, int32_t(v));
        }
        __syncthreads();
    }
}

// ---- small samples: whole samples staged in LDS ----
//
// When one sample's input and output (and the filter bank) are a few KB, as
// in the page's example network (64 x 2 input, 16 x 2 filters), a workgroup
// copies SPB whole samples from HBM into LDS with wide loads and computes
// from there: every input byte is read from HBM once per workgroup instead
// of once per output that touches it, and the byte gathers hit LDS.

constexpr int kSmallLds = 32768;                 // LDS bytes per workgroup
constexpr int kSmallMaxBytes = 4096;             // per-sample input and output bytes
constexpr int kSmallMaxW = 16384;                // filter bank bytes
constexpr int kSmallMaxG = 1024;                 // weights held by one workgroup's wgrad

struct SmallGeo {
    int H, W, Cin, Cout, KH, KW, P, Ho, Wo;
    int in_b, out_b, w_b;                        // bytes per sample in / out, filter bank
    int spb;                                     // samples per group
};

__device__ __forceinline__ void copy_to_lds(int8_t *dst, const int8_t *src, int nbytes) {
    if (((reinterpret_cast<uintptr_t>(src) | uintptr_t(nbytes)) & 15) == 0) {
        for (int i = threadIdx.x; i < nbytes / 16; i += blockDim.x)
            reinterpret_cast<uint4 *>(dst)[i] = reinterpret_cast<const uint4 *>(src)[i];
    } else {
        for (int i = threadIdx.x; i < nbytes; i += blockDim.x) dst[i] = src[i];
    }
}

__device__ __forceinline__ int round16(int x) { return (x + 15) & ~15; }

// nbytes from src to LDS at dst + (src mod 4), whatever src's alignment:
// aligned dwords (dst is 4-byte aligned; the copy's first dword starts at
// dst, its leading src mod 4 bytes are not part of the data), the last,
// partial dword by bytes so nothing past src + nbytes is read.  Returns the
// offset (src mod 4) at which the data starts.
__device__ __forceinline__ int copy_to_lds_u(int8_t *dst, const int8_t *src, int nbytes) {
    const int off = int(reinterpret_cast<uintptr_t>(src) & 3);
    const uint32_t *a = reinterpret_cast<const uint32_t *>(src - off);
    const int end = off + nbytes, full = end / 4;  // dwords wholly inside [src - off, src + nbytes)
    uint32_t *d = reinterpret_cast<uint32_t *>(dst);
    int q = threadIdx.x;
    for (; q + 3 * int(blockDim.x) < full; q += 4 * blockDim.x) {
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = a[q + u * blockDim.x];
#pragma unroll
        for (int u = 0; u < 4; ++u) d[q + u * blockDim.x] = w[u];
    }
    for (; q < full; q += blockDim.x) d[q] = a[q];
    if (threadIdx.x < uint32_t(end - 4 * full)) dst[4 * full + threadIdx.x] = src[4 * full + threadIdx.x - off];
    return off;
}

// Y for groups of g.spb samples, one output element per thread and step.
__global__ __launch_bounds__(256) void conv_small_fwd(const int8_t *__restrict__ X, const int8_t *__restrict__ Wt,
                                                      int32_t *__restrict__ Y, int64_t N, SmallGeo g,
                                                      uint32_t *__restrict__ absmax) {
    __shared__ __attribute__((aligned(16))) int8_t lds[kSmallLds];
    int8_t *ws = lds, *xs = lds + round16(g.w_b);
    copy_to_lds(ws, Wt, g.w_b);
    uint32_t amax = 0;
    for (int64_t n0 = int64_t(blockIdx.x) * g.spb; n0 < N; n0 += int64_t(gridDim.x) * g.spb) {
        const int ns = int(N - n0 < g.spb ? N - n0 : g.spb);
        __syncthreads();  // the previous group's reads are done
        copy_to_lds(xs, X + n0 * g.in_b, ns * g.in_b);
        __syncthreads();
        const int nout = ns * g.out_b;
        for (int o = threadIdx.x; o < nout; o += blockDim.x) {
            const int sm = o / g.out_b, r = o - sm * g.out_b;
            const int co = r % g.Cout, t = r / g.Cout, wo = t % g.Wo, ho = t / g.Wo;
            const int8_t *xsm = xs + sm * g.in_b;
            uint32_t acc = 0;
            for (int kh = 0; kh < g.KH; ++kh) {
                const int y = ho + kh - g.P;
                if (y < 0 || y >= g.H) continue;
                for (int kw = 0; kw < g.KW; ++kw) {
                    const int x = wo + kw - g.P;
                    if (x < 0 || x >= g.W) continue;
                    const int8_t *xp = xsm + (y * g.W + x) * g.Cin;
                    const int8_t *wp = ws + ((co * g.KH + kh) * g.KW + kw) * g.Cin;
                    for (int ci = 0; ci < g.Cin; ++ci) acc += uint32_t(int32_t(xp[ci]) * int32_t(wp[ci]));
                }
            }
            Y[n0 * g.out_b + o] = int32_t(acc);
            amax = max(amax, abs_u32(int32_t(acc)));
        }
    }
    if (absmax) {
        amax = wave_max_u32(amax);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, amax);
    }
}

// dX for groups of samples: the output error staged, one input element per
// thread and step.
__global__ __launch_bounds__(256) void conv_small_dgrad(const int8_t *__restrict__ dY, const int8_t *__restrict__ Wt,
                                                        int32_t *__restrict__ dX, int64_t N, SmallGeo g,
                                                        uint32_t *__restrict__ absmax) {
    __shared__ __attribute__((aligned(16))) int8_t lds[kSmallLds];
    int8_t *ws = lds, *ds = lds + round16(g.w_b);
    copy_to_lds(ws, Wt, g.w_b);
    uint32_t amax = 0;
    const int wstride = g.KH * g.KW * g.Cin;
    for (int64_t n0 = int64_t(blockIdx.x) * g.spb; n0 < N; n0 += int64_t(gridDim.x) * g.spb) {
        const int ns = int(N - n0 < g.spb ? N - n0 : g.spb);
        __syncthreads();
        copy_to_lds(ds, dY + n0 * g.out_b, ns * g.out_b);
        __syncthreads();
        const int nin = ns * g.in_b;
        for (int o = threadIdx.x; o < nin; o += blockDim.x) {
            const int sm = o / g.in_b, r = o - sm * g.in_b;
            const int ci = r % g.Cin, t = r / g.Cin, w = t % g.W, h = t / g.W;
            const int8_t *dsm = ds + sm * g.out_b;
            uint32_t acc = 0;
            for (int kh = 0; kh < g.KH; ++kh) {
                const int y = h - kh + g.P;
                if (y < 0 || y >= g.Ho) continue;
                for (int kw = 0; kw < g.KW; ++kw) {
                    const int x = w - kw + g.P;
                    if (x < 0 || x >= g.Wo) continue;
                    const int8_t *dp = dsm + (y * g.Wo + x) * g.Cout;
                    const int8_t *wp = ws + (kh * g.KW + kw) * g.Cin + ci;
                    for (int co = 0; co < g.Cout; ++co) acc += uint32_t(int32_t(dp[co]) * int32_t(wp[co * wstride]));
                }
            }
            dX[n0 * g.in_b + o] = int32_t(acc);
            amax = max(amax, abs_u32(int32_t(acc)));
        }
    }
    if (absmax) {
        amax = wave_max_u32(amax);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, amax);
    }
}

// G (zeroed) += this workgroup's samples.  Thread t holds weights
// w = t % NW + 256 j... of a chunk layout like conv_direct_wgrad: weight
// chunk c covers [256 c, 256 c + 256), thread t takes weight t % NW of it
// and every S-th sample of the group from t / NW on; sums stay in
// registers across groups, meet in LDS at the end, one atomic per weight.
__global__ __launch_bounds__(256) void conv_small_wgrad(const int8_t *__restrict__ dY, const int8_t *__restrict__ X,
                                                        int32_t *__restrict__ G, int64_t N, SmallGeo g, int n_g) {
    __shared__ __attribute__((aligned(16))) int8_t lds[kSmallLds];
    __shared__ uint32_t red[256];
    int8_t *xs = lds, *ds = lds + round16(g.spb * g.in_b);
    const int t = threadIdx.x;
    constexpr int MAXC = kSmallMaxG / 256;
    uint32_t acc[MAXC] = {};
    for (int64_t n0 = int64_t(blockIdx.x) * g.spb; n0 < N; n0 += int64_t(gridDim.x) * g.spb) {
        const int ns = int(N - n0 < g.spb ? N - n0 : g.spb);
        __syncthreads();
        copy_to_lds(xs, X + n0 * g.in_b, ns * g.in_b);
        copy_to_lds(ds, dY + n0 * g.out_b, ns * g.out_b);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int wc = 256 * c;
            if (wc >= n_g) break;
            const int NW = n_g - wc < 256 ? n_g - wc : 256, S = 256 / NW;
            const int wl = t % NW, sub = t / NW;
            if (sub >= S) continue;
            const int i = wc + wl;
            const int ci = i % g.Cin, q = i / g.Cin, kw = q % g.KW, q2 = q / g.KW, kh = q2 % g.KH, co = q2 / g.KH;
            uint32_t a = 0;
            for (int sm = sub; sm < ns; sm += S) {
                const int8_t *dsm = ds + sm * g.out_b + co, *xsm = xs + sm * g.in_b + ci;
                for (int ho = 0; ho < g.Ho; ++ho) {
                    const int y = ho + kh - g.P;
                    if (y < 0 || y >= g.H) continue;
                    for (int wo = 0; wo < g.Wo; ++wo) {
                        const int x = wo + kw - g.P;
                        if (x >= 0 && x < g.W)
                            a += uint32_t(int32_t(dsm[(ho * g.Wo + wo) * g.Cout]) * int32_t(xsm[(y * g.W + x) * g.Cin]));
                    }
                }
            }
            acc[c] += a;
        }
    }
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int wc = 256 * c;
        if (wc >= n_g) break;
        const int NW = n_g - wc < 256 ? n_g - wc : 256, S = 256 / NW;
        __syncthreads();
        red[t] = t / NW < S ? acc[c] : 0u;
        __syncthreads();
        if (t < NW) {
            uint32_t v = 0;
            for (int k = 0; k < S; ++k) v += red[t + k * NW];
            if (v) atomicAdd(G + wc + t, int32_t(v));
        }
    }
}

// The small-sample geometry of a descriptor, or spb = 0 when it does not fit.
// Full-row windows (no padding and KW = W, so every window spans whole input
// rows): output row ho of sample n reads the contiguous bytes
// X[n][ho RB .. ho RB + L) with RB = W Cin and L = KH RB, and channel co's
// filter is the contiguous Wt[co][0 .. L) (OHWI).  L is a multiple of 4.
constexpr int kRowsMaxCout = 8;

__device__ __forceinline__ bool rows_geo(const SmallGeo &g) { return g.P == 0 && g.KW == g.W; }

// Y (int32, [n][ho][co]) for groups of g.spb staged samples: one (sample,
// output row) per thread, its L / 4 window words read as two aligned LDS
// dwords and v_alignbyte, one v_dot4 per word and channel.
// CO = Cout (1 .. kRowsMaxCout) as a template parameter: the per-channel
// loop is then straight-line, so each window word's CO weight reads are in
// flight together (with a run-time channel test around each, every v_dot4
// waited for its own LDS read).
template <int CO>
__global__ __launch_bounds__(256) void conv_rows_fwd(const int8_t *__restrict__ X, const int8_t *__restrict__ Wt,
                                                     int32_t *__restrict__ Y, int64_t N, SmallGeo g,
                                                     uint32_t *__restrict__ absmax) {
    __shared__ __attribute__((aligned(16))) int8_t lds[kSmallLds];
    int8_t *ws = lds, *xs = lds + round16(g.w_b);
    copy_to_lds(ws, Wt, g.w_b);
    const uint32_t *w32 = reinterpret_cast<const uint32_t *>(ws);
    const int RB = g.W * g.Cin, LW = g.KH * RB / 4;
    constexpr int Cout = CO;
    const int dsm = 256 / g.Ho, dho = 256 - dsm * g.Ho;  // (sample, row) step per 256 pairs
    uint32_t amax = 0;
    for (int64_t n0 = int64_t(blockIdx.x) * g.spb; n0 < N; n0 += int64_t(gridDim.x) * g.spb) {
        const int ns = int(N - n0 < g.spb ? N - n0 : g.spb);
        __syncthreads();
        const int x0 = copy_to_lds_u(xs, X + n0 * g.in_b, ns * g.in_b);
        __syncthreads();
        int sm = int(threadIdx.x) / g.Ho, ho = int(threadIdx.x) - sm * g.Ho;
        for (; sm < ns;) {
            const int start = x0 + sm * g.in_b + ho * RB;
            const uint32_t *d = reinterpret_cast<const uint32_t *>(xs + (start & ~3));
            const uint32_t sh = uint32_t(start & 3);
            int32_t acc[CO];
#pragma unroll
            for (int co = 0; co < CO; ++co) acc[co] = 0;
            uint32_t lo = d[0];
#pragma unroll 4
            for (int i = 0; i < LW; ++i) {
                const uint32_t hi = d[i + 1];
                const int w = int(__builtin_amdgcn_alignbyte(hi, lo, sh));  // window bytes 4i .. 4i + 3
                lo = hi;
#pragma unroll
                for (int co = 0; co < CO; ++co)
                    acc[co] = __builtin_amdgcn_sdot4(w, int(w32[co * LW + i]), acc[co], false);
            }
            int32_t *yp = Y + ((n0 + sm) * g.Ho + ho) * Cout;
#pragma unroll
            for (int co = 0; co < CO; ++co) {
                yp[co] = acc[co];
                amax = max(amax, abs_u32(acc[co]));
            }
            sm += dsm;
            ho += dho;
            if (ho >= g.Ho) {
                ho -= g.Ho;
                ++sm;
            }
        }
    }
    if (absmax) {
        amax = wave_max_u32(amax);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, amax);
    }
}

// G += (int32, OHWI, zeroed by the caller) over groups of staged samples, or
// (part not null) each workgroup's sums to part[blockIdx.x][Cout L]:
// thread slot s = (co, word jw) keeps the four sums of G[co][4 jw .. 4 jw + 3];
// the 1024 / slots slices of a workgroup take every (1024 / slots)-th output
// row and meet in LDS; the workgroup adds its sums with integer atomics
// (exact in any order).
constexpr int kRowsWgradThreads = 1024;

__global__ __launch_bounds__(kRowsWgradThreads) void conv_rows_wgrad(const int8_t *__restrict__ dY,
                                                                     const int8_t *__restrict__ X,
                                                                     int32_t *__restrict__ G, int64_t N, SmallGeo g,
                                                                     int32_t *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) int8_t lds[kSmallLds];
    __shared__ uint32_t red[4][kRowsWgradThreads];
    int8_t *xs = lds, *ds = lds + round16(g.spb * g.in_b + 16);
    const int RB = g.W * g.Cin, LW = g.KH * RB / 4, L = 4 * LW;
    const int slots = g.Cout * LW, S = kRowsWgradThreads / slots;
    const int t = threadIdx.x, slot = t % slots, sub = t / slots;
    const int co = slot / LW, jw = slot - co * LW;
    uint32_t a[4] = {0, 0, 0, 0};
    for (int64_t n0 = int64_t(blockIdx.x) * g.spb; n0 < N; n0 += int64_t(gridDim.x) * g.spb) {
        const int ns = int(N - n0 < g.spb ? N - n0 : g.spb);
        __syncthreads();
        const int8_t *xsd = xs + copy_to_lds_u(xs, X + n0 * g.in_b, ns * g.in_b);
        const int8_t *dsd = ds + copy_to_lds_u(ds, dY + n0 * g.out_b, ns * g.out_b);
        __syncthreads();
        if (sub < S) {
            for (int sm = 0; sm < ns; ++sm) {
                for (int ho = sub; ho < g.Ho; ho += S) {
                    const int start = int(xsd - xs) + sm * g.in_b + ho * RB + 4 * jw;
                    const uint32_t *d = reinterpret_cast<const uint32_t *>(xs + (start & ~3));
                    const uint32_t w = __builtin_amdgcn_alignbyte(d[1], d[0], uint32_t(start & 3));
                    const int32_t dy = dsd[(sm * g.Ho + ho) * g.Cout + co];
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] += uint32_t(dy * int32_t(int8_t(uint8_t(w >> (8 * e)))));
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) red[e][t] = sub < S ? a[e] : 0u;
    __syncthreads();
    if (sub == 0 && slot < slots) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t tot = 0;
            for (int z = 0; z < S; ++z) tot += red[e][z * slots + slot];
            if (part)
                part[int64_t(blockIdx.x) * g.Cout * L + co * L + 4 * jw + e] = int32_t(tot);
            else if (tot)
                atomicAdd(G + co * L + 4 * jw + e, int32_t(tot));
        }
    }
}

SmallGeo small_geo(const ionn_conv_desc *d, int which) {
    SmallGeo g{};
    const int64_t Ho = d->H + 2 * int64_t(d->pad) - d->KH + 1, Wo = d->W + 2 * int64_t(d->pad) - d->KW + 1;
    const int64_t in_b = d->H * d->W * d->Cin, out_b = Ho * Wo * d->Cout;
    const int64_t w_b = d->Cout * d->KH * d->KW * d->Cin;
    if (Ho <= 0 || Wo <= 0 || in_b < 1 || out_b < 1 || in_b > kSmallMaxBytes || out_b > kSmallMaxBytes ||
        w_b > kSmallMaxW)
        return g;
    int64_t per = which == 0 ? in_b : which == 1 ? out_b : in_b + out_b + 32;   // staged bytes per sample
    const int64_t room = which == 2 ? kSmallLds - 16 : kSmallLds - ((w_b + 15) & ~15);
    if (which == 2 && w_b > kSmallMaxG) return g;
    int64_t spb = room / per;
    if (spb > 64) spb = 64;
    if (spb < 1) return g;
    g = SmallGeo{int(d->H), int(d->W), int(d->Cin), int(d->Cout), d->KH, d->KW, d->pad, int(Ho), int(Wo),
                 int(in_b), int(out_b), int(w_b), int(spb)};
    return g;
}

// Whether the full-row-window kernels take the geometry: no padding, KW = W,
// a window length L = KH W Cin that is a multiple of 4 (at most 1024 bytes),
// at most 8 output channels and at most 256 (channel, window word) slots.
bool rows_path(const ionn_conv_desc *d) {
    const int64_t L = int64_t(d->KH) * d->W * d->Cin;
    return d->pad == 0 && d->KW == d->W && L % 4 == 0 && L <= 1024 && d->Cout >= 1 &&
           d->Cout <= kRowsMaxCout && d->Cout * (L / 4) <= 256;
}

unsigned small_blocks(int64_t N, int spb, int64_t cap) {
    int64_t b = (N + spb - 1) / spb;
    if (b > cap) b = cap;
    return unsigned(b < 1 ? 1 : b);
}

unsigned direct_blocks(int64_t n) {
    int64_t b = (n + 255) / 256;
    return unsigned(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

// The 64-channel halo-tiled kernel applies (see conv3x3.h).
bool fast_c64(const ionn_conv_desc *d, const void *in, const void *w, const void *out) {
    return geom33(d) && d->Cin == 64 && d->Cout == 64 && c3::fits(d->W) && aligned(in, 16) &&
           aligned(w, 16) && aligned(out, 16);
}

// fwd / dgrad fast path: 64 -> 64 channels, the halo in one LDS buffer and
// 32-bit byte offsets into the input and the int32 output.
bool fast_c64_fd(const ionn_conv_desc *d, const void *in, const void *w, const void *out) {
    return fast_c64(d, in, w, out) && c3::fits_fd(d->W, d->N * d->H * d->W * 64);
}

unsigned c3_grid(const ionn_conv_desc *d) {
    const int64_t tiles = d->N * ((d->H * d->W + c3::TP - 1) / c3::TP);
    const int64_t g = tiles < device_cus() ? tiles : device_cus();
    return unsigned(g < 1 ? 1 : g);
}

}  // namespace
}  // namespace ionn

using namespace ionn;
using namespace ionn::gemm;

// Workspace of the one-pass fused requantisation: a rounding-bit word per
// lane and a shift per wavefront, for every tile.
size_t requant_ws_bytes(const ionn_conv_desc *d) {
    const int64_t tiles = d->N * ((d->H * d->W + c3::TP - 1) / c3::TP);
    return size_t(tiles) * 8 * (64 * 4 + 4);
}

// The 64-channel halo-tiled kernel with the NITI requantisation fused; the
// int32 accumulator is never stored.  With a workspace and target_bits <= 7:
// one contraction pass storing each wavefront block's int8 asr(acc, s_b)
// with its rounding bits, then a streaming pass that applies the tensor's
// shift (conv3x3.h, PARTIAL).  Otherwise two contraction passes: max |acc|
// only, then the contraction again with int8 output.
template <bool DGRAD>
int conv_requant(const int8_t *in, const int8_t *Wt, int8_t *out8, const ionn_conv_desc *desc,
                 int target_bits, int relu, uint32_t *absmax, int32_t *shift_out, void *workspace,
                 size_t workspace_bytes, void *stream, const char *name) {
    clear_error();
    if (int rc = check_desc(desc, name)) return rc;
    IONN_REQUIRE(geom33(desc) && desc->Cin == 64 && desc->Cout == 64 && c3::fits_fd(desc->W, desc->N * desc->H * desc->W * 64),
                 IONN_ERR_UNSUPPORTED,
                 "%s: fused path needs 3x3 / stride 1 / pad 1, 64 -> 64 channels and a width whose halo fits "
                 "(use the int32 contraction and niti_quantize otherwise)", name);
    IONN_REQUIRE(target_bits >= 1 && target_bits <= 31, IONN_ERR_RANGE, "%s: target_bits = %d outside [1, 31]",
                 name, target_bits);
    IONN_REQUIRE(relu == 0 || relu == 1, IONN_ERR_ARG, "%s: relu = %d", name, relu);
    IONN_REQUIRE(absmax != nullptr, IONN_ERR_ARG, "%s: absmax is NULL", name);
    const int64_t npix = desc->N * desc->H * desc->W;
    IONN_REQUIRE(npix == 0 || (in && Wt && out8), IONN_ERR_ARG, "%s: NULL tensor", name);
    IONN_REQUIRE(aligned(in, 16) && aligned(Wt, 16) && aligned(out8, 4) && aligned(absmax, 4) &&
                     aligned(shift_out, 4),
                 IONN_ERR_ALIGN, "%s: in/W must be 16-byte, out/absmax/shift 4-byte aligned", name);
    hipStream_t st = as_stream(stream);
    if (npix == 0)  // max |acc| = 0, so s = 0
        return shift_out ? ionn_fill_u32(reinterpret_cast<uint32_t *>(shift_out), 1, 0, stream) : IONN_OK;
    const dim3 grid(c3_grid(desc)), block(c3::NTF);
    const int N = int(desc->N), H = int(desc->H), W = int(desc->W);
    // the pipelined kernel when its halo fits (80-byte slots), else the
    // eight-wavefront one (64-byte slots)
    const bool pipe = c3::pipe_fits(desc->W, npix * 64);
    if (workspace != nullptr && target_bits <= 7) {
        const size_t need = requant_ws_bytes(desc);
        IONN_REQUIRE(workspace_bytes >= need && aligned(workspace, 16) && aligned(out8, 16), IONN_ERR_WORKSPACE,
                     "%s: the one-pass path needs a 16-byte aligned workspace of %zu bytes and a 16-byte aligned "
                     "output", name, need);
        const int64_t tiles = desc->N * ((desc->H * desc->W + c3::TP - 1) / c3::TP);
        uint32_t *bits = static_cast<uint32_t *>(workspace);
        int32_t *sblk = reinterpret_cast<int32_t *>(bits + tiles * 8 * 64);
        if (pipe)
            c3::launch_pipe(DGRAD, c3::PARTIAL, in, Wt, out8, N, H, W, absmax, target_bits, relu, nullptr, bits,
                            sblk, grid.x, st);
        else
            c3::conv3x3_kernel<DGRAD, c3::PARTIAL><<<grid, block, 0, st>>>(in, Wt, out8, N, H, W, absmax,
                                                                           target_bits, relu, nullptr, bits, sblk);
        if (int rc = check_launch(name)) return rc;
        const int64_t nchunks = npix * 4;
        int64_t fb = (nchunks + 255) / 256;
        if (fb > 2048) fb = 2048;
        c3::conv3x3_requant_fix<<<dim3(unsigned(fb)), dim3(256), 0, st>>>(
            out8, bits, sblk, absmax, target_bits, relu, uint32_t(desc->H * desc->W),
            uint32_t((desc->H * desc->W + c3::TP - 1) / c3::TP), uint32_t(nchunks), shift_out);
        return check_launch(name);
    }
    if (pipe) {
        c3::launch_pipe(DGRAD, c3::MAXONLY, in, Wt, nullptr, N, H, W, absmax, 0, 0, nullptr, nullptr, nullptr,
                        grid.x, st);
        if (int rc = check_launch(name)) return rc;
        c3::launch_pipe(DGRAD, c3::REQUANT, in, Wt, out8, N, H, W, absmax, target_bits, relu, shift_out, nullptr,
                        nullptr, grid.x, st);
        return check_launch(name);
    }
    c3::conv3x3_kernel<DGRAD, c3::MAXONLY><<<grid, block, 0, st>>>(in, Wt, nullptr, N, H, W, absmax);
    if (int rc = check_launch(name)) return rc;
    c3::conv3x3_kernel<DGRAD, c3::REQUANT><<<grid, block, 0, st>>>(in, Wt, out8, N, H, W, absmax, target_bits,
                                                                   relu, shift_out);
    return check_launch(name);
}

extern "C" {

int int_conv_fwd(const int8_t *X, const int8_t *Wt, int32_t *Y, const ionn_conv_desc *desc,
                 uint32_t *absmax_Y, void *stream) {
    clear_error();
    if (int rc = check_desc(desc, "int_conv_fwd")) return rc;
    const int npix = int(desc->N * desc->H * desc->W), Cin = int(desc->Cin), Cout = int(desc->Cout);
    if (!geom33(desc)) {
        const int64_t Ho = out_h(desc), Wo = out_w(desc), n_out = desc->N * Ho * Wo * Cout;
        if (Ho <= 0 || Wo <= 0 || n_out == 0) return IONN_OK;
        IONN_REQUIRE(Y && (Cin == 0 || (X && Wt)), IONN_ERR_ARG, "int_conv_fwd: NULL tensor");
        IONN_REQUIRE(aligned(Y, 4) && aligned(absmax_Y, 4), IONN_ERR_ALIGN,
                     "int_conv_fwd: Y/absmax must be 4-byte aligned");
        const SmallGeo sg = small_geo(desc, 0);
        if (sg.spb > 0 && Cin > 0 && rows_path(desc)) {
            // the window reads run up to 3 bytes past the staged samples
            SmallGeo rg = sg;
            while (rg.spb > 1 && ((rg.w_b + 15) & ~15) + int64_t(rg.spb) * rg.in_b + 16 > kSmallLds) --rg.spb;
            const dim3 grid(small_blocks(desc->N, rg.spb, 2048)), block(256);
            hipStream_t st = as_stream(stream);
            switch (rg.Cout) {
            case 1: conv_rows_fwd<1><<<grid, block, 0, st>>>(X, Wt, Y, desc->N, rg, absmax_Y); break;
            case 2: conv_rows_fwd<2><<<grid, block, 0, st>>>(X, Wt, Y, desc->N, rg, absmax_Y); break;
            case 3: conv_rows_fwd<3><<<grid, block, 0, st>>>(X, Wt, Y, desc->N, rg, absmax_Y); break;
            case 4: conv_rows_fwd<4><<<grid, block, 0, st>>>(X, Wt, Y, desc->N, rg, absmax_Y); break;
            case 5: conv_rows_fwd<5><<<grid, block, 0, st>>>(X, Wt, Y, desc->N, rg, absmax_Y); break;
            case 6: conv_rows_fwd<6><<<grid, block, 0, st>>>(X, Wt, Y, desc->N, rg, absmax_Y); break;
            case 7: conv_rows_fwd<7><<<grid, block, 0, st>>>(X, Wt, Y, desc->N, rg, absmax_Y); break;
            default: conv_rows_fwd<8><<<grid, block, 0, st>>>(X, Wt, Y, desc->N, rg, absmax_Y); break;
            }
            return check_launch("int_conv_fwd");
        }
        if (sg.spb > 0 && Cin > 0) {
            conv_small_fwd<<<dim3(small_blocks(desc->N, sg.spb, 2048)), dim3(256), 0, as_stream(stream)>>>(
                X, Wt, Y, desc->N, sg, absmax_Y);
            return check_launch("int_conv_fwd");
        }
        conv_direct_fwd<<<dim3(direct_blocks(n_out)), dim3(256), 0, as_stream(stream)>>>(
            X, Wt, Y, int(desc->H), int(desc->W), Cin, Cout, desc->KH, desc->KW, desc->pad, int(Ho), int(Wo),
            n_out, absmax_Y);
        return check_launch("int_conv_fwd");
    }
    if (npix == 0 || Cout == 0) return IONN_OK;
    IONN_REQUIRE(X && Wt && Y, IONN_ERR_ARG, "int_conv_fwd: NULL tensor");
    IONN_REQUIRE(aligned(X, 16) && aligned(Wt, 16) && aligned(Y, 16) && aligned(absmax_Y, 4),
                 IONN_ERR_ALIGN, "int_conv_fwd: tensors must be 16-byte aligned");
    hipStream_t st = as_stream(stream);
    if (Cin == 0) {
        zero_i32_kernel<<<dim3(4096), dim3(256), 0, st>>>(Y, int64_t(npix) * Cout);
        return check_launch("int_conv_fwd");
    }
    if (fast_c64_fd(desc, X, Wt, Y)) {
        c3::conv3x3_kernel<false><<<dim3(c3_grid(desc)), dim3(c3::NTF), 0, st>>>(
            X, Wt, Y, int(desc->N), int(desc->H), int(desc->W), absmax_Y);
        return check_launch("int_conv_fwd");
    }
    const int M = npix, N = Cout, K = 9 * Cin;
    SrcIm2colK sa{X, npix, int(desc->H), int(desc->W), Cin, +1};
    SrcRowK sb{Wt, K, N, K, true};
    Epi ep{Y, Cout, M, N, true, nullptr, absmax_Y, false};
    if (M % 256 == 0 && N % 64 == 0 && K % 64 == 0)
        launch<256, 64, 64, 4, 1, false>(sa, sb, ep, M, N, K, 1, st);
    else
        launch<256, 64, 64, 4, 1, true>(sa, sb, ep, M, N, K, 1, st);
    return check_launch("int_conv_fwd");
}

int int_conv_dgrad(const int8_t *dY, const int8_t *Wt, int32_t *dX, const ionn_conv_desc *desc,
                   uint32_t *absmax_dX, void *stream) {
    clear_error();
    if (int rc = check_desc(desc, "int_conv_dgrad")) return rc;
    const int npix = int(desc->N * desc->H * desc->W), Cin = int(desc->Cin), Cout = int(desc->Cout);
    if (!geom33(desc)) {
        const int64_t Ho = out_h(desc), Wo = out_w(desc), n_in = int64_t(npix) * Cin;
        if (n_in == 0) return IONN_OK;
        const bool any_out = Ho > 0 && Wo > 0 && Cout > 0;
        IONN_REQUIRE(dX && (!any_out || (dY && Wt)), IONN_ERR_ARG, "int_conv_dgrad: NULL tensor");
        IONN_REQUIRE(aligned(dX, 4) && aligned(absmax_dX, 4), IONN_ERR_ALIGN,
                     "int_conv_dgrad: dX/absmax must be 4-byte aligned");
        hipStream_t st = as_stream(stream);
        if (!any_out) {
            zero_i32_kernel<<<dim3(direct_blocks(n_in)), dim3(256), 0, st>>>(dX, n_in);
            return check_launch("int_conv_dgrad");
        }
        const SmallGeo sg = small_geo(desc, 1);
        if (sg.spb > 0) {
            conv_small_dgrad<<<dim3(small_blocks(desc->N, sg.spb, 2048)), dim3(256), 0, st>>>(dY, Wt, dX, desc->N,
                                                                                              sg, absmax_dX);
            return check_launch("int_conv_dgrad");
        }
        conv_direct_dgrad<<<dim3(direct_blocks(n_in)), dim3(256), 0, st>>>(
            dY, Wt, dX, int(desc->H), int(desc->W), Cin, Cout, desc->KH, desc->KW, desc->pad, int(Ho), int(Wo),
            n_in, absmax_dX);
        return check_launch("int_conv_dgrad");
    }
    if (npix == 0 || Cin == 0) return IONN_OK;
    IONN_REQUIRE(dY && Wt && dX, IONN_ERR_ARG, "int_conv_dgrad: NULL tensor");
    IONN_REQUIRE(aligned(dY, 16) && aligned(Wt, 16) && aligned(dX, 16) && aligned(absmax_dX, 4),
                 IONN_ERR_ALIGN, "int_conv_dgrad: tensors must be 16-byte aligned");
    hipStream_t st = as_stream(stream);
    if (Cout == 0) {
        zero_i32_kernel<<<dim3(4096), dim3(256), 0, st>>>(dX, int64_t(npix) * Cin);
        return check_launch("int_conv_dgrad");
    }
    if (fast_c64_fd(desc, dY, Wt, dX)) {
        c3::conv3x3_kernel<true><<<dim3(c3_grid(desc)), dim3(c3::NTF), 0, st>>>(
            dY, Wt, dX, int(desc->N), int(desc->H), int(desc->W), absmax_dX);
        return check_launch("int_conv_dgrad");
    }
    const int M = npix, N = Cin, K = 9 * Cout;
    SrcIm2colK sa{dY, npix, int(desc->H), int(desc->W), Cout, -1};
    SrcConvWT sb{Wt, Cin, Cout};
    Epi ep{dX, Cin, M, N, true, nullptr, absmax_dX, false};
    if (M % 256 == 0 && N % 64 == 0 && K % 64 == 0)
        launch<256, 64, 64, 4, 1, false>(sa, sb, ep, M, N, K, 1, st);
    else
        launch<256, 64, 64, 4, 1, true>(sa, sb, ep, M, N, K, 1, st);
    return check_launch("int_conv_dgrad");
}

size_t int_conv_requant_workspace_bytes(const ionn_conv_desc *desc) {
    if (desc == nullptr || desc->N < 0 || desc->H < 0 || desc->W < 0 || desc->N > kMaxDim ||
        desc->H > kMaxDim || desc->W > kMaxDim || desc->stride != 1 || desc->dilation != 1 ||
        desc->groups != 1 || !geom33(desc) || desc->Cin != 64 || desc->Cout != 64 ||
        desc->H * desc->W > kMaxDim / (desc->N > 0 ? desc->N : 1) ||
        !c3::fits_fd(desc->W, desc->N * desc->H * desc->W * 64))
        return 0;
    return requant_ws_bytes(desc);
}

int int_conv_fwd_requant(const int8_t *X, const int8_t *Wt, int8_t *Y8, const ionn_conv_desc *desc,
                         int target_bits, int relu, uint32_t *absmax_Y, int32_t *shift_out, void *workspace,
                         size_t workspace_bytes, void *stream) {
    return conv_requant<false>(X, Wt, Y8, desc, target_bits, relu, absmax_Y, shift_out, workspace,
                               workspace_bytes, stream, "int_conv_fwd_requant");
}

int int_conv_dgrad_requant(const int8_t *dY, const int8_t *Wt, int8_t *dX8, const ionn_conv_desc *desc,
                           int target_bits, uint32_t *absmax_dX, int32_t *shift_out, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return conv_requant<true>(dY, Wt, dX8, desc, target_bits, 0, absmax_dX, shift_out, workspace,
                              workspace_bytes, stream, "int_conv_dgrad_requant");
}

// Workgroups of the full-row-window wgrad (one group of staged samples per
// workgroup and step; at most 1024 with per-workgroup partials, 256 when they
// add into G with atomics), or 0 when the geometry is not one.
int64_t rows_wgrad_groups(const ionn_conv_desc *d, int64_t cap = 1024) {
    if (geom33(d) || !rows_path(d)) return 0;
    const int64_t Ho = out_h(d), Wo = out_w(d);
    if (Ho <= 0 || Wo <= 0 || d->N <= 0) return 0;
    const SmallGeo sg = small_geo(d, 2);
    if (sg.spb <= 0) return 0;
    return small_blocks(d->N, sg.spb, cap);
}

size_t int_conv_wgrad_workspace_bytes(const ionn_conv_desc *desc) {
    if (desc == nullptr) return 0;
    if (const int64_t nb = rows_wgrad_groups(desc))
        return size_t(nb) * size_t(desc->Cout * desc->KH * desc->KW * desc->Cin) * sizeof(int32_t);
    if (!geom33(desc) || desc->Cin != 64 || desc->Cout != 64 || !c3::fits(desc->W)) return 0;
    return size_t(c3::wgrad_rows(device_cus())) * c3::GSZ * sizeof(int32_t);
}

int int_conv_wgrad(const int8_t *dY, const int8_t *X, int32_t *G, const ionn_conv_desc *desc,
                   uint32_t *absmax_G, void *workspace, size_t ws_bytes, void *stream) {
    clear_error();
    if (int rc = check_desc(desc, "int_conv_wgrad")) return rc;
    const int npix = int(desc->N * desc->H * desc->W), Cin = int(desc->Cin), Cout = int(desc->Cout);
    if (Cin == 0 || Cout == 0) return IONN_OK;
    if (!geom33(desc)) {
        const int64_t Ho = out_h(desc), Wo = out_w(desc);
        const int64_t n_g = int64_t(Cout) * desc->KH * desc->KW * Cin;
        const int64_t rows = (Ho > 0 && Wo > 0) ? desc->N * Ho : 0;
        IONN_REQUIRE(G && (rows == 0 || (dY && X)), IONN_ERR_ARG, "int_conv_wgrad: NULL tensor");
        IONN_REQUIRE(aligned(G, 4) && aligned(absmax_G, 4), IONN_ERR_ALIGN,
                     "int_conv_wgrad: G/absmax must be 4-byte aligned");
        hipStream_t st = as_stream(stream);
        const SmallGeo sg = small_geo(desc, 2);
        const int64_t rg = rows > 0 ? rows_wgrad_groups(desc) : 0;
        if (rg > 0 && workspace != nullptr && aligned(workspace, 4) &&
            ws_bytes >= size_t(rg) * size_t(n_g) * sizeof(int32_t)) {
            // per-workgroup partials, summed with the max in one pass
            int32_t *part = static_cast<int32_t *>(workspace);
            conv_rows_wgrad<<<dim3(unsigned(rg)), dim3(kRowsWgradThreads), 0, st>>>(dY, X, G, desc->N, sg, part);
            if (int rc = check_launch("int_conv_wgrad")) return rc;
            wl::sum_partials(part, int(rg), n_g, G, absmax_G, st);
            return check_launch("int_conv_wgrad");
        }
        zero_i32_kernel<<<dim3(direct_blocks(n_g)), dim3(256), 0, st>>>(G, n_g);
        if (int rc = check_launch("int_conv_wgrad")) return rc;
        if (rg > 0) {
            const int64_t ra = rows_wgrad_groups(desc, 256);
            conv_rows_wgrad<<<dim3(unsigned(ra)), dim3(kRowsWgradThreads), 0, st>>>(dY, X, G, desc->N, sg, nullptr);
            if (int rc = check_launch("int_conv_wgrad")) return rc;
        } else if (rows > 0 && sg.spb > 0) {
            conv_small_wgrad<<<dim3(small_blocks(desc->N, sg.spb, 1024)), dim3(256), 0, st>>>(dY, X, G, desc->N, sg,
                                                                                              int(n_g));
            if (int rc = check_launch("int_conv_wgrad")) return rc;
        } else if (rows > 0) {
            // up to 1024 workgroups of at least 16 output rows each
            int64_t nb = (rows + 15) / 16;
            if (nb > 1024) nb = 1024;
            const int64_t per = (rows + nb - 1) / nb;
            nb = (rows + per - 1) / per;
            conv_direct_wgrad<<<dim3(unsigned(nb)), dim3(256), 0, st>>>(dY, X, G, int(desc->H), int(desc->W), Cin,
                                                                      Cout, desc->KH, desc->KW, desc->pad, int(Ho),
                                                                      int(Wo), rows, per, n_g);
            if (int rc = check_launch("int_conv_wgrad")) return rc;
        }
        if (absmax_G) return launch_absmax_i32(G, n_g, absmax_G, st);
        return IONN_OK;
    }
    IONN_REQUIRE(G && (npix == 0 || (dY && X)), IONN_ERR_ARG, "int_conv_wgrad: NULL tensor");
    IONN_REQUIRE(aligned(dY, 16) && aligned(X, 16) && aligned(G, 16) && aligned(absmax_G, 4),
                 IONN_ERR_ALIGN, "int_conv_wgrad: tensors must be 16-byte aligned");
    hipStream_t st = as_stream(stream);
    if (npix > 0 && workspace != nullptr && fast_c64(desc, dY, X, G) && aligned(workspace, 16) &&
        ws_bytes >= int_conv_wgrad_workspace_bytes(desc)) {
        const unsigned P = c3_grid(desc);
        int32_t *part = static_cast<int32_t *>(workspace);
        c3::conv3x3_wgrad_kernel<<<dim3(P), dim3(c3::NTF), 0, st>>>(dY, X, part, int(desc->N),
                                                                    int(desc->H), int(desc->W));
        if (int rc = check_launch("int_conv_wgrad")) return rc;
        // one pass over the P partial rows, with the max
        wl::sum_partials(part, int(P), c3::GSZ, G, absmax_G, st);
        return check_launch("int_conv_wgrad");
    }
    const int M = Cout, N = 9 * Cin, K = npix;
    zero_i32_kernel<<<dim3(64), dim3(256), 0, st>>>(G, int64_t(M) * N);
    if (int rc = check_launch("int_conv_wgrad")) return rc;
    if (K > 0) {
        SrcColK sa{dY, Cout, M, K, true};
        SrcIm2colM sb{X, npix, int(desc->H), int(desc->W), Cin};
        Epi ep{G, N, M, N, true, nullptr, nullptr, true};
        const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
        const int ksteps = (K + 63) / 64;
        int split = (1024 + tiles - 1) / tiles;
        if (split > ksteps / 4) split = ksteps / 4;
        if (split < 1) split = 1;
        if (M % 64 == 0 && N % 64 == 0 && K % 64 == 0)
            launch<64, 64, 64, 2, 2, false>(sa, sb, ep, M, N, K, split, st);
        else
            launch<64, 64, 64, 2, 2, true>(sa, sb, ep, M, N, K, split, st);
        if (int rc = check_launch("int_conv_wgrad")) return rc;
    }
    if (absmax_G) return launch_absmax_i32(G, int64_t(M) * N, absmax_G, st);
    return IONN_OK;
}

}  // extern "C"
