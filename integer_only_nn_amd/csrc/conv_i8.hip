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
#include "gemm_core.h"
#include "conv3x3.h"

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

int check_desc(const ionn_conv_desc *d, const char *name) {
    IONN_REQUIRE(d != nullptr, IONN_ERR_ARG, "%s: desc is NULL", name);
    IONN_REQUIRE(d->N >= 0 && d->H >= 0 && d->W >= 0 && d->Cin >= 0 && d->Cout >= 0,
                 IONN_ERR_SHAPE, "%s: negative size", name);
    IONN_REQUIRE(d->KH == 3 && d->KW == 3 && d->stride == 1 && d->pad == 1 && d->dilation == 1 &&
                     d->groups == 1,
                 IONN_ERR_UNSUPPORTED,
                 "%s: only 3x3 kernels, stride 1, pad 1, dilation 1, groups 1 are implemented "
                 "(got %dx%d s%d p%d d%d g%d)",
                 name, d->KH, d->KW, d->stride, d->pad, d->dilation, d->groups);
    IONN_REQUIRE(d->Cin % 16 == 0 && d->Cout % 16 == 0, IONN_ERR_UNSUPPORTED,
                 "%s: Cin and Cout must be multiples of 16 (got %lld, %lld)", name,
                 (long long)d->Cin, (long long)d->Cout);
    const int64_t npix = d->N * d->H * d->W;
    IONN_REQUIRE(npix <= kMaxDim && npix * d->Cin <= kMaxDim && npix * d->Cout <= kMaxDim &&
                     9 * d->Cin * d->Cout <= kMaxDim,
                 IONN_ERR_SHAPE, "%s: tensors must hold fewer than 2^31 elements", name);
    return IONN_OK;
}

// Compute units of the current device (persistent grids).
int device_cus() {
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

// The 64-channel halo-tiled kernel applies (see conv3x3.h).
bool fast_c64(const ionn_conv_desc *d, const void *in, const void *w, const void *out) {
    return d->Cin == 64 && d->Cout == 64 && c3::fits(d->W) && aligned(in, 16) && aligned(w, 16) &&
           aligned(out, 16);
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

extern "C" {

int int_conv_fwd(const int8_t *X, const int8_t *Wt, int32_t *Y, const ionn_conv_desc *desc,
                 uint32_t *absmax_Y, void *stream) {
    clear_error();
    if (int rc = check_desc(desc, "int_conv_fwd")) return rc;
    const int npix = int(desc->N * desc->H * desc->W), Cin = int(desc->Cin), Cout = int(desc->Cout);
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

size_t int_conv_wgrad_workspace_bytes(const ionn_conv_desc *desc) {
    if (desc == nullptr || desc->Cin != 64 || desc->Cout != 64 || !c3::fits(desc->W)) return 0;
    return size_t(c3::wgrad_rows(device_cus())) * c3::GSZ * sizeof(int32_t);
}

int int_conv_wgrad(const int8_t *dY, const int8_t *X, int32_t *G, const ionn_conv_desc *desc,
                   uint32_t *absmax_G, void *workspace, size_t ws_bytes, void *stream) {
    clear_error();
    if (int rc = check_desc(desc, "int_conv_wgrad")) return rc;
    const int npix = int(desc->N * desc->H * desc->W), Cin = int(desc->Cin), Cout = int(desc->Cout);
    if (Cin == 0 || Cout == 0) return IONN_OK;
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
        const int xb = c3::GSZ / 1024;
        if (P > 16) {
            const unsigned P2 = (P + 15) / 16;
            int32_t *part2 = part + int64_t(P) * c3::GSZ;
            c3::conv3x3_wgrad_reduce<<<dim3(xb, P2), dim3(256), 0, st>>>(part, int(P), part2, nullptr);
            if (int rc = check_launch("int_conv_wgrad")) return rc;
            c3::conv3x3_wgrad_reduce<<<dim3(xb, 1), dim3(256), 0, st>>>(part2, int(P2), G, absmax_G);
        } else {
            c3::conv3x3_wgrad_reduce<<<dim3(xb, 1), dim3(256), 0, st>>>(part, int(P), G, absmax_G);
        }
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
