// int8 x int8 -> int32 contractions of a Linear layer ("Integer On-Device
// Training: Overview", sections 3-4 and 7; weight index W[oc*IC + ic] as on
// the TiGrIS "Compilation Pipeline" page) on gfx950 matrix cores.
//
//   fwd   Y  = X  W^T : A = X  [M=B][K=IN]  (K-major), B = W [N=OUT][K=IN] (K-major)
//   dgrad dX = dY W   : A = dY [M=B][K=OUT] (K-major), B = W [K=OUT][N=IN] (N-major)
//   wgrad G  = dY^T X : A = dY [K=B][M=OUT] (M-major), B = X [K=B][N=IN]   (N-major)
//
// Tile-aligned problems take the 256x256x128 direct-to-LDS kernel of
// gemm256.h (v_mfma_i32_32x32x32_i8); a long batch through layers of at most
// 160 inputs and outputs takes gemm_skinny.h; other large problems run
// 256x256x64 bounds-checked tiles of the generic mainloop (gemm_core.h),
// small ones 64x64 tiles.  The epilogue fuses dgrad's ReLU mask and the max-abs that
// feeds the NITI shift.
#include "gemm256.h"
#include "gemm_skinny.h"
#include "wgrad_long.h"

namespace ionn {

int launch_absmax_i32(const int32_t *x, int64_t n, uint32_t *absmax, hipStream_t st);
namespace {

using namespace gemm;

template <class SA, class SB>
void launch_linear(const SA &sa, const SB &sb, const Epi &ep, int M, int N, int K, bool fast,
                   hipStream_t st) {
    // 256 x 256 tiles only with at least 16 of them: a 256 x 256 output as
    // one workgroup took 25 us where 16 tiles of 64 x 64 take 8
    if (fast && M >= 1024 && N >= 1024)
        launch<256, 256, 64, 2, 2, false>(sa, sb, ep, M, N, K, 1, st);
    else if (M >= 1024 && N >= 1024)
        launch<256, 256, 64, 2, 2, true>(sa, sb, ep, M, N, K, 1, st);
    else if (K >= 128)
        // few, small tiles: each K step is a load round trip the workgroup
        // waits for, so 256-deep steps (a 784-long reduction in 4 of them
        // instead of 13)
        launch<64, 64, 256, 2, 2, true>(sa, sb, ep, M, N, K, 1, st);
    else
        launch<64, 64, 64, 2, 2, true>(sa, sb, ep, M, N, K, 1, st);
}

__global__ void zero_i32_kernel(int32_t *C, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        C[i] = 0;
}

// Empty reduction (K == 0): C = 0, which leaves any max-abs unchanged.
int zero_output(int32_t *C, int64_t n, hipStream_t st, const char *name) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    zero_i32_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, st>>>(C, n);
    return check_launch(name);
}

bool dims_ok(int64_t B, int64_t IN, int64_t OUT) {
    return B >= 0 && IN >= 0 && OUT >= 0 && B <= kMaxDim && IN <= kMaxDim && OUT <= kMaxDim;
}

bool tile_aligned(int M, int N, int K) { return M % 256 == 0 && N % 256 == 0 && K % 64 == 0; }

// The 256x256x128 direct-to-LDS path: whole tiles (an even number of 128-deep
// K steps), operands below 2^31 bytes (32-bit buffer offsets), 16-byte aligned operands
// with row pitches that are multiples of 16, 16-byte aligned output rows.
bool fast256(int M, int N, int K, const void *A, int64_t lda, const void *B, int64_t ldb,
             const Epi &ep) {
    return M % 256 == 0 && N % 256 == 0 && K % 256 == 0 && aligned(A, 16) && aligned(B, 16) &&
           lda % 16 == 0 && ldb % 16 == 0 && aligned(ep.C, 16) && ep.ldc % 4 == 0 &&
           (ep.act == nullptr || aligned(ep.act, 4)) && int64_t(M) * lda < (int64_t(1) << 31) &&
           int64_t(K) * lda < (int64_t(1) << 31) && int64_t(N) * ldb < (int64_t(1) << 31) &&
           int64_t(K) * ldb < (int64_t(1) << 31);
}

}  // namespace
}  // namespace ionn

using namespace ionn;
using namespace ionn::gemm;

extern "C" {

int int_linear_fwd(const int8_t *X, const int8_t *W, int32_t *Y, int64_t B, int64_t IN,
                   int64_t OUT, uint32_t *absmax_Y, void *stream) {
    clear_error();
    IONN_REQUIRE(dims_ok(B, IN, OUT), IONN_ERR_SHAPE,
                 "int_linear_fwd: sizes must be in [0, 2^31): B=%lld IN=%lld OUT=%lld",
                 (long long)B, (long long)IN, (long long)OUT);
    if (B == 0 || OUT == 0) return IONN_OK;
    IONN_REQUIRE(Y && (IN == 0 || (X && W)), IONN_ERR_ARG, "int_linear_fwd: NULL tensor");
    IONN_REQUIRE(aligned(Y, 4) && aligned(absmax_Y, 4), IONN_ERR_ALIGN,
                 "int_linear_fwd: Y/absmax must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    if (IN == 0) return zero_output(Y, B * OUT, st, "int_linear_fwd");
    const int M = int(B), N = int(OUT), K = int(IN);
    SrcRowK sa{X, IN, M, K, aligned(X, 16) && IN % 16 == 0};
    SrcRowK sb{W, IN, N, K, aligned(W, 16) && IN % 16 == 0};
    Epi ep{Y, OUT, M, N, aligned(Y, 16) && OUT % 4 == 0, nullptr, absmax_Y, false};
    if (fast256(M, N, K, X, IN, W, IN, ep)) {
        g256::launch<true, true>(X, IN, W, IN, ep, M, N, K, st);
        return check_launch("int_linear_fwd");
    }
    if (sk::skinny_fits(M, N, K, X, W, Y, nullptr)) {
        sk::skinny_launch(false, X, W, Y, nullptr, absmax_Y, M, N, K, st);
        return check_launch("int_linear_fwd");
    }
    launch_linear(sa, sb, ep, M, N, K, tile_aligned(M, N, K) && sa.vec && sb.vec && ep.vec, st);
    return check_launch("int_linear_fwd");
}

size_t int_linear_fwd_oss_workspace_bytes(int64_t B, int64_t IN, int64_t OUT) {
    if (!dims_ok(B, IN, OUT)) return 0;
    const bool tile = B % 256 == 0 && OUT % 256 == 0 && IN % 256 == 0 && IN > 0;
    return tile ? 0 : size_t(B * OUT) * sizeof(int32_t);
}

int int_linear_fwd_oss(const int8_t *X, const int8_t *W, const int32_t *offset, const int32_t *mult,
                       const int8_t *k, int relu, int8_t *Y, int64_t B, int64_t IN, int64_t OUT,
                       void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    IONN_REQUIRE(dims_ok(B, IN, OUT), IONN_ERR_SHAPE,
                 "int_linear_fwd_oss: sizes must be in [0, 2^31): B=%lld IN=%lld OUT=%lld",
                 (long long)B, (long long)IN, (long long)OUT);
    IONN_REQUIRE(relu == 0 || relu == 1, IONN_ERR_ARG, "int_linear_fwd_oss: relu = %d", relu);
    if (B == 0 || OUT == 0) return IONN_OK;
    IONN_REQUIRE(Y && offset && mult && k && (IN == 0 || (X && W)), IONN_ERR_ARG,
                 "int_linear_fwd_oss: NULL tensor");
    IONN_REQUIRE(aligned(offset, 4) && aligned(mult, 4), IONN_ERR_ALIGN,
                 "int_linear_fwd_oss: offset/mult must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    const int M = int(B), N = int(OUT), K = int(IN);
    Epi ep{nullptr, OUT, M, N, false, nullptr, nullptr, false,
           Y, offset, mult, k, relu ? 0 : -128};
    if (M % 256 == 0 && N % 256 == 0 && K % 256 == 0 && K > 0 && aligned(X, 16) && aligned(W, 16) &&
        aligned(Y, 4) && aligned(offset, 16) && aligned(mult, 16) && aligned(k, 4) &&
        int64_t(M) * K < (int64_t(1) << 31) && int64_t(N) * K < (int64_t(1) << 31)) {
        g256::launch<true, true>(X, IN, W, IN, ep, M, N, K, st);
        return check_launch("int_linear_fwd_oss");
    }
    // other shapes: the int32 product into the workspace, then the OSS pass
    IONN_REQUIRE(workspace != nullptr && aligned(workspace, 16) &&
                     workspace_bytes >= size_t(B * OUT) * sizeof(int32_t),
                 IONN_ERR_WORKSPACE,
                 "int_linear_fwd_oss: this shape or alignment needs a 16-byte aligned workspace of %zu bytes",
                 size_t(B * OUT) * sizeof(int32_t));
    int32_t *acc = static_cast<int32_t *>(workspace);
    if (int rc = int_linear_fwd(X, W, acc, B, IN, OUT, nullptr, stream)) return rc;
    return ionn_oss_requant(acc, offset, mult, k, B, OUT, relu, Y, stream);
}

int int_linear_dgrad(const int8_t *dY, const int8_t *W, const int8_t *relu_act, int32_t *dX,
                     int64_t B, int64_t IN, int64_t OUT, uint32_t *absmax_dX, void *stream) {
    clear_error();
    IONN_REQUIRE(dims_ok(B, IN, OUT), IONN_ERR_SHAPE,
                 "int_linear_dgrad: sizes must be in [0, 2^31): B=%lld IN=%lld OUT=%lld",
                 (long long)B, (long long)IN, (long long)OUT);
    if (B == 0 || IN == 0) return IONN_OK;
    IONN_REQUIRE(dX && (OUT == 0 || (dY && W)), IONN_ERR_ARG, "int_linear_dgrad: NULL tensor");
    IONN_REQUIRE(aligned(dX, 4) && aligned(absmax_dX, 4), IONN_ERR_ALIGN,
                 "int_linear_dgrad: dX/absmax must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    if (OUT == 0) return zero_output(dX, B * IN, st, "int_linear_dgrad");
    const int M = int(B), N = int(IN), K = int(OUT);
    SrcRowK sa{dY, OUT, M, K, aligned(dY, 16) && OUT % 16 == 0};
    SrcColK sb{W, IN, N, K, aligned(W, 4) && IN % 4 == 0};
    Epi ep{dX, IN, M, N,
           aligned(dX, 16) && IN % 4 == 0 && (relu_act == nullptr || aligned(relu_act, 4)),
           relu_act, absmax_dX, false};
    if (fast256(M, N, K, dY, OUT, W, IN, ep)) {
        g256::launch<true, false>(dY, OUT, W, IN, ep, M, N, K, st);
        return check_launch("int_linear_dgrad");
    }
    if (sk::skinny_fits(M, N, K, dY, W, dX, relu_act)) {
        sk::skinny_launch(true, dY, W, dX, relu_act, absmax_dX, M, N, K, st);
        return check_launch("int_linear_dgrad");
    }
    launch_linear(sa, sb, ep, M, N, K, tile_aligned(M, N, K) && sa.vec && sb.vec && ep.vec, st);
    return check_launch("int_linear_dgrad");
}

int int_linear_wgrad(const int8_t *dY, const int8_t *X, int32_t *G, int64_t B, int64_t IN,
                     int64_t OUT, uint32_t *absmax_G, void *stream) {
    clear_error();
    IONN_REQUIRE(dims_ok(B, IN, OUT), IONN_ERR_SHAPE,
                 "int_linear_wgrad: sizes must be in [0, 2^31): B=%lld IN=%lld OUT=%lld",
                 (long long)B, (long long)IN, (long long)OUT);
    if (OUT == 0 || IN == 0) return IONN_OK;
    IONN_REQUIRE(G && (B == 0 || (dY && X)), IONN_ERR_ARG, "int_linear_wgrad: NULL tensor");
    IONN_REQUIRE(aligned(G, 4) && aligned(absmax_G, 4), IONN_ERR_ALIGN,
                 "int_linear_wgrad: G/absmax must be 4-byte aligned");
    hipStream_t st = as_stream(stream);
    if (B == 0) return zero_output(G, OUT * IN, st, "int_linear_wgrad");
    const int M = int(OUT), N = int(IN), K = int(B);
    SrcColK sa{dY, OUT, M, K, aligned(dY, 4) && OUT % 4 == 0};
    SrcColK sb{X, IN, N, K, aligned(X, 4) && IN % 4 == 0};
    Epi ep{G, IN, M, N, aligned(G, 16) && IN % 4 == 0, nullptr, absmax_G, false};
    if (fast256(M, N, K, dY, OUT, X, IN, ep)) {
        g256::launch<false, false>(dY, OUT, X, IN, ep, M, N, K, st);
        return check_launch("int_linear_wgrad");
    }
    // A small G over a long batch (a layer of a few hundred units trained on
    // a large batch): batch ranges reduced by the matrix cores from row
    // copies in LDS, added into the zeroed G with integer atomics (exact in
    // any order), then the max in its own pass.
    if (wl::wgrad_long_fits(K, M, N, dY, X)) {
        if (int rc = zero_output(G, OUT * IN, st, "int_linear_wgrad")) return rc;
        wl::wgrad_long_launch(dY, X, K, M, N, G, nullptr, st);
        if (int rc = check_launch("int_linear_wgrad")) return rc;
        if (absmax_G) return launch_absmax_i32(G, OUT * IN, absmax_G, st);
        return IONN_OK;
    }
    // Otherwise too few 64 x 64 tiles to fill the chip: split the batch over
    // up to 32 ranges of the generic kernel, with the same atomics.
    const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
    const int ksteps = (K + 63) / 64;
    if (tiles < 64 && ksteps >= 64) {
        int split = (512 + tiles - 1) / tiles;
        if (split > ksteps / 8) split = ksteps / 8;
        if (split > 32) split = 32;
        if (int rc = zero_output(G, OUT * IN, st, "int_linear_wgrad")) return rc;
        Epi epa{G, IN, M, N, aligned(G, 16) && IN % 4 == 0, nullptr, nullptr, true};
        launch<64, 64, 64, 2, 2, true>(sa, sb, epa, M, N, K, split, st);
        if (int rc = check_launch("int_linear_wgrad")) return rc;
        if (absmax_G) return launch_absmax_i32(G, OUT * IN, absmax_G, st);
        return IONN_OK;
    }
    launch_linear(sa, sb, ep, M, N, K, tile_aligned(M, N, K) && sa.vec && sb.vec && ep.vec, st);
    return check_launch("int_linear_wgrad");
}

size_t int_linear_wgrad_workspace_bytes(int64_t B, int64_t IN, int64_t OUT) {
    if (!dims_ok(B, IN, OUT) || !wl::wgrad_long_fits(B, OUT, IN, nullptr, nullptr)) return 0;
    return size_t(wl::wgrad_long_groups(B)) * size_t(wl::wgrad_long_part_elems(OUT, IN)) * sizeof(int32_t);
}

int int_linear_wgrad_ws(const int8_t *dY, const int8_t *X, int32_t *G, int64_t B, int64_t IN, int64_t OUT,
                        uint32_t *absmax_G, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    IONN_REQUIRE(dims_ok(B, IN, OUT), IONN_ERR_SHAPE,
                 "int_linear_wgrad_ws: sizes must be in [0, 2^31): B=%lld IN=%lld OUT=%lld", (long long)B,
                 (long long)IN, (long long)OUT);
    const size_t need = int_linear_wgrad_workspace_bytes(B, IN, OUT);
    if (need == 0 || OUT == 0 || IN == 0 || !wl::wgrad_long_fits(B, OUT, IN, dY, X))
        return int_linear_wgrad(dY, X, G, B, IN, OUT, absmax_G, stream);
    IONN_REQUIRE(G && dY && X, IONN_ERR_ARG, "int_linear_wgrad_ws: NULL tensor");
    IONN_REQUIRE(aligned(G, 4) && aligned(absmax_G, 4), IONN_ERR_ALIGN,
                 "int_linear_wgrad_ws: G/absmax must be 4-byte aligned");
    IONN_REQUIRE(workspace != nullptr && aligned(workspace, 4) && workspace_bytes >= need, IONN_ERR_WORKSPACE,
                 "int_linear_wgrad_ws: needs a 4-byte aligned workspace of %zu bytes", need);
    hipStream_t st = as_stream(stream);
    int32_t *part = static_cast<int32_t *>(workspace);
    const int nw = wl::wgrad_long_launch(dY, X, B, int(OUT), int(IN), G, part, st);
    if (int rc = check_launch("int_linear_wgrad_ws")) return rc;
    if (wl::wgrad_long_blocked(OUT, IN, part))
        wl::sum_partials_blocked(part, nw, int(((OUT + 31) / 32) * ((IN + 31) / 32)), int((IN + 31) / 32), int(OUT),
                                 int(IN), G, absmax_G, st);
    else
        wl::sum_partials(part, nw, OUT * IN, G, absmax_G, st);
    return check_launch("int_linear_wgrad_ws");
}

}  // extern "C"
