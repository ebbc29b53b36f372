// One whole NITI step of a small int8 Linear layer in a single launch
// ("Integer On-Device Training: Overview", section 3 "The NITI Algorithm",
// steps 1-5, in the order the step takes them; weight index W[o*IN + i]).
//
// A layer of microcontroller size (the pages' own setting: tens of inputs
// and outputs, a batch of a few dozen) is latency-bound on this chip: the
// step as separate contractions, quantiser and update is five or six
// launches of a few microseconds each for a few ten thousand products.  Here
// one workgroup of 1024 threads stages X, W and dY in LDS and runs
//   fwd    Y  = X W^T                      (int32, max |Y|)
//   dgrad  dX = dY W                       (int32, max |dX|, pre-update W)
//          delta = sat8(rhu(dX, s_d)),     s_d = max(0, bitlen(max |dX|) - tb_d)
//   wgrad  G  = dY^T X                     (int32, max |G|)
//   update s = max(0, bitlen(max |G|) - tb_w), ws = max(0, s - mu),
//          W = sat8(W - rhu(rhu(G, s), ws))
// with the maxima reduced inside the workgroup (so nothing is max-combined
// and nothing needs clearing first).  Every product is an int8 x int8
// multiply-add into int32; with every dimension below 2^15 (the three
// operands share 32 KiB of LDS) no sum can leave the int32 range.
#include "common.h"

namespace ionn {
namespace {

constexpr int kStepThreads = 1024;
constexpr int64_t kStepLds = 32768;  // bytes of X, W and dY together

__device__ __forceinline__ uint32_t wg_max(uint32_t v, uint32_t *red) {
    v = wave_max_u32(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();  // red may still be read from the previous reduction
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    uint32_t m = red[0];
    for (int i = 1; i < kStepThreads / 64; ++i) m = max(m, red[i]);
    return m;
}

__global__ __launch_bounds__(kStepThreads) void linear_step_small_kernel(
    const int8_t *__restrict__ X, int8_t *__restrict__ W, const int8_t *__restrict__ dY, int B, int IN, int OUT,
    int tb_w, int mu, int tb_d, int32_t *__restrict__ Y, int32_t *__restrict__ dX, int8_t *__restrict__ delta,
    int32_t *__restrict__ G, int32_t *__restrict__ gq, uint32_t *__restrict__ maxima,
    int32_t *__restrict__ shifts) {
    __shared__ int8_t lds[kStepLds];
    __shared__ uint32_t red[kStepThreads / 64];
    const int tid = threadIdx.x;
    const int nx = B * IN, nw = OUT * IN, ny = B * OUT;
    int8_t *xs = lds, *ws_ = lds + nx, *ds = lds + nx + nw;
    for (int e = tid; e < nx; e += kStepThreads) xs[e] = X[e];
    for (int e = tid; e < nw; e += kStepThreads) ws_[e] = W[e];
    for (int e = tid; e < ny; e += kStepThreads) ds[e] = dY[e];
    __syncthreads();

    // fwd: Y[b][o] = sum_i X[b][i] W[o][i]
    uint32_t my = 0;
    for (int e = tid; e < ny; e += kStepThreads) {
        const int b = e / OUT, o = e - b * OUT;
        const int8_t *xr = xs + b * IN, *wr = ws_ + o * IN;
        int32_t s = 0;
        for (int i = 0; i < IN; ++i) s += int32_t(xr[i]) * int32_t(wr[i]);
        Y[e] = s;
        my = max(my, abs_u32(s));
    }
    // dgrad: dX[b][i] = sum_o dY[b][o] W[o][i] (W before the update)
    uint32_t mdx = 0;
    for (int e = tid; e < nx; e += kStepThreads) {
        const int b = e / IN, i = e - b * IN;
        const int8_t *dr = ds + b * OUT;
        int32_t s = 0;
        for (int o = 0; o < OUT; ++o) s += int32_t(dr[o]) * int32_t(ws_[o * IN + i]);
        dX[e] = s;
        mdx = max(mdx, abs_u32(s));
    }
    // wgrad: G[o][i] = sum_b dY[b][o] X[b][i]
    uint32_t mg = 0;
    for (int e = tid; e < nw; e += kStepThreads) {
        const int o = e / IN, i = e - o * IN;
        int32_t s = 0;
        for (int b = 0; b < B; ++b) s += int32_t(ds[b * OUT + o]) * int32_t(xs[b * IN + i]);
        G[e] = s;
        mg = max(mg, abs_u32(s));
    }
    my = wg_max(my, red);
    mdx = wg_max(mdx, red);
    mg = wg_max(mg, red);

    // each thread reads back only the int32 values it wrote above
    const int sd = niti_shift(mdx, tb_d);
    for (int e = tid; e < nx; e += kStepThreads) delta[e] = int8_t(sat8(rhu(dX[e], sd)));
    const int s = niti_shift(mg, tb_w), wsh = s > mu ? s - mu : 0;
    for (int e = tid; e < nw; e += kStepThreads) {
        const int32_t q = rhu(G[e], s);
        if (gq) gq[e] = q;
        W[e] = int8_t(sat8(int32_t(ws_[e]) - rhu(q, wsh)));
    }
    if (tid == 0) {
        maxima[0] = my;
        maxima[1] = mdx;
        maxima[2] = mg;
        shifts[0] = sd;
        shifts[1] = s;
        shifts[2] = wsh;
    }
}

bool step_small_fits(int64_t B, int64_t IN, int64_t OUT) {
    if (B < 1 || IN < 1 || OUT < 1 || B > kStepLds || IN > kStepLds || OUT > kStepLds) return false;
    return B * IN + OUT * IN + B * OUT <= kStepLds;
}

}  // namespace
}  // namespace ionn

using namespace ionn;

extern "C" {

int int_linear_step_small_fits(int64_t B, int64_t IN, int64_t OUT) { return step_small_fits(B, IN, OUT) ? 1 : 0; }

int int_linear_step_small(const int8_t *X, int8_t *W, const int8_t *dY, int64_t B, int64_t IN, int64_t OUT,
                          int tb_w, int mu_weight, int tb_d, int32_t *Y, int32_t *dX, int8_t *delta, int32_t *G,
                          int32_t *gq, uint32_t *maxima, int32_t *shifts, void *stream) {
    clear_error();
    IONN_REQUIRE(step_small_fits(B, IN, OUT), IONN_ERR_SHAPE,
                 "int_linear_step_small: B=%lld IN=%lld OUT=%lld (X, W and dY must fit together in %lld bytes)",
                 (long long)B, (long long)IN, (long long)OUT, (long long)kStepLds);
    IONN_REQUIRE(X && W && dY && Y && dX && delta && G && maxima && shifts, IONN_ERR_ARG,
                 "int_linear_step_small: NULL argument");
    IONN_REQUIRE(tb_w >= 1 && tb_w <= 31 && tb_d >= 1 && tb_d <= 31, IONN_ERR_RANGE,
                 "int_linear_step_small: target bits %d, %d outside [1, 31]", tb_w, tb_d);
    IONN_REQUIRE(mu_weight >= 0 && mu_weight <= 31, IONN_ERR_RANGE, "int_linear_step_small: mu_weight = %d",
                 mu_weight);
    IONN_REQUIRE(aligned(Y, 4) && aligned(dX, 4) && aligned(G, 4) && aligned(gq, 4) && aligned(maxima, 4) &&
                     aligned(shifts, 4),
                 IONN_ERR_ALIGN, "int_linear_step_small: int32 pointers must be 4-byte aligned");
    linear_step_small_kernel<<<dim3(1), dim3(kStepThreads), 0, as_stream(stream)>>>(
        X, W, dY, int(B), int(IN), int(OUT), tb_w, mu_weight, tb_d, Y, dX, delta, G, gq, maxima, shifts);
    return check_launch("int_linear_step_small");
}

}  // extern "C"
