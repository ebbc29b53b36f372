// Model-level training driver over an array of layer descriptors, the
// INT_LAYERS forward and backward of "Integer On-Device Training: Overview"
// (section 7: Conv2D, Conv2D+ReLU, Linear and Linear+ReLU layers with int8
// weights, int32 offsets and per-filter OSS shifts / multipliers; section 8:
// the OSS chain and the per-class TARGET_MAG loss; section 3: the NITI
// updates), as a sequence of the library's own calls on one stream.  The
// caller owns every tensor and one workspace; the driver allocates nothing.
//
// Forward, layer l: int32 contraction of the previous activation, then the
// OSS chain (the ReLU clip for the *_RELU types) into the layer's int8
// activation (a conv output [B][Ho][Wo][Cout] is the next Linear's input
// row, NHWC order).  Backward: the MSE gradient against the per-class
// targets, requantised to int8 (NITI, tb_delta bits); then for l = L..1 the
// offset gradient, wgrad, and for l > 1 dgrad with the pre-update weights,
// masked by a_{l-1} > 0 when layer l-1 has a ReLU and requantised; then the
// NITI updates of the weights (int8) and offsets (int32).
#include "common.h"

namespace ionn {
namespace {

__global__ __launch_bounds__(256) void mse_grad_kernel(const int8_t *__restrict__ out,
                                                       const int32_t *__restrict__ labels, int64_t B, int64_t C,
                                                       const int8_t *__restrict__ tmc,
                                                       const int8_t *__restrict__ tmw, int32_t *__restrict__ g,
                                                       uint32_t *__restrict__ absmax) {
    // B C < 2^31: 32-bit indices; both targets of the column are loaded with
    // the label and the output, so no load waits for another
    uint32_t m = 0;
    const uint32_t n = uint32_t(B * C), Cu = uint32_t(C);
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        const uint32_t b = i / Cu, c = i - b * Cu;
        const int32_t lab = labels[b], o = out[i], tc = tmc[c], tw = tmw[c];
        const int32_t v = o - (int32_t(c) == lab ? tc : tw);
        g[i] = v;
        m = max(m, abs_u32(v));
    }
    if (absmax) {
        m = wave_max_u32(m);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, m);
    }
}

__global__ __launch_bounds__(256) void relu_mask_kernel(int32_t *__restrict__ d, const int8_t *__restrict__ act,
                                                        int64_t n, uint32_t *__restrict__ absmax) {
    uint32_t m = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
        const int32_t v = act[i] > 0 ? d[i] : 0;
        d[i] = v;
        m = max(m, abs_u32(v));
    }
    if (absmax) {
        m = wave_max_u32(m);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, m);
    }
}

unsigned blocks_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    return unsigned(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

bool is_conv(const ionn_layer &L) { return L.type == IONN_LAYER_CONV2D || L.type == IONN_LAYER_CONV2D_RELU; }
bool has_relu(const ionn_layer &L) { return L.type == IONN_LAYER_CONV2D_RELU || L.type == IONN_LAYER_LINEAR_RELU; }

ionn_conv_desc desc_of(const ionn_layer &L, int64_t B) {
    ionn_conv_desc d;
    d.N = B;
    d.H = L.H;
    d.W = L.W;
    d.Cin = L.Cin;
    d.Cout = L.Cout;
    d.KH = L.KH;
    d.KW = L.KW;
    d.stride = 1;
    d.pad = L.pad;
    d.dilation = 1;
    d.groups = 1;
    return d;
}

int64_t in_size(const ionn_layer &L) { return L.H * L.W * L.Cin; }
int64_t out_hw(const ionn_layer &L) {
    if (!is_conv(L)) return 1;
    return (L.H + 2 * int64_t(L.pad) - L.KH + 1) * (L.W + 2 * int64_t(L.pad) - L.KW + 1);
}
int64_t out_size(const ionn_layer &L) { return out_hw(L) * L.Cout; }
int64_t weight_size(const ionn_layer &L) { return is_conv(L) ? L.Cout * L.KH * L.KW * L.Cin : L.Cout * in_size(L); }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace carving; base == nullptr only measures.
struct Plan {
    int8_t *act[IONN_MAX_LAYERS];
    int32_t *z32, *g32, *gb, *e32;
    int8_t *delta[2];
    uint32_t *scal;
    void *bgws, *cws, *lws;
    size_t bg_bytes, cw_bytes, lw_bytes, z_bytes;
    size_t total;
};

Plan plan(const ionn_layer *layers, int L, int64_t B, void *base) {
    Plan p{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return base ? static_cast<char *>(base) + o : nullptr;
    };
    int64_t max_io = 0, max_out = 0, max_w = 0, max_c = 0;
    size_t bg = 0, cw = 0, lw = 0;
    for (int l = 0; l < L; ++l) {
        const ionn_layer &Ly = layers[l];
        max_io = max(max_io, max(in_size(Ly), out_size(Ly)));
        max_out = max(max_out, out_size(Ly));
        max_w = max(max_w, weight_size(Ly));
        max_c = max(max_c, Ly.Cout);
        bg = max(bg, ionn_bias_grad_workspace_bytes(B * out_hw(Ly), Ly.Cout));
        if (is_conv(Ly)) {
            const ionn_conv_desc d = desc_of(Ly, B);
            cw = max(cw, int_conv_wgrad_workspace_bytes(&d));
        } else {
            lw = max(lw, int_linear_wgrad_workspace_bytes(B, Ly.Cin, Ly.Cout));
        }
    }
    for (int l = 0; l < L; ++l) p.act[l] = reinterpret_cast<int8_t *>(take(size_t(B * out_size(layers[l]))));
    p.z_bytes = size_t(B * max_io) * 4;
    p.z32 = reinterpret_cast<int32_t *>(take(p.z_bytes));
    p.g32 = reinterpret_cast<int32_t *>(take(size_t(max_w) * 4));
    p.gb = reinterpret_cast<int32_t *>(take(size_t(max_c) * 4));
    p.delta[0] = reinterpret_cast<int8_t *>(take(size_t(B * max_out)));
    p.delta[1] = reinterpret_cast<int8_t *>(take(size_t(B * max_out)));
    p.e32 = reinterpret_cast<int32_t *>(take(size_t(B * layers[L - 1].Cout) * 4));
    p.scal = reinterpret_cast<uint32_t *>(take(size_t(3 * L + 1) * 4));
    p.bg_bytes = bg;
    p.bgws = take(bg);
    p.cw_bytes = cw;
    p.cws = cw ? take(cw) : nullptr;
    p.lw_bytes = lw;
    p.lws = lw ? take(lw) : nullptr;
    p.total = off;
    return p;
}

int check_model(const ionn_layer *layers, int L, int64_t B, const char *name) {
    IONN_REQUIRE(layers != nullptr && L >= 1 && L <= IONN_MAX_LAYERS, IONN_ERR_ARG,
                 "%s: need 1..%d layers (got %d)", name, IONN_MAX_LAYERS, L);
    IONN_REQUIRE(B >= 1 && B <= kMaxDim, IONN_ERR_SHAPE, "%s: batch %lld", name, (long long)B);
    for (int l = 0; l < L; ++l) {
        const ionn_layer &Ly = layers[l];
        IONN_REQUIRE(Ly.type >= IONN_LAYER_CONV2D && Ly.type <= IONN_LAYER_LINEAR_RELU, IONN_ERR_ARG,
                     "%s: layer %d has type %d", name, l, Ly.type);
        IONN_REQUIRE(Ly.H >= 1 && Ly.W >= 1 && Ly.Cin >= 1 && Ly.Cout >= 1, IONN_ERR_SHAPE,
                     "%s: layer %d has an empty dimension", name, l);
        IONN_REQUIRE(Ly.weight && Ly.offset && Ly.mult && Ly.k, IONN_ERR_ARG, "%s: layer %d: NULL parameter", name, l);
        if (is_conv(Ly)) {
            IONN_REQUIRE(Ly.KH >= 1 && Ly.KW >= 1 && Ly.pad >= 0 && out_hw(Ly) >= 1 &&
                             Ly.H + 2 * int64_t(Ly.pad) - Ly.KH + 1 >= 1,
                         IONN_ERR_SHAPE, "%s: layer %d: kernel %dx%d pad %d leaves no output", name, l, Ly.KH,
                         Ly.KW, Ly.pad);
        } else {
            IONN_REQUIRE(Ly.H == 1 && Ly.W == 1, IONN_ERR_SHAPE,
                         "%s: layer %d: a Linear layer takes H = W = 1 and Cin = its input features", name, l);
        }
        IONN_REQUIRE(B * max(in_size(Ly), out_size(Ly)) <= kMaxDim && weight_size(Ly) <= kMaxDim,
                     IONN_ERR_SHAPE, "%s: layer %d: tensors must hold fewer than 2^31 elements", name, l);
        if (l > 0)
            IONN_REQUIRE(in_size(Ly) == out_size(layers[l - 1]), IONN_ERR_SHAPE,
                         "%s: layer %d reads %lld values per sample, layer %d writes %lld", name, l,
                         (long long)in_size(Ly), l - 1, (long long)out_size(layers[l - 1]));
    }
    return IONN_OK;
}

// ---------------------------------------------------------------------------
// Small models (the on-device training page's networks at their batch of a
// few samples): the whole forward, and the whole backward, in one workgroup
// each.  Every contraction of a layer is staged in LDS as two zero-padded
// byte matrices P [n1][kb] and Q [n2][kb] (kb a multiple of 16) with
// out[i][j] = sum_k P[i][k] Q[j][k]:
//   forward  P = im2col rows of the input [B*Ho*Wo][K], Q = weights [Cout][K]
//            (K = KH*KW*Cin, terms in the weight's (kh, kw, ci) order);
//   offsets  P = delta transposed [Cout][B*Ho*Wo], Q = a row of ones;
//   wgrad    P = delta transposed, Q = im2col transposed [K][B*Ho*Wo];
//   dgrad    P = rows of the delta seen through the flipped kernel
//            [B*H*W][KH*KW*Cout], Q = weights regrouped per input channel
//            [Cin][KH*KW*Cout].
// A Linear layer is the 1x1 case (H = W = 1).  A term group is one 16-byte
// LDS read of each operand and four v_dot4 (int8 products summed in int32,
// exact), the quantisers and updates are block-strided loops with the same
// integer arithmetic as the multi-kernel driver, each per-tensor maximum a
// block reduction; the phases are separated by barriers.  Same bits as the
// multi-kernel driver.
// ---------------------------------------------------------------------------
constexpr int kSmallLayers = 8;
constexpr int kSmallThreads = 1024;
constexpr int64_t kSmallMacs = int64_t(1) << 22;  // multiply-adds per step, fwd + bwd
constexpr int kStageBytes = 96 * 1024;            // the operand matrices of one layer
constexpr int kZWords = 8192;                     // int32 outputs of a phase kept in LDS

struct SmallModel {
    int L;
    int64_t B;
    ionn_layer ly[kSmallLayers];
    int8_t *act[kSmallLayers];
    const int8_t *X;
    int8_t *out;
    int32_t *g32, *gb;
    int8_t *delta[2];
    const int32_t *labels;
    const int8_t *tmc, *tmw;
    int tb_delta, tb_weight, mu;
    int32_t *shifts_out;
};

struct Geo {  // per-layer sizes (a Linear layer: H = W = KH = KW = Ho = Wo = 1)
    int H, W, Cin, Cout, KH, KW, P, Ho, Wo;
    bool conv, relu;
};

__host__ __device__ inline Geo geo(const ionn_layer &L) {
    Geo g;
    g.conv = L.type == IONN_LAYER_CONV2D || L.type == IONN_LAYER_CONV2D_RELU;
    g.relu = L.type == IONN_LAYER_CONV2D_RELU || L.type == IONN_LAYER_LINEAR_RELU;
    g.H = g.conv ? int(L.H) : 1;
    g.W = g.conv ? int(L.W) : 1;
    g.Cin = g.conv ? int(L.Cin) : int(L.H * L.W * L.Cin);
    g.Cout = int(L.Cout);
    g.KH = g.conv ? L.KH : 1; g.KW = g.conv ? L.KW : 1; g.P = g.conv ? L.pad : 0;
    g.Ho = g.H + 2 * g.P - g.KH + 1;
    g.Wo = g.W + 2 * g.P - g.KW + 1;
    return g;
}

__host__ __device__ inline int64_t pad16(int64_t n) { return (n + 15) & ~int64_t(15); }

// LDS operand sizes of one layer.
struct SmallSizes {
    int64_t R, K, Kf, Rb, Kd, npix, nx;  // rows B*Ho*Wo, K, padded K, padded R, padded KH*KW*Cout, B*H*W, B*H*W*Cin
    int64_t fwd_bytes, bwd_bytes, dgrad_bytes;
};

__host__ __device__ inline SmallSizes small_sizes(const Geo &g, int64_t B) {
    SmallSizes z;
    z.R = B * g.Ho * g.Wo;
    z.K = int64_t(g.KH) * g.KW * g.Cin;
    z.Kf = pad16(z.K);
    z.Rb = pad16(z.R);
    z.Kd = pad16(int64_t(g.KH) * g.KW * g.Cout);
    z.npix = B * g.H * g.W;
    z.nx = z.npix * g.Cin;
    z.fwd_bytes = (z.R + g.Cout) * z.Kf;
    z.bwd_bytes = (g.Cout + z.K) * z.Rb;
    z.dgrad_bytes = (z.npix + g.Cin) * z.Kd;
    return z;
}

// Quotient of 0 <= x < 2^22 by d >= 1: a float estimate (error below one)
// corrected both ways.
struct FastDiv {
    int d;
    float r;
    __device__ explicit FastDiv(int d_) : d(d_), r(1.0f / float(d_)) {}
    __device__ __forceinline__ int div(int x) const {
        int q = int(float(x) * r);
        q -= q * d > x ? 1 : 0;
        q += (q + 1) * d <= x ? 1 : 0;
        return q;
    }
};

// Max over the workgroup of one value per thread (every thread gets it).
__device__ uint32_t block_max(uint32_t v) {
    __shared__ uint32_t red[kSmallThreads / 64];
    v = wave_max_u32(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t m = 0;
    for (int i = 0; i < int(blockDim.x >> 6); ++i) m = max(m, red[i]);
    return m;
}

// Fill the LDS matrix S [rows][kb] one dword per step: row(i) prepares row
// i, byte(ctx, k) returns its byte k (zero in the padding).
template <class Row, class Byte>
__device__ __forceinline__ void stage(int8_t *S, int rows, int kb, Row row, Byte byte) {
    const int wpr = kb >> 2, nw = rows * wpr;
    const FastDiv dw(wpr);
    for (int w = threadIdx.x; w < nw; w += blockDim.x) {
        const int i = dw.div(w), k0 = (w - i * wpr) << 2;
        const auto ctx = row(i);
        const uint32_t v = uint32_t(uint8_t(byte(ctx, k0))) | (uint32_t(uint8_t(byte(ctx, k0 + 1))) << 8) |
                           (uint32_t(uint8_t(byte(ctx, k0 + 2))) << 16) |
                           (uint32_t(uint8_t(byte(ctx, k0 + 3))) << 24);
        reinterpret_cast<uint32_t *>(S)[w] = v;
    }
}

struct Pix {  // an output (or input) pixel (n, y, x)
    int n, y, x;
};

__device__ __forceinline__ int32_t dot16(const int4 &a, const int4 &b, int32_t t) {
    t = __builtin_amdgcn_sdot4(a.x, b.x, t, false);
    t = __builtin_amdgcn_sdot4(a.y, b.y, t, false);
    t = __builtin_amdgcn_sdot4(a.z, b.z, t, false);
    return __builtin_amdgcn_sdot4(a.w, b.w, t, false);
}

__device__ __forceinline__ int4 ones16() { return make_int4(0x01010101, 0x01010101, 0x01010101, 0x01010101); }

// f(e, j, out[e]) for every output e = i * n2 + j of out[i][j] = sum_k
// P[i][k] Q[j][k] (P, Q: LDS byte matrices [n1][kb], [n2][kb], kb a multiple
// of 16; Q == nullptr: a row of ones), block-strided, four outputs per
// thread at a time so that their LDS reads are in flight together.
template <class F>
__device__ __forceinline__ void each_dot(const int8_t *P, const int8_t *Q, int n1, int n2, int kb, F f) {
    const int nt = blockDim.x, n = n1 * n2, ng = kb >> 4;
    const FastDiv dn2(n2);
    for (int e0 = threadIdx.x; e0 < n; e0 += 4 * nt) {
        const int4 *p[4], *q[4];
        int jj[4];
        int32_t t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = min(e0 + u * nt, n - 1), i = dn2.div(e);
            jj[u] = e - i * n2;
            p[u] = reinterpret_cast<const int4 *>(P + i * kb);
            q[u] = reinterpret_cast<const int4 *>(Q ? Q + jj[u] * kb : P);
            t[u] = 0;
        }
        for (int gq = 0; gq < ng; ++gq) {
#pragma unroll
            for (int u = 0; u < 4; ++u) t[u] = dot16(p[u][gq], Q ? q[u][gq] : ones16(), t[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (e0 + u * nt < n) f(e0 + u * nt, jj[u], t[u]);
    }
}

// The same outputs, each finished one passed to fin(e, j, v), which returns
// the value whose magnitude enters the per-thread maximum that the call
// returns.  With fewer than two outputs per thread the term groups are split
// into ranges and the partial sums of an output meet in Z by LDS atomics
// (exact in any order; n < 2 * threads <= kZWords then).  Ends with a
// barrier.
template <class Fin>
__device__ uint32_t contract(const int8_t *P, const int8_t *Q, int n1, int n2, int kb, int32_t *Z, Fin fin) {
    const int nt = blockDim.x, tid = threadIdx.x;
    const int n = n1 * n2, ng = kb >> 4;
    int ns = max(1, min((2 * nt + n - 1) / n, ng));
    const int gs = (ng + ns - 1) / ns;
    ns = (ng + gs - 1) / gs;
    uint32_t mx = 0;
    if (ns == 1) {
        each_dot(P, Q, n1, n2, kb, [&](int e, int j, int32_t v) { mx = max(mx, abs_u32(fin(e, j, v))); });
        __syncthreads();
        return mx;
    }
    const FastDiv dn(n), dn2(n2);
    const int4 ones = ones16();
    for (int e = tid; e < n; e += nt) Z[e] = 0;
    __syncthreads();
    for (int it = tid; it < n * ns; it += nt) {
        const int r = dn.div(it), e = it - r * n;
        const int i = dn2.div(e), j = e - i * n2;
        const int g0 = r * gs, g1 = min(ng, g0 + gs);
        const int4 *p = reinterpret_cast<const int4 *>(P + i * kb);
        int32_t t = 0;
        if (Q) {
            const int4 *q = reinterpret_cast<const int4 *>(Q + j * kb);
#pragma unroll 2
            for (int gq = g0; gq < g1; ++gq) t = dot16(p[gq], q[gq], t);
        } else {
#pragma unroll 2
            for (int gq = g0; gq < g1; ++gq) t = dot16(p[gq], ones, t);
        }
        atomicAdd(&Z[e], t);
    }
    __syncthreads();
    for (int e = tid; e < n; e += nt) {
        const int j = e - dn2.div(e) * n2;
        mx = max(mx, abs_u32(fin(e, j, Z[e])));
    }
    __syncthreads();
    return mx;
}

// im2col rows of the input a [B][H][W][Cin]: row r = (n, ho, wo), byte k =
// (kh * KW + kw) * Cin + ci.
__device__ __forceinline__ void stage_cols(int8_t *S, const int8_t *a, const Geo &g, const SmallSizes &z) {
    const FastDiv dWo(g.Wo), dHo(g.Ho), dCin(g.Cin), dKW(g.KW);
    const int K = int(z.K);
    stage(S, int(z.R), int(z.Kf),
          [&](int r) {
              const int q = dWo.div(r), n = dHo.div(q);
              return Pix{n, q - n * g.Ho, r - q * g.Wo};
          },
          [&](const Pix &p, int k) -> int8_t {
              if (k >= K) return 0;
              if (!g.conv) return a[p.n * g.Cin + k];
              const int tap = dCin.div(k), ci = k - tap * g.Cin, kh = dKW.div(tap), kw = tap - kh * g.KW;
              const int h = p.y + kh - g.P, x = p.x + kw - g.P;
              return (h >= 0 && h < g.H && x >= 0 && x < g.W) ? a[((p.n * g.H + h) * g.W + x) * g.Cin + ci] : 0;
          });
}

// The same matrix transposed: row k, byte r.
__device__ __forceinline__ void stage_cols_t(int8_t *S, const int8_t *a, const Geo &g, const SmallSizes &z) {
    const FastDiv dWo(g.Wo), dHo(g.Ho), dCin(g.Cin), dKW(g.KW);
    const int R = int(z.R);
    struct Tap {
        int kh, kw, ci;
    };
    stage(S, int(z.K), int(z.Rb),
          [&](int k) {
              const int tap = dCin.div(k), kh = dKW.div(tap);
              return Tap{kh, tap - kh * g.KW, k - tap * g.Cin};
          },
          [&](const Tap &t, int r) -> int8_t {
              if (r >= R) return 0;
              if (!g.conv) return a[r * g.Cin + t.ci];
              const int q = dWo.div(r), n = dHo.div(q), ho = q - n * g.Ho, wo = r - q * g.Wo;
              const int h = ho + t.kh - g.P, x = wo + t.kw - g.P;
              return (h >= 0 && h < g.H && x >= 0 && x < g.W) ? a[((n * g.H + h) * g.W + x) * g.Cin + t.ci] : 0;
          });
}

// Zero-padded rows of a row-major [rows][cols] byte matrix.
__device__ __forceinline__ void stage_rows(int8_t *S, const int8_t *src, int rows, int cols, int kb) {
    stage(S, rows, kb, [&](int i) { return src + i * cols; },
          [&](const int8_t *row, int k) -> int8_t { return k < cols ? row[k] : 0; });
}

// Transpose of a row-major [rows][cols] byte matrix: row c, byte i.
__device__ __forceinline__ void stage_rows_t(int8_t *S, const int8_t *src, int rows, int cols, int kb) {
    stage(S, cols, kb, [&](int c) { return src + c; },
          [&](const int8_t *col, int i) -> int8_t { return i < rows ? col[i * cols] : 0; });
}

// dgrad rows: input pixel p = (n, h, x), byte k = (kh * KW + kw) * Cout + co
// holds d[n][h + P - kh][x + P - kw][co] (zero outside the output).
__device__ __forceinline__ void stage_dgrad_rows(int8_t *S, const int8_t *d, const Geo &g, const SmallSizes &z) {
    const FastDiv dW(g.W), dH(g.H), dCout(g.Cout), dKW(g.KW);
    const int Kd = g.KH * g.KW * g.Cout;
    stage(S, int(z.npix), int(z.Kd),
          [&](int p) {
              const int q = dW.div(p), n = dH.div(q);
              return Pix{n, q - n * g.H, p - q * g.W};
          },
          [&](const Pix &p, int k) -> int8_t {
              if (k >= Kd) return 0;
              if (!g.conv) return d[p.n * g.Cout + k];
              const int tap = dCout.div(k), co = k - tap * g.Cout, kh = dKW.div(tap), kw = tap - kh * g.KW;
              const int ho = p.y + g.P - kh, wo = p.x + g.P - kw;
              return (ho >= 0 && ho < g.Ho && wo >= 0 && wo < g.Wo) ? d[((p.n * g.Ho + ho) * g.Wo + wo) * g.Cout + co]
                                                                     : 0;
          });
}

// Weights regrouped per input channel: row ci, byte (kh * KW + kw) * Cout + co
// holds w[co][kh][kw][ci].
__device__ __forceinline__ void stage_dgrad_w(int8_t *S, const int8_t *w, const Geo &g, const SmallSizes &z) {
    const FastDiv dCout(g.Cout);
    const int taps = g.KH * g.KW, Kd = taps * g.Cout;
    stage(S, g.Cin, int(z.Kd), [&](int ci) { return ci; },
          [&](int ci, int k) -> int8_t {
              if (k >= Kd) return 0;
              const int tap = dCout.div(k), co = k - tap * g.Cout;
              return w[(co * taps + tap) * g.Cin + ci];
          });
}

__global__ __launch_bounds__(kSmallThreads) void small_forward_kernel(SmallModel m) {
    __shared__ __attribute__((aligned(16))) int8_t S[kStageBytes];
    __shared__ int32_t Z[kZWords];
    const int B = int(m.B);
    for (int l = 0; l < m.L; ++l) {
        const ionn_layer &Ly = m.ly[l];
        const Geo g = geo(Ly);
        const SmallSizes z = small_sizes(g, B);
        int8_t *A = S, *Wm = S + z.R * z.Kf;
        stage_cols(A, l == 0 ? m.X : m.act[l - 1], g, z);
        stage_rows(Wm, Ly.weight, g.Cout, int(z.K), int(z.Kf));
        __syncthreads();
        // the OSS chain (static shift) into the layer's int8 activation
        const int32_t lo = g.relu ? 0 : -128;
        int8_t *act = m.act[l], *out = l == m.L - 1 ? m.out : nullptr;
        contract(A, Wm, int(z.R), g.Cout, int(z.Kf), Z, [&](int e, int c, int32_t v) {
            const int8_t y = int8_t(oss_elem(v, Ly.offset[c], Ly.mult[c], int(Ly.k[c]), lo));
            act[e] = y;
            if (out) out[e] = y;
            return 0;
        });
    }
}

__global__ __launch_bounds__(kSmallThreads) void small_backward_kernel(SmallModel m) {
    __shared__ __attribute__((aligned(16))) int8_t S[kStageBytes];
    __shared__ int32_t Z[kZWords];
    const int L = m.L, B = int(m.B);
    const int tid = threadIdx.x, nt = blockDim.x;
    if (m.shifts_out)
        for (int i = tid; i < 5 * L + 1; i += nt) m.shifts_out[i] = -1;
    // loss gradient against the per-class targets, requantised
    const int C = int(m.ly[L - 1].Cout), ne = B * C;
    uint32_t mx = 0;
    for (int i = tid; i < ne; i += nt) {
        const int b = i / C, c = i - b * C;
        const int32_t t = c == m.labels[b] ? int32_t(m.tmc[c]) : int32_t(m.tmw[c]);
        const int32_t v = int32_t(m.act[L - 1][i]) - t;
        Z[i] = v;
        mx = max(mx, abs_u32(v));
    }
    const int s = niti_shift(block_max(mx), m.tb_delta);
    for (int i = tid; i < ne; i += nt) m.delta[0][i] = int8_t(sat8(rhu(Z[i], s)));
    if (m.shifts_out && tid == 0) m.shifts_out[0] = s;
    __syncthreads();
    int cur = 0;
    for (int l = L - 1; l >= 0; --l) {
        const ionn_layer &Ly = m.ly[l];
        const Geo g = geo(Ly);
        const SmallSizes z = small_sizes(g, B);
        const int8_t *a = l == 0 ? m.X : m.act[l - 1];
        const int8_t *d = m.delta[cur];
        int32_t *sh = m.shifts_out ? m.shifts_out + 1 + 5 * l : nullptr;
        const int Rb = int(z.Rb), K = int(z.K), nw = g.Cout * K;
        int8_t *dT = S, *aT = S + g.Cout * z.Rb, *Pd = aT + z.K * z.Rb, *Qd = Pd + z.npix * z.Kd;
        stage_rows_t(dT, d, int(z.R), g.Cout, Rb);
        stage_cols_t(aT, a, g, z);
        if (l > 0) {
            stage_dgrad_rows(Pd, d, g, z);
            stage_dgrad_w(Qd, Ly.weight, g, z);  // pre-update weights
        }
        __syncthreads();
        // offset gradient: column sums of the delta
        int32_t *gb = m.gb, *g32 = m.g32;
        const uint32_t mb = contract(dT, nullptr, g.Cout, 1, Rb, Z, [&](int e, int, int32_t v) {
            gb[e] = v;
            return v;
        });
        // weight gradient
        const uint32_t mg = contract(dT, aT, g.Cout, K, Rb, Z, [&](int e, int, int32_t v) {
            g32[e] = v;
            return v;
        });
        // propagated delta with the pre-update weights, masked by the previous
        // layer's ReLU, requantised
        if (l > 0) {
            const bool mask = m.ly[l - 1].type == IONN_LAYER_CONV2D_RELU ||
                              m.ly[l - 1].type == IONN_LAYER_LINEAR_RELU;
            const uint32_t md = contract(Pd, Qd, int(z.npix), g.Cin, int(z.Kd), Z, [&](int e, int, int32_t v) {
                if (mask && a[e] <= 0) v = 0;
                Z[e] = v;
                return v;
            });
            const int sd = niti_shift(block_max(md), m.tb_delta);
            int8_t *dn = m.delta[cur ^ 1];
            for (int e = tid; e < int(z.nx); e += nt) dn[e] = int8_t(sat8(rhu(Z[e], sd)));
            if (sh && tid == 0) sh[0] = sd;
        }
        // updates (each thread reads back the gradients it wrote)
        const uint32_t amg = block_max(mg), amb = block_max(mb);
        const int sw = niti_shift(amg, m.tb_weight), wsw = sw > m.mu ? sw - m.mu : 0;
        for (int e = tid; e < nw; e += nt)
            Ly.weight[e] = int8_t(sat8(int32_t(Ly.weight[e]) - rhu(rhu(g32[e], sw), wsw)));
        const int sb = niti_shift(amb, m.tb_weight), wsb = sb > m.mu ? sb - m.mu : 0;
        for (int c = tid; c < g.Cout; c += nt) {
            const int64_t v = int64_t(Ly.offset[c]) - int64_t(rhu(rhu(gb[c], sb), wsb));
            Ly.offset[c] = v < INT32_MIN ? INT32_MIN : (v > INT32_MAX ? INT32_MAX : int32_t(v));
        }
        if (sh && tid == 0) {
            sh[1] = sw; sh[2] = wsw; sh[3] = sb; sh[4] = wsb;
        }
        __syncthreads();
        cur ^= 1;
    }
}

int64_t step_macs(const ionn_layer *layers, int L, int64_t B) {
    int64_t t = 0;
    for (int l = 0; l < L; ++l) {
        const ionn_layer &Ly = layers[l];
        const int64_t per = is_conv(Ly) ? int64_t(Ly.KH) * Ly.KW * Ly.Cin : in_size(Ly);
        t += 3 * B * out_size(Ly) * per;
    }
    return t;
}

// The one-workgroup path applies: few layers, little work.
// The one-workgroup path applies: few layers, little work, and every layer's
// operand matrices and LDS-held outputs within their LDS regions.
bool small_model(const ionn_layer *layers, int L, int64_t B) {
    if (L > kSmallLayers || step_macs(layers, L, B) > kSmallMacs) return false;
    for (int l = 0; l < L; ++l) {
        const Geo g = geo(layers[l]);
        const SmallSizes z = small_sizes(g, B);
        if (z.fwd_bytes > kStageBytes || z.bwd_bytes + (l > 0 ? z.dgrad_bytes : 0) > kStageBytes) return false;
        if (l > 0 && z.nx > kZWords) return false;
    }
    return B * layers[L - 1].Cout <= kZWords;
}

SmallModel small_args(const ionn_layer *layers, int L, int64_t B, const int8_t *X, const Plan &p) {
    SmallModel m{};
    m.L = L;
    m.B = B;
    for (int l = 0; l < L; ++l) {
        m.ly[l] = layers[l];
        m.act[l] = p.act[l];
    }
    m.X = X;
    m.g32 = p.g32; m.gb = p.gb;
    m.delta[0] = p.delta[0]; m.delta[1] = p.delta[1];
    return m;
}

}  // namespace
}  // namespace ionn

using namespace ionn;

extern "C" {

int ionn_mse_grad_targets(const int8_t *out, const int32_t *labels, int64_t B, int64_t C, const int8_t *tmc,
                          const int8_t *tmw, int32_t *g, uint32_t *absmax_g, void *stream) {
    clear_error();
    IONN_REQUIRE(B >= 0 && C >= 0 && B <= kMaxDim && C <= kMaxDim && B * C <= kMaxDim, IONN_ERR_SHAPE,
                 "ionn_mse_grad_targets: bad shape B=%lld C=%lld", (long long)B, (long long)C);
    if (B * C == 0) return IONN_OK;
    IONN_REQUIRE(out && labels && tmc && tmw && g, IONN_ERR_ARG, "ionn_mse_grad_targets: NULL argument");
    IONN_REQUIRE(aligned(labels, 4) && aligned(g, 4) && aligned(absmax_g, 4), IONN_ERR_ALIGN,
                 "ionn_mse_grad_targets: int32 pointers must be 4-byte aligned");
    mse_grad_kernel<<<dim3(blocks_for(B * C)), dim3(256), 0, as_stream(stream)>>>(out, labels, B, C, tmc, tmw, g,
                                                                                  absmax_g);
    return check_launch("ionn_mse_grad_targets");
}

int ionn_relu_mask_i32(int32_t *d, const int8_t *act, int64_t n, uint32_t *absmax_d, void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 0 && n <= kMaxDim, IONN_ERR_SHAPE, "ionn_relu_mask_i32: n = %lld", (long long)n);
    if (n == 0) return IONN_OK;
    IONN_REQUIRE(d && act, IONN_ERR_ARG, "ionn_relu_mask_i32: NULL argument");
    IONN_REQUIRE(aligned(d, 4) && aligned(absmax_d, 4), IONN_ERR_ALIGN,
                 "ionn_relu_mask_i32: int32 pointers must be 4-byte aligned");
    relu_mask_kernel<<<dim3(blocks_for(n)), dim3(256), 0, as_stream(stream)>>>(d, act, n, absmax_d);
    return check_launch("ionn_relu_mask_i32");
}

size_t ionn_model_workspace_bytes(const ionn_layer *layers, int L, int64_t B) {
    clear_error();
    if (check_model(layers, L, B, "ionn_model_workspace_bytes")) return 0;
    return plan(layers, L, B, nullptr).total;
}

int ionn_model_forward(const ionn_layer *layers, int L, const int8_t *X, int64_t B, int8_t *out, void *workspace,
                       size_t workspace_bytes, void *stream) {
    clear_error();
    if (int rc = check_model(layers, L, B, "ionn_model_forward")) return rc;
    IONN_REQUIRE(X != nullptr, IONN_ERR_ARG, "ionn_model_forward: X is NULL");
    const Plan p0 = plan(layers, L, B, nullptr);
    IONN_REQUIRE(workspace && aligned(workspace, 256) && workspace_bytes >= p0.total, IONN_ERR_WORKSPACE,
                 "ionn_model_forward: needs a 256-byte aligned workspace of %zu bytes", p0.total);
    const Plan p = plan(layers, L, B, workspace);
    if (small_model(layers, L, B)) {
        SmallModel m = small_args(layers, L, B, X, p);
        m.out = out;
        small_forward_kernel<<<dim3(1), dim3(kSmallThreads), 0, as_stream(stream)>>>(m);
        return check_launch("ionn_model_forward");
    }
    for (int l = 0; l < L; ++l) {
        const ionn_layer &Ly = layers[l];
        const int8_t *a_in = l == 0 ? X : p.act[l - 1];
        const int relu = has_relu(Ly) ? 1 : 0;
        if (is_conv(Ly)) {
            const ionn_conv_desc d = desc_of(Ly, B);
            if (int rc = int_conv_fwd(a_in, Ly.weight, p.z32, &d, nullptr, stream)) return rc;
            if (int rc = ionn_oss_requant(p.z32, Ly.offset, Ly.mult, Ly.k, B * out_hw(Ly), Ly.Cout, relu, p.act[l],
                                          stream))
                return rc;
        } else {
            if (int rc = int_linear_fwd_oss(a_in, Ly.weight, Ly.offset, Ly.mult, Ly.k, relu, p.act[l], B, Ly.Cin,
                                            Ly.Cout, p.z32, p.z_bytes, stream))
                return rc;
        }
    }
    if (out) {
        const size_t bytes = size_t(B * out_size(layers[L - 1]));
        IONN_REQUIRE(hipMemcpyAsync(out, p.act[L - 1], bytes, hipMemcpyDeviceToDevice, as_stream(stream)) ==
                         hipSuccess,
                     IONN_ERR_HIP, "ionn_model_forward: copy of the output failed");
    }
    return IONN_OK;
}

int ionn_model_backward(const ionn_layer *layers, int L, const int8_t *X, int64_t B, const int32_t *labels,
                        const int8_t *tmc, const int8_t *tmw, int tb_delta, int tb_weight, int mu, void *workspace,
                        size_t workspace_bytes, int32_t *shifts_out, void *stream) {
    clear_error();
    if (int rc = check_model(layers, L, B, "ionn_model_backward")) return rc;
    IONN_REQUIRE(X && labels && tmc && tmw, IONN_ERR_ARG, "ionn_model_backward: NULL argument");
    IONN_REQUIRE(tb_delta >= 1 && tb_delta <= 31 && tb_weight >= 1 && tb_weight <= 31 && mu >= 0 && mu <= 31,
                 IONN_ERR_RANGE, "ionn_model_backward: tb_delta %d, tb_weight %d, mu %d", tb_delta, tb_weight, mu);
    IONN_REQUIRE(aligned(shifts_out, 4), IONN_ERR_ALIGN, "ionn_model_backward: shifts_out must be 4-byte aligned");
    const Plan p0 = plan(layers, L, B, nullptr);
    IONN_REQUIRE(workspace && aligned(workspace, 256) && workspace_bytes >= p0.total, IONN_ERR_WORKSPACE,
                 "ionn_model_backward: needs a 256-byte aligned workspace of %zu bytes", p0.total);
    const Plan p = plan(layers, L, B, workspace);
    if (small_model(layers, L, B)) {
        SmallModel m = small_args(layers, L, B, X, p);
        m.labels = labels;
        m.tmc = tmc;
        m.tmw = tmw;
        m.tb_delta = tb_delta;
        m.tb_weight = tb_weight;
        m.mu = mu;
        m.shifts_out = shifts_out;
        small_backward_kernel<<<dim3(1), dim3(kSmallThreads), 0, as_stream(stream)>>>(m);
        return check_launch("ionn_model_backward");
    }
    if (int rc = ionn_fill_u32(p.scal, 3 * L + 1, 0u, stream)) return rc;
    if (shifts_out)
        if (int rc = ionn_fill_u32(reinterpret_cast<uint32_t *>(shifts_out), 5 * L + 1, 0xffffffffu, stream))
            return rc;
    const ionn_layer &Lt = layers[L - 1];
    uint32_t *am_err = p.scal + 3 * L;
    if (int rc = ionn_mse_grad_targets(p.act[L - 1], labels, B, Lt.Cout, tmc, tmw, p.e32, am_err, stream)) return rc;
    int cur = 0;
    if (int rc = niti_quantize(p.e32, B * Lt.Cout, am_err, tb_delta, 0, p.delta[cur], shifts_out, stream)) return rc;
    for (int l = L - 1; l >= 0; --l) {
        const ionn_layer &Ly = layers[l];
        const int8_t *a_in = l == 0 ? X : p.act[l - 1];
        const int8_t *dl = p.delta[cur];
        uint32_t *am_g = p.scal + 3 * l, *am_b = am_g + 1, *am_d = am_g + 2;
        int32_t *sh = shifts_out ? shifts_out + 1 + 5 * l : nullptr;
        const int64_t rows = B * out_hw(Ly);
        // offset gradient and its max
        if (int rc = ionn_bias_grad(dl, rows, Ly.Cout, p.gb, p.bgws, p.bg_bytes, stream)) return rc;
        if (int rc = ionn_absmax_i32(p.gb, Ly.Cout, am_b, stream)) return rc;
        // weight gradient
        if (is_conv(Ly)) {
            const ionn_conv_desc d = desc_of(Ly, B);
            if (int rc = int_conv_wgrad(dl, a_in, p.g32, &d, am_g, p.cws, p.cw_bytes, stream)) return rc;
        } else {
            if (int rc = int_linear_wgrad_ws(dl, a_in, p.g32, B, Ly.Cin, Ly.Cout, am_g, p.lws, p.lw_bytes, stream))
                return rc;
        }
        // propagated delta, with the pre-update weights
        if (l > 0) {
            const bool mask = has_relu(layers[l - 1]);
            const int64_t n_in = B * in_size(Ly);
            if (is_conv(Ly)) {
                const ionn_conv_desc d = desc_of(Ly, B);
                if (int rc = int_conv_dgrad(dl, Ly.weight, p.z32, &d, mask ? nullptr : am_d, stream)) return rc;
                if (mask)
                    if (int rc = ionn_relu_mask_i32(p.z32, a_in, n_in, am_d, stream)) return rc;
            } else {
                if (int rc = int_linear_dgrad(dl, Ly.weight, mask ? a_in : nullptr, p.z32, B, Ly.Cin, Ly.Cout, am_d,
                                              stream))
                    return rc;
            }
            if (int rc = niti_quantize(p.z32, n_in, am_d, tb_delta, 0, p.delta[cur ^ 1], sh, stream)) return rc;
        }
        // updates
        if (int rc = niti_quantize_update(p.g32, weight_size(Ly), am_g, tb_weight, mu, Ly.weight,
                                          sh ? sh + 1 : nullptr, nullptr, stream))
            return rc;
        if (int rc = niti_quantize_update_i32(p.gb, Ly.Cout, am_b, tb_weight, mu, Ly.offset, sh ? sh + 3 : nullptr,
                                              nullptr, stream))
            return rc;
        cur ^= 1;
    }
    return IONN_OK;
}

}  // extern "C"
