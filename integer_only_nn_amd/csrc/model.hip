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
    uint32_t m = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < B * C;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t b = i / C, c = i - b * C;
        const int32_t t = c == int64_t(labels[b]) ? int32_t(tmc[c]) : int32_t(tmw[c]);
        const int32_t v = int32_t(out[i]) - t;
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
    void *bgws, *cws;
    size_t bg_bytes, cw_bytes, z_bytes;
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
    size_t bg = 0, cw = 0;
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
            if (int rc = int_linear_wgrad(dl, a_in, p.g32, B, Ly.Cin, Ly.Cout, am_g, stream)) return rc;
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
