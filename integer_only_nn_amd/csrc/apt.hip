// Adaptive per-layer precision ("Adaptive Precision Training for Resource
// Constrained Devices"): each layer's weights are k-bit signed mantissas m
// with one shared exponent e (the grid step, eps = 2^e, of Equation 2); the
// update W <- W - lr * g of Equation 1 lands on that grid (Equation 3) with
// lr = 2^-lr_shift; Gavg (Equation 4) is sampled on chosen steps and summed
// per layer; between epochs Algorithm 1 moves every layer's k by one bit on
// the mean of its samples and rescales the weights to the new grid.
//
// All layers of a model go through one launch.  The per-layer pointers and
// sizes travel in the kernel arguments; every workgroup belongs to exactly
// one layer and covers kBlockElems of its weights, so a layer of any size
// and a model of many small layers both fill the grid.  The weights, the
// gradient and the per-layer precision state stay on the device, and the
// precision change is decided on the device too, so steps and epochs chain
// on a stream without a host synchronisation.
#include "common.h"

namespace ionn {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 1;                         // 16-byte vectors per thread
constexpr int kBlockElems = kThreads * kVecPerThread * 8;  // 8 int16 per vector
constexpr int kKMinBits = 2, kKMaxBits = 16;
constexpr int64_t kMaxLayerElems = int64_t(1) << 36;    // sum |g| < 2^53 stays exact in a double

struct Table {
    void *W[IONN_MAX_LAYERS];            // int16 mantissas, or int8 for the layers in i8
    const int16_t *G[IONN_MAX_LAYERS];
    int64_t n[IONN_MAX_LAYERS];
    int32_t first[IONN_MAX_LAYERS + 1];  // first workgroup of each layer; first[L] = grid size
    uint64_t vec;                        // bit l: layer l takes the vector path (aligned W and G)
    uint64_t i8;                         // bit l: layer l's W is int8 (k held in [2, 8])
    int32_t L;
};

__device__ __forceinline__ int layer_of(const Table &t, int b) {
    int l = 0;
    while (l + 1 < t.L && b >= t.first[l + 1]) ++l;
    return l;
}

constexpr int kKMaxBits8 = 8;  // int8 storage holds at most 8-bit mantissas

__device__ __forceinline__ int max_bits(const Table &t, int l) { return (t.i8 >> l) & 1 ? kKMaxBits8 : kKMaxBits; }

__device__ __forceinline__ int clamp_bits(int k, int kmax) {
    return k < kKMinBits ? kKMinBits : (k > kmax ? kmax : k);
}

// The change of a weight in grid steps for sigma = e_w + lr_shift - e_g,
// as one formula for both signs of sigma: c = ((g << left) + bias) >> right
// with left = -sigma, right = 0 when sigma < 0 (exact) and left = 0,
// right = sigma, bias = 2^(sigma-1) when sigma > 0 (rhu: floor((g +
// 2^(sigma-1)) / 2^sigma)).  Past a right shift of 20 every int16 g rounds
// to 0, as it does for any larger shift.  Past a left shift of 16, and past
// |c| = 2^17, a nonzero change saturates the weight on the side opposite to
// g whatever its size (|m| <= 2^15), so both are clamped there and every
// step stays in 32-bit arithmetic.
struct Rule {
    int left, right;
    int32_t bias, lo, hi;
};

__device__ __forceinline__ Rule make_rule(int k, int32_t e_w, int32_t e_g, int lr_shift) {
    const int64_t sigma = int64_t(e_w) + lr_shift - int64_t(e_g);
    Rule r;
    r.right = sigma > 0 ? int(sigma > 20 ? 20 : sigma) : 0;
    r.left = sigma < 0 ? int(-sigma > 16 ? 16 : -sigma) : 0;
    r.bias = r.right > 0 ? int32_t(1) << (r.right - 1) : 0;
    r.lo = -(int32_t(1) << (k - 1));
    r.hi = (int32_t(1) << (k - 1)) - 1;
    return r;
}

__device__ __forceinline__ int32_t clamp32(int32_t v, int32_t lo, int32_t hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

__device__ __forceinline__ int32_t apply(const Rule &r, int32_t m, int32_t g) {
    const int32_t c = clamp32((int32_t(uint32_t(g) << r.left) + r.bias) >> r.right, -(1 << 17), 1 << 17);
    return clamp32(m - c, r.lo, r.hi);
}

__device__ __forceinline__ int32_t lo16(uint32_t x) { return int32_t(x << 16) >> 16; }
__device__ __forceinline__ int32_t hi16(uint32_t x) { return int32_t(x) >> 16; }
__device__ __forceinline__ uint32_t pack16(int32_t a, int32_t b) {
    return (uint32_t(a) & 0xffffu) | (uint32_t(b) << 16);
}
__device__ __forceinline__ int32_t iabs(int32_t v) { return v < 0 ? -v : v; }

// Block sum of one int32 per thread (|sum| < 2^31 by the block's size).
__device__ __forceinline__ int32_t block_sum(int32_t v) {
    __shared__ int32_t part[kThreads / 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    return part[0] + part[1] + part[2] + part[3];
}

// One step's update of every layer; with SAMPLE, each workgroup also writes
// the sum of |g| over its weights to part[blockIdx.x].
template <bool SAMPLE>
__global__ __launch_bounds__(kThreads) void update_kernel(Table t, const int32_t *__restrict__ kbits,
                                                          const int32_t *__restrict__ e_w,
                                                          const int32_t *__restrict__ e_g, int lr_shift,
                                                          int64_t *__restrict__ part) {
    const int l = layer_of(t, blockIdx.x);
    const Rule r = make_rule(clamp_bits(kbits[l], max_bits(t, l)), e_w[l], e_g[l], lr_shift);
    const int64_t n = t.n[l];
    const int64_t b0 = int64_t(int(blockIdx.x) - t.first[l]) * kBlockElems;
    int16_t *__restrict__ W = static_cast<int16_t *>(t.W[l]);
    int8_t *__restrict__ W8 = static_cast<int8_t *>(t.W[l]);
    const int16_t *__restrict__ G = t.G[l];
    int32_t asum = 0;
    if ((t.i8 >> l) & 1) {
        // int8 weights: 8 per thread (8 bytes of W, 16 of G)
        const int64_t e = b0 + int64_t(threadIdx.x) * 8;
        if (((t.vec >> l) & 1) && e + 8 <= n) {
            const uint2 w = *reinterpret_cast<const uint2 *>(W8 + e);
            const v4i gv = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(G + e));
            const uint32_t gd[4] = {uint32_t(gv.x), uint32_t(gv.y), uint32_t(gv.z), uint32_t(gv.w)};
            uint32_t o[2] = {0, 0};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t g = j & 1 ? hi16(gd[j >> 1]) : lo16(gd[j >> 1]);
                const int32_t m = int32_t(int8_t(uint8_t((j < 4 ? w.x : w.y) >> (8 * (j & 3)))));
                if (SAMPLE) asum += iabs(g);
                o[j >> 2] |= (uint32_t(apply(r, m, g)) & 0xffu) << (8 * (j & 3));
            }
            *reinterpret_cast<uint2 *>(W8 + e) = make_uint2(o[0], o[1]);
        } else {
            const int64_t end = e + 8 < n ? e + 8 : n;
            for (int64_t j = e; j < end; ++j) {
                const int32_t g = G[j];
                if (SAMPLE) asum += iabs(g);
                W8[j] = int8_t(apply(r, W8[j], g));
            }
        }
    } else if ((t.vec >> l) & 1) {
        v4i wv[kVecPerThread], gv[kVecPerThread];
#pragma unroll
        for (int i = 0; i < kVecPerThread; ++i) {
            const int64_t e = b0 + (int64_t(i) * kThreads + threadIdx.x) * 8;
            if (e + 8 <= n) {
                wv[i] = *reinterpret_cast<const v4i *>(W + e);
                gv[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(G + e));
            }
        }
#pragma unroll
        for (int i = 0; i < kVecPerThread; ++i) {
            const int64_t e = b0 + (int64_t(i) * kThreads + threadIdx.x) * 8;
            if (e + 8 <= n) {
                uint32_t wd[4] = {uint32_t(wv[i].x), uint32_t(wv[i].y), uint32_t(wv[i].z), uint32_t(wv[i].w)};
                const uint32_t gd[4] = {uint32_t(gv[i].x), uint32_t(gv[i].y), uint32_t(gv[i].z),
                                        uint32_t(gv[i].w)};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int32_t g0 = lo16(gd[j]), g1 = hi16(gd[j]);
                    if (SAMPLE) asum += iabs(g0) + iabs(g1);
                    wd[j] = pack16(apply(r, lo16(wd[j]), g0), apply(r, hi16(wd[j]), g1));
                }
                *reinterpret_cast<uint4 *>(W + e) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            } else if (e < n) {  // the layer's ragged tail: fewer than 8 weights
                for (int64_t j = e; j < n; ++j) {
                    const int32_t g = G[j];
                    if (SAMPLE) asum += iabs(g);
                    W[j] = int16_t(apply(r, W[j], g));
                }
            }
        }
    } else {
        const int64_t end = b0 + kBlockElems < n ? b0 + kBlockElems : n;
        for (int64_t j = b0 + threadIdx.x; j < end; j += kThreads) {
            const int32_t g = G[j];
            if (SAMPLE) asum += iabs(g);
            W[j] = int16_t(apply(r, W[j], g));
        }
    }
    if (SAMPLE) {
        const int32_t s = block_sum(asum);
        if (threadIdx.x == 0) part[blockIdx.x] = s;
    }
}

// Gavg of layer blockIdx.x from its workgroups' partial sums, added to the
// epoch's sum: mean(|g|) * 2^(e_g - e_w), the power of two applied one
// factor at a time (exact), then one double addition.  The partials are
// read kFinishUnroll at a time per thread so the loads overlap.
constexpr int kFinishThreads = 512, kFinishUnroll = 8;

__global__ __launch_bounds__(kFinishThreads) void gavg_add_kernel(Table t, const int64_t *__restrict__ part,
                                                                  const int32_t *__restrict__ e_w,
                                                                  const int32_t *__restrict__ e_g,
                                                                  double *gavg_sum, int32_t *gavg_count) {
    __shared__ int64_t red[kFinishThreads / 64];
    const int l = blockIdx.x;
    const int end = t.first[l + 1];
    int64_t s = 0;
    for (int b0 = t.first[l] + int(threadIdx.x); b0 < end; b0 += kFinishThreads * kFinishUnroll) {
        int64_t v[kFinishUnroll];
#pragma unroll
        for (int u = 0; u < kFinishUnroll; ++u) {
            const int b = b0 + u * kFinishThreads;
            v[u] = b < end ? part[b] : 0;
        }
#pragma unroll
        for (int u = 0; u < kFinishUnroll; ++u) s += v[u];
    }
    s = wave_sum_i64(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t tot = 0;
        for (int w = 0; w < kFinishThreads / 64; ++w) tot += red[w];
        double v = double(tot) / double(t.n[l]);
        int e = e_g[l] - e_w[l];
        for (; e > 0; --e) v *= 2.0;
        for (; e < 0; ++e) v *= 0.5;
        gavg_sum[l] = gavg_sum[l] + v;
        gavg_count[l] = gavg_count[l] + 1;
    }
}

// Algorithm 1 for one layer: +1, 0 or -1 from the mean of its samples.
__device__ __forceinline__ int decide(double sum, int32_t count, int k, double t_min, double t_max, int k_min,
                                      int k_max) {
    if (count <= 0) return 0;
    const double mean = sum / double(count);
    if (mean < t_min && k < k_max) return 1;
    if (mean > t_max && k > k_min) return -1;
    return 0;
}

struct Policy {
    double t_min, t_max;
    int k_min, k_max;
};

// The weights of every layer whose precision moves, at the new precision
// with the same range: m -> 2m for one more bit, sat(rhu(m, 1)) for one less.
__global__ __launch_bounds__(kThreads) void rescale_kernel(Table t, const int32_t *__restrict__ kbits,
                                                           const double *__restrict__ gavg_sum,
                                                           const int32_t *__restrict__ gavg_count, Policy p) {
    const int l = layer_of(t, blockIdx.x);
    const int kmax = max_bits(t, l);
    const int k = clamp_bits(kbits[l], kmax);
    const int dk = decide(gavg_sum[l], gavg_count[l], k, p.t_min, p.t_max, p.k_min,
                          p.k_max < kmax ? p.k_max : kmax);
    if (dk == 0) return;
    const int kn = k + dk;
    const int32_t lo = -(int32_t(1) << (kn - 1)), hi = (int32_t(1) << (kn - 1)) - 1;
    auto one = [&](int32_t m) {
        const int32_t v = dk > 0 ? 2 * m : rhu(m, 1);
        return v < lo ? lo : (v > hi ? hi : v);
    };
    const int64_t n = t.n[l];
    const int64_t b0 = int64_t(int(blockIdx.x) - t.first[l]) * kBlockElems;
    int16_t *__restrict__ W = static_cast<int16_t *>(t.W[l]);
    if ((t.i8 >> l) & 1) {
        int8_t *__restrict__ W8 = static_cast<int8_t *>(t.W[l]);
        const int64_t end = b0 + kBlockElems < n ? b0 + kBlockElems : n;
        for (int64_t j = b0 + threadIdx.x; j < end; j += kThreads) W8[j] = int8_t(one(W8[j]));
    } else if ((t.vec >> l) & 1) {
#pragma unroll
        for (int i = 0; i < kVecPerThread; ++i) {
            const int64_t e = b0 + (int64_t(i) * kThreads + threadIdx.x) * 8;
            if (e + 8 <= n) {
                uint4 v = *reinterpret_cast<const uint4 *>(W + e);
                v.x = pack16(one(lo16(v.x)), one(hi16(v.x)));
                v.y = pack16(one(lo16(v.y)), one(hi16(v.y)));
                v.z = pack16(one(lo16(v.z)), one(hi16(v.z)));
                v.w = pack16(one(lo16(v.w)), one(hi16(v.w)));
                *reinterpret_cast<uint4 *>(W + e) = v;
            } else if (e < n) {
                for (int64_t j = e; j < n; ++j) W[j] = int16_t(one(W[j]));
            }
        }
    } else {
        const int64_t end = b0 + kBlockElems < n ? b0 + kBlockElems : n;
        for (int64_t j = b0 + threadIdx.x; j < end; j += kThreads) W[j] = int16_t(one(W[j]));
    }
}

// After the rescale: the same decision moves k and the exponent, reports
// the change, and clears the sums for the next epoch.
__global__ void commit_kernel(int L, uint64_t i8, int32_t *kbits, int32_t *e_w, double *gavg_sum,
                              int32_t *gavg_count, int32_t *dk_out, Policy p) {
    const int l = blockIdx.x * blockDim.x + threadIdx.x;
    if (l >= L) return;
    const int kmax = (i8 >> l) & 1 ? kKMaxBits8 : kKMaxBits;
    const int k = clamp_bits(kbits[l], kmax);
    const int dk = decide(gavg_sum[l], gavg_count[l], k, p.t_min, p.t_max, p.k_min, p.k_max < kmax ? p.k_max : kmax);
    kbits[l] = k + dk;
    e_w[l] = e_w[l] - dk;
    gavg_sum[l] = 0.0;
    gavg_count[l] = 0;
    if (dk_out) dk_out[l] = dk;
}

// Fill the table from host arrays; returns 0 or an IONN_ERR_* code.
int make_table(const char *who, int L, void *const *W, const int32_t *wbytes, const int16_t *const *G,
               const int64_t *n, Table &t) {
    IONN_REQUIRE(L >= 1 && L <= IONN_MAX_LAYERS, IONN_ERR_SHAPE, "%s: L = %d outside [1, %d]", who, L,
                 IONN_MAX_LAYERS);
    IONN_REQUIRE(W && n, IONN_ERR_ARG, "%s: NULL layer array", who);
    memset(&t, 0, sizeof(t));
    t.L = L;
    int64_t blocks = 0;
    for (int l = 0; l < L; ++l) {
        IONN_REQUIRE(n[l] >= 1 && n[l] <= kMaxLayerElems, IONN_ERR_SHAPE, "%s: layer %d has n = %lld", who, l,
                     (long long)n[l]);
        IONN_REQUIRE(W[l] != nullptr && (G == nullptr || G[l] != nullptr), IONN_ERR_ARG,
                     "%s: layer %d has a NULL tensor", who, l);
        const int wb = wbytes ? wbytes[l] : 2;
        IONN_REQUIRE(wb == 1 || wb == 2, IONN_ERR_ARG, "%s: layer %d has %d bytes per weight (1 or 2)", who, l,
                     wb);
        IONN_REQUIRE(aligned(W[l], size_t(wb)) && (G == nullptr || aligned(G[l], 2)), IONN_ERR_ALIGN,
                     "%s: layer %d tensors must be aligned to their element size", who, l);
        t.W[l] = W[l];
        if (wb == 1) t.i8 |= uint64_t(1) << l;
        t.G[l] = G ? G[l] : nullptr;
        t.n[l] = n[l];
        t.first[l] = int32_t(blocks);
        blocks += (n[l] + kBlockElems - 1) / kBlockElems;
        IONN_REQUIRE(blocks <= 0x7fffffff, IONN_ERR_SHAPE, "%s: too many weights", who);
        if (aligned(W[l], wb == 1 ? 8 : 16) && (G == nullptr || aligned(G[l], 16))) t.vec |= uint64_t(1) << l;
    }
    t.first[L] = int32_t(blocks);
    return IONN_OK;
}

}  // namespace
}  // namespace ionn

using namespace ionn;

extern "C" {

size_t apt_workspace_bytes(int L, const int64_t *n) {
    if (L < 1 || L > IONN_MAX_LAYERS || n == nullptr) return 0;
    int64_t blocks = 0;
    for (int l = 0; l < L; ++l) {
        if (n[l] < 1 || n[l] > kMaxLayerElems) return 0;
        blocks += (n[l] + kBlockElems - 1) / kBlockElems;
    }
    return size_t(blocks) * sizeof(int64_t);
}

int apt_update_mixed(int L, void *const *W, const int32_t *wbytes, const int16_t *const *G, const int64_t *n,
                     const int32_t *k, const int32_t *e_w, const int32_t *e_g, int lr_shift, double *gavg_sum,
                     int32_t *gavg_count, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    IONN_REQUIRE(G != nullptr, IONN_ERR_ARG, "apt_update: NULL gradient array");
    Table t;
    if (int rc = make_table("apt_update", L, W, wbytes, G, n, t)) return rc;
    IONN_REQUIRE(k && e_w && e_g, IONN_ERR_ARG, "apt_update: NULL k / e_w / e_g");
    IONN_REQUIRE(aligned(k, 4) && aligned(e_w, 4) && aligned(e_g, 4), IONN_ERR_ALIGN,
                 "apt_update: k / e_w / e_g must be 4-byte aligned");
    IONN_REQUIRE(lr_shift >= 0 && lr_shift <= 62, IONN_ERR_RANGE, "apt_update: lr_shift = %d outside [0, 62]",
                 lr_shift);
    IONN_REQUIRE((gavg_sum == nullptr) == (gavg_count == nullptr), IONN_ERR_ARG,
                 "apt_update: gavg_sum and gavg_count must both be given or both be NULL");
    hipStream_t st = as_stream(stream);
    const dim3 grid(unsigned(t.first[L])), block(kThreads);
    if (gavg_sum == nullptr) {
        update_kernel<false><<<grid, block, 0, st>>>(t, k, e_w, e_g, lr_shift, nullptr);
        return check_launch("apt_update");
    }
    IONN_REQUIRE(aligned(gavg_sum, 8) && aligned(gavg_count, 4), IONN_ERR_ALIGN,
                 "apt_update: gavg_sum must be 8-byte and gavg_count 4-byte aligned");
    const size_t need = size_t(t.first[L]) * sizeof(int64_t);
    IONN_REQUIRE(workspace != nullptr && aligned(workspace, 8) && workspace_bytes >= need, IONN_ERR_WORKSPACE,
                 "apt_update: sampling needs an 8-byte aligned workspace of %zu bytes", need);
    int64_t *part = static_cast<int64_t *>(workspace);
    update_kernel<true><<<grid, block, 0, st>>>(t, k, e_w, e_g, lr_shift, part);
    if (int rc = check_launch("apt_update")) return rc;
    gavg_add_kernel<<<dim3(unsigned(L)), dim3(kFinishThreads), 0, st>>>(t, part, e_w, e_g, gavg_sum, gavg_count);
    return check_launch("apt_update");
}

int apt_update(int L, int16_t *const *W, const int16_t *const *G, const int64_t *n, const int32_t *k,
               const int32_t *e_w, const int32_t *e_g, int lr_shift, double *gavg_sum, int32_t *gavg_count,
               void *workspace, size_t workspace_bytes, void *stream) {
    return apt_update_mixed(L, reinterpret_cast<void *const *>(W), nullptr, G, n, k, e_w, e_g, lr_shift, gavg_sum,
                            gavg_count, workspace, workspace_bytes, stream);
}

int apt_adjust_mixed(int L, void *const *W, const int32_t *wbytes, const int64_t *n, int32_t *k, int32_t *e_w,
                     double *gavg_sum, int32_t *gavg_count, double t_min, double t_max, int k_min, int k_max,
                     int32_t *dk_out, void *stream) {
    clear_error();
    Table t;
    if (int rc = make_table("apt_adjust", L, W, wbytes, nullptr, n, t)) return rc;
    IONN_REQUIRE(k && e_w && gavg_sum && gavg_count, IONN_ERR_ARG, "apt_adjust: NULL state array");
    IONN_REQUIRE(aligned(k, 4) && aligned(e_w, 4) && aligned(gavg_sum, 8) && aligned(gavg_count, 4) &&
                     aligned(dk_out, 4),
                 IONN_ERR_ALIGN, "apt_adjust: misaligned state array");
    IONN_REQUIRE(k_min >= kKMinBits && k_max <= kKMaxBits && k_min <= k_max, IONN_ERR_RANGE,
                 "apt_adjust: need %d <= k_min <= k_max <= %d (got %d, %d)", kKMinBits, kKMaxBits, k_min, k_max);
    IONN_REQUIRE(t_min == t_min && t_max == t_max && t_min <= t_max, IONN_ERR_RANGE,
                 "apt_adjust: need t_min <= t_max, neither NaN");
    const Policy p{t_min, t_max, k_min, k_max};
    hipStream_t st = as_stream(stream);
    rescale_kernel<<<dim3(unsigned(t.first[L])), dim3(kThreads), 0, st>>>(t, k, gavg_sum, gavg_count, p);
    if (int rc = check_launch("apt_adjust")) return rc;
    commit_kernel<<<dim3(1), dim3(64), 0, st>>>(L, t.i8, k, e_w, gavg_sum, gavg_count, dk_out, p);
    return check_launch("apt_adjust");
}

int apt_adjust(int L, int16_t *const *W, const int64_t *n, int32_t *k, int32_t *e_w, double *gavg_sum,
               int32_t *gavg_count, double t_min, double t_max, int k_min, int k_max, int32_t *dk_out,
               void *stream) {
    return apt_adjust_mixed(L, reinterpret_cast<void *const *>(W), nullptr, n, k, e_w, gavg_sum, gavg_count, t_min,
                            t_max, k_min, k_max, dk_out, stream);
}

}  // extern "C"
