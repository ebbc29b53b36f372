// Matrix-core mainloop shared by the int8 Linear GEMMs and the implicit-GEMM
// 3x3 convolutions (gfx950, v_mfma_i32_16x16x64_i8).
//
// C[m][n] = sum_k A(m,k) * B(k,n), int32 accumulation modulo 2^32.
//
// Operands are produced by loader policies that move one BM x BK (or BN x BK)
// tile from HBM into registers and then into LDS in a single K-major layout
// ([row][BK + kPad] bytes).  Two families exist:
//   * K-major loaders fetch 16-byte chunks (16 consecutive k of one row);
//   * M-major loaders fetch 4-byte words (4 consecutive rows at one k) for
//     16 consecutive k and transpose the 16x4 byte block in registers, so an
//     operand whose contraction index is its outer dimension (dgrad's W,
//     wgrad's dY and X) lands in LDS in the same K-major layout.
// Loader policies differ only in where element (row, k) lives: a plain
// matrix, or an im2col gather of an NHWC image for the convolutions.
//
// Every wavefront owns a (BM/WGM) x (BN/WGN) sub-tile of 16x16 blocks.  The
// B fragment is passed as the MFMA's first operand, so the 16x16 result has
// n along its rows: each lane holds C[m][n..n+3] (m = lane % 16) and stores
// 16 contiguous bytes.
#pragma once

#include "common.h"

namespace ionn {
namespace gemm {

constexpr int kPad = 16;  // LDS row padding: conflict-free ds_read_b128 fragment reads

// r[i] = bytes (k = i, col 0..3) -> o[j] = bytes (k = 0..3, col j).  Plain
// shifts and masks; the compiler emits v_perm_b32.
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             uint32_t &o0, uint32_t &o1, uint32_t &o2,
                                             uint32_t &o3) {
    o0 = (r0 & 0xffu) | ((r1 & 0xffu) << 8) | ((r2 & 0xffu) << 16) | (r3 << 24);
    o1 = ((r0 >> 8) & 0xffu) | (r1 & 0xff00u) | ((r2 & 0xff00u) << 8) | ((r3 & 0xff00u) << 16);
    o2 = ((r0 >> 16) & 0xffu) | ((r1 >> 8) & 0xff00u) | (r2 & 0xff0000u) | ((r3 & 0xff0000u) << 8);
    o3 = (r0 >> 24) | ((r1 >> 16) & 0xff00u) | ((r2 >> 8) & 0xff0000u) | (r3 & 0xff000000u);
}

__device__ __forceinline__ uint32_t ldbyte(const int8_t *p) { return uint32_t(uint8_t(*p)); }

// ---------------------------------------------------------------------------
// Operand sources.  Each provides, for a tile whose rows start at r0:
//   K-major:  v4i chunk(row r, k)  -> bytes k..k+15 of row r (0 outside)
//   M-major:  uint32 word(k, row r) -> rows r..r+3 at k (0 outside)
// `rows` / `kdim` are the logical extents; `vec` says whole-chunk loads are
// aligned and allowed.
// ---------------------------------------------------------------------------

// Plain matrix, element (r, k) at base[r * ld + k].
struct SrcRowK {
    const int8_t *base;
    int64_t ld;
    int rows, kdim;
    bool vec;
    template <bool EDGE>
    __device__ __forceinline__ v4i chunk(int r, int k) const {
        const int8_t *p = base + int64_t(r) * ld + k;
        if (!EDGE || (r < rows && k + 16 <= kdim && vec)) return *reinterpret_cast<const v4i *>(p);
        uint32_t w[4] = {0, 0, 0, 0};
        if (r < rows)
            for (int b = 0; b < 16; ++b)
                if (k + b < kdim) w[b >> 2] |= ldbyte(p + b) << (8 * (b & 3));
        return v4i{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
    }
};

// Plain matrix, element (r, k) at base[k * ld + r].
struct SrcColK {
    const int8_t *base;
    int64_t ld;
    int rows, kdim;
    bool vec;
    template <bool EDGE>
    __device__ __forceinline__ uint32_t word(int k, int r) const {
        const int8_t *p = base + int64_t(k) * ld + r;
        if (!EDGE || (k < kdim && r + 4 <= rows && vec)) return *reinterpret_cast<const uint32_t *>(p);
        uint32_t x = 0;
        if (k < kdim)
            for (int b = 0; b < 4; ++b)
                if (r + b < rows) x |= ldbyte(p + b) << (8 * b);
        return x;
    }
};

// NHWC image seen as an im2col matrix for a 3x3, stride-1, pad-1 convolution.
// Row r = output pixel (n, h, w); k = tap * C + c with tap = 3 * kh + kw.
// The pixel read is (h + s*(kh - 1), w + s*(kw - 1)), s = +1 for the forward
// product and -1 for delta propagation.  C is a multiple of 16, so a 16-byte
// chunk never straddles two taps.
struct SrcIm2colK {
    const int8_t *img;
    int npix, H, W, C, sign;
    template <bool EDGE>
    __device__ __forceinline__ v4i chunk(int r, int k) const {
        v4i v = {0, 0, 0, 0};
        if (r >= npix || k >= 9 * C) return v;
        const int tap = k / C, c = k - tap * C;
        const int kh = tap / 3, kw = tap - 3 * kh;
        const int hw = H * W;
        const int n = r / hw, rem = r - n * hw;
        const int h = rem / W, w = rem - h * W;
        const int hh = h + sign * (kh - 1), ww = w + sign * (kw - 1);
        if (hh < 0 || hh >= H || ww < 0 || ww >= W) return v;
        return *reinterpret_cast<const v4i *>(img + ((int64_t(n) * H + hh) * W + ww) * C + c);
    }
};

// The weight gradient's second operand: row r = tap * C + c, k = pixel
// (n, h, w); element = img[n, h + kh - 1, w + kw - 1, c] (zero outside).
struct SrcIm2colM {
    const int8_t *img;
    int npix, H, W, C;
    template <bool EDGE>
    __device__ __forceinline__ uint32_t word(int k, int r) const {
        if (k >= npix || r >= 9 * C) return 0;
        const int tap = r / C, c = r - tap * C;
        const int kh = tap / 3, kw = tap - 3 * kh;
        const int hw = H * W;
        const int n = k / hw, rem = k - n * hw;
        const int h = rem / W, w = rem - h * W;
        const int hh = h + kh - 1, ww = w + kw - 1;
        if (hh < 0 || hh >= H || ww < 0 || ww >= W) return 0;
        return *reinterpret_cast<const uint32_t *>(img + ((int64_t(n) * H + hh) * W + ww) * C + c);
    }
};

// Conv weights W[Cout][3][3][Cin] seen as delta propagation's second operand:
// row r = ci, k = tap * Cout + co; element = W[co][tap][ci].
struct SrcConvWT {
    const int8_t *w;
    int Cin, Cout;
    template <bool EDGE>
    __device__ __forceinline__ uint32_t word(int k, int r) const {
        if (k >= 9 * Cout || r >= Cin) return 0;
        const int tap = k / Cout, co = k - tap * Cout;
        return *reinterpret_cast<const uint32_t *>(w + (int64_t(co) * 9 + tap) * Cin + r);
    }
};

template <class S> struct is_kmajor { static constexpr bool value = false; };
template <> struct is_kmajor<SrcRowK> { static constexpr bool value = true; };
template <> struct is_kmajor<SrcIm2colK> { static constexpr bool value = true; };

// ---------------------------------------------------------------------------
// Tile loader: registers <- HBM, then LDS <- registers.
// ---------------------------------------------------------------------------
template <class Src, int R, int BK, int NT, bool EDGE, bool KMAJOR = is_kmajor<Src>::value>
struct Loader;

template <class Src, int R, int BK, int NT, bool EDGE>
struct Loader<Src, R, BK, NT, EDGE, true> {
    static constexpr int kChunks = R * BK / 16;
    static constexpr int kPer = (kChunks + NT - 1) / NT;
    v4i reg[kPer];
    __device__ __forceinline__ void load(const Src &s, int r0, int k0, int tid) {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int id = it * NT + tid;
            v4i v = {0, 0, 0, 0};
            if (kChunks % NT == 0 || id < kChunks) {
                const int r = id / (BK / 16), c = id % (BK / 16);
                v = s.template chunk<EDGE>(r0 + r, k0 + 16 * c);
            }
            reg[it] = v;
        }
    }
    __device__ __forceinline__ void store(int8_t *lds, int tid) const {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int id = it * NT + tid;
            if (kChunks % NT == 0 || id < kChunks) {
                const int r = id / (BK / 16), c = id % (BK / 16);
                *reinterpret_cast<v4i *>(lds + r * (BK + kPad) + 16 * c) = reg[it];
            }
        }
    }
};

template <class Src, int R, int BK, int NT, bool EDGE>
struct Loader<Src, R, BK, NT, EDGE, false> {
    static constexpr int kUnits = (BK / 16) * (R / 4);
    static constexpr int kPer = (kUnits + NT - 1) / NT;
    v4i reg[4 * kPer];
    __device__ __forceinline__ void load(const Src &s, int r0, int k0, int tid) {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int u = it * NT + tid;
            const bool live = kUnits % NT == 0 || u < kUnits;
            const int kq = u / (R / 4), rq = u % (R / 4);
            uint32_t d[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                d[i] = live ? s.template word<EDGE>(k0 + 16 * kq + i, r0 + 4 * rq) : 0u;
            uint32_t o[4][4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                transpose4x4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3], o[0][q], o[1][q],
                             o[2][q], o[3][q]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                reg[4 * it + j] = v4i{int(o[j][0]), int(o[j][1]), int(o[j][2]), int(o[j][3])};
        }
    }
    __device__ __forceinline__ void store(int8_t *lds, int tid) const {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int u = it * NT + tid;
            if (kUnits % NT == 0 || u < kUnits) {
                const int kq = u / (R / 4), rq = u % (R / 4);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<v4i *>(lds + (4 * rq + j) * (BK + kPad) + 16 * kq) =
                        reg[4 * it + j];
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Epilogue.
// ---------------------------------------------------------------------------
struct Epi {
    int32_t *C;
    int64_t ldc;
    int M, N;
    bool vec;            // 16-byte stores allowed
    const int8_t *act;   // ReLU-mask source with C's layout (nullable)
    uint32_t *absmax;    // max-combined (nullable)
    bool atomic;         // split-K: atomicAdd into C (absmax handled separately)
    // static OSS epilogue (256x256 path only): int8 out8[m][n] =
    // oss_elem(C[m][n], oss_off[n], oss_mult[n], oss_k[n], oss_lo); C is not written
    int8_t *out8;
    const int32_t *oss_off, *oss_mult;
    const int8_t *oss_k;
    int oss_lo;
};

// Tile index remap: workgroups that are resident on one XCD at the same time
// (ids congruent mod 8) get a contiguous, M-grouped block of tiles so they
// share operand rows/columns in that XCD's L2.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int ntiles = tiles_m * tiles_n;
    if (ntiles % 8 == 0) pid = (pid % 8) * (ntiles / 8) + pid / 8;
    constexpr int GROUP_M = 4;
    const int group = pid / (GROUP_M * tiles_n);
    const int first_m = group * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int local = pid % (GROUP_M * tiles_n);
    tm = first_m + local % gsize;
    tn = local / gsize;
}

template <int BM, int BN, int BK, int WGM, int WGN>
struct Shape {
    static constexpr int NT = WGM * WGN * 64;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int LDS_A = BM * (BK + kPad), LDS_B = BN * (BK + kPad);
    static constexpr int LDS_BYTES = 2 * (LDS_A + LDS_B);
    static_assert(BK % 64 == 0, "BK must be a multiple of the MFMA depth 64");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wavefront tile must be 16-aligned");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// The mainloop.  k_begin/k_end: the K range of this workgroup (split-K).
template <int BM, int BN, int BK, int WGM, int WGN, bool EDGE, class SA, class SB>
__device__ __forceinline__ void mainloop(const SA &sa, const SB &sb, const Epi &ep, int m0, int n0,
                                         int k_begin, int k_end, int8_t *lds) {
    using S = Shape<BM, BN, BK, WGM, WGN>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    Loader<SA, BM, BK, S::NT, EDGE> la;
    Loader<SB, BN, BK, S::NT, EDGE> lb;

    v4i acc[S::FM][S::FN];
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int j = 0; j < S::FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int nk = (k_end - k_begin + BK - 1) / BK;
    if (nk > 0) {
        la.load(sa, m0, k_begin, tid);
        lb.load(sb, n0, k_begin, tid);
        la.store(lds, tid);
        lb.store(lds + S::LDS_A, tid);
    }
    __syncthreads();

    const int frow = lane & 15, fk = (lane >> 4) * 16;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const int8_t *As = lds + cur * (S::LDS_A + S::LDS_B);
        const int8_t *Bs = As + S::LDS_A;
        if (kt + 1 < nk) {
            la.load(sa, m0, k_begin + (kt + 1) * BK, tid);
            lb.load(sb, n0, k_begin + (kt + 1) * BK, tid);
        }
#pragma unroll
        for (int ks = 0; ks < BK; ks += 64) {
            v4i af[S::FM];
#pragma unroll
            for (int i = 0; i < S::FM; ++i)
                af[i] = *reinterpret_cast<const v4i *>(
                    As + (wm * S::WTM + i * 16 + frow) * (BK + kPad) + ks + fk);
#pragma unroll
            for (int j = 0; j < S::FN; ++j) {
                const v4i bf = *reinterpret_cast<const v4i *>(
                    Bs + (wn * S::WTN + j * 16 + frow) * (BK + kPad) + ks + fk);
#pragma unroll
                for (int i = 0; i < S::FM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf, af[i], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) {
            int8_t *An = lds + (cur ^ 1) * (S::LDS_A + S::LDS_B);
            la.store(An, tid);
            lb.store(An + S::LDS_A, tid);
        }
        __syncthreads();
    }

    // Epilogue: lane holds C[m][n .. n+3], m = .. + lane % 16.
    uint32_t amax = 0;
    const int em = lane & 15, en = (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < S::FM; ++i) {
        const int m = m0 + wm * S::WTM + i * 16 + em;
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            const int n = n0 + wn * S::WTN + j * 16 + en;
            v4i v = acc[i][j];
            const bool full = !EDGE || (m < ep.M && n + 4 <= ep.N && ep.vec);
            int32_t *cp = ep.C + int64_t(m) * ep.ldc + n;
            if (ep.act) {
                const int8_t *ap = ep.act + int64_t(m) * ep.ldc + n;
                if (full) {
                    const uint32_t a = *reinterpret_cast<const uint32_t *>(ap);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (int8_t(uint8_t(a >> (8 * c))) <= 0) v[c] = 0;
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (m < ep.M && n + c < ep.N && ap[c] <= 0) v[c] = 0;
                }
            }
            if (ep.atomic) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (!EDGE || (m < ep.M && n + c < ep.N)) atomicAdd(cp + c, v[c]);
            } else if (full) {
                *reinterpret_cast<v4i *>(cp) = v;
#pragma unroll
                for (int c = 0; c < 4; ++c) amax = max(amax, abs_u32(v[c]));
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (m < ep.M && n + c < ep.N) {
                        cp[c] = v[c];
                        amax = max(amax, abs_u32(v[c]));
                    }
            }
        }
    }
    if (ep.absmax && !ep.atomic) {
        amax = wave_max_u32(amax);
        if (lane == 0) publish_max_u32(ep.absmax, amax);
    }
}

// Grid: one workgroup per (tile, K-split).  blockIdx.x = tile, blockIdx.y = split.
template <int BM, int BN, int BK, int WGM, int WGN, bool EDGE, class SA, class SB>
__global__ __launch_bounds__(WGM *WGN * 64) void gemm_kernel(SA sa, SB sb, Epi ep, int M, int N,
                                                             int K, int k_split) {
    using S = Shape<BM, BN, BK, WGM, WGN>;
    __shared__ __attribute__((aligned(16))) int8_t lds[S::LDS_BYTES];
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int kb = int((int64_t(K) * blockIdx.y / k_split) / BK * BK);
    const int ke = blockIdx.y + 1 == unsigned(k_split) ? K
                                                      : int((int64_t(K) * (blockIdx.y + 1) / k_split) / BK * BK);
    mainloop<BM, BN, BK, WGM, WGN, EDGE>(sa, sb, ep, tm * BM, tn * BN, kb, ke, lds);
}

template <int BM, int BN, int BK, int WGM, int WGN, bool EDGE, class SA, class SB>
void launch(const SA &sa, const SB &sb, const Epi &ep, int M, int N, int K, int k_split,
            hipStream_t st) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_kernel<BM, BN, BK, WGM, WGN, EDGE, SA, SB>
        <<<dim3(tiles, k_split), dim3(WGM * WGN * 64), 0, st>>>(sa, sb, ep, M, N, K, k_split);
}

}  // namespace gemm
}  // namespace ionn
