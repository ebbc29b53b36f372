// Weight gradient of a small layer over a long reduction: G[M][N] = sum over
// k of A[k][m] * B[k][n] for row-major int8 operands A [K][M] and B [K][N]
// (a Linear layer's dY and X over the batch: "Integer On-Device Training:
// Overview", section 4), when G has at most 32 blocks of 32 x 32 and the
// reduction is long.  The batch-major layout puts the reduction on the row
// index of both operands, so a workgroup copies whole rows of a range of k
// into LDS (coalesced along a row; any row length, padded LDS pitches) and
// the matrix cores contract 32-row K steps read back transposed
// (ds_read_b64_tr_b8).  Each workgroup reduces one range of k and adds its
// partial G into the zeroed G with integer atomics (exact in any order).
// Operands: contiguous rows (pitch M and N), 4-byte aligned bases.
#pragma once

#include "common.h"

namespace ionn {
namespace wl {

constexpr int NT = 256;     // four wavefronts
constexpr int R = 64;       // rows of k per LDS stage (two 32-row K steps)
constexpr int MAXB = 8;     // blocks of 32 per side of G
constexpr int MAXBLK = 32;  // blocks of G in all (8 per wavefront)
constexpr int PMAX = 32 * MAXB + 16;

typedef int v2i __attribute__((ext_vector_type(2)));

struct Args {
    const int8_t *a, *b;  // A [K][M], B [K][N], both with contiguous rows
    int64_t K, rows;      // reduction length; rows of k per workgroup (a multiple of R)
    int M, N, mb, nb;     // G is M x N, mb x nb blocks of 32
    int pa, pb;           // LDS pitches (multiples of 16)
    int32_t *G;           // atomics into the zeroed G, or (part != nullptr)
    int32_t *part;        // the workgroup's partial G: part[w][M][N], or blocked
    int blk;              // partials blocked: part[w][block][lane][16] (see wgrad_long_blocked)
};

// One stage of a row-major operand [K][C] with contiguous rows (pitch C):
// rows k0 .. k0 + R - 1 form one block of R C bytes starting at a multiple
// of 4 (k0 is a multiple of R = 64 and the base is 4-byte aligned), read as
// dwords into registers (thread t holds dwords t, t + NT, ...) and then
// spread over the stage's rows in LDS (pitch P); bytes of rows at or past
// kend read as 0.  ND: dwords per thread for the widest rows (R * 256 / 4 / NT).
template <int ND>
struct Stage {
    uint32_t w[ND];
    __device__ __forceinline__ void load(const int8_t *base, int C, int64_t k0, int64_t kend) {
        const int nd = R * C / 4;                           // dwords of the stage
        const int64_t valid = (kend - k0 < R ? kend - k0 : R) * int64_t(C);  // bytes
        const uint32_t *p = reinterpret_cast<const uint32_t *>(base + k0 * C);
#pragma unroll
        for (int j = 0; j < ND; ++j) {
            const int q = int(threadIdx.x) + j * NT;
            uint32_t v = 0;
            if (q < nd) {
                if (4 * int64_t(q) + 3 < valid) {
                    v = p[q];
                } else {  // the stage's last valid dword may end the tensor: byte loads
                    for (int e = 0; e < 4; ++e)
                        if (4 * int64_t(q) + e < valid) v |= uint32_t(uint8_t(base[k0 * C + 4 * q + e])) << (8 * e);
                }
            }
            w[j] = v;
        }
    }
    // VEC (C a multiple of 4): a dword never straddles two rows.  Byte f of
    // the block is row f / C, column f % C; dword t + j NT starts at byte
    // 4 t + 4 NT j, so the row and column advance by a fixed step per j.
    template <bool VEC>
    __device__ __forceinline__ void store(int C, int8_t *st, int P) const {
        const int nd = R * C / 4;
        int r = 4 * int(threadIdx.x) / C, c = 4 * int(threadIdx.x) - r * C;
        const int dr = 4 * NT / C, dc = 4 * NT - dr * C;
#pragma unroll
        for (int j = 0; j < ND; ++j) {
            const int q = int(threadIdx.x) + j * NT;
            if (q < nd) {
                if (VEC) {
                    *reinterpret_cast<uint32_t *>(st + r * P + c) = w[j];
                } else {  // C >= 2: a dword spans at most two rows
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int cc = c + e, wrap = cc >= C;
                        st[(r + wrap) * P + cc - wrap * C] = int8_t(uint8_t(w[j] >> (8 * e)));
                    }
                }
            }
            r += dr;
            c += dc;
            if (c >= C) {
                c -= C;
                ++r;
            }
        }
    }
};

// Matrix-core operand of rows (of G) rb0 .. rb0 + 31 and k = k0 + 16 (lane / 32)
// .. + 15 from a stage laid out [k][row] with pitch P: two transposing reads,
// each giving a lane 8 consecutive k of its row.
__device__ __forceinline__ v4i frag_t(const int8_t *st, int P, int rb0, int k0, int lane) {
    typedef __attribute__((address_space(3))) v2i lds_v2i_t;
    const int g = lane >> 4, i = lane & 15;
    const int8_t *p = st + (k0 + 16 * (g >> 1) + (i >> 1)) * P + rb0 + 16 * (g & 1) + 8 * (i & 1);
    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p));
    const v2i y = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p + 8 * P));
    return v4i{x.x, x.y, y.x, y.y};
}

// Workgroup w reduces k in [w rows, (w + 1) rows); wavefront v owns blocks
// q = v, v + 4, ... (q = bm * nb + bn) of G.  Two LDS buffers: the next
// stage's dwords are in flight while the current stage is contracted.
template <bool VA, bool VB>
__global__ __launch_bounds__(NT) void wgrad_long_kernel(Args g) {
    __shared__ __attribute__((aligned(16))) int8_t lds[2][2 * R * PMAX];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int nblk = g.mb * g.nb;
    v16i acc[MAXBLK / 4];
#pragma unroll
    for (int i = 0; i < MAXBLK / 4; ++i) acc[i] = v16i{};
    const int64_t k0 = int64_t(blockIdx.x) * g.rows;
    const int64_t k1 = k0 + g.rows < g.K ? k0 + g.rows : g.K;
    constexpr int ND = R * 32 * MAXB / 4 / NT;
    Stage<ND> ra, rb;
    ra.load(g.a, g.M, k0, k1);
    rb.load(g.b, g.N, k0, k1);
    int buf = 0;
    for (int64_t s = k0; s < k1; s += R) {
        int8_t *sta = lds[buf], *stb = lds[buf] + R * g.pa;
        ra.template store<VA>(g.M, sta, g.pa);
        rb.template store<VB>(g.N, stb, g.pb);
        __syncthreads();
        if (s + R < k1) {
            ra.load(g.a, g.M, s + R, k1);
            rb.load(g.b, g.N, s + R, k1);
        }
#pragma unroll
        for (int ks = 0; ks < R; ks += 32) {
#pragma unroll
            for (int i = 0; i < MAXBLK / 4; ++i) {
                const int q = wave + 4 * i;
                if (q < nblk) {
                    const int bm = q / g.nb, bn = q - bm * g.nb;
                    const v4i fa = frag_t(sta, g.pa, 32 * bm, ks, lane);
                    const v4i fb = frag_t(stb, g.pb, 32 * bn, ks, lane);
                    acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb, fa, acc[i], 0, 0, 0);
                }
            }
        }
        buf ^= 1;
    }
    // lane holds G[m][n .. n + 3] for m = 32 bm + lane % 32 and
    // n = 32 bn + 8 (v / 4) + 4 (lane / 32)
    if (g.part && g.blk) {
        // the accumulators as they lie: block q's 16 values of each lane at
        // part[w][q][lane], 64 contiguous bytes a lane (values outside G
        // included; the sum pass drops them)
#pragma unroll
        for (int i = 0; i < MAXBLK / 4; ++i) {
            const int q = wave + 4 * i;
            if (q < nblk) {
                v4i *dst = reinterpret_cast<v4i *>(g.part + ((int64_t(blockIdx.x) * nblk + q) * 64 + lane) * 16);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    dst[c] = v4i{acc[i][4 * c], acc[i][4 * c + 1], acc[i][4 * c + 2], acc[i][4 * c + 3]};
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < MAXBLK / 4; ++i) {
        const int q = wave + 4 * i;
        if (q < nblk) {
            const int bm = q / g.nb, bn = q - bm * g.nb;
            const int m = 32 * bm + (lane & 31);
            if (m < g.M) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int n = 32 * bn + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    if (n >= g.N) continue;
                    if (g.part)
                        g.part[(int64_t(blockIdx.x) * g.M + m) * g.N + n] = acc[i][v];
                    else if (acc[i][v] != 0)
                        atomicAdd(g.G + int64_t(m) * g.N + n, acc[i][v]);
                }
            }
        }
    }
}

// G[i] = sum over the nw workgroup partials part[w][i] (modulo 2^32), with
// max |G| max-combined into *absmax (nullable).  A workgroup step takes
// E = 4 (256 / SL) consecutive i: thread (slice z, group q) adds
// part[w][i .. i + 3] for i = i0 + 4 q and w = z, z + SL, ... (eight loads
// in flight), and the SL slices meet in LDS.  More slices suit fewer
// outputs over more partials (sum_partials picks SL).
// BLK: the partial rows are blocked (see wgrad_long_kernel): element j is
// block j / 1024 (bm, bn of nb blocks a row), lane (j / 16) % 64, value
// j % 16, i.e. G[32 bm + lane % 32][32 bn + 8 (v / 4) + 4 (lane / 32) + v % 4]
// when inside the M x N of G, else dropped.
template <int SL, bool BLK = false>
__global__ __launch_bounds__(256) void wgrad_long_sum(const int32_t *__restrict__ part, int nw, int64_t n,
                                                      int32_t *__restrict__ G, uint32_t *__restrict__ absmax,
                                                      int nb = 0, int M = 0, int N = 0) {
    static_assert(SL == 16 || SL == 64, "16 or 64 slices");
    constexpr int GR = 256 / SL, E = 4 * GR;
    typedef unsigned v4u __attribute__((ext_vector_type(4)));  // sums wrap modulo 2^32
    __shared__ uint32_t red[SL][E];
    const int q = threadIdx.x % GR, z = threadIdx.x / GR;
    // whole 16-byte groups when every partial row starts 16-byte aligned
    const bool vec = (n & 3) == 0 && (reinterpret_cast<uintptr_t>(part) & 15) == 0;
    uint32_t amax = 0;
    for (int64_t i0 = int64_t(blockIdx.x) * E; i0 < n; i0 += int64_t(gridDim.x) * E) {
        const int64_t i = i0 + 4 * q;
        uint32_t t[4] = {0, 0, 0, 0};
        int w = z;
        if (vec && i0 + E <= n) {
            v4u tv = {0, 0, 0, 0};
            for (; w + SL * 7 < nw; w += SL * 8) {
                v4u x[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const v4u *>(part + int64_t(w + SL * u) * n + i);
#pragma unroll
                for (int u = 0; u < 8; ++u) tv += x[u];
            }
            for (; w < nw; w += SL) tv += *reinterpret_cast<const v4u *>(part + int64_t(w) * n + i);
            t[0] = tv.x;
            t[1] = tv.y;
            t[2] = tv.z;
            t[3] = tv.w;
            w = nw;
        }
        for (; w + SL * 7 < nw; w += SL * 8) {
            uint32_t x[8][4];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[u][e] = i + e < n ? uint32_t(part[int64_t(w + SL * u) * n + i + e]) : 0u;
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] += x[u][e];
        }
        for (; w < nw; w += SL)
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] += i + e < n ? uint32_t(part[int64_t(w) * n + i + e]) : 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) red[z][4 * q + e] = t[e];
        __syncthreads();
        if (threadIdx.x < E && i0 + threadIdx.x < n) {
            uint32_t tot = 0;
#pragma unroll
            for (int zz = 0; zz < SL; ++zz) tot += red[zz][threadIdx.x];
            if (BLK) {
                const int64_t j = i0 + threadIdx.x;
                const int q = int(j >> 10), ln = int(j >> 4) & 63, v = int(j) & 15;
                const int bm = q / nb, bn = q - bm * nb;
                const int m = 32 * bm + (ln & 31), c = 32 * bn + 8 * (v >> 2) + 4 * (ln >> 5) + (v & 3);
                if (m < M && c < N) {
                    G[int64_t(m) * N + c] = int32_t(tot);
                    amax = max(amax, abs_u32(int32_t(tot)));
                }
            } else {
                G[i0 + threadIdx.x] = int32_t(tot);
                amax = max(amax, abs_u32(int32_t(tot)));
            }
        }
    }
    if (absmax) {
        amax = wave_max_u32(amax);
        if ((threadIdx.x & 63) == 0) publish_max_u32(absmax, amax);
    }
}

// Launches the sum of nw partial rows of n elements into G (with the max
// when absmax is not null), at most 2048 workgroups (each then loops):
// 16 slices (256-byte segments of each partial row) when that still gives
// 256 workgroups, else 64 (64-byte segments; 32 slices measured slower than
// 16 on 36864-element rows).
inline void sum_partials(const int32_t *part, int nw, int64_t n, int32_t *G, uint32_t *absmax, hipStream_t st) {
    auto blocks = [n](int64_t e) {
        const int64_t b = (n + e - 1) / e;
        return unsigned(b < 1 ? 1 : (b > 2048 ? 2048 : b));
    };
    if (n >= 16384)
        wgrad_long_sum<16><<<dim3(blocks(64)), dim3(256), 0, st>>>(part, nw, n, G, absmax);
    else
        wgrad_long_sum<64><<<dim3(blocks(16)), dim3(256), 0, st>>>(part, nw, n, G, absmax);
}

// The same sum over blocked partials (nblk blocks of 1024 a row, nb a row
// of G's blocks) into the M x N of G.
inline void sum_partials_blocked(const int32_t *part, int nw, int nblk, int nb, int M, int N, int32_t *G,
                                 uint32_t *absmax, hipStream_t st) {
    const int64_t n = int64_t(nblk) * 1024;
    const int64_t b = (n + 63) / 64;
    wgrad_long_sum<16, true><<<dim3(unsigned(b > 2048 ? 2048 : b)), dim3(256), 0, st>>>(part, nw, n, G, absmax,
                                                                                       nb, M, N);
}

// Whether the partials are kept blocked: the accumulators' own layout
// (each lane's 16 values of a block in 64 contiguous bytes) instead of rows
// of G, whose 16-byte pieces do not line up with G's rows for N not a
// multiple of 4 (one dword store per value: 16 us for 160 x 147 partials,
// a third of the kernel).  Blocks pad G to multiples of 32, so only when
// that adds at most a quarter.
// The blocked partials take 16-byte stores, so also a 16-byte aligned
// workspace (part == nullptr: the size query, which covers both layouts).
inline bool wgrad_long_blocked(int64_t M, int64_t N, const void *part = nullptr) {
    const int64_t nblk = ((M + 31) / 32) * ((N + 31) / 32);
    return nblk * 1024 * 4 <= 5 * M * N && (part == nullptr || aligned(part, 16));
}

// int32 elements of one workgroup's partial G (the blocked layout's when
// the shape takes it, never fewer than the rows' M N).
inline int64_t wgrad_long_part_elems(int64_t M, int64_t N) {
    return wgrad_long_blocked(M, N) ? ((M + 31) / 32) * ((N + 31) / 32) * 1024 : M * N;
}

// Workgroups of a launch over a reduction of length K: at least 256 rows
// (four stages) each, at most 256.  A stage carries little work, so each
// workgroup's chain of stage loads sets the time: 128 workgroups of 512
// rows took 46 us on 65536 x 147 x 160.
inline int64_t wgrad_long_groups(int64_t K) {
    const int64_t wgs = (K + 255) / 256;
    return wgs > 256 ? 256 : wgs;
}

// Whether the kernel takes the shape: G within 32 blocks of 32 x 32, at most
// 256 per side, at least 2 (a staged dword then spans at most two rows), and
// a reduction long enough to split.
inline bool wgrad_long_fits(int64_t K, int64_t M, int64_t N, const void *a, const void *b) {
    const int64_t mb = (M + 31) / 32, nb = (N + 31) / 32;
    return M >= 2 && N >= 2 && mb <= MAXB && nb <= MAXB && mb * nb <= MAXBLK && K >= 4096 && aligned(a, 4) &&
           aligned(b, 4) && K * (M > N ? M : N) < (int64_t(1) << 31);
}

// Partial sums go to part when it is not null (it holds wgrad_long_groups(K)
// x wgrad_long_part_elems(M, N) int32, blocked when wgrad_long_blocked(M, N,
// part); the caller sums them), else into the zeroed G by atomics.
// Returns the number of workgroups (of partials).
inline int wgrad_long_launch(const int8_t *a, const int8_t *b, int64_t K, int M, int N, int32_t *G,
                              int32_t *part, hipStream_t st) {
    Args g;
    g.a = a;
    g.b = b;
    g.part = part;
    g.K = K;
    g.M = M;
    g.N = N;
    g.mb = (M + 31) / 32;
    g.nb = (N + 31) / 32;
    g.pa = 32 * g.mb + 16;
    g.pb = 32 * g.nb + 16;
    g.G = G;
    g.blk = part != nullptr && wgrad_long_blocked(M, N, part);
    int64_t wgs = wgrad_long_groups(K);
    g.rows = ((K + wgs - 1) / wgs + R - 1) / R * R;
    wgs = (K + g.rows - 1) / g.rows;  // at most wgrad_long_groups(K)
    const bool va = M % 4 == 0, vb = N % 4 == 0;
    const dim3 grid{unsigned(wgs), 1u, 1u}, block{unsigned(NT), 1u, 1u};
    if (va && vb) wgrad_long_kernel<true, true><<<grid, block, 0, st>>>(g);
    else if (va) wgrad_long_kernel<true, false><<<grid, block, 0, st>>>(g);
    else if (vb) wgrad_long_kernel<false, true><<<grid, block, 0, st>>>(g);
    else wgrad_long_kernel<false, false><<<grid, block, 0, st>>>(g);
    return int(wgs);
}

}  // namespace wl
}  // namespace ionn
