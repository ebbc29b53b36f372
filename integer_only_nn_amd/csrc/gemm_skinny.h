// Linear-layer contractions with a long batch and narrow layers ("Integer
// On-Device Training: Overview", sections 4 and 7: the forward product and
// the delta product of a Linear layer), C[M][N] = sum_k A[m][k] * B(n, k),
// for M rows of A with contiguous K-byte rows and at most 160 outputs and
// 160 reduction terms per row:
//   fwd    A = X  [B][IN],  B(n, k) = W[n][k]   (W [OUT][IN], rows of K bytes)
//   dgrad  A = dY [B][OUT], B(n, k) = W[k][n]   (W [OUT][IN], rows of N bytes)
// Rows of 147 or 160 bytes have no 16-byte aligned path in the tiled
// kernels, which then read them byte by byte.  Here a workgroup copies 128
// consecutive rows of A (one contiguous, 16-byte aligned run of 128 K bytes)
// into LDS as it lies in memory, and builds each lane's 16-byte fragment of
// a row from five aligned dwords with v_alignbyte (bytes past K masked to
// 0); the whole B operand, read once per workgroup, stays in registers as
// matrix-core fragments; each wavefront contracts 32 rows against all of B
// with v_mfma_i32_32x32x32_i8.  The epilogue is the tiled kernels': ReLU
// mask from an int8 tensor with C's layout (value set to 0 where it is
// <= 0) and the max |C| max-combined.
#pragma once

#include "common.h"

namespace ionn {
namespace sk {

constexpr int NT = 256;                 // four wavefronts
constexpr int RS = 128;                 // rows of A per stage (32 per wavefront)
constexpr int MAXB = 5;                 // blocks of 32 per side: N, K <= 160
constexpr int PA = 32 * MAXB + 16;      // LDS pitch of the staged B rows (bytes)
constexpr int SA = RS * 32 * MAXB + 32; // one A stage (bytes), with slack for the last row's reads
constexpr int NQ = RS * 32 * MAXB / 16 / NT;  // 16-byte pieces per thread, widest rows
constexpr int PO = 32 * MAXB + 4;       // int32 pitch of a wavefront's output rows in LDS
constexpr int NP = 32 * 32 * MAXB / 4 / 64;  // 16-byte pieces per lane of a wavefront's 32 x N block
static_assert(NP % 2 == 0, "the epilogue takes the pieces in two halves");

struct Args {
    const int8_t *a;      // A [M][K], contiguous rows, 16-byte aligned, M K a multiple of 16
    const int8_t *w;      // W: [N][K] (fwd) or [K][N] (dgrad), 4-byte aligned
    int32_t *c;           // C [M][N] (pitch N), 16-byte aligned
    const int8_t *act;    // ReLU mask source [M][N] (nullable), 4-byte aligned
    uint32_t *absmax;     // nullable
    int M, N, K, nb, ks;  // nb = ceil(N / 32), ks = ceil(K / 32)
};

// Rows m0 .. m0 + RS - 1 of A, RS K contiguous bytes from a multiple of 16
// (m0 is a multiple of RS = 128, the base is 16-byte aligned): thread t holds
// pieces t, t + NT, ... of 16 bytes.  M K is a multiple of 16, so a piece
// lies wholly before or wholly past the end of A (then it is not loaded).
__device__ __forceinline__ void stage_load(v4i (&v)[NQ], const int8_t *a, int K, int64_t m0, int M) {
    const int64_t rows = M - m0 < RS ? M - m0 : RS;
    const int nq = int(rows * K / 16);
    const v4i *p = reinterpret_cast<const v4i *>(a + m0 * K);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int q = int(threadIdx.x) + j * NT;
        v[j] = q < nq ? p[q] : v4i{0, 0, 0, 0};
    }
}

// The pieces to LDS as they lie in memory.
__device__ __forceinline__ void stage_store(const v4i (&v)[NQ], int K, int8_t *st) {
    const int nq = RS * K / 16;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int q = int(threadIdx.x) + j * NT;
        if (q < nq) reinterpret_cast<v4i *>(st)[q] = v[j];
    }
}

// Row r (of the stage), bytes c0 .. c0 + 15 of A from the stage as it lies
// in memory (row pitch K bytes), bytes at or past column K set to 0.
__device__ __forceinline__ v4i a_frag(const int8_t *st, int K, int r, int c0) {
    const int o = r * K + c0, b = o & ~3;
    const uint32_t *d = reinterpret_cast<const uint32_t *>(st + b);
    const uint32_t d0 = d[0], d1 = d[1], d2 = d[2], d3 = d[3], d4 = d[4];
    const uint32_t sh = uint32_t(o & 3);
    uint32_t w[4] = {__builtin_amdgcn_alignbyte(d1, d0, sh), __builtin_amdgcn_alignbyte(d2, d1, sh),
                     __builtin_amdgcn_alignbyte(d3, d2, sh), __builtin_amdgcn_alignbyte(d4, d3, sh)};
    const int nv = K - c0;  // valid bytes of the 16 (the row may end inside them)
    if (nv < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = nv - 4 * i;
            w[i] &= k >= 4 ? 0xffffffffu : (k <= 0 ? 0u : (1u << (8 * k)) - 1u);
        }
    }
    return v4i{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
}

// W (rows x cols bytes, contiguous, 4-byte aligned) into LDS rows of pitch
// PA at st, through a linear copy at lin: every dword of W loaded at once
// (the last rows x cols mod 4 bytes one per thread) and stored as it lies;
// then dword d of padded row r is the four bytes at r cols + 4 d of the copy,
// v_alignbyte of the two dwords around them, bytes at or past cols cleared.
constexpr int NW = 32 * MAXB * 32 * MAXB / 4 / NT;  // dwords per thread, largest W
__device__ __forceinline__ void stage_w(int8_t *st, int8_t *lin, const int8_t *w, int rows, int cols) {
    const int t = int(threadIdx.x);
    const int n4 = rows * cols / 4, tail = rows * cols - 4 * n4;
    const uint32_t *w32 = reinterpret_cast<const uint32_t *>(w);
    uint32_t v[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int q = t + j * NT;
        v[j] = q < n4 ? w32[q] : 0u;
    }
    uint32_t *l32 = reinterpret_cast<uint32_t *>(lin);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int q = t + j * NT;
        if (q < n4) l32[q] = v[j];
    }
    if (t < tail) lin[4 * n4 + t] = w[4 * n4 + t];
    __syncthreads();
    const int dpr = (cols + 3) / 4;  // dwords per padded row
    const int items = rows * dpr;
    int r = t / dpr, d = t - r * dpr;
    const int dr = NT / dpr, dd = NT - dr * dpr;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        if (t + j * NT < items) {
            const int o = r * cols + 4 * d;
            const uint32_t lo = l32[o >> 2], hi = l32[(o >> 2) + 1];
            uint32_t x = __builtin_amdgcn_alignbyte(hi, lo, uint32_t(o & 3));
            const int nv = cols - 4 * d;
            if (nv < 4) x &= (1u << (8 * nv)) - 1u;
            *reinterpret_cast<uint32_t *>(st + r * PA + 4 * d) = x;
        }
        r += dr;
        d += dd;
        if (d >= dpr) {
            d -= dpr;
            ++r;
        }
    }
}

// The four mask bytes of values e0 .. e0 + 3 of a run of `valid` values
// (past its end: any), as one word.
__device__ __forceinline__ uint32_t mask_word(const int8_t *ab, int e0, int valid) {
    if (e0 + 4 <= valid) return *reinterpret_cast<const uint32_t *>(ab + e0);
    uint32_t a = 0x01010101u;
    for (int e = 0; e < 4; ++e)
        if (e0 + e < valid) a = (a & ~(0xffu << (8 * e))) | (uint32_t(uint8_t(ab[e0 + e])) << (8 * e));
    return a;
}

// One workgroup per group of stages (persistent over m0 = RS (blockIdx.x +
// i gridDim.x)).  B is staged once through LDS (fwd: rows n of K bytes;
// dgrad: rows k of N bytes, read back transposed) into registers; the next
// stage's dwords are in flight while the current one is contracted.
template <bool BT>
__global__ __launch_bounds__(NT, 1) void skinny_kernel(Args g) {
    typedef int v2i_ __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i_ lds_v2i_t;
    // the two A stages; before them, B staged at pitch PA (32 MAXB rows)
    __shared__ __attribute__((aligned(16))) int8_t lds[2][SA];
    // each wavefront's 32 output rows, for the contiguous store
    __shared__ __attribute__((aligned(16))) int32_t out_lds[4 * 32 * PO];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int nb = g.nb, ks = g.ks;

    // B staged over both buffers as one region of 32 MAXB rows of pitch PA
    // (fwd: rows n of K bytes; dgrad: rows k of N bytes), zero-padded
    static_assert(32 * MAXB * PA <= 2 * SA, "B fits the two stage buffers");
    int8_t *bst = &lds[0][0];
    for (int i = int(threadIdx.x); i < 2 * SA / 16; i += NT)
        reinterpret_cast<v4i *>(bst)[i] = v4i{0, 0, 0, 0};
    __syncthreads();
    // the first A stage's loads go out first, so that their round trip
    // overlaps B's staging
    const int64_t nstages = (int64_t(g.M) + RS - 1) / RS;
    int64_t sidx = blockIdx.x;
    v4i v[NQ];
    if (sidx < nstages) stage_load(v, g.a, g.K, sidx * RS, g.M);
    stage_w(bst, reinterpret_cast<int8_t *>(out_lds), g.w, BT ? g.K : g.N, BT ? g.N : g.K);
    __syncthreads();
    v4i bf[MAXB][MAXB];  // [column block][k step]
#pragma unroll
    for (int j = 0; j < MAXB; ++j)
#pragma unroll
        for (int s = 0; s < MAXB; ++s) {
            if (j < nb && s < ks) {
                if (!BT) {
                    bf[j][s] = *reinterpret_cast<const v4i *>(bst + (32 * j + (lane & 31)) * PA + 32 * s +
                                                              16 * (lane >> 5));
                } else {
                    // rows n = 32 j + lane % 32, k = 32 s + 16 (lane / 32) .. + 15 from [k][n]
                    const int q = lane >> 4, i = lane & 15;
                    const int8_t *p = bst + (32 * s + 16 * (q >> 1) + (i >> 1)) * PA + 32 * j + 16 * (q & 1) +
                                      8 * (i & 1);
                    const v2i_ x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p));
                    const v2i_ y = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p + 8 * PA));
                    bf[j][s] = v4i{x.x, x.y, y.x, y.y};
                }
            } else {
                bf[j][s] = v4i{0, 0, 0, 0};
            }
        }
    __syncthreads();

    int buf = 0;
    uint32_t amax = 0;
    while (sidx < nstages) {
        stage_store(v, g.K, lds[buf]);
        __syncthreads();
        const int64_t m0 = sidx * RS;
        const int64_t nxt = sidx + gridDim.x;
        if (nxt < nstages) stage_load(v, g.a, g.K, nxt * RS, g.M);
        // the wavefront's block of C: rows mb .. mb + 31, one contiguous run
        // of `valid` values; its mask words are fetched now, used at the end
        const int64_t mb = m0 + 32 * wave;
        const int64_t brows = g.M - mb < 32 ? g.M - mb : 32;
        const int valid = brows > 0 ? int(brows) * g.N : 0;
        const int8_t *ab = g.act ? g.act + mb * g.N : nullptr;
        uint32_t mk[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int e0 = 4 * (lane + 64 * i);
            mk[i] = (ab && e0 < valid) ? mask_word(ab, e0, valid) : 0x01010101u;
        }
        v16i acc[MAXB];
#pragma unroll
        for (int j = 0; j < MAXB; ++j) acc[j] = v16i{};
#pragma unroll
        for (int s = 0; s < MAXB; ++s) {
            if (s < ks) {
                const v4i af = a_frag(lds[buf], g.K, 32 * wave + (lane & 31), 32 * s + 16 * (lane >> 5));
#pragma unroll
                for (int j = 0; j < MAXB; ++j)
                    if (j < nb) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j][s], af, acc[j], 0, 0, 0);
            }
        }
        // lane holds C[m][n .. n + 3] for m = row lane % 32 of the wavefront's
        // block and n = 32 j + 8 q + 4 (lane / 32).  The block (32 rows of N)
        // goes through the wavefront's LDS area so that it leaves as one
        // contiguous run of 32 N int32: rows at pitch N + 4 when N is a
        // multiple of 4 (16-byte pieces never straddle rows), else at pitch N
        // (the run itself, written a value at a time).
        int32_t *ob = out_lds + wave * 32 * PO;
        const bool n4 = (g.N & 3) == 0;
        const int pn = n4 ? g.N + 4 : g.N;
        {
            const int r = lane & 31;
#pragma unroll
            for (int j = 0; j < MAXB; ++j) {
                if (j >= nb) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = 32 * j + 8 * q + 4 * (lane >> 5);
                    if (n >= g.N) continue;
                    if (n4) {
                        *reinterpret_cast<v4i *>(ob + r * pn + n) =
                            v4i{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < g.N) ob[r * pn + n + e] = acc[j][4 * q + e];
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wavefront's LDS writes done
        __builtin_amdgcn_wave_barrier();
        {
            // piece p = lane + 64 i holds values 4 p .. 4 p + 3 of the run:
            // in two halves, all of a half's LDS reads first, then its stores
            const int q4 = g.N >> 2;
            int32_t *cb = g.c + mb * g.N;
#pragma unroll
            for (int h = 0; h < NP; h += NP / 2) {
                v4i r4[NP / 2];
#pragma unroll
                for (int i = 0; i < NP / 2; ++i) {
                    const int p = lane + 64 * (h + i);
                    if (4 * p < valid) {
                        if (n4) {
                            const int row = int(uint32_t(p) / uint32_t(q4)), col = 4 * (p - row * q4);
                            r4[i] = *reinterpret_cast<const v4i *>(ob + row * pn + col);
                        } else {
                            r4[i] = *reinterpret_cast<const v4i *>(ob + 4 * p);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < NP / 2; ++i) {
                    const int e0 = 4 * (lane + 64 * (h + i));
                    if (e0 >= valid) continue;
                    v4i r = r4[i];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (int8_t(uint8_t(mk[h + i] >> (8 * e))) <= 0) r[e] = 0;
                    if (e0 + 4 <= valid) {
                        *reinterpret_cast<v4i *>(cb + e0) = r;
#pragma unroll
                        for (int e = 0; e < 4; ++e) amax = max(amax, abs_u32(r[e]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (e0 + e < valid) {
                                cb[e0 + e] = r[e];
                                amax = max(amax, abs_u32(r[e]));
                            }
                    }
                }
            }
        }
        __syncthreads();
        buf ^= 1;
        sidx = nxt;
    }
    if (g.absmax) {
        amax = wave_max_u32(amax);
        if (lane == 0) publish_max_u32(g.absmax, amax);
    }
}

// Whether the kernel takes the product: N, K in [2, 160], a long batch, a
// 16-byte aligned A of a multiple of 16 bytes, a 4-byte aligned W, a 16-byte
// aligned C, a 4-byte aligned mask, and C below 2^31 elements.
inline bool skinny_fits(int64_t M, int64_t N, int64_t K, const void *a, const void *w, const void *c,
                        const void *act) {
    return M >= 4096 && N >= 2 && N <= 32 * MAXB && K >= 2 && K <= 32 * MAXB && aligned(a, 16) && aligned(w, 4) &&
           (M * K) % 16 == 0 && aligned(c, 16) && (act == nullptr || aligned(act, 4)) &&
           M * (N > K ? N : K) < (int64_t(1) << 31);
}

inline void skinny_launch(bool bt, const int8_t *a, const int8_t *w, int32_t *c, const int8_t *act,
                          uint32_t *absmax, int M, int N, int K, hipStream_t st) {
    Args g{a, w, c, act, absmax, M, N, K, (N + 31) / 32, (K + 31) / 32};
    const int64_t nstages = (int64_t(M) + RS - 1) / RS;
    const int64_t cus = device_cus();
    const unsigned grid = unsigned(nstages < cus ? nstages : cus);
    if (bt) skinny_kernel<true><<<dim3(grid), dim3(NT), 0, st>>>(g);
    else skinny_kernel<false><<<dim3(grid), dim3(NT), 0, st>>>(g);
}

}  // namespace sk
}  // namespace ionn
