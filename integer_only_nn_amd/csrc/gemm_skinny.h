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

// A buffer offset past the end of every resource built here: loads from it
// return 0 and stores to it are dropped, so lanes outside a tensor need no
// branch (a lane-dependent branch around a load or store leaves the compiler
// unable to count the memory operations in flight, and it then drains them
// all before the next use of a loaded value).
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, int(bytes), 0x00020000);
}

// Rows m0 .. m0 + RS - 1 of A, RS K contiguous bytes from a multiple of 16
// (m0 is a multiple of RS = 128, the base is 16-byte aligned): thread t holds
// pieces t, t + NT, ... of 16 bytes.  M K is a multiple of 16, so a piece
// lies wholly before or wholly past the end of A (then it reads as zeros).
__device__ __forceinline__ void stage_load(v4i (&v)[NQ], __amdgpu_buffer_rsrc_t ar, int K, int64_t m0, int M) {
    const int64_t rows = M - m0 < RS ? M - m0 : RS;
    const int nq = rows > 0 ? int(rows * K / 16) : 0;
    const uint32_t base = uint32_t(m0 * K);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int q = int(threadIdx.x) + j * NT;
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(ar, int(q < nq ? base + 16u * uint32_t(q) : OOB), 0, 0);
    }
}

// The pieces to LDS as they lie in memory (all NQ NT pieces: those past the
// stage's rows are zeros and stay inside the stage buffer).
__device__ __forceinline__ void stage_store(const v4i (&v)[NQ], int8_t *st) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) reinterpret_cast<v4i *>(st)[int(threadIdx.x) + j * NT] = v[j];
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
    const __amdgpu_buffer_rsrc_t wr = rsrc(w, int64_t(rows) * cols);
    uint32_t v[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int q = t + j * NT;
        v[j] = __builtin_amdgcn_raw_buffer_load_b32(wr, int(q < n4 ? 4u * uint32_t(q) : OOB), 0, 0);
    }
    const uint8_t tb = __builtin_amdgcn_raw_buffer_load_b8(wr, int(t < tail ? uint32_t(4 * n4 + t) : OOB), 0, 0);
    uint32_t *l32 = reinterpret_cast<uint32_t *>(lin);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int q = t + j * NT;
        if (q < n4) l32[q] = v[j];
    }
    if (t < tail) lin[4 * n4 + t] = int8_t(tb);
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

// One workgroup per group of stages (persistent over m0 = RS (blockIdx.x +
// i gridDim.x)).  B is staged once through LDS (fwd: rows n of K bytes;
// dgrad: rows k of N bytes, read back transposed) into registers; the next
// stage's dwords are in flight while the current one is contracted.
template <bool BT, bool N4>
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
    static_assert(NQ * NT * 16 <= SA, "a stage's pieces fit its buffer");
    int8_t *bst = &lds[0][0];
    for (int i = int(threadIdx.x); i < 2 * SA / 16; i += NT)
        reinterpret_cast<v4i *>(bst)[i] = v4i{0, 0, 0, 0};
    __syncthreads();
    // the first A stage's loads go out first, so that their round trip
    // overlaps B's staging
    const int64_t nstages = (int64_t(g.M) + RS - 1) / RS;
    int64_t sidx = blockIdx.x;
    const __amdgpu_buffer_rsrc_t ar = rsrc(g.a, int64_t(g.M) * g.K);
    v4i v[NQ];
    if (sidx < nstages) stage_load(v, ar, g.K, sidx * RS, g.M);
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
        stage_store(v, lds[buf]);
        __syncthreads();
        const int64_t m0 = sidx * RS;
        const int64_t nxt = sidx + gridDim.x;
        // (past the last stage the loads read zeros: no branch around them)
        stage_load(v, ar, g.K, nxt * RS, g.M);
        // the wavefront's block of C: rows mb .. mb + 31, one contiguous run
        // of `valid` values; its mask words are fetched now, used at the end
        const int64_t mb = m0 + 32 * wave;
        const int64_t brows = g.M - mb < 32 ? g.M - mb : 32;
        const int valid = brows > 0 ? int(brows) * g.N : 0;
        const int8_t *ab = g.act ? g.act + mb * g.N : nullptr;
        // (whole words in one pass, so that no lane takes a path of byte
        // loads: the compiler then waits for each word by count, where a
        // per-lane choice between a word and its bytes made it drain every
        // load and store before each of the 20 stores below; ab is 4-byte
        // aligned, as act is and 32 N is a multiple of 4)
        // Every path issues the same loads (none without a mask: an empty
        // resource), so that the compiler's count of the memory operations
        // after the next stage's loads is exact, not the least over the paths.
        const __amdgpu_buffer_rsrc_t mr = g.act ? rsrc(g.act, int64_t(g.M) * g.N) : rsrc(g.a, 0);
        const bool masked = g.act != nullptr;
        uint32_t mk[NP];
        uint32_t tb = 0;
        if (N4) {
            // word (j, q): the mask bytes of row lane % 32, columns
            // n = 32 j + 8 q + 4 (lane / 32) .. + 3, which the lane stores
            // (past the block's rows or N: read as 0, never stored)
            const int r = lane & 31;
            const uint32_t rb = uint32_t((mb + r) * g.N);
#pragma unroll
            for (int j = 0; j < MAXB; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = 32 * j + 8 * q + 4 * (lane >> 5);
                    mk[4 * j + q] = __builtin_amdgcn_raw_buffer_load_b32(
                        mr, int(j < nb && n < g.N && r < brows ? rb + uint32_t(n) : OOB), 0, 0);
                }
        } else {
            // word i: the mask bytes of values 4 p .. 4 p + 3 of the run,
            // p = lane + 64 i, when the run holds all four; of the word the
            // run ends inside (a last block of brows N values, not a multiple
            // of 4), value e goes to lane e (tb)
            const uint32_t rb = uint32_t(mb * g.N);
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int e0 = 4 * (lane + 64 * i);
                mk[i] = __builtin_amdgcn_raw_buffer_load_b32(mr, int(e0 + 4 <= valid ? rb + uint32_t(e0) : OOB), 0, 0);
            }
            const int wq = valid >> 2;
            tb = __builtin_amdgcn_raw_buffer_load_b8(
                mr, int(lane < (valid & 3) ? rb + uint32_t(4 * wq + lane) : OOB), 0, 0);
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
        // block and n = 32 j + 8 q + 4 (lane / 32).  The stage's rows of C
        // are one resource (their bytes stay below 2^31).
        const int64_t srows = g.M - m0 < RS ? g.M - m0 : RS;
        const __amdgpu_buffer_rsrc_t cr = rsrc(g.c + m0 * g.N, srows * g.N * 4);
        if (N4) {
            // N a multiple of 4: the four values leave as one aligned 16-byte
            // store (a wavefront writes 32 bytes of each of 32 rows per
            // instruction, and the L2 joins the rows' pieces); rows past M
            // and columns past N are not stored.  Rows past M and columns
            // past N hold 0 (zero A rows, zero-padded B), so the max and min
            // run over every value without a test.
            const int r = lane & 31;
            const uint32_t rb = uint32_t((32 * wave + r) * g.N) * 4u;
            // (20 stores on every path, those outside C dropped; blocks past
            // nb hold zeros)
            int32_t mx = 0, mn = 0;
#pragma unroll
            for (int j = 0; j < MAXB; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = 32 * j + 8 * q + 4 * (lane >> 5);
                    v4i x = {acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
                    const uint32_t w = masked ? mk[4 * j + q] : 0x01010101u;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = int8_t(uint8_t(w >> (8 * e))) > 0 ? x[e] : 0;
                    mx = max(mx, max(max(x[0], x[1]), max(x[2], x[3])));
                    mn = min(mn, min(min(x[0], x[1]), min(x[2], x[3])));
                    __builtin_amdgcn_raw_buffer_store_b128(
                        x, cr, int(j < nb && n < g.N && r < brows ? rb + 4u * uint32_t(n) : OOB), 0, 0);
                }
            }
            amax = max(amax, max(uint32_t(mx), 0u - uint32_t(mn)));
            buf ^= 1;
            sidx = nxt;
            __syncthreads();
            continue;
        }
        // Otherwise the block (32 rows of N) goes through the wavefront's LDS
        // area, the run itself at pitch N written a value at a time, so that
        // it leaves as one contiguous, 16-byte aligned run of 32 N int32.
        int32_t *ob = out_lds + wave * 32 * PO;
        {
            // (blocks wholly inside N: four values a lane, no test)
            const int r = lane & 31;
#pragma unroll
            for (int j = 0; j < MAXB; ++j) {
                if (j >= nb) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = 32 * j + 8 * q + 4 * (lane >> 5);
                    if (32 * (j + 1) <= g.N) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) ob[r * g.N + n + e] = acc[j][4 * q + e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < g.N) ob[r * g.N + n + e] = acc[j][4 * q + e];
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wavefront's LDS writes done
        __builtin_amdgcn_wave_barrier();
        {
            // piece p = lane + 64 i holds values 4 p .. 4 p + 3 of the run
            // (the LDS area holds 1280 pieces, so every read stays inside
            // it): in two halves, a half's LDS reads first, then its stores;
            // pieces past the run are neither stored nor counted in the max
            const uint32_t cb = uint32_t(32 * wave * g.N) * 4u;
            int32_t mx = 0, mn = 0;
#pragma unroll
            for (int h = 0; h < NP; h += NP / 2) {
                v4i r4[NP / 2];
#pragma unroll
                for (int i = 0; i < NP / 2; ++i)
                    r4[i] = *reinterpret_cast<const v4i *>(ob + 4 * (lane + 64 * (h + i)));
#pragma unroll
                for (int i = 0; i < NP / 2; ++i) {
                    const int e0 = 4 * (lane + 64 * (h + i));
                    const bool in = e0 + 4 <= valid;
                    // a value is kept where its mask byte is positive: all
                    // ones without a mask, none past the run
                    uint32_t w = masked ? mk[h + i] : 0x01010101u;
                    w = in ? w : 0u;
                    v4i x = r4[i];
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = int8_t(uint8_t(w >> (8 * e))) > 0 ? x[e] : 0;
                    mx = max(mx, max(max(x[0], x[1]), max(x[2], x[3])));
                    mn = min(mn, min(min(x[0], x[1]), min(x[2], x[3])));
                    __builtin_amdgcn_raw_buffer_store_b128(x, cr, int(in ? cb + 4u * uint32_t(e0) : OOB), 0, 0);
                }
            }
            // the word the run ends inside: lane e < valid mod 4 stores value
            // 4 wq + e (one store on every lane, the rest dropped)
            {
                const int wq = valid >> 2;
                const bool ok = lane < (valid & 3);
                int32_t x = ok ? ob[4 * wq + (lane & 3)] : 0;
                // (used here, not earlier: waiting for tb, the last load
                // issued, would wait for every load before it)
                asm volatile("" : "+v"(tb));
                if (masked && int8_t(uint8_t(tb)) <= 0) x = 0;
                mx = max(mx, x);
                mn = min(mn, x);
                __builtin_amdgcn_raw_buffer_store_b32(x, cr, int(ok ? cb + 4u * uint32_t(4 * wq + lane) : OOB), 0, 0);
            }
            amax = max(amax, max(uint32_t(mx), 0u - uint32_t(mn)));
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
    const bool n4 = N % 4 == 0;
    if (bt && n4) skinny_kernel<true, true><<<dim3(grid), dim3(NT), 0, st>>>(g);
    else if (bt) skinny_kernel<true, false><<<dim3(grid), dim3(NT), 0, st>>>(g);
    else if (n4) skinny_kernel<false, true><<<dim3(grid), dim3(NT), 0, st>>>(g);
    else skinny_kernel<false, false><<<dim3(grid), dim3(NT), 0, st>>>(g);
}

}  // namespace sk
}  // namespace ionn
