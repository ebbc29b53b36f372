// Fast path of the int8 Linear contractions: 256x256 output tiles, 128-deep
// K steps, gfx950 direct-to-LDS loads and LDS transpose reads.
//
// C[m][n] = sum_k A(m,k) * B(k,n), int32 modulo 2^32.  Each operand is either
//   K-major: element (r, k) at base[r * ld + k]   (contiguous along k), or
//   M-major: element (r, k) at base[k * ld + r]   (contiguous along r).
// Requires M, N multiples of 256, K a multiple of 256, 16-byte aligned bases,
// ld a multiple of 16 and each operand below 2^31 bytes (the caller checks).
//
// Data movement.  Every operand tile goes HBM -> LDS with
// buffer_load_dwordx4 ... lds (each instruction writes 64 lanes x 16 B = 1 KiB of
// LDS contiguously and uses no VGPRs for data), double-buffered in two static
// LDS stages of 64 KiB (A 32 KiB + B 32 KiB).  The loop is unrolled by two so
// the two stages are distinct arrays: the compiler can then prove that the
// loads in flight into one stage do not alias the reads of the other and
// waits for them only where the algorithm needs to.
//
// LDS layouts (bank-conflict free for the 16-lane and 8-lane phases of
// 128-bit reads and the 32-lane phases of 64-bit reads):
//   K-major tile [256 rows][128 B]: 16-byte chunk c of row r is stored at
//     chunk position c ^ fK(r & 15), fK(r) = (r >> 1) ^ ((r & 1) << 2).
//     Fragment read: one ds_read_b128 per 16x64 fragment.
//   M-major tile [128 k][256 B]: 16-byte chunk c of k-row k is stored at
//     position c ^ fM(k), fM(k) = (k & 7) | ((k & 1) << 3).
//     Fragment read: two ds_read_b64_tr_b8.  Within each 16-lane group the
//     instruction returns, to lane j, byte (j mod 8) of the 8-byte rows
//     addressed by lanes 2b + j/8 (b = 0..7); pointing lane i at
//     T[k0 + i/2][m0 + 8 (i mod 2)] therefore hands lane j the eight values
//     T[k0 .. k0+7][m0 + j], which is the matrix-core fragment layout (row =
//     lane mod 16, consecutive k) without any register shuffling.
// Both swizzles depend only on lane bits and on compile-time indices, so every
// address is a uniform (scalar) part plus one of a few per-lane offsets.
//
// Compute: 4 wavefronts in a 2x2 grid, 128x128 each: 4x4 blocks of 32x32 on
// v_mfma_i32_32x32x32_i8 (256 int32 accumulators per lane, in AGPRs).  On
// gfx950 this shape runs int8 at full rate; the 16x16x64 shape measures at
// half of it.  A 128-deep K step is 4 slices of 32; per slice a wavefront
// reads 4 A and 4 B fragments (16 bytes per lane each: row = lane % 32,
// k = 16 (lane / 32) .. +15) and issues 16 MFMAs.  The next slice's fragments
// are read while the current slice's MFMAs run, and the next step's loads go
// out over the first two slices: one memory instruction between consecutive
// MFMAs, because a wavefront stalls on the issue of a load into LDS for
// about as long as an MFMA takes, and a burst of them starves the matrix core
// (measured: 16 loads issued back to back cost a third of the loop time).
// At the last slice the stage barrier, the first loads of the step after
// next and the next step's first fragments are tucked in before its last MFMAs.
#pragma once

#include "gemm_core.h"

namespace ionn {
namespace g256 {

constexpr int BM = 256, BN = 256, BK = 128, NT = 256;
constexpr int TILE_BYTES = BM * BK;  // 32 KiB per operand per stage

__host__ __device__ constexpr int fK(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }
__host__ __device__ constexpr int fM(int k) { return (k & 7) | ((k & 1) << 3); }

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// One buffer_load_dwordx4 ... lds: every lane fetches 16 bytes at
// rsrc.base + soff + voff and the wavefront writes them to LDS at m0 + 16 *
// lane.  Issued through inline asm so the compiler does not track it: the
// kernel orders these loads itself (each wavefront waits for vmcnt(0), then
// all meet at s_barrier, before a stage is read), and a compiler that cannot
// tell the two LDS stages apart would otherwise wait for the prefetch in
// flight before every LDS read.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr), "s"(soff)
                 : "memory", "m0");
}

// Two loads under one m0: the second lands 1 KiB further in LDS through the
// instruction offset, which also adds 1 KiB to its global address, so the
// caller passes that load's SGPR offset less 1 KiB.
__device__ __forceinline__ void dma16x2(v4i rsrc, uint32_t voff0, uint32_t soff0, uint32_t voff1,
                                        uint32_t soff1m, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds\n\t"
                 "buffer_load_dwordx4 %4, %1, %5 offen offset:1024 lds"
                 :
                 : "v"(voff0), "s"(rsrc), "s"(lds_addr), "s"(soff0), "v"(voff1), "s"(soff1m)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const int8_t *p) {
    return uint32_t(uintptr_t((__attribute__((address_space(3))) const int8_t *)(p)));
}

// This wavefront's share (8 of the 32 1-KiB load instructions) of one
// operand tile.  The operand is one buffer resource (base and byte size in
// SGPRs: an offset past the end reads zeros instead of faulting); each
// instruction adds a uniform SGPR offset (row or k-row position of the
// instruction, plus k0) to a per-lane 32-bit VGPR offset.  The instruction
// index enters the swizzle only through its parity, so two per-lane offsets
// serve all eight instructions.
template <bool KMAJOR>
struct TileSrc {
    v4i rsrc;
    int ld;
    uint32_t wave_off;
    uint32_t lane_off[2];
    __device__ __forceinline__ void init(const int8_t *b, int ldv, uint32_t bytes, int r0, int wave,
                                         int lane) {
        const uint64_t a = uint64_t(uintptr_t(b));
        rsrc = v4i{__builtin_amdgcn_readfirstlane(int(uint32_t(a))),
                   __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffffu)),  // stride 0
                   __builtin_amdgcn_readfirstlane(int(bytes)),                        // num_records
                   0x00020000};                                                       // 32-bit data format
        ld = ldv;
        if (KMAJOR) {
            // instruction q = 8*wave + qq covers rows 8q .. 8q+7; lane -> row 8q + lane/8,
            // row & 15 = 8*(qq & 1) + lane/8
            wave_off = uint32_t(r0 + 64 * wave) * uint32_t(ld);
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int r15 = 8 * p + (lane >> 3);
                lane_off[p] = uint32_t((lane >> 3) * ld + 16 * ((lane & 7) ^ fK(r15)));
            }
        } else {
            // instruction q = 8*wave + qq covers k-rows 4q .. 4q+3; lane -> k = 4q + lane/16;
            // k & 7 = 4*(qq & 1) + lane/16, so fM(k) depends on qq & 1 only
            wave_off = uint32_t(32 * wave) * uint32_t(ld) + uint32_t(r0);
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int k = 4 * p + (lane >> 4);
                lane_off[p] = uint32_t((lane >> 4) * ld + 16 * ((lane & 15) ^ fM(k)));
            }
        }
    }
    __device__ __forceinline__ uint32_t soff_of(int k0, int qq) const {
        return KMAJOR ? wave_off + uint32_t(8 * qq * ld + k0) : wave_off + uint32_t((k0 + 4 * qq) * ld);
    }
    __device__ __forceinline__ uint32_t lds_of(int8_t *dst, int wave, int qq) const {
        return lds_addr(dst) + uint32_t(wave * 8 * 1024 + qq * 1024);
    }
    // instruction qq
    __device__ __forceinline__ void issue_one(int k0, int8_t *dst, int wave, int qq) const {
        dma16(rsrc, lane_off[qq & 1], soff_of(k0, qq), lds_of(dst, wave, qq));
    }
    // instructions qq (even) and qq + 1 under one m0; soff_of(k0, qq + 1) >= 1 KiB
    // because it includes at least 8 rows (or 4 k-rows) of a pitch >= 256
    __device__ __forceinline__ void issue_two(int k0, int8_t *dst, int wave, int qq) const {
        dma16x2(rsrc, lane_off[0], soff_of(k0, qq), lane_off[1], soff_of(k0, qq + 1) - 1024u,
                lds_of(dst, wave, qq));
    }
    // all eight instructions
    __device__ __forceinline__ void issue(int k0, int8_t *dst, int wave) const {
#pragma unroll
        for (int qq = 0; qq < 8; qq += 2) issue_two(k0, dst, wave, qq);
    }
};

// Fragment reader for one operand of one wavefront (rows rw .. rw+127 of the
// tile): fragment fi covers rows rw + 32 fi .. +31, slice sl covers k
// 32 sl .. 32 sl + 31; lane takes row lane % 32 and k 16 (lane / 32) .. +15.
template <bool KMAJOR>
struct FragSrc {
    uint32_t off[2];
    __device__ __forceinline__ void init(int rw, int lane) {
        if (KMAJOR) {
            // row = rw + 32 fi + (lane & 31), row & 15 = lane & 15;
            // chunk = 2 sl + lane/32, position chunk ^ fK(row & 15).
            // off[p]: slices with (sl & 1) == p; (2 sl) ^ f keeps bit 2 of 2 sl
            // separate only through the XOR, so both parities are precomputed
            // and slices 2, 3 add 4 chunks (64 bytes) XOR-free: chunk bits
            // 0-1 come from (lane/32, sl & 1), bit 2 from sl >> 1.
            const int r15 = lane & 15;
#pragma unroll
            for (int p = 0; p < 2; ++p)
                off[p] = uint32_t((rw + (lane & 31)) * BK + 16 * ((2 * p + (lane >> 5)) ^ fK(r15)));
        } else {
            // 16-lane group g = lane / 16 reads m-chunk 2 fi + (g & 1) (+ rw/16)
            // at k = 32 sl + 16 (g >> 1) + 8 h + i/2, i = lane & 15; k & 7 = i/2,
            // so fM(k) = i/2 | (i/2 & 1) << 3 per lane and the position is
            // (rw/16 + (g & 1) ^ fM) ^ 2 fi.
            const int g = lane >> 4, i = lane & 15;
            const int f = fM(i >> 1);
            const int base_c = ((rw >> 4) + (g & 1)) ^ f;
            off[0] = uint32_t((16 * (g >> 1) + (i >> 1)) * BM + 8 * (i & 1));
            off[1] = uint32_t(16 * base_c);  // XORed with 32 * fi
        }
    }
    __device__ __forceinline__ v4i read(const int8_t *tile, int fi, int sl) const {
        if (KMAJOR) {
            // positions of slices 2, 3 = positions of slices 0, 1 with bit 2
            // flipped: fK only uses bits 0-2, so flip via XOR on the offset
            const uint32_t o = off[sl & 1] ^ uint32_t((sl >> 1) * 64);
            return *reinterpret_cast<const v4i *>(tile + o + fi * 32 * BK);
        } else {
            const uint32_t o = off[0] + (off[1] ^ uint32_t(32 * fi));
            v4i out;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int8_t *p = tile + o + (32 * sl + 8 * h) * BM;
                const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(p));
                out[2 * h] = v.x;
                out[2 * h + 1] = v.y;
            }
            return out;
        }
    }
};

// Fragments of one 32-deep slice: A blocks 0..3 then B blocks 0..3.
template <bool A_KM, bool B_KM>
struct Frags {
    v4i a[4], b[4];
    __device__ __forceinline__ void read(int idx, const int8_t *As, const int8_t *Bs,
                                         const FragSrc<A_KM> &fa, const FragSrc<B_KM> &fb, int sl) {
        if (idx < 4) a[idx] = fa.read(As, idx, sl);
        else b[idx - 4] = fb.read(Bs, idx - 4, sl);
    }
};

#define IONN_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Issue order of one slice: 16 MFMAs in 4 groups, and the next slice's 8
// fragments read in the order a0 b0 a1 b1 a2 b2 b3 a3.  Group g needs only
// fragments that are read early: group 0 uses a0 a1 b0 b1, group 1 adds a2
// b2, group 2 adds b3 and group 3 a3, so the first MFMAs of a slice wait for
// reads issued two groups earlier.
constexpr int GI[16] = {0, 0, 1, 1, 0, 1, 2, 2, 2, 0, 1, 2, 3, 3, 3, 3};
constexpr int GJ[16] = {0, 1, 0, 1, 2, 2, 0, 1, 2, 3, 3, 3, 0, 1, 2, 3};
constexpr int RO[8] = {0, 4, 1, 5, 2, 6, 7, 3};

// MFMA t of group g.  The B fragment goes first, so the 32x32 result has n
// along its rows: lane holds m = lane % 32 and, for q = 0..3,
// n = 8 q + 4 (lane / 32) .. +3.
template <bool A_KM, bool B_KM>
__device__ __forceinline__ void mfma_gt(const Frags<A_KM, B_KM> &f, int g, int t, v16i (&acc)[4][4]) {
    const int i = GI[4 * g + t], j = GJ[4 * g + t];
    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

template <bool A_KM, bool B_KM, bool RELU, bool OSS>
__global__ __launch_bounds__(NT, 1) void gemm256_kernel(const int8_t *__restrict__ A, int64_t lda,
                                                        const int8_t *__restrict__ B, int64_t ldb,
                                                        uint32_t a_bytes, uint32_t b_bytes,
                                                        gemm::Epi ep, int M, int N, int K) {
    __shared__ __attribute__((aligned(1024))) int8_t sA0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) int8_t sB0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) int8_t sA1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) int8_t sB1[TILE_BYTES];
    // static OSS: the tile's 256 columns of offset, multiplier and k (as
    // int32 each), loaded with the first step, so that the epilogue reads
    // them from LDS (a global load there, issued after earlier stores,
    // would wait for those stores as well: the counter retires in order)
    __shared__ __attribute__((aligned(16))) int32_t sP[OSS ? 3 * BN : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    gemm::tile_coords(blockIdx.x, M / BM, N / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    TileSrc<A_KM> ta;
    TileSrc<B_KM> tb;
    ta.init(A, int(lda), a_bytes, m0, wave, lane);
    tb.init(B, int(ldb), b_bytes, n0, wave, lane);
    FragSrc<A_KM> fa;
    FragSrc<B_KM> fb;
    fa.init(wm * 128, lane);
    fb.init(wn * 128, lane);

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};

    Frags<A_KM, B_KM> F[2];  // fragments of the current / next slice
    const int nk = K / BK;   // even and >= 2 (checked by the caller)

    // Load instruction q (0..15) of this wavefront's share of a step: q < 8
    // are the A tile's, q >= 8 the B tile's; pairs (q, q+1), q even, share m0.
    auto dma1 = [&](int q, int k0, int8_t *Ad, int8_t *Bd) __attribute__((always_inline)) {
        if (q < 8) ta.issue_one(k0, Ad, wave, q);
        else tb.issue_one(k0, Bd, wave, q - 8);
    };
    auto dma2 = [&](int q, int k0, int8_t *Ad, int8_t *Bd) __attribute__((always_inline)) {
        if (q < 8) ta.issue_two(k0, Ad, wave, q);
        else tb.issue_two(k0, Bd, wave, q - 8);
    };

    // Prologue: step 0 -> stage 0, wait, the first 4 loads of step 1 ->
    // stage 1, then the slice-0 fragments of step 0.  No scalar load may be
    // pending into the loop (it would force a full LDS wait at its head).
    ta.issue(0, sA0, wave);
    tb.issue(0, sB0, wave);
    int32_t po = 0, pm = 0, pk = 0;
    if (OSS) {
        po = ep.oss_off[n0 + tid];
        pm = ep.oss_mult[n0 + tid];
        pk = int(uint8_t(ep.oss_k[n0 + tid]));  // k as the byte it is (0..255)
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    if (OSS) {
        sP[tid] = po;
        sP[BN + tid] = pm;
        sP[2 * BN + tid] = pk;
    }
    __builtin_amdgcn_s_barrier();
    dma2(0, BK, sA1, sB1);
    dma2(2, BK, sA1, sB1);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
#pragma unroll
    for (int r = 0; r < 8; ++r) F[0].read(RO[r], sA0, sB0, fa, fb, 0);

    // One K step held in stage (Ac, Bc); stage (An, Bn) receives the next
    // step.  Exactly one memory instruction (a fragment read, or one or two
    // loads under one m0) sits between consecutive MFMAs, so no issue gap is
    // longer than an MFMA and the matrix core never waits on the issue of a
    // load.  Slices 0..2: the next slice's fragment reads, and over slices 0
    // and 1 the remaining 12 loads of the next step (its first 4 went out at
    // the end of the previous step).  Slice 3: groups 0, 1; wait for this
    // wave's loads and reads and meet at the barrier (the next step's data is
    // in, nobody reads this stage any more); then the first 4 loads of step
    // + 2 into this stage and the next step's slice-0 reads, interleaved with
    // groups 2, 3.  Reading the next stage on the last step reads stale LDS,
    // which is harmless and keeps the schedule branch-free.
    auto step = [&](const int8_t *Ac, const int8_t *Bc, const int8_t *An, const int8_t *Bn,
                    int8_t *Adst, int8_t *Bdst, int kt) __attribute__((always_inline)) {
        int8_t *Anw = const_cast<int8_t *>(An), *Bnw = const_cast<int8_t *>(Bn);
        const bool more1 = kt + 1 < nk, more2 = kt + 2 < nk;
#pragma unroll
        for (int sl = 0; sl < 3; ++sl) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = 4 * sl + g;
                mfma_gt(F[sl & 1], g, 0, acc);
                IONN_SCHED_FENCE();
                F[(sl + 1) & 1].read(RO[2 * g], Ac, Bc, fa, fb, sl + 1);
                IONN_SCHED_FENCE();
                mfma_gt(F[sl & 1], g, 1, acc);
                IONN_SCHED_FENCE();
                if (c < 8 && more1) {
                    if (c < 4) dma2(4 + 2 * c, (kt + 1) * BK, Anw, Bnw);
                    else dma1(12 + (c - 4), (kt + 1) * BK, Anw, Bnw);
                }
                IONN_SCHED_FENCE();
                mfma_gt(F[sl & 1], g, 2, acc);
                IONN_SCHED_FENCE();
                F[(sl + 1) & 1].read(RO[2 * g + 1], Ac, Bc, fa, fb, sl + 1);
                IONN_SCHED_FENCE();
                mfma_gt(F[sl & 1], g, 3, acc);
                IONN_SCHED_FENCE();
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) mfma_gt(F[1], t >> 2, t & 3, acc);
        IONN_SCHED_FENCE();
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        IONN_SCHED_FENCE();
#pragma unroll
        for (int g = 2; g < 4; ++g) {
            if (more2) dma2(2 * (g - 2), (kt + 2) * BK, Adst, Bdst);
            IONN_SCHED_FENCE();
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                mfma_gt(F[1], g, t, acc);
                IONN_SCHED_FENCE();
                F[0].read(RO[4 * (g - 2) + t], An, Bn, fa, fb, 0);
                IONN_SCHED_FENCE();
            }
        }
    };

    for (int kt = 0; kt < nk; kt += 2) {
        step(sA0, sB0, sA1, sB1, sA0, sB0, kt);
        step(sA1, sB1, sA0, sB0, sA1, sB1, kt + 1);
    }

    // ---- epilogue: lane holds C[m][n .. n+3] for m = .. + lane % 32 and
    // n = .. + 8 q + 4 (lane / 32), q = 0..3.  The max-abs is taken as the
    // larger magnitude of the running max and min (v_max3 / v_min3 over pairs
    // of values: one instruction per value instead of abs + max per value);
    // |INT32_MIN| = 2^31 is exact in uint32.  Row pointers are formed once
    // per 32-row block; column offsets are immediates. ----
    const int em = lane & 31, en = (lane >> 5) * 4;
    if (OSS) {
        // static OSS: int8 out, four columns per dword; per-column parameters
        // from LDS (the same 16 column groups for every row block)
        const int cl = wn * 128 + en;  // the lane's first column within the tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + wm * 128 + i * 32 + em;
            const int64_t nb = n0 + cl;
            int8_t *orow = ep.out8 + m * ep.ldc + nb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int dn = j * 32 + 8 * q;
                    const v4i o = *reinterpret_cast<const v4i *>(sP + cl + dn);
                    const v4i mu = *reinterpret_cast<const v4i *>(sP + BN + cl + dn);
                    const v4i kk = *reinterpret_cast<const v4i *>(sP + 2 * BN + cl + dn);
                    const int lo = ep.oss_lo;
                    *reinterpret_cast<uint32_t *>(orow + dn) =
                        pack4_u8(oss_elem(acc[i][j][4 * q], o.x, mu.x, kk.x, lo),
                                 oss_elem(acc[i][j][4 * q + 1], o.y, mu.y, kk.y, lo),
                                 oss_elem(acc[i][j][4 * q + 2], o.z, mu.z, kk.z, lo),
                                 oss_elem(acc[i][j][4 * q + 3], o.w, mu.w, kk.w, lo));
                }
            }
        }
        return;
    }
    int32_t vmax = INT32_MIN, vmin = INT32_MAX;
    // ReLU mask: every word of the lane loaded before the first store, so
    // that waiting for a word never waits for a store (the counter retires
    // in order)
    uint32_t mk[RELU ? 4 : 1][RELU ? 16 : 1];
    if (RELU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int8_t *arow = ep.act + (m0 + wm * 128 + i * 32 + em) * ep.ldc + n0 + wn * 128 + en;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    mk[RELU ? i : 0][RELU ? 4 * j + q : 0] = *reinterpret_cast<const uint32_t *>(arow + j * 32 + 8 * q);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + i * 32 + em;
        const int64_t nb = n0 + wn * 128 + en;
        int32_t *row = ep.C + m * ep.ldc + nb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int dn = j * 32 + 8 * q;
                v4i v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                if (RELU) {
                    const uint32_t a = mk[RELU ? i : 0][RELU ? 4 * j + q : 0];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (int8_t(uint8_t(a >> (8 * c))) <= 0) v[c] = 0;
                }
                *reinterpret_cast<v4i *>(row + dn) = v;
                vmax = max(vmax, max(v[0], v[1]));
                vmax = max(vmax, max(v[2], v[3]));
                vmin = min(vmin, min(v[0], v[1]));
                vmin = min(vmin, min(v[2], v[3]));
            }
        }
    }
    if (ep.absmax) {
        uint32_t amax = max(abs_u32(vmax), abs_u32(vmin));
        amax = wave_max_u32(amax);
        if (lane == 0) publish_max_u32(ep.absmax, amax);
    }
}

// ep.out8 selects the static OSS epilogue (int8 out, C unused); ep.act the
// ReLU-masked one (dgrad): C = 0 where act <= 0.
template <bool A_KM, bool B_KM>
void launch(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb, const gemm::Epi &ep, int M,
            int N, int K, hipStream_t st) {
    const uint32_t a_bytes = uint32_t((A_KM ? int64_t(M) : int64_t(K)) * lda);
    const uint32_t b_bytes = uint32_t((B_KM ? int64_t(N) : int64_t(K)) * ldb);
    const dim3 grid((M / BM) * (N / BN)), block(NT);
    if (ep.out8)
        gemm256_kernel<A_KM, B_KM, false, true><<<grid, block, 0, st>>>(A, lda, B, ldb, a_bytes, b_bytes, ep, M, N, K);
    else if (ep.act)
        gemm256_kernel<A_KM, B_KM, true, false><<<grid, block, 0, st>>>(A, lda, B, ldb, a_bytes, b_bytes, ep, M, N, K);
    else
        gemm256_kernel<A_KM, B_KM, false, false><<<grid, block, 0, st>>>(A, lda, B, ldb, a_bytes, b_bytes, ep, M, N, K);
}

}  // namespace g256
}  // namespace ionn
