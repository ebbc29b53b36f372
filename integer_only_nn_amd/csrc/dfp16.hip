// DFP-16 shared-exponent contractions ("Mixed Precision Training of
// Convolutional Neural Networks using Integer Operations", sections 3, 3.1
// and 4 "Handling overflows") and the Gavg metric ("Adaptive Precision
// Training for Resource Constrained Devices", Equation 4).
//
// gfx950 has no int16 matrix instruction, so each int16 mantissa is split
// exactly into two int8 digits: the signed high byte ah = a >> 8 and a low
// digit al from the low byte.  The integer form takes al = 127 - (a & 255),
// so a = 256 ah + 127 - al and every correction term of a 64-term chunk is an
// int8 product against a fragment of -127 (see dfpi_kernel): the matrix
// cores produce H, X2, L2 with p = 65536 H - 256 X2 + L2 (mod 2^32).  The
// FP32 forms and the general-shape kernel take al = (a & 255) - 128, so
// a = 256 ah + al + 128 and
//   sum a*b = 65536*sum(ah*bh) + 256*sum(ah*bl + al*bh) + sum(al*bl)
//             + 128*sum(A') + 128*sum(B') + 2^20                  (mod 2^32)
// with the sums of A' = a - 128 and B' = b - 128 taken on the VALU or against
// an all-ones fragment.  Both splits are exact for every int16, zero
// included, so zero padding contributes exactly 0 and every chunk is
// evaluated as a full 64-term chunk.
//
// Overflow management: each chunk's int32 partial p_c is shifted down by
// r = ceil(log2(number of chunks)) with round-half-up before it joins the
// int32 accumulator, so the sum of chunks stays in range.  The accumulator
// then goes through adaptive down-conversion: Rs = max(0, bitlen(max|acc|)
// - 15), out = sat16(rhu(acc, Rs)), E_out = Ea + Eb + r + Rs.
#include "common.h"

namespace ionn {

int launch_absmax_i32(const int32_t *x, int64_t n, uint32_t *absmax, hipStream_t st);

namespace {

constexpr int kChunk = 64;
constexpr int kPad = 16;

// fl(v * 2^e), one rounding: the product is exact in double (e clamped to
// the double range, where a larger |e| gives the same single result).
__device__ __forceinline__ float scale_f32(float v, int e) {
    e = e < -1022 ? -1022 : (e > 1023 ? 1023 : e);
    return float(double(v) * __longlong_as_double(int64_t(e + 1023) << 52));
}

// rhu(a, 1) of 8 int16 held in a v4i (the input shifted by one bit):
// (a >> 1) + (a & 1) in every 16-bit half, which cannot carry across.
__device__ __forceinline__ v4i rhu1_x8(v4i r) {
    typedef short v2s __attribute__((ext_vector_type(2)));
    int w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const v2s a = __builtin_bit_cast(v2s, w[q]);
        w[q] = __builtin_bit_cast(int, v2s((a >> 1) + (a & 1)));
    }
    return v4i{w[0], w[1], w[2], w[3]};
}

// Split 8 int16 (4 dwords) into 8 high bytes and 8 flipped low bytes.
__device__ __forceinline__ void split8(v4i w, uint32_t &h0, uint32_t &h1, uint32_t &l0,
                                       uint32_t &l1) {
    auto hi = [](uint32_t a, uint32_t b) {
        return ((a >> 8) & 0xffu) | ((a >> 16) & 0xff00u) | ((b << 8) & 0xff0000u) | (b & 0xff000000u);
    };
    auto lo = [](uint32_t a, uint32_t b) {
        return ((a & 0xffu) | ((a >> 8) & 0xff00u) | ((b & 0xffu) << 16) | ((b << 8) & 0xff000000u)) ^
               0x80808080u;
    };
    h0 = hi(uint32_t(w.x), uint32_t(w.y));
    h1 = hi(uint32_t(w.z), uint32_t(w.w));
    l0 = lo(uint32_t(w.x), uint32_t(w.y));
    l1 = lo(uint32_t(w.z), uint32_t(w.w));
}

// K-major int16 operand: element (r, k) at base[r * ld + k].
struct Src16 {
    const int16_t *base;
    int64_t ld;
    int rows, kdim;
    bool vec;  // base 16-byte aligned and ld % 8 == 0
    template <bool EDGE>
    __device__ __forceinline__ v4i chunk(int r, int k) const {  // 8 elements k..k+7
        const int16_t *p = base + int64_t(r) * ld + k;
        if (!EDGE || (r < rows && k + 8 <= kdim && vec)) return *reinterpret_cast<const v4i *>(p);
        uint32_t w[4] = {0, 0, 0, 0};
        if (r < rows)
            for (int e = 0; e < 8; ++e)
                if (k + e < kdim) w[e >> 1] |= uint32_t(uint16_t(p[e])) << (16 * (e & 1));
        return v4i{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
    }
};

// Tile of R rows x 64 k (int16) -> LDS planes hi[R][64+kPad], lo[R][64+kPad].
template <int R, int NT, bool EDGE>
struct Loader16 {
    static constexpr int kChunks = R * kChunk / 8;
    static constexpr int kPer = (kChunks + NT - 1) / NT;
    v4i reg[kPer];
    __device__ __forceinline__ void load(const Src16 &s, int r0, int k0, int tid) {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int id = it * NT + tid;
            v4i v = {0, 0, 0, 0};
            if (kChunks % NT == 0 || id < kChunks) v = s.template chunk<EDGE>(r0 + id / 8, k0 + 8 * (id % 8));
            reg[it] = v;
        }
    }
    __device__ __forceinline__ void rhu1() {
#pragma unroll
        for (int it = 0; it < kPer; ++it) reg[it] = rhu1_x8(reg[it]);
    }
    __device__ __forceinline__ void store(int8_t *hi, int8_t *lo, int tid) const {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int id = it * NT + tid;
            if (kChunks % NT == 0 || id < kChunks) {
                uint32_t h0, h1, l0, l1;
                split8(reg[it], h0, h1, l0, l1);
                const int off = (id / 8) * (kChunk + kPad) + 8 * (id % 8);
                *reinterpret_cast<uint2 *>(hi + off) = make_uint2(h0, h1);
                *reinterpret_cast<uint2 *>(lo + off) = make_uint2(l0, l1);
            }
        }
    }
};

struct DfpArgs {
    Src16 a, b;          // A [M][L], B [N][L], both K-major
    int32_t *acc;        // [M][N], ldc = N
    uint32_t *absmax;    // max-combined (non-atomic epilogue only)
    int M, N, L;
    int r;               // per-chunk shift
    int split;           // K splits (gridDim.y)
    bool atomic;         // accumulate with atomicAdd (split > 1)
    // FP32 form: acc holds floats, [split][M][N] partial sums when split > 1
    // (no atomics: the splits are added in order afterwards), else the
    // result scaled by 2^(*ea + shift + *eb)
    int shift;
    const int32_t *ea, *eb;
    // Blocked-DFP form: exponents bea[m * nch + c], beb[n * nch + c]
    const int32_t *bea, *beb;
    int nch;
};

template <int BM, int BN, int WGM, int WGN, bool EDGE, bool F32, bool BLK = false>
__global__ __launch_bounds__(WGM *WGN * 64) void dfp16_kernel(DfpArgs g) {
    constexpr int NT = WGM * WGN * 64;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int ROW = kChunk + kPad;
    constexpr int PLANE_A = BM * ROW, PLANE_B = BN * ROW;
    constexpr int STAGE = 2 * PLANE_A + 2 * PLANE_B;
    __shared__ __attribute__((aligned(16))) int8_t lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int tiles_n = (g.N + BN - 1) / BN;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nchunks = (g.L + kChunk - 1) / kChunk;
    const int c_begin = int(int64_t(nchunks) * blockIdx.y / g.split);
    const int c_end = int(int64_t(nchunks) * (blockIdx.y + 1) / g.split);

    Loader16<BM, NT, EDGE> la;
    Loader16<BN, NT, EDGE> lb;
    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    if (c_begin < c_end) {
        la.load(g.a, m0, c_begin * kChunk, tid);
        lb.load(g.b, n0, c_begin * kChunk, tid);
        if (F32 && g.shift) la.rhu1();
        la.store(lds, lds + PLANE_A, tid);
        lb.store(lds + 2 * PLANE_A, lds + 2 * PLANE_A + PLANE_B, tid);
    }
    __syncthreads();

    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const v4i zero = {0, 0, 0, 0};
    const int frow = lane & 15, fk = (lane >> 4) * 16;
    const int r = g.r;
    for (int c = c_begin; c < c_end; ++c) {
        const int cur = (c - c_begin) & 1;
        const int8_t *Ah = lds + cur * STAGE, *Al = Ah + PLANE_A;
        const int8_t *Bh = Ah + 2 * PLANE_A, *Bl = Bh + PLANE_B;
        if (c + 1 < c_end) {
            la.load(g.a, m0, (c + 1) * kChunk, tid);
            lb.load(g.b, n0, (c + 1) * kChunk, tid);
        }
        v4i ah[FM], al[FM], rt[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int off = (wm * WTM + i * 16 + frow) * ROW + fk;
            ah[i] = *reinterpret_cast<const v4i *>(Ah + off);
            al[i] = *reinterpret_cast<const v4i *>(Al + off);
            // row sums of A' = 256*ah + al, every value of the fragment is the
            // sum for this lane's row m
            v4i sh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, ah[i], zero, 0, 0, 0);
            v4i sl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, al[i], zero, 0, 0, 0);
            const uint32_t ra = (uint32_t(sh.x) << 8) + uint32_t(sl.x);
            rt[i].x = int(ra * 128u + (1u << 20));
        }
        int32_t eai[FM], ebv[FN][4];
        if (BLK) {  // this chunk's exponents of the lane's rows and columns
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = m0 + wm * WTM + i * 16 + (lane & 15);
                eai[i] = m < g.M ? g.bea[int64_t(m) * g.nch + c] + g.shift : 0;
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = n0 + wn * WTN + j * 16 + (lane >> 4) * 4 + v;
                    ebv[j][v] = n < g.N ? g.beb[int64_t(n) * g.nch + c] : 0;
                }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int off = (wn * WTN + j * 16 + frow) * ROW + fk;
            const v4i bh = *reinterpret_cast<const v4i *>(Bh + off);
            const v4i bl = *reinterpret_cast<const v4i *>(Bl + off);
            // column sums of B' for this lane's four columns
            const v4i ch = __builtin_amdgcn_mfma_i32_16x16x64_i8(bh, ones, zero, 0, 0, 0);
            const v4i cl = __builtin_amdgcn_mfma_i32_16x16x64_i8(bl, ones, zero, 0, 0, 0);
            uint32_t ct[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) ct[v] = ((uint32_t(ch[v]) << 8) + uint32_t(cl[v])) * 128u;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v4i hh = __builtin_amdgcn_mfma_i32_16x16x64_i8(bh, ah[i], zero, 0, 0, 0);
                v4i x = __builtin_amdgcn_mfma_i32_16x16x64_i8(bl, ah[i], zero, 0, 0, 0);
                x = __builtin_amdgcn_mfma_i32_16x16x64_i8(bh, al[i], x, 0, 0, 0);
                const v4i ll = __builtin_amdgcn_mfma_i32_16x16x64_i8(bl, al[i], zero, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t p = (uint32_t(hh[v]) << 16) + (uint32_t(x[v]) << 8) +
                                       uint32_t(ll[v]) + uint32_t(rt[i].x) + ct[v];
                    if (BLK)
                        acc[i][j][v] = __float_as_int(__fadd_rn(
                            __int_as_float(acc[i][j][v]),
                            __builtin_amdgcn_ldexpf(float(int32_t(p)), eai[i] + ebv[j][v])));
                    else if (F32)
                        acc[i][j][v] = __float_as_int(__fadd_rn(__int_as_float(acc[i][j][v]), float(int32_t(p))));
                    else
                        acc[i][j][v] += rhu(int32_t(p), r);
                }
            }
        }
        if (c + 1 < c_end) {
            int8_t *nxt = lds + (cur ^ 1) * STAGE;
            if (F32 && g.shift) la.rhu1();
            la.store(nxt, nxt + PLANE_A, tid);
            lb.store(nxt + 2 * PLANE_A, nxt + 2 * PLANE_A + PLANE_B, tid);
        }
        __syncthreads();
    }

    uint32_t amax = 0;
    const int em = lane & 15, en = (lane >> 4) * 4;
    if (F32) {
        const int e = !BLK && g.split == 1 ? *g.ea + g.shift + *g.eb : 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * WTM + i * 16 + em;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WTN + j * 16 + en;
                float *cp = reinterpret_cast<float *>(g.acc) + (int64_t(blockIdx.y) * g.M + m) * g.N + n;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float f = __int_as_float(acc[i][j][v]);
                    if (m < g.M && n + v < g.N) cp[v] = !BLK && g.split == 1 ? scale_f32(f, e) : f;
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WTM + i * 16 + em;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WTN + j * 16 + en;
            int32_t *cp = g.acc + int64_t(m) * g.N + n;
            if (g.atomic) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (m < g.M && n + v < g.N) atomicAdd(cp + v, acc[i][j][v]);
            } else if (!EDGE || (m < g.M && n + 4 <= g.N)) {
                *reinterpret_cast<v4i *>(cp) = acc[i][j];
#pragma unroll
                for (int v = 0; v < 4; ++v) amax = max(amax, abs_u32(acc[i][j][v]));
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (m < g.M && n + v < g.N) {
                        cp[v] = acc[i][j][v];
                        amax = max(amax, abs_u32(acc[i][j][v]));
                    }
            }
        }
    }
    if (!g.atomic && g.absmax) {
        amax = wave_max_u32(amax);
        if (lane == 0) publish_max_u32(g.absmax, amax);
    }
}

// ---------------------------------------------------------------------------
// Tile-aligned path on v_mfma_i32_32x32x32_i8 (full int8 rate on gfx950).
//
// 128 x 128 output tile per workgroup, 4 wavefronts of 64 x 64 (2 x 2 blocks
// of 32 x 32); one 64-term chunk per K step, double-buffered in LDS as four
// int8 digit planes (A hi/lo, B hi/lo).  A K-major operand lands as
// [row][80 bytes] (16 consecutive rows hit 16 distinct bank groups) and is
// read with ds_read_b128; an M-major operand (dgrad's W, wgrad's dY and X)
// lands as [k][row + 16 bytes] and is read with two ds_read_b64_tr_b8 per
// fragment, so no operand is ever transposed in memory.  The digit split
// happens once per element on the way into LDS (v_perm_b32 picks the high
// and low bytes of four int16 at a time).
//
// Per chunk and 32 x 32 block: 8 MFMAs give sum(ah bh), sum(ah bl + al bh)
// and sum(al bl) over the 64 terms.  The row sums of A' and the column sums
// of B' come from v_dot4 on the fragments (a fragment row is one row or
// column, so each is one value per lane); the column sums then pass through
// a small per-wave LDS row to the lanes that hold those columns in the MFMA
// result.  Per element p = 65536 hh + 256 x + ll + 128 sum A' + 128 sum B' +
// 2^20 (mod 2^32) and acc += rhu(p, r): six VALU operations, the bound of
// this kernel.
// ---------------------------------------------------------------------------
namespace d2 {

typedef int v2i __attribute__((ext_vector_type(2)));
constexpr int BM = 128, BN = 128, NT = 512;  // 8 wavefronts, 2 per SIMD
constexpr int KP = 80;            // K-major plane: bytes per row
constexpr int MP = 128 + 16;      // M-major plane: bytes per k-row
constexpr int PLANE = 128 * KP;   // >= 64 * MP
constexpr int STAGE = 4 * PLANE;

// hi / lo digit bytes of 4 int16 held in two dwords.  The lo digit is the
// low byte with its top bit flipped (low - 128) for the FP32 forms, or with
// its low 7 bits flipped (127 - low) for the integer form (lox selects).
__device__ __forceinline__ uint32_t hi4(uint32_t w0, uint32_t w1) { return __builtin_amdgcn_perm(w1, w0, 0x07050301u); }
__device__ __forceinline__ uint32_t lo4(uint32_t w0, uint32_t w1, uint32_t lox = 0x80808080u) {
    return __builtin_amdgcn_perm(w1, w0, 0x06040200u) ^ lox;
}

// One operand tile (128 rows x 64 k of int16) global -> registers -> digit planes.
template <bool KM>
struct Ld {
    static constexpr int IT = 128 * 64 / 8 / NT;  // 16-byte chunks per thread
    v4i reg[IT];
    __device__ __forceinline__ void load(const int16_t *base, int64_t ld, int r0, int k0, int tid) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int id = it * NT + tid;
            const int16_t *p = KM ? base + int64_t(r0 + (id >> 3)) * ld + k0 + 8 * (id & 7)
                                  : base + int64_t(k0 + (id >> 4)) * ld + r0 + 8 * (id & 15);
            reg[it] = *reinterpret_cast<const v4i *>(p);
        }
    }
    __device__ __forceinline__ void rhu1() {
#pragma unroll
        for (int it = 0; it < IT; ++it) reg[it] = rhu1_x8(reg[it]);
    }
    __device__ __forceinline__ void store(int8_t *hi, int8_t *lo, int tid, uint32_t lox = 0x80808080u) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int id = it * NT + tid;
            const int off = KM ? (id >> 3) * KP + 8 * (id & 7) : (id >> 4) * MP + 8 * (id & 15);
            const uint32_t w0 = reg[it].x, w1 = reg[it].y, w2 = reg[it].z, w3 = reg[it].w;
            *reinterpret_cast<uint2 *>(hi + off) = make_uint2(hi4(w0, w1), hi4(w2, w3));
            *reinterpret_cast<uint2 *>(lo + off) = make_uint2(lo4(w0, w1, lox), lo4(w2, w3, lox));
        }
    }
};

// Fragment of rows rb0 .. rb0+31, k = 32 kh + 16 (lane / 32) .. +15.
template <bool KM>
__device__ __forceinline__ v4i frag(const int8_t *plane, int rb0, int kh, int lane) {
    if (KM) return *reinterpret_cast<const v4i *>(plane + (rb0 + (lane & 31)) * KP + 32 * kh + 16 * (lane >> 5));
    typedef __attribute__((address_space(3))) v2i lds_v2i_t;
    const int g = lane >> 4, i = lane & 15;
    const int8_t *p = plane + (32 * kh + 16 * (g >> 1) + (i >> 1)) * MP + rb0 + 16 * (g & 1) + 8 * (i & 1);
    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p));
    const v2i y = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p + 8 * MP));
    return v4i{x.x, x.y, y.x, y.y};
}

__device__ __forceinline__ int32_t dot16(v4i f, int32_t s) {  // s + sum of the 16 signed bytes
    s = __builtin_amdgcn_sdot4(f.x, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(f.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(f.z, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(f.w, 0x01010101, s, false);
    return s;
}

// v + (the same value in lane l ^ 32)
__device__ __forceinline__ uint32_t add_half_swap(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] + r[1];
}

// Makes v opaque to the optimiser (no instruction): keeps (a << s) + v as one
// v_lshl_add_u32 instead of letting the compiler fold v's adds into a v_add3
// and leave the shift on its own.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

struct Args {
    const int16_t *a, *b;
    int64_t lda, ldb;
    int32_t *acc;        // [M][N] (split == 1) or split partial tiles [split][M][N]
    uint32_t *absmax;    // max-combined (split == 1)
    int M, N, L, r, split;
    // FP32 form only: A's one-bit shift and the exponents of the final
    // scaling 2^(*ea + shift + *eb) (split == 1; acc then holds floats)
    int shift;
    const int32_t *ea, *eb;
    // Blocked-DFP form: one exponent per row and 64-term chunk,
    // bea[m * nch + c] and beb[n * nch + c]; each chunk's term is scaled on
    // its own and the output is not scaled again
    const int32_t *bea, *beb;
    int nch;
    // Block-shift int16 form (integer, split == 1): each wavefront's 32 x 64
    // block of acc gets its own shift s_b = max(0, bitlen(max |acc|) - 15);
    // out16 [M][N] receives asr(acc, s_b), bits the rounding bits (bit
    // 16 j + v of word blk * 64 + lane for value v of column block j), shifts
    // s_b of block blk = tile * 8 + wave, slots max |acc| of each workgroup
    int16_t *out16;
    uint32_t *bits;
    int32_t *shifts;
    uint32_t *slots;
};


// FP32 forms (digits with lo = low byte - 128, corrections from the digit
// sums on the VALU).  Persistent: workgroup w takes work units w,
// w + gridDim.x, ...; a unit is one output tile and one range of chunks (a K
// split).  The chunk loop runs across unit boundaries, so the first chunk of
// the next unit is loaded while the last chunk of the current one computes and
// its result is stored.
template <bool A_KM, bool B_KM, bool BLK = false>
__global__ __launch_bounds__(NT, 1) void dfp_kernel(Args g) {
    __shared__ __attribute__((aligned(16))) int8_t lds[2 * STAGE];
    // Blocked form, per stage: the chunk's exponents of the tile's 128 rows
    // of A, then of its 128 rows of B
    __shared__ __attribute__((aligned(16))) int32_t bexp[BLK ? 2 : 1][BLK ? 256 : 4];
    __shared__ __attribute__((aligned(16))) uint32_t csum[NT / 64][64];  // per wave: 128 * sum(B') of its 64 columns
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;  // 32-row block wm of 4, 64-column half wn of 2
    const int tiles_n = g.N / BN;
    const int ntiles = (g.M / BM) * tiles_n;
    const int nunits = ntiles * g.split;
    const int nch = g.L / 64;

    // unit u -> tile origin and chunk range
    auto unit = [&](int u, int &m0, int &n0, int &c0, int &c1) __attribute__((always_inline)) {
        const int t = u % ntiles, sp = u / ntiles;
        const int tm = t / tiles_n;
        m0 = tm * BM;
        n0 = (t - tm * tiles_n) * BN;
        c0 = int(int64_t(nch) * sp / g.split);
        c1 = int(int64_t(nch) * (sp + 1) / g.split);
    };

    int u = blockIdx.x;
    if (u >= nunits) return;
    int m0, n0, c0, c1;
    unit(u, m0, n0, c0, c1);

    Ld<A_KM> la;
    Ld<B_KM> lb;
    v16i acc[2];
    acc[0] = v16i{};
    acc[1] = v16i{};

    int32_t ereg = 0;
    auto eload = [&](int em0, int en0, int ec) __attribute__((always_inline)) {
        if (tid < 128) ereg = g.bea[int64_t(em0 + tid) * g.nch + ec];
        else if (tid < 256) ereg = g.beb[int64_t(en0 + tid - 128) * g.nch + ec];
    };
    la.load(g.a, g.lda, m0, 64 * c0, tid);
    lb.load(g.b, g.ldb, n0, 64 * c0, tid);
    // the output exponent of the one-range form, read once here: read at
    // each store, the compiler reloads it after every earlier store (which
    // might alias it) and waits for that store with it
    const int e_out = !BLK && g.split == 1 ? *g.ea + g.shift + *g.eb : 0;
    if (BLK) {
        eload(m0, n0, c0);
        if (tid < 256) bexp[0][tid] = ereg;
    }
    if (g.shift) la.rhu1();
    la.store(lds, lds + PLANE, tid);
    lb.store(lds + 2 * PLANE, lds + 3 * PLANE, tid);
    __syncthreads();

    const v16i zero16 = {};
    int c = c0, stage = 0;
    while (true) {
        // the work item after (u, c)
        int nu = u, nm0 = m0, nn0 = n0, nc = c + 1, nc1 = c1;
        bool more = true;
        if (nc >= c1) {
            nu = u + gridDim.x;
            more = nu < nunits;
            if (more) unit(nu, nm0, nn0, nc, nc1);
        }
        if (more) {
            la.load(g.a, g.lda, nm0, 64 * nc, tid);
            lb.load(g.b, g.ldb, nn0, 64 * nc, tid);
            if (BLK) eload(nm0, nn0, nc);
        }
        const int8_t *st = lds + stage * STAGE;
        v4i ah[2], al[2], bh[2][2], bl[2][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            ah[kh] = frag<A_KM>(st, 32 * wm, kh, lane);
            al[kh] = frag<A_KM>(st + PLANE, 32 * wm, kh, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bh[j][kh] = frag<B_KM>(st + 2 * PLANE, 64 * wn + 32 * j, kh, lane);
                bl[j][kh] = frag<B_KM>(st + 3 * PLANE, 64 * wn + 32 * j, kh, lane);
            }
        }
        // Sums over the chunk's 64 terms (lanes l and l + 32 hold the two
        // 16-term halves of a fragment row): 128 * sum(A') + 2^20 for this
        // lane's row, and 128 * sum(B') for column 32 j + lane % 32 of the
        // wave's half, which goes through the wave's own LDS row to reach the
        // lanes that hold that column in the MFMA result layout.
        // (256 sum(hi digits) + sum(lo digits)) over the lane's 32 terms
        const uint32_t sa = dot16(al[1], dot16(al[0], int32_t(uint32_t(dot16(ah[1], dot16(ah[0], 0))) << 8)));
        const uint32_t rt = (add_half_swap(sa) << 7) + (1u << 20);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t sb =
                dot16(bl[j][1], dot16(bl[j][0], int32_t(uint32_t(dot16(bh[j][1], dot16(bh[j][0], 0))) << 8)));
            const uint32_t cs = add_half_swap(sb);
            csum[wave][32 * j + (lane & 31)] = cs << 7;  // lanes l and l + 32 hold the same value
        }
        const int32_t ea_lane = BLK ? bexp[BLK ? stage : 0][32 * wm + (lane & 31)] + g.shift : 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            v4i cb[4], eb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cb[q] = *reinterpret_cast<const v4i *>(&csum[wave][32 * j + 8 * q + 4 * (lane >> 5)]);
                if (BLK)
                    eb[q] = *reinterpret_cast<const v4i *>(
                        &bexp[BLK ? stage : 0][128 + 64 * wn + 32 * j + 8 * q + 4 * (lane >> 5)]);
            }
            v16i hh = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][0], ah[0], zero16, 0, 0, 0);
            hh = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][1], ah[1], hh, 0, 0, 0);
            v16i x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][0], ah[0], zero16, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][0], al[0], x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][1], ah[1], x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][1], al[1], x, 0, 0, 0);
            v16i ll = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][0], al[0], zero16, 0, 0, 0);
            ll = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][1], al[1], ll, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                // p mod 2^32, then acc = fl(acc + fl(float(p)))
                const uint32_t t = opaque((uint32_t(x[v]) << 8) + uint32_t(ll[v]));
                const uint32_t p = (uint32_t(hh[v]) << 16) + opaque(t + rt + uint32_t(cb[v >> 2][v & 3]));
                if (BLK)  // the chunk's term scaled on its own (v_ldexp_f32: one rounding)
                    acc[j][v] = __float_as_int(__fadd_rn(
                        __int_as_float(acc[j][v]),
                        __builtin_amdgcn_ldexpf(float(int32_t(p)), ea_lane + eb[v >> 2][v & 3])));
                else
                    acc[j][v] = __float_as_int(__fadd_rn(__int_as_float(acc[j][v]), float(int32_t(p))));
            }
        }

        // the prefetched chunk goes to the other stage before the unit's
        // stores are issued, so its wait does not include them
        int8_t *nx = lds + (stage ^ 1) * STAGE;
        if (more) {
            if (g.shift) la.rhu1();
            la.store(nx, nx + PLANE, tid);
            lb.store(nx + 2 * PLANE, nx + 3 * PLANE, tid);
            if (BLK && tid < 256) bexp[BLK ? stage ^ 1 : 0][tid] = ereg;
        }
        if (c + 1 >= c1) {
            // unit done: lane holds acc[m][n .. n+3] for m = row lane % 32 of the
            // wave's block, n = block col 8 q + 4 (lane / 32)
            const int m = m0 + 32 * wm + (lane & 31);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + 64 * wn + 32 * j + 8 * q + 4 * (lane >> 5);
                    int32_t *cp = g.acc + (int64_t(u / ntiles) * g.M + m) * g.N + n;
                    v4i v = {acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
                    if (!BLK && g.split == 1) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[i] = __float_as_int(scale_f32(__int_as_float(v[i]), e_out));
                    }
                    *reinterpret_cast<v4i *>(cp) = v;
                }
                acc[j] = v16i{};
            }
        }
        if (!more) break;
        __syncthreads();
        u = nu; m0 = nm0; n0 = nn0; c = nc; c1 = nc1; stage ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Integer form, corrections on the matrix cores.  With the lo digit
// al = 127 - (a & 255) (in [-128, 127]), a = 256 ah + 127 - al and per term
//   a b = 65536 ah bh - 256 (ah bl + al bh - 127 ah - 127 bh)
//         + (al bl - 127 al - 127 bl) + 127^2,
// so over a 64-term chunk, with every correction an int8 product against a
// fragment of -127:
//   H  = 16 + sum ah bh
//   X2 = 64 + sum (ah bl + al bh) + sum (-127) ah + sum (-127) bh
//   L2 = 64 + sum al bl + sum (-127) al + sum (-127) bl
//   p  = 65536 H - 256 X2 + L2                                  (mod 2^32)
// (the constants 16, 64, 64 are the accumulators' starting values and sum to
// 65536*16 - 256*64 + 64 = 64 * 127^2).  |X2| < 2^23, so L2 - 256 X2 is one
// 24-bit multiply-add; |H| < 2^21.  Per output and chunk the VALU does 5
// operations: the two of p, and acc += (p >> r) + bit (r - 1) of p.
// ---------------------------------------------------------------------------
template <bool A_KM, bool B_KM, bool B16>
__global__ __launch_bounds__(NT, 1) void dfpi_kernel(Args g) {
    __shared__ __attribute__((aligned(16))) int8_t lds[2 * STAGE];
    __shared__ uint32_t wmax[NT / 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;  // 32-row block wm of 4, 64-column half wn of 2
    const int tiles_n = g.N / BN;
    const int ntiles = (g.M / BM) * tiles_n;
    const int nunits = ntiles * g.split;
    const int nch = g.L / 64;
    constexpr uint32_t LOX = 0x7f7f7f7fu;

    auto unit = [&](int u, int &m0, int &n0, int &c0, int &c1) __attribute__((always_inline)) {
        const int t = u % ntiles, sp = u / ntiles;
        const int tm = t / tiles_n;
        m0 = tm * BM;
        n0 = (t - tm * tiles_n) * BN;
        c0 = int(int64_t(nch) * sp / g.split);
        c1 = int(int64_t(nch) * (sp + 1) / g.split);
    };

    int u = blockIdx.x;
    if (u >= nunits) return;
    int m0, n0, c0, c1;
    unit(u, m0, n0, c0, c1);

    Ld<A_KM> la;
    Ld<B_KM> lb;
    v16i acc[2];
    acc[0] = v16i{};
    acc[1] = v16i{};
    uint32_t amax = 0;
    la.load(g.a, g.lda, m0, 64 * c0, tid);
    lb.load(g.b, g.ldb, n0, 64 * c0, tid);
    la.store(lds, lds + PLANE, tid, LOX);
    lb.store(lds + 2 * PLANE, lds + 3 * PLANE, tid, LOX);
    __syncthreads();

    const v4i cm = {int(0x81818181u), int(0x81818181u), int(0x81818181u), int(0x81818181u)};  // -127 bytes
    const v16i c16 = {16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16};
    const v16i c64 = {64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64};
    const int r = g.r;
    const uint32_t rm1 = r > 0 ? r - 1 : 0, rw = r > 0 ? 1 : 0;  // rounding bit (none for r = 0)
    // -256 kept opaque, so that L2 - 256 X2 stays one v_mad_i32_i24 instead
    // of a shift and a subtraction
    int m256 = -256;
    asm volatile("" : "+s"(m256));
    int c = c0, stage = 0;
    while (true) {
        int nu = u, nm0 = m0, nn0 = n0, nc = c + 1, nc1 = c1;
        bool more = true;
        if (nc >= c1) {
            nu = u + gridDim.x;
            more = nu < nunits;
            if (more) unit(nu, nm0, nn0, nc, nc1);
        }
        if (more) {
            la.load(g.a, g.lda, nm0, 64 * nc, tid);
            lb.load(g.b, g.ldb, nn0, 64 * nc, tid);
        }
        const int8_t *st = lds + stage * STAGE;
        v4i ah[2], al[2], bh[2][2], bl[2][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            ah[kh] = frag<A_KM>(st, 32 * wm, kh, lane);
            al[kh] = frag<A_KM>(st + PLANE, 32 * wm, kh, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bh[j][kh] = frag<B_KM>(st + 2 * PLANE, 64 * wn + 32 * j, kh, lane);
                bl[j][kh] = frag<B_KM>(st + 3 * PLANE, 64 * wn + 32 * j, kh, lane);
            }
        }
        // the row corrections of A (sum (-127) ah, sum (-127) al over the
        // chunk) are the same for both column blocks: formed once, with the
        // starting value 64, and the start of both blocks' X2 and L2 chains
        v16i rx = __builtin_amdgcn_mfma_i32_32x32x32_i8(cm, ah[0], c64, 0, 0, 0);
        v16i rl = __builtin_amdgcn_mfma_i32_32x32x32_i8(cm, al[0], c64, 0, 0, 0);
        rx = __builtin_amdgcn_mfma_i32_32x32x32_i8(cm, ah[1], rx, 0, 0, 0);
        rl = __builtin_amdgcn_mfma_i32_32x32x32_i8(cm, al[1], rl, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            v16i h = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][0], ah[0], c16, 0, 0, 0);
            v16i x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][0], ah[0], rx, 0, 0, 0);
            v16i l = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][0], al[0], rl, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][0], al[0], x, 0, 0, 0);
            h = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][1], ah[1], h, 0, 0, 0);
            l = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][0], cm, l, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][0], cm, x, 0, 0, 0);
            l = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][1], al[1], l, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][1], ah[1], x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][1], al[1], x, 0, 0, 0);
            l = __builtin_amdgcn_mfma_i32_32x32x32_i8(bl[j][1], cm, l, 0, 0, 0);
            x = __builtin_amdgcn_mfma_i32_32x32x32_i8(bh[j][1], cm, x, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const uint32_t p = (uint32_t(h[v]) << 16) + opaque(uint32_t(__mul24(x[v], m256) + l[v]));
                acc[j][v] = int32_t(uint32_t(acc[j][v]) + uint32_t(int32_t(p) >> r) + __builtin_amdgcn_ubfe(p, rm1, rw));
            }
        }

        // the prefetched chunk goes to the other stage before the unit's
        // stores are issued, so its wait does not include them
        int8_t *nx = lds + (stage ^ 1) * STAGE;
        if (more) {
            la.store(nx, nx + PLANE, tid, LOX);
            lb.store(nx + 2 * PLANE, nx + 3 * PLANE, tid, LOX);
        }
        if (B16 && c + 1 >= c1) {
            // unit done, block-shift form: the shift of the wave's block, then
            // int16 asr(acc, s_b); lanes l and l + 32 trade halves so that each
            // stores 8 consecutive columns (16 bytes)
            uint32_t bm = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) bm = max(bm, abs_u32(acc[j][v]));
            bm = wave_max_u32(bm);
            amax = max(amax, bm);
            const int sb = niti_shift(bm, 15);
            const uint32_t sm1 = sb > 0 ? sb - 1 : 0, sw = sb > 0 ? 1 : 0;
            const int blk = ((m0 / BM) * tiles_n + n0 / BN) * 8 + wave;
            const int m = m0 + 32 * wm + (lane & 31);
            uint32_t bw = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint32_t pk[8];  // int16 pairs, two words per column group q
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    bw |= __builtin_amdgcn_ubfe(uint32_t(acc[j][v]), sm1, sw) << (16 * j + v);
                    bw |= __builtin_amdgcn_ubfe(uint32_t(acc[j][v + 1]), sm1, sw) << (16 * j + v + 1);
                    pk[v >> 1] = __builtin_amdgcn_perm(uint32_t(acc[j][v + 1] >> sb), uint32_t(acc[j][v] >> sb),
                                                       0x05040100u);
                }
#pragma unroll
                for (int pq = 0; pq < 2; ++pq) {
                    const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * pq], pk[4 * pq + 2], false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * pq + 1], pk[4 * pq + 3], false, false);
                    const int n = n0 + 64 * wn + 32 * j + 8 * (2 * pq + (lane >> 5));
                    *reinterpret_cast<v4i *>(g.out16 + int64_t(m) * g.N + n) =
                        v4i{int(s0[0]), int(s1[0]), int(s0[1]), int(s1[1])};
                }
                acc[j] = v16i{};
            }
            g.bits[int64_t(blk) * 64 + lane] = bw;
            if (lane == 0) g.shifts[blk] = sb;
        }
        if (!B16 && c + 1 >= c1) {
            // unit done (K-split partial tiles): lane holds acc[m][n .. n+3] for
            // m = row lane % 32 of the wave's block, n = block col 8 q + 4 (lane / 32)
            const int m = m0 + 32 * wm + (lane & 31);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + 64 * wn + 32 * j + 8 * q + 4 * (lane >> 5);
                    int32_t *cp = g.acc + (int64_t(u / ntiles) * g.M + m) * g.N + n;
                    *reinterpret_cast<v4i *>(cp) = v4i{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2],
                                                       acc[j][4 * q + 3]};
                }
                acc[j] = v16i{};
            }
        }
        if (!more) break;
        __syncthreads();
        u = nu; m0 = nm0; n0 = nn0; c = nc; c1 = nc1; stage ^= 1;
    }
    if (B16) {  // the workgroup's max |acc| to its slot
        if (lane == 0) wmax[wave] = amax;
        __syncthreads();
        if (tid == 0) {
            uint32_t mx = 0;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) mx = max(mx, wmax[w]);
            g.slots[blockIdx.x] = mx;
        }
    }
}


// FP32 form: out[e] = fl(total * 2^(*ea + shift + *eb)) with total the split
// partial sums added in split order to 0.
__global__ __launch_bounds__(256) void split_reduce_f32(const float *__restrict__ part, int split, int64_t n,
                                                        float *__restrict__ out, const int32_t *__restrict__ ea,
                                                        int shift, const int32_t *__restrict__ eb) {
    const int e = ea ? *ea + shift + *eb : 0;  // no exponents: the blocked form, already scaled
    const int64_t nt = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += nt) {
        float s = 0.0f;
        for (int p = 0; p < split; ++p) s = __fadd_rn(s, __builtin_nontemporal_load(part + int64_t(p) * n + i));
        out[i] = scale_f32(s, e);
    }
}

// acc[e] = sum over the split partial tiles (modulo 2^32), with the max |acc|
// of each workgroup in slots[blockIdx.x].
__global__ __launch_bounds__(256) void split_reduce(const int32_t *__restrict__ part, int split, int64_t n,
                                                    int32_t *__restrict__ acc, uint32_t *__restrict__ slots) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    __shared__ uint32_t red[4];
    uint32_t amax = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; 4 * i < n; i += int64_t(gridDim.x) * blockDim.x) {
        v4u s = {0, 0, 0, 0};
#pragma unroll 8
        for (int p = 0; p < split; ++p) s += __builtin_nontemporal_load(reinterpret_cast<const v4u *>(part + int64_t(p) * n + 4 * i));
        *reinterpret_cast<v4u *>(acc + 4 * i) = s;
        amax = max(max(amax, max(abs_u32(int32_t(s.x)), abs_u32(int32_t(s.y)))),
                   max(abs_u32(int32_t(s.z)), abs_u32(int32_t(s.w))));
    }
    amax = wave_max_u32(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) slots[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

}  // namespace d2

// The max over nslots per-workgroup maxima, for every thread of a block of
// at most 256 threads (1D or 2D; waves are taken in linear thread order).
__device__ __forceinline__ uint32_t slots_max(const uint32_t *__restrict__ slots, int nslots) {
    __shared__ uint32_t red[4];
    const int t = threadIdx.y * blockDim.x + threadIdx.x, nt = blockDim.x * blockDim.y;
    uint32_t mx = 0;
    for (int i = t; i < nslots; i += nt) mx = max(mx, slots[i]);
    mx = wave_max_u32(mx);
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    const int nw = (nt + 63) >> 6;
    uint32_t r = red[0];
    for (int w = 1; w < nw; ++w) r = max(r, red[w]);
    return r;
}

// Block-shift form, second pass (in place over out [M][N], tile-aligned):
// with Rs = max(0, bitlen(max |acc|) - 15) from the workgroup maxima and s_b
// the shift of the element's block, d = Rs - s_b >= 0 and
//   rhu(acc, Rs) = sat16(f + bit)    for d = 0  (f = asr(acc, s_b), bit = bit s_b - 1 of acc)
//                = rhu(f, d)          for d > 0  (the bits of acc below s_b cannot reach
//                                                 the rounding position s_b + d - 1)
// A thread takes 8 consecutive columns (16 bytes) of a row, as int16 pairs:
// the pair arithmetic never carries across halves (|rhu(f, d)| <= 2^14; the
// d = 0 sum saturates per half).  Threads (x, y) of a block cover column
// groups x and rows y; exponent bookkeeping as in the two-pass form.
__global__ __launch_bounds__(256) void block16_fix_kernel(int16_t *__restrict__ out, int M, int N,
                                                          const uint32_t *__restrict__ bits,
                                                          const int32_t *__restrict__ shifts,
                                                          const uint32_t *__restrict__ slots, int nslots,
                                                          const int32_t *__restrict__ ea,
                                                          const int32_t *__restrict__ eb, int r,
                                                          int32_t *__restrict__ e_out,
                                                          int32_t *__restrict__ status) {
    typedef short v2s __attribute__((ext_vector_type(2)));
    const int rs = niti_shift(slots_max(slots, nslots), 15);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && threadIdx.y == 0) {
        const int e = *ea + *eb + r + rs;
        *e_out = e;
        if (status) *status = (e < -128 || e > 127) ? 1 : 0;
    }
    const uint32_t cpr = uint32_t(N) >> 3, tiles_n = uint32_t(N) >> 7;
    const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= cpr) return;
    const uint32_t n = c << 3;
    const uint32_t pos = 16 * ((n >> 5) & 1) + 4 * ((n >> 3) & 3);
    for (uint32_t m = blockIdx.y * blockDim.y + threadIdx.y; m < uint32_t(M); m += gridDim.y * blockDim.y) {
        const uint32_t blk = ((m >> 7) * tiles_n + (n >> 7)) * 8 + ((m >> 5) & 3) * 2 + ((n >> 6) & 1);
        const int d = rs - shifts[blk];
        v4i *p = reinterpret_cast<v4i *>(out + int64_t(m) * N + n);
        const v4i x = *p;
        v4i y;
        if (d == 0) {
            // pair q of the 8 columns: bits 2 (q & 1) and 2 (q & 1) + 1 of the
            // word of lane m % 32 (q < 2) or m % 32 + 32 (q >= 2)
            const uint32_t b0 = bits[blk * 64 + (m & 31)] >> pos, b1 = bits[blk * 64 + 32 + (m & 31)] >> pos;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t bw = (q < 2 ? b0 : b1) >> (2 * (q & 1));
                const v2s bit = __builtin_bit_cast(v2s, (bw & 1u) | ((bw & 2u) << 15));
                const int xq = x[q];  // a scalar copy: bit_cast of a vector element reads element 0
                y[q] = __builtin_bit_cast(int, __builtin_elementwise_add_sat(__builtin_bit_cast(v2s, xq), bit));
            }
        } else if (d < 16) {
            // packed 16-bit shifts take their count modulo 16, so d < 16 here
            const v2s dv = {short(d), short(d)}, dm = {short(d - 1), short(d - 1)}, one = {1, 1};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int xq = x[q];
                const v2s f = __builtin_bit_cast(v2s, xq);
                y[q] = __builtin_bit_cast(int, v2s((f >> dv) + ((f >> dm) & one)));
            }
        } else {
            // |f| <= 2^15 and d >= 16: f + 2^(d-1) lies in [0, 2^d), so rhu(f, d) = 0
            y = v4i{0, 0, 0, 0};
        }
        *p = y;
    }
}

// out = sat16(rhu(acc, Rs)), Rs from the tensor max (the max over nslots
// partial maxima); exponent bookkeeping.
__global__ __launch_bounds__(256) void downconvert_kernel(const int32_t *__restrict__ acc, int64_t n,
                                                          const uint32_t *__restrict__ slots, int nslots,
                                                          const int32_t *__restrict__ ea,
                                                          const int32_t *__restrict__ eb, int r,
                                                          int16_t *__restrict__ out,
                                                          int32_t *__restrict__ e_out,
                                                          int32_t *__restrict__ status) {
    const int rs = niti_shift(slots_max(slots, nslots), 15);
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nt = int64_t(gridDim.x) * blockDim.x;
    if (tid == 0) {
        const int e = *ea + *eb + r + rs;
        *e_out = e;
        if (status) *status = (e < -128 || e > 127) ? 1 : 0;
    }
    const int64_t n8 = n / 8;
    const v4i *av = reinterpret_cast<const v4i *>(acc);
    v4i *ov = reinterpret_cast<v4i *>(out);
    for (int64_t g = tid; g < n8; g += nt) {
        const v4i a0 = av[2 * g], a1 = av[2 * g + 1];
        auto q = [&](int32_t v) { return uint32_t(uint16_t(int16_t(sat16(rhu(v, rs))))); };
        ov[g] = v4i{int(q(a0.x) | (q(a0.y) << 16)), int(q(a0.z) | (q(a0.w) << 16)),
                    int(q(a1.x) | (q(a1.y) << 16)), int(q(a1.z) | (q(a1.w) << 16))};
    }
    for (int64_t i = n8 * 8 + tid; i < n; i += nt) out[i] = int16_t(sat16(rhu(acc[i], rs)));
}

// dst[c][r] = src[r][c] for an R x C int16 matrix (64x64 tiles through LDS).
__global__ __launch_bounds__(256) void transpose16_kernel(const int16_t *__restrict__ src,
                                                          int16_t *__restrict__ dst, int R, int C) {
    __shared__ int16_t t[64][65];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4)
        if (r0 + i < R && c0 + tx < C) t[i][tx] = src[int64_t(r0 + i) * C + c0 + tx];
    __syncthreads();
    for (int i = ty; i < 64; i += 4)
        if (c0 + i < C && r0 + tx < R) dst[int64_t(c0 + i) * R + r0 + tx] = t[tx][i];
}

__global__ void zero_i32_kernel(int32_t *C, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        C[i] = 0;
}

// Gavg in three stream-ordered steps, exact: the output's 8 bytes first hold
// the int64 sum of |g| (zeroed, then one atomic add per workgroup; integer
// sums are order-free), then the last step turns the sum into
// mean(|g|) * 2^(E_g - E_w) as a double.
__global__ void gavg_zero_kernel(unsigned long long *acc) { *acc = 0ull; }

__global__ __launch_bounds__(256) void gavg_sum_kernel(const int16_t *__restrict__ g, int64_t n,
                                                       unsigned long long *__restrict__ acc) {
    __shared__ int64_t part[4];
    int64_t s = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int32_t v = g[i];
        s += v < 0 ? -v : v;
    }
    s = wave_sum_i64(s);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int64_t tot = part[0] + part[1] + part[2] + part[3];
        if (tot) atomicAdd(acc, (unsigned long long)tot);
    }
}

// mean(|g|) * 2^(E_g - E_w) from the exact sum (one rounding in the
// division; the power-of-two scaling is exact short of the double range).
__device__ double gavg_value(int64_t tot, int64_t n, const int32_t *__restrict__ eg, const int32_t *__restrict__ ew) {
    double v = double(tot) / double(n);
    int e = *eg - *ew;
    for (; e > 0; --e) v *= 2.0;
    for (; e < 0; ++e) v *= 0.5;
    return v;
}

__global__ void gavg_finish_kernel(double *out, int64_t n, const int32_t *__restrict__ eg,
                                   const int32_t *__restrict__ ew) {
    *out = gavg_value(int64_t(*reinterpret_cast<const unsigned long long *>(out)), n, eg, ew);
}

// The whole Gavg in one workgroup, for tensors small enough that one compute
// unit streams them faster than three dependent launches complete.
constexpr int64_t kGavgOneBlock = int64_t(1) << 21;

__global__ __launch_bounds__(1024) void gavg_one_kernel(const int16_t *__restrict__ g, int64_t n, double *out,
                                                        const int32_t *__restrict__ eg,
                                                        const int32_t *__restrict__ ew) {
    __shared__ int64_t part[16];
    int64_t s = 0;
    const int64_t n8 = n / 8;
    const v4i *gv = reinterpret_cast<const v4i *>(g);
    auto add8 = [&](const v4i w) {
        int32_t t = 0;  // 8 magnitudes below 2^15 each
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int32_t lo = int32_t(uint32_t(w[q]) << 16) >> 16, hi = w[q] >> 16;
            t += (lo < 0 ? -lo : lo) + (hi < 0 ? -hi : hi);
        }
        s += t;
    };
    int64_t i = threadIdx.x;
    for (; i + 7 * 1024 < n8; i += 8 * 1024) {  // eight 16-byte loads in flight per thread
        v4i w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = gv[i + k * 1024];
#pragma unroll
        for (int k = 0; k < 8; ++k) add8(w[k]);
    }
    for (; i < n8; i += 1024) add8(gv[i]);
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += 1024) {
        const int32_t v = g[i];
        s += v < 0 ? -v : v;
    }
    s = wave_sum_i64(s);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t tot = 0;
        for (int w = 0; w < 16; ++w) tot += part[w];
        *out = gavg_value(tot, n, eg, ew);
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int chunk_shift(int64_t L) {
    const int64_t nc = (L + kChunk - 1) / kChunk;
    int r = 0;
    while ((int64_t(1) << r) < nc) ++r;
    return nc <= 1 ? 0 : r;
}

// acc[M][N] = sum_c rhu(p_c, r) for A [M][L], B [N][L] (K-major int16).
int contract(const Src16 &a, const Src16 &b, int M, int N, int L, int32_t *acc, uint32_t *absmax,
             hipStream_t st) {
    DfpArgs g{a, b, acc, absmax, M, N, L, chunk_shift(L), 1, false, 0, nullptr, nullptr};
    const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
    const int nchunks = (L + kChunk - 1) / kChunk;
    if (tiles < 512 && nchunks >= 16) {
        int split = (1024 + tiles - 1) / tiles;
        if (split > nchunks / 4) split = nchunks / 4;
        g.split = split < 1 ? 1 : split;
    }
    g.atomic = g.split > 1;
    if (g.atomic) {
        zero_i32_kernel<<<dim3(1024), dim3(256), 0, st>>>(acc, int64_t(M) * N);
        if (int rc = check_launch("dfp16 contraction")) return rc;
    }
    const bool even = M % 128 == 0 && N % 128 == 0 && L % kChunk == 0 && a.vec && b.vec;
    dim3 grid(tiles, g.split), block(256);
    if (even) dfp16_kernel<128, 128, 2, 2, false, false><<<grid, block, 0, st>>>(g);
    else dfp16_kernel<128, 128, 2, 2, true, false><<<grid, block, 0, st>>>(g);
    if (int rc = check_launch("dfp16 contraction")) return rc;
    if (g.atomic) return launch_absmax_i32(acc, int64_t(M) * N, absmax, st);
    return IONN_OK;
}

// Tile-aligned contraction on the 32x32x32 path: acc[M][N] = sum_c rhu(p_c, r)
// with A (M rows) and B (N rows) each K-major (element (row, k) at
// base[row * ld + k]) or M-major (at base[k * ld + row]); reduction length L.
bool fast2(int M, int N, int L, const void *a, int64_t lda, const void *b, int64_t ldb) {
    return M % d2::BM == 0 && N % d2::BN == 0 && L % 64 == 0 && aligned(a, 16) && aligned(b, 16) &&
           lda % 8 == 0 && ldb % 8 == 0;
}

// K splits of the tile-aligned path: enough work units to cover 256 compute
// units when the output has few tiles, at least 4 chunks per unit.
int split2(int64_t M, int64_t N, int64_t L) {
    if (M % d2::BM || N % d2::BN || L % 64 || M < 1 || N < 1 || L < 1) return 1;
    const int64_t tiles = (M / d2::BM) * (N / d2::BN), nch = L / 64;
    if (tiles >= 256 || nch < 8) return 1;
    int64_t split = (256 + tiles - 1) / tiles;
    if (split > nch / 4) split = nch / 4;
    return split < 1 ? 1 : int(split);
}

// Workgroup maxima of the tile-aligned path (one per persistent workgroup
// of the contraction, or per workgroup of the split sum).
constexpr int kMaxSlots = 4096;

struct Workspace {
    int32_t *acc;
    uint32_t *absmax;
    int16_t *t0, *t1;
    int32_t *part;     // split partial tiles of the tile-aligned path
    uint32_t *bits;    // block-shift form: rounding bits, one word per lane and 32 x 64 block
    int32_t *shifts;   // block-shift form: s_b per block
    uint32_t *slots;   // workgroup maxima
};

size_t ws_bytes(int64_t M, int64_t K, int64_t N, int which, Workspace *w, void *base) {
    int64_t out = which == IONN_DFP16_FWD ? M * N : which == IONN_DFP16_DGRAD ? M * K : N * K;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return base ? static_cast<char *>(base) + o : nullptr;
    };
    char *acc = take(size_t(out) * 4);
    char *am = take(4);
    const int split = which == IONN_DFP16_FWD ? split2(M, N, K) : which == IONN_DFP16_DGRAD ? split2(M, K, N)
                                                                                           : split2(N, K, M);
    char *part = split > 1 ? take(size_t(split) * out * 4) : nullptr;
    char *t0 = nullptr, *t1 = nullptr;
    if (which == IONN_DFP16_DGRAD) t0 = take(size_t(N) * K * 2);           // W^T [K][N]
    if (which == IONN_DFP16_WGRAD) {
        t0 = take(size_t(N) * M * 2);                                        // dY^T [N][M]
        t1 = take(size_t(K) * M * 2);                                        // X^T  [K][M]
    }
    char *bits = take(size_t((out + 7) / 8));           // 256 bytes per 2048-element block
    char *shifts = take(size_t((out + 2047) / 2048) * 4);
    char *slots = take(size_t(kMaxSlots) * 4);
    if (w) *w = Workspace{reinterpret_cast<int32_t *>(acc), reinterpret_cast<uint32_t *>(am),
                          reinterpret_cast<int16_t *>(t0), reinterpret_cast<int16_t *>(t1),
                          reinterpret_cast<int32_t *>(part), reinterpret_cast<uint32_t *>(bits),
                          reinterpret_cast<int32_t *>(shifts), reinterpret_cast<uint32_t *>(slots)};
    return off;
}

// Tile-aligned contraction of an M x N output with reduction length L and
// its down-conversion to out (int16) with the exponent bookkeeping.  Without
// K splits the contraction writes the block-shift int16 form straight into
// out and a second pass applies the tensor's shift in place; with K splits it
// writes int32 partial tiles, the split sum forms acc and the down-conversion
// reads it.  Either way the max |acc| travels through per-workgroup slots, so
// nothing needs clearing first.
template <bool A_KM, bool B_KM>
int contract2(const int16_t *a, int64_t lda, const int16_t *b, int64_t ldb, int M, int N, int L,
              const Workspace &w, const int32_t *ea, const int32_t *eb, int16_t *out, int32_t *e_out,
              int32_t *status, hipStream_t st) {
    const int split = split2(M, N, L);
    const int r = chunk_shift(L);
    d2::Args g{a, b, lda, ldb, split > 1 ? w.part : w.acc, nullptr, M, N, L, r, split, 0, nullptr, nullptr};
    const int tiles = (M / d2::BM) * (N / d2::BN);
    int cus = 256;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    const int units = tiles * split;
    int grid = units < cus ? units : cus;
    if (grid > kMaxSlots) grid = kMaxSlots;
    const int64_t n = int64_t(M) * N;
    if (split == 1) {
        g.out16 = out;
        g.bits = w.bits;
        g.shifts = w.shifts;
        g.slots = w.slots;
        d2::dfpi_kernel<A_KM, B_KM, true><<<dim3(grid), dim3(d2::NT), 0, st>>>(g);
        if (int rc = check_launch("dfp16 contraction")) return rc;
        const unsigned cpr = unsigned(N) / 8, bx = cpr < 256 ? cpr : 256, by = 256 / bx;
        unsigned gy = (unsigned(M) + by - 1) / by;
        if (gy > 4096) gy = 4096;
        block16_fix_kernel<<<dim3((cpr + bx - 1) / bx, gy), dim3(bx, by), 0, st>>>(
            out, M, N, w.bits, w.shifts, w.slots, grid, ea, eb, r, e_out, status);
        return check_launch("dfp16 down-conversion");
    }
    d2::dfpi_kernel<A_KM, B_KM, false><<<dim3(grid), dim3(d2::NT), 0, st>>>(g);
    if (int rc = check_launch("dfp16 contraction")) return rc;
    // four 16-byte groups per thread: fewer requests in flight than one
    // group per thread, which measured twice as fast on 16 partials
    int64_t blocks = (n / 4 + 1023) / 1024;
    if (blocks > 2048) blocks = 2048;
    d2::split_reduce<<<dim3(unsigned(blocks)), dim3(256), 0, st>>>(w.part, split, n, w.acc, w.slots);
    if (int rc = check_launch("dfp16 contraction")) return rc;
    int64_t dblocks = (n / 8 + 255) / 256;
    if (dblocks < 1) dblocks = 1;
    if (dblocks > 8192) dblocks = 8192;
    downconvert_kernel<<<dim3(unsigned(dblocks)), dim3(256), 0, st>>>(w.acc, n, w.slots, int(blocks), ea, eb, r,
                                                                     out, e_out, status);
    return check_launch("dfp16 down-conversion");
}

int transpose16(const int16_t *src, int16_t *dst, int R, int C, hipStream_t st) {
    dim3 grid((C + 63) / 64, (R + 63) / 64);
    transpose16_kernel<<<grid, dim3(256), 0, st>>>(src, dst, R, C);
    return check_launch("dfp16 transpose");
}

int finish(const Workspace &w, int64_t n, const int32_t *ea, const int32_t *eb, int r, int16_t *out,
           int32_t *e_out, int32_t *status, hipStream_t st) {
    int64_t blocks = (n / 8 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 8192) blocks = 8192;
    downconvert_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, st>>>(w.acc, n, w.absmax, 1, ea, eb, r,
                                                                    out, e_out, status);
    return check_launch("dfp16 down-conversion");
}

// ---------------------------------------------------------------------------
// FP32 form: chunk partials summed in FP32 over S consecutive chunk ranges,
// the ranges added in order, the total scaled by 2^(eA + shift + eB).
// ---------------------------------------------------------------------------

// Default range count: a function of the shape alone (so the result never
// depends on which kernel runs), equal to split2 on tile-aligned shapes.
int split_f32(int64_t M, int64_t N, int64_t L) {
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128), nch = (L + 63) / 64;
    if (tiles >= 256 || nch < 8) return 1;
    int64_t s = (256 + tiles - 1) / tiles;
    if (s > nch / 4) s = nch / 4;
    return s < 1 ? 1 : int(s);
}

// Output rows, output columns and reduction length of a role.
void role_dims(int64_t M, int64_t K, int64_t N, int which, int64_t &R, int64_t &C, int64_t &L) {
    if (which == IONN_DFP16_FWD) { R = M; C = N; L = K; }
    else if (which == IONN_DFP16_DGRAD) { R = M; C = K; L = N; }
    else { R = N; C = K; L = M; }
}

struct WsF32 {
    float *part;
    int16_t *t0, *t1;
};

size_t ws_f32_bytes(int64_t M, int64_t K, int64_t N, int which, int S, WsF32 *w, void *base) {
    int64_t R, C, L;
    role_dims(M, K, N, which, R, C, L);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align256(bytes);
        return base ? static_cast<char *>(base) + o : nullptr;
    };
    char *part = S > 1 ? take(size_t(S) * R * C * 4) : nullptr;
    char *t0 = nullptr, *t1 = nullptr;
    if (which == IONN_DFP16_DGRAD) t0 = take(size_t(N) * K * 2);
    if (which == IONN_DFP16_WGRAD) {
        t0 = take(size_t(N) * M * 2);
        t1 = take(size_t(K) * M * 2);
    }
    if (w) *w = WsF32{reinterpret_cast<float *>(part), reinterpret_cast<int16_t *>(t0),
                      reinterpret_cast<int16_t *>(t1)};
    return off ? off : 256;
}

template <bool A_KM, bool B_KM>
int contract2_f32(const int16_t *a, int64_t lda, const int16_t *b, int64_t ldb, int M, int N, int L, int S,
                  int shift, const int32_t *ea, const int32_t *eb, float *out, float *part, hipStream_t st) {
    d2::Args g{a, b, lda, ldb, reinterpret_cast<int32_t *>(S > 1 ? part : out), nullptr, M, N, L, 0, S,
               shift, ea, eb};
    const int tiles = (M / d2::BM) * (N / d2::BN);
    int cus = 256, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    const int units = tiles * S;
    d2::dfp_kernel<A_KM, B_KM><<<dim3(units < cus ? units : cus), dim3(d2::NT), 0, st>>>(g);
    return check_launch("dfp16 FP32 contraction");
}

int contract_f32(const Src16 &a, const Src16 &b, int M, int N, int L, int S, int shift, const int32_t *ea,
                 const int32_t *eb, float *out, float *part, hipStream_t st) {
    DfpArgs g{a, b, reinterpret_cast<int32_t *>(S > 1 ? part : out), nullptr, M, N, L, 0, S, false,
              shift, ea, eb};
    // 64 x 64 tiles: the FP32 accumulators of a 128 x 128 tile spill here
    const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
    const bool even = M % 64 == 0 && N % 64 == 0 && L % kChunk == 0 && a.vec && b.vec;
    dim3 grid(tiles, S), block(256);
    if (even) dfp16_kernel<64, 64, 2, 2, false, true><<<grid, block, 0, st>>>(g);
    else dfp16_kernel<64, 64, 2, 2, true, true><<<grid, block, 0, st>>>(g);
    return check_launch("dfp16 FP32 contraction");
}

int reduce_f32(const float *part, int S, int64_t n, float *out, const int32_t *ea, int shift, const int32_t *eb,
               hipStream_t st) {
    if (S <= 1) return IONN_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    d2::split_reduce_f32<<<dim3(unsigned(blocks)), dim3(256), 0, st>>>(part, S, n, out, ea, shift, eb);
    return check_launch("dfp16 FP32 split sum");
}

int check_f32(const void *A, const int32_t *eA, const void *B, const int32_t *eB, const float *out, int64_t M,
              int64_t K, int64_t N, int input_shift, int nsplit, void *ws, size_t ws_size, int which,
              const char *name, int &S) {
    IONN_REQUIRE(M >= 1 && K >= 1 && N >= 1 && M <= kMaxDim && K <= kMaxDim && N <= kMaxDim &&
                     M * N <= kMaxDim && M * K <= kMaxDim && N * K <= kMaxDim,
                 IONN_ERR_SHAPE, "%s: sizes must be >= 1 with every tensor below 2^31 elements", name);
    IONN_REQUIRE(A && eA && B && eB && out, IONN_ERR_ARG, "%s: NULL argument", name);
    IONN_REQUIRE(input_shift == 0 || input_shift == 1, IONN_ERR_RANGE, "%s: input_shift = %d (0 or 1)", name,
                 input_shift);
    int64_t R, C, L;
    role_dims(M, K, N, which, R, C, L);
    const int64_t nch = (L + kChunk - 1) / kChunk;
    IONN_REQUIRE(nsplit >= 0 && nsplit <= nch && nsplit <= 4096, IONN_ERR_RANGE,
                 "%s: nsplit = %d outside [0, %lld]", name, nsplit, (long long)(nch < 4096 ? nch : 4096));
    S = nsplit ? nsplit : split_f32(R, C, L);
    IONN_REQUIRE(S * R * C <= (int64_t(1) << 40), IONN_ERR_SHAPE, "%s: split partials too large", name);
    const size_t need = ws_f32_bytes(M, K, N, which, S, nullptr, nullptr);
    IONN_REQUIRE(ws != nullptr && aligned(ws, 256) && ws_size >= need, IONN_ERR_WORKSPACE,
                 "%s: workspace must be 256-byte aligned and hold %zu bytes", name, need);
    IONN_REQUIRE(aligned(A, 2) && aligned(B, 2) && aligned(out, 16) && aligned(eA, 4) && aligned(eB, 4),
                 IONN_ERR_ALIGN, "%s: misaligned pointer (out needs 16 bytes)", name);
    return IONN_OK;
}

int check_common(const void *A, const int32_t *eA, const void *B, const int32_t *eB, void *out,
                 int32_t *eout, int64_t M, int64_t K, int64_t N, int chunk, void *ws,
                 size_t ws_size, int which, const char *name) {
    IONN_REQUIRE(M >= 1 && K >= 1 && N >= 1 && M <= kMaxDim && K <= kMaxDim && N <= kMaxDim &&
                     M * N <= kMaxDim && M * K <= kMaxDim && N * K <= kMaxDim,
                 IONN_ERR_SHAPE, "%s: sizes must be >= 1 with every tensor below 2^31 elements",
                 name);
    IONN_REQUIRE(chunk == kChunk, IONN_ERR_RANGE, "%s: chunk must be 64 (got %d)", name, chunk);
    IONN_REQUIRE(A && eA && B && eB && out && eout, IONN_ERR_ARG, "%s: NULL argument", name);
    IONN_REQUIRE(ws != nullptr && aligned(ws, 256) &&
                     ws_size >= ws_bytes(M, K, N, which, nullptr, nullptr),
                 IONN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned and hold %zu bytes",
                 name, ws_bytes(M, K, N, which, nullptr, nullptr));
    IONN_REQUIRE(aligned(A, 2) && aligned(B, 2) && aligned(out, 16) && aligned(eA, 4) &&
                     aligned(eB, 4) && aligned(eout, 4),
                 IONN_ERR_ALIGN, "%s: misaligned pointer (out needs 16 bytes)", name);
    return IONN_OK;
}

}  // namespace
}  // namespace ionn

using namespace ionn;

extern "C" {

size_t dfp16_workspace_bytes(int64_t M, int64_t K, int64_t N, int which) {
    if (M < 1 || K < 1 || N < 1 || which < 0 || which > 2) return 0;
    return ws_bytes(M, K, N, which, nullptr, nullptr);
}

int dfp16_gemm_fwd(const int16_t *X, const int32_t *eX, const int16_t *W, const int32_t *eW,
                   int16_t *Y, int32_t *eY, int64_t M, int64_t K, int64_t N, int chunk,
                   void *workspace, size_t workspace_bytes, int32_t *status_out, void *stream) {
    clear_error();
    if (int rc = check_common(X, eX, W, eW, Y, eY, M, K, N, chunk, workspace, workspace_bytes,
                              IONN_DFP16_FWD, "dfp16_gemm_fwd"))
        return rc;
    hipStream_t st = as_stream(stream);
    Workspace w;
    ws_bytes(M, K, N, IONN_DFP16_FWD, &w, workspace);
    if (fast2(int(M), int(N), int(K), X, K, W, K))
        return contract2<true, true>(X, K, W, K, int(M), int(N), int(K), w, eX, eW, Y, eY, status_out, st);
    zero_i32_kernel<<<dim3(1), dim3(64), 0, st>>>(reinterpret_cast<int32_t *>(w.absmax), 1);
    Src16 a{X, K, int(M), int(K), aligned(X, 16) && K % 8 == 0};
    Src16 b{W, K, int(N), int(K), aligned(W, 16) && K % 8 == 0};
    if (int rc = contract(a, b, int(M), int(N), int(K), w.acc, w.absmax, st)) return rc;
    return finish(w, M * N, eX, eW, chunk_shift(K), Y, eY, status_out, st);
}

int dfp16_gemm_dgrad(const int16_t *dY, const int32_t *edY, const int16_t *W, const int32_t *eW,
                     int16_t *dX, int32_t *edX, int64_t M, int64_t K, int64_t N, int chunk,
                     void *workspace, size_t workspace_bytes, int32_t *status_out, void *stream) {
    clear_error();
    if (int rc = check_common(dY, edY, W, eW, dX, edX, M, K, N, chunk, workspace, workspace_bytes,
                              IONN_DFP16_DGRAD, "dfp16_gemm_dgrad"))
        return rc;
    hipStream_t st = as_stream(stream);
    Workspace w;
    ws_bytes(M, K, N, IONN_DFP16_DGRAD, &w, workspace);
    if (fast2(int(M), int(K), int(N), dY, N, W, K))  // B = W seen M-major: (k, n) at W[n * K + k]
        return contract2<true, false>(dY, N, W, K, int(M), int(K), int(N), w, edY, eW, dX, edX, status_out, st);
    zero_i32_kernel<<<dim3(1), dim3(64), 0, st>>>(reinterpret_cast<int32_t *>(w.absmax), 1);
    if (int rc = transpose16(W, w.t0, int(N), int(K), st)) return rc;  // W^T [K][N]
    Src16 a{dY, N, int(M), int(N), aligned(dY, 16) && N % 8 == 0};
    Src16 b{w.t0, N, int(K), int(N), N % 8 == 0};
    if (int rc = contract(a, b, int(M), int(K), int(N), w.acc, w.absmax, st)) return rc;
    return finish(w, M * K, edY, eW, chunk_shift(N), dX, edX, status_out, st);
}

int dfp16_gemm_wgrad(const int16_t *dY, const int32_t *edY, const int16_t *X, const int32_t *eX,
                     int16_t *G, int32_t *eG, int64_t M, int64_t K, int64_t N, int chunk,
                     void *workspace, size_t workspace_bytes, int32_t *status_out, void *stream) {
    clear_error();
    if (int rc = check_common(dY, edY, X, eX, G, eG, M, K, N, chunk, workspace, workspace_bytes,
                              IONN_DFP16_WGRAD, "dfp16_gemm_wgrad"))
        return rc;
    hipStream_t st = as_stream(stream);
    Workspace w;
    ws_bytes(M, K, N, IONN_DFP16_WGRAD, &w, workspace);
    if (fast2(int(N), int(K), int(M), dY, N, X, K))  // A = dY, B = X, both M-major over m
        return contract2<false, false>(dY, N, X, K, int(N), int(K), int(M), w, edY, eX, G, eG, status_out, st);
    zero_i32_kernel<<<dim3(1), dim3(64), 0, st>>>(reinterpret_cast<int32_t *>(w.absmax), 1);
    if (int rc = transpose16(dY, w.t0, int(M), int(N), st)) return rc;  // dY^T [N][M]
    if (int rc = transpose16(X, w.t1, int(M), int(K), st)) return rc;   // X^T  [K][M]
    Src16 a{w.t0, M, int(N), int(M), M % 8 == 0};
    Src16 b{w.t1, M, int(K), int(M), M % 8 == 0};
    if (int rc = contract(a, b, int(N), int(K), int(M), w.acc, w.absmax, st)) return rc;
    return finish(w, N * K, edY, eX, chunk_shift(M), G, eG, status_out, st);
}

int dfp16_f32_splits(int64_t M, int64_t K, int64_t N, int which) {
    if (M < 1 || K < 1 || N < 1 || which < 0 || which > 2) return 0;
    int64_t R, C, L;
    role_dims(M, K, N, which, R, C, L);
    return split_f32(R, C, L);
}

size_t dfp16_f32_workspace_bytes(int64_t M, int64_t K, int64_t N, int which, int nsplit) {
    if (M < 1 || K < 1 || N < 1 || which < 0 || which > 2 || nsplit < 0) return 0;
    const int S = nsplit ? nsplit : dfp16_f32_splits(M, K, N, which);
    return ws_f32_bytes(M, K, N, which, S, nullptr, nullptr);
}

int dfp16_gemm_fwd_f32(const int16_t *X, const int32_t *eX, const int16_t *W, const int32_t *eW, float *Y,
                       int64_t M, int64_t K, int64_t N, int input_shift, int nsplit, void *workspace,
                       size_t workspace_bytes, void *stream) {
    clear_error();
    int S = 1;
    if (int rc = check_f32(X, eX, W, eW, Y, M, K, N, input_shift, nsplit, workspace, workspace_bytes,
                           IONN_DFP16_FWD, "dfp16_gemm_fwd_f32", S))
        return rc;
    hipStream_t st = as_stream(stream);
    WsF32 w;
    ws_f32_bytes(M, K, N, IONN_DFP16_FWD, S, &w, workspace);
    if (fast2(int(M), int(N), int(K), X, K, W, K)) {
        if (int rc = contract2_f32<true, true>(X, K, W, K, int(M), int(N), int(K), S, input_shift, eX, eW, Y,
                                               w.part, st))
            return rc;
    } else {
        Src16 a{X, K, int(M), int(K), aligned(X, 16) && K % 8 == 0};
        Src16 b{W, K, int(N), int(K), aligned(W, 16) && K % 8 == 0};
        if (int rc = contract_f32(a, b, int(M), int(N), int(K), S, input_shift, eX, eW, Y, w.part, st)) return rc;
    }
    return reduce_f32(w.part, S, M * N, Y, eX, input_shift, eW, st);
}

int dfp16_gemm_dgrad_f32(const int16_t *dY, const int32_t *edY, const int16_t *W, const int32_t *eW, float *dX,
                         int64_t M, int64_t K, int64_t N, int input_shift, int nsplit, void *workspace,
                         size_t workspace_bytes, void *stream) {
    clear_error();
    int S = 1;
    if (int rc = check_f32(dY, edY, W, eW, dX, M, K, N, input_shift, nsplit, workspace, workspace_bytes,
                           IONN_DFP16_DGRAD, "dfp16_gemm_dgrad_f32", S))
        return rc;
    hipStream_t st = as_stream(stream);
    WsF32 w;
    ws_f32_bytes(M, K, N, IONN_DFP16_DGRAD, S, &w, workspace);
    if (fast2(int(M), int(K), int(N), dY, N, W, K)) {
        if (int rc = contract2_f32<true, false>(dY, N, W, K, int(M), int(K), int(N), S, input_shift, edY, eW, dX,
                                                w.part, st))
            return rc;
    } else {
        if (int rc = transpose16(W, w.t0, int(N), int(K), st)) return rc;
        Src16 a{dY, N, int(M), int(N), aligned(dY, 16) && N % 8 == 0};
        Src16 b{w.t0, N, int(K), int(N), N % 8 == 0};
        if (int rc = contract_f32(a, b, int(M), int(K), int(N), S, input_shift, edY, eW, dX, w.part, st)) return rc;
    }
    return reduce_f32(w.part, S, M * K, dX, edY, input_shift, eW, st);
}

int dfp16_gemm_wgrad_f32(const int16_t *dY, const int32_t *edY, const int16_t *X, const int32_t *eX, float *G,
                         int64_t M, int64_t K, int64_t N, int input_shift, int nsplit, void *workspace,
                         size_t workspace_bytes, void *stream) {
    clear_error();
    int S = 1;
    if (int rc = check_f32(dY, edY, X, eX, G, M, K, N, input_shift, nsplit, workspace, workspace_bytes,
                           IONN_DFP16_WGRAD, "dfp16_gemm_wgrad_f32", S))
        return rc;
    hipStream_t st = as_stream(stream);
    WsF32 w;
    ws_f32_bytes(M, K, N, IONN_DFP16_WGRAD, S, &w, workspace);
    if (fast2(int(N), int(K), int(M), dY, N, X, K)) {
        if (int rc = contract2_f32<false, false>(dY, N, X, K, int(N), int(K), int(M), S, input_shift, edY, eX, G,
                                                 w.part, st))
            return rc;
    } else {
        if (int rc = transpose16(dY, w.t0, int(M), int(N), st)) return rc;
        if (int rc = transpose16(X, w.t1, int(M), int(K), st)) return rc;
        Src16 a{w.t0, M, int(N), int(M), M % 8 == 0};
        Src16 b{w.t1, M, int(K), int(M), M % 8 == 0};
        if (int rc = contract_f32(a, b, int(N), int(K), int(M), S, input_shift, edY, eX, G, w.part, st)) return rc;
    }
    return reduce_f32(w.part, S, N * K, G, edY, input_shift, eX, st);
}

int dfp16_gemm_fwd_f32_blocked(const int16_t *X, const int32_t *eX, const int16_t *W, const int32_t *eW, float *Y,
                               int64_t M, int64_t K, int64_t N, int input_shift, int nsplit, void *workspace,
                               size_t workspace_bytes, void *stream) {
    clear_error();
    int S = 1;
    if (int rc = check_f32(X, eX, W, eW, Y, M, K, N, input_shift, nsplit, workspace, workspace_bytes,
                           IONN_DFP16_FWD, "dfp16_gemm_fwd_f32_blocked", S))
        return rc;
    hipStream_t st = as_stream(stream);
    WsF32 w;
    ws_f32_bytes(M, K, N, IONN_DFP16_FWD, S, &w, workspace);
    const int nch = int((K + kChunk - 1) / kChunk);
    float *dst = S > 1 ? w.part : Y;
    if (fast2(int(M), int(N), int(K), X, K, W, K)) {
        d2::Args g{X, W, K, K, reinterpret_cast<int32_t *>(dst), nullptr, int(M), int(N), int(K), 0, S,
                   input_shift, nullptr, nullptr, eX, eW, nch};
        const int tiles = int(M / d2::BM) * int(N / d2::BN);
        int cus = 256, dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        const int units = tiles * S;
        d2::dfp_kernel<true, true, true><<<dim3(units < cus ? units : cus), dim3(d2::NT), 0, st>>>(g);
    } else {
        Src16 a{X, K, int(M), int(K), aligned(X, 16) && K % 8 == 0};
        Src16 b{W, K, int(N), int(K), aligned(W, 16) && K % 8 == 0};
        DfpArgs g{a, b, reinterpret_cast<int32_t *>(dst), nullptr, int(M), int(N), int(K), 0, S, false,
                  input_shift, nullptr, nullptr, eX, eW, nch};
        const int tiles = int((M + 63) / 64) * int((N + 63) / 64);
        const bool even = M % 64 == 0 && N % 64 == 0 && K % kChunk == 0 && a.vec && b.vec;
        dim3 grid(tiles, S), block(256);
        if (even) dfp16_kernel<64, 64, 2, 2, false, true, true><<<grid, block, 0, st>>>(g);
        else dfp16_kernel<64, 64, 2, 2, true, true, true><<<grid, block, 0, st>>>(g);
    }
    if (int rc = check_launch("dfp16_gemm_fwd_f32_blocked")) return rc;
    return reduce_f32(w.part, S, M * N, Y, nullptr, 0, nullptr, st);
}

int dfp16_gavg(const int16_t *G, const int32_t *eG, const int32_t *eW, int64_t n, double *gavg_out,
               void *stream) {
    clear_error();
    IONN_REQUIRE(n >= 1, IONN_ERR_SHAPE, "dfp16_gavg: n = %lld < 1", (long long)n);
    IONN_REQUIRE(G && eG && eW && gavg_out, IONN_ERR_ARG, "dfp16_gavg: NULL argument");
    IONN_REQUIRE(aligned(G, 2) && aligned(eG, 4) && aligned(eW, 4) && aligned(gavg_out, 8),
                 IONN_ERR_ALIGN, "dfp16_gavg: misaligned pointer");
    hipStream_t st = as_stream(stream);
    if (n <= kGavgOneBlock && aligned(G, 16)) {
        gavg_one_kernel<<<dim3(1), dim3(1024), 0, st>>>(G, n, gavg_out, eG, eW);
        return check_launch("dfp16_gavg");
    }
    unsigned long long *acc = reinterpret_cast<unsigned long long *>(gavg_out);
    gavg_zero_kernel<<<dim3(1), dim3(1), 0, st>>>(acc);
    int64_t blocks = (n + 256 * 8 - 1) / (256 * 8);
    if (blocks > 1024) blocks = 1024;
    gavg_sum_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, st>>>(G, n, acc);
    gavg_finish_kernel<<<dim3(1), dim3(1), 0, st>>>(gavg_out, n, eG, eW);
    return check_launch("dfp16_gavg");
}

}  // extern "C"
