// Fast path of the 3x3 / stride 1 / pad 1 convolution contractions for 64
// input and 64 output channels ("Integer On-Device Training: Overview",
// section 7: Conv2D layers; NHWC activations and OHWI weights as on the
// TiGrIS "Compilation Pipeline" page), on v_mfma_i32_32x32x32_i8.
//
//   fwd    out[p][co] = sum_{tap, ci} in[p + off(tap)][ci] * W[co][tap][ci]
//   dgrad  out[p][ci] = sum_{tap, co} in[p + off(tap)][co] * W[co][8 - tap][ci]
//
// off(tap) = (kh - 1, kw - 1) for tap = 3 kh + kw, zero outside the image.
// dgrad is the same sum over the mirrored kernel (off(8 - tap) = -off(tap)),
// so both run one kernel; only the weight fragments differ.
//
// A persistent workgroup per compute unit walks tiles of 256 consecutive
// output pixels of one image.  For each tile the input rows it touches, plus
// one row above and below, are staged in LDS as a zero-padded halo: (W + 2)
// slots per row (the two outer slots are zero) and zero rows outside the
// image, so every tap of every pixel reads its operand at
// slot(pixel) + dy (W + 2) + dx with no bounds test.
//
// fwd / dgrad: the 64 x 576 weight matrix lives in registers for the whole
// kernel (36 16-byte fragments per lane), so LDS serves only the pixel
// operand.  Halos are loaded straight into LDS two tiles ahead, into one of
// three buffers, with 64-byte slots whose 16-byte chunks are XOR-swizzled
// against bank conflicts.  Eight wavefronts, two per SIMD so that one's
// memory waits overlap the other's matrix work; each owns 32 pixels x 64
// channels (two blocks of 32 x 32); K = 9 taps x 64 = 18 steps of 32.
//
// wgrad: 80-byte slots (64 channels + 16 bytes of padding, which makes 16
// consecutive slots hit 16 distinct 16-byte bank groups), double-buffered
// through registers.
#pragma once

#include "conv3x3_common.h"

namespace ionn {
namespace c3 {

template <bool DGRAD, int MODE = STORE32>
__global__ __launch_bounds__(NTF, 1) void conv3x3_kernel(const int8_t *__restrict__ in,
                                                         const int8_t *__restrict__ wgt,
                                                         void *__restrict__ out_any, int N, int H,
                                                         int W, uint32_t *__restrict__ absmax,
                                                         int target_bits = 0, int relu = 0,
                                                         int32_t *__restrict__ shift_out = nullptr,
                                                         uint32_t *__restrict__ bits_out = nullptr,
                                                         int32_t *__restrict__ shifts_blk = nullptr) {
    __shared__ __attribute__((aligned(1024))) int8_t halo[NB][HBUF];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int HW = H * W;
    const int tpi = (HW + TP - 1) / TP;
    const int ntiles = N * tpi;
    const int W2 = W + 2;
    const int G = gridDim.x;

    // ---- weight fragments: wf[cb][ks] = 16 bytes of row (cb*32 + lane%32),
    // k = ks*32 + 16*(lane/32) of the operand B[row][k] (k = tap*64 + channel).
    v4i wf[2][KS];
    if (!DGRAD) {
        // B[co][tap*64 + ci] = W[co][tap][ci]: the weight rows as stored.
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                wf[cb][ks] = *reinterpret_cast<const v4i *>(
                    wgt + (cb * 32 + (MODE == PARTIAL ? part_row(lane & 31) : (lane & 31))) * 576 + ks * 32 +
                    16 * (lane >> 5));
    } else {
        // B[ci][tap*64 + co] = W[co][8 - tap][ci].  W is staged in LDS as stored
        // (rows of 576 bytes per co) and every fragment comes out with two
        // ds_read_b64_tr_b8: lane i of a 16-lane group addresses co row
        // co0 + i/2 at ci0 + 8 (i mod 2), and lane j receives
        // W[co0 .. co0+7][8 - tap][ci0 + j], eight consecutive k of row ci0 + j.
        typedef __attribute__((address_space(3))) v2i lds_v2i_t;
        int8_t *stage = &halo[0][0];
        if (MODE == PARTIAL) {
            // the channels of every 32-byte block in the order part_row
            // reads them: staged dword b holds channel dword 4 (b & 1) + b / 2
            for (int i = tid; i < 64 * 576 / 32; i += NTF) {
                const v4i x = *reinterpret_cast<const v4i *>(wgt + 32 * i);
                const v4i y = *reinterpret_cast<const v4i *>(wgt + 32 * i + 16);
                *reinterpret_cast<v4i *>(stage + 32 * i) = v4i{x[0], y[0], x[1], y[1]};
                *reinterpret_cast<v4i *>(stage + 32 * i + 16) = v4i{x[2], y[2], x[3], y[3]};
            }
        } else {
            for (int i = tid; i < 64 * 576 / 16; i += NTF)
                *reinterpret_cast<v4i *>(stage + 16 * i) = *reinterpret_cast<const v4i *>(wgt + 16 * i);
        }
        __syncthreads();
        const int g = lane >> 4, i = lane & 15;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int co = (ks & 1) * 32 + 16 * (g >> 1) + (i >> 1);
                const int ci = cb * 32 + 16 * (g & 1) + 8 * (i & 1);
                const int8_t *p = stage + co * 576 + (8 - (ks >> 1)) * 64 + ci;
                const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p));
                const v2i y = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t *)(p + 8 * 576));
                wf[cb][ks] = v4i{x.x, x.y, y.x, y.y};
            }
        __syncthreads();
    }

    // The weight loads are complete before the halo loads start, so that no
    // wait inside the tile loop has to cover them.
    wait_vm<0>();

    // Buffer resource over the input: offsets at or past its end read zeros.
    const uint64_t abase = uint64_t(uintptr_t(in));
    const v4i rsrc = {__builtin_amdgcn_readfirstlane(int(uint32_t(abase))),
                      __builtin_amdgcn_readfirstlane(int(uint32_t(abase >> 32) & 0xffffu)),
                      __builtin_amdgcn_readfirstlane(int(uint32_t(int64_t(N) * HW * C))),
                      0x00020000};
    // Load i of this wavefront fills chunk positions q = (8 i + wave) * 64 + lane:
    // slot s = q / 4, halo row s / W2, column s % W2 - 1, channel chunk
    // (q % 4) ^ ((s / 4) % 4); hoff = byte offset of that chunk within its
    // image row, or -1 for the pad slots.
    int hrow[NI], hoff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int q = (8 * i + wave) * 64 + lane, sl = q >> 2;
        hrow[i] = sl / W2;
        const int w = sl - hrow[i] * W2 - 1;
        hoff[i] = (w >= 0 && w < W) ? w * 64 + 16 * ((q & 3) ^ ((sl >> 2) & 3)) : -1;
    }
    // Halo of tile t into buffer bf; every wavefront issues exactly NI loads,
    // also past the last tile (all zeros then), so the wait counts below hold.
    auto fetch = [&](int t, int bf) __attribute__((always_inline)) {
        int n = 0, hf = 0, nrows = 0;
        if (t < ntiles) {
            n = t / tpi;
            const int p0 = (t - n * tpi) * TP, valid = min(TP, HW - p0);
            hf = p0 / W;
            nrows = (p0 + valid - 1) / W - hf + 3;
        }
        const uint32_t lds0 = uint32_t(uintptr_t((__attribute__((address_space(3))) const int8_t *)(&halo[bf][0])));
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int h = hf - 1 + hrow[i];
            const bool ok = hrow[i] < nrows && hoff[i] >= 0 && h >= 0 && h < H;
            const uint32_t voff = ok ? uint32_t((n * H + h) * W) * 64u + uint32_t(hoff[i]) : OOB;
            dma_lds16(rsrc, voff, lds0 + uint32_t((8 * i + wave) * 1024));
        }
    };

    // Output through a buffer resource as well (see the epilogue): int32 or,
    // requantised, int8 elements.
    constexpr int OB = MODE == REQUANT || MODE == PARTIAL ? 1 : 4;
    const __amdgpu_buffer_rsrc_t orsrc =
        __builtin_amdgcn_make_buffer_rsrc(out_any, 0, int(int64_t(N) * HW * C * OB), 0x00020000);
    // requantisation shift from the finished max |acc| (NITI steps 2-3)
    int rs = 0;
    if (MODE == REQUANT) {
        rs = __builtin_amdgcn_readfirstlane(niti_shift(*absmax, target_bits));
        if (blockIdx.x == 0 && tid == 0 && shift_out) *shift_out = rs;
    }

    // PARTIAL side outputs: one rounding-bit word per lane and one shift per
    // wavefront and tile
    const __amdgpu_buffer_rsrc_t brsrc =
        __builtin_amdgcn_make_buffer_rsrc(bits_out, 0, MODE == PARTIAL ? ntiles * 8 * 64 * 4 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t srsrc =
        __builtin_amdgcn_make_buffer_rsrc(shifts_blk, 0, MODE == PARTIAL ? ntiles * 8 * 4 : 0, 0x00020000);
    uint32_t gmax = 0;

    int t = blockIdx.x;
    fetch(t, 0);
    fetch(t + G, 1);

    int32_t vmax = INT32_MIN, vmin = INT32_MAX;
    int b = 0;
    for (int k = 0; t < ntiles; t += G, ++k) {
        // This tile's loads are done when at most the next tile's (NI) and the
        // previous tile's stores (8, none without output) are still outstanding.
        if (k == 0) wait_vm<NI>(); else wait_vm<NI + stores_per_tile(MODE)>();
        __syncthreads();
        fetch(t + 2 * G, b == 0 ? 2 : b - 1);

        const int n = t / tpi, p0 = (t - n * tpi) * TP;
        const int valid = min(TP, HW - p0);
        const int hf = p0 / W;
        const int8_t *buf = halo[b];

        // centre slot of this lane's pixel; slot 0 (a pad, all zero) past the
        // tile's valid pixels
        const int pl = 32 * wave + (lane & 31);
        int sc = -1;
        if (pl < valid) {
            const int p = p0 + pl, h = p / W, w = p - h * W;
            sc = (h - hf + 1) * W2 + w + 1;
        }
        // operand fragment at step ks: tap ks/2, channel chunk 2 (ks & 1) + lane/32
        auto afrag = [&](int ks) __attribute__((always_inline)) {
            const int tap = ks >> 1, dy = tap / 3 - 1, dx = tap % 3 - 1;
            const int sl = sc >= 0 ? sc + dy * W2 + dx : 0;
            return *reinterpret_cast<const v4i *>(buf + 16 * chunk_pos(sl, 2 * (ks & 1) + (lane >> 5)));
        };

        v16i acc[2] = {v16i{}, v16i{}};
        v4i a[2];
        a[0] = afrag(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks & 1;
            if (ks + 1 < KS) a[c ^ 1] = afrag(ks + 1);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[cb][ks], a[c], acc[cb], 0, 0, 0);
        }

        // epilogue: lane holds out[p][co .. co+3], p = pixel pl,
        // co = cb*32 + 8 q + 4 (lane / 32); a lane past the valid pixels
        // stores to an offset beyond the end (dropped), so every wavefront
        // issues exactly eight stores per tile
        const uint32_t obase = pl < valid ? uint32_t(((n * HW + p0 + pl) * C + 4 * (lane >> 5)) * OB) : OOB;
        if (MODE == STORE32) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v4i v = {acc[cb][4 * q], acc[cb][4 * q + 1], acc[cb][4 * q + 2], acc[cb][4 * q + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, int(obase + uint32_t((cb * 32 + 8 * q) * 4)), 0, 0);
                }
        } else if (MODE == REQUANT) {
            // out = sat8(rhu(acc, s)), then max(out, 0) with ReLU; four
            // channels per dword
            auto rq = [&](int32_t v) __attribute__((always_inline)) {
                const int32_t q8 = sat8(rhu(v, rs));
                return relu ? max(q8, 0) : q8;
            };
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w = pack4_u8(rq(acc[cb][4 * q]), rq(acc[cb][4 * q + 1]), rq(acc[cb][4 * q + 2]),
                                                rq(acc[cb][4 * q + 3]));
                    __builtin_amdgcn_raw_buffer_store_b32(w, orsrc, int(obase + uint32_t(cb * 32 + 8 * q)), 0, 0);
                }
        } else if (MODE == PARTIAL) {
            // this wavefront's max |acc| over its valid pixels, its shift, and
            // the int8 f = asr(acc, sb) with the rounding bits
            int32_t bmax = INT32_MIN, bmin = INT32_MAX;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    bmax = max(bmax, max(acc[cb][v], acc[cb][v + 1]));
                    bmin = min(bmin, min(acc[cb][v], acc[cb][v + 1]));
                }
            const uint32_t bm = wave_max_u32(pl < valid ? max(abs_u32(bmax), abs_u32(bmin)) : 0u);
            gmax = max(gmax, bm);
            const int sb = __builtin_amdgcn_readfirstlane(niti_shift(bm, target_bits));
            const int sh1 = sb > 0 ? sb - 1 : 0;
            const uint32_t one = sb > 0 ? 1u : 0u;
            uint32_t bits = 0;
            const uint32_t ob = pl < valid ? uint32_t((n * HW + p0 + pl) * C + 16 * (lane >> 5)) : OOB;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                v4i f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f[q] = int(pack4_u8(acc[cb][4 * q] >> sb, acc[cb][4 * q + 1] >> sb, acc[cb][4 * q + 2] >> sb,
                                        acc[cb][4 * q + 3] >> sb));
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        bits |= ((uint32_t(acc[cb][4 * q + j]) >> sh1) & one) << (16 * cb + 4 * q + j);
                }
                __builtin_amdgcn_raw_buffer_store_b128(f, orsrc, int(ob + uint32_t(32 * cb)), 0, 0);
            }
            const int blk = t * 8 + wave;
            __builtin_amdgcn_raw_buffer_store_b32(bits, brsrc, int(uint32_t(blk * 64 + lane) * 4u), 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(uint32_t(sb), srsrc, int(lane == 0 ? uint32_t(blk) * 4u : OOB),
                                                  0, 0);
        }
        if (MODE != REQUANT && MODE != PARTIAL && pl < valid) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    vmax = max(vmax, max(acc[cb][v], acc[cb][v + 1]));
                    vmin = min(vmin, min(acc[cb][v], acc[cb][v + 1]));
                }
        }
        b = b == 2 ? 0 : b + 1;
    }
    wait_vm<0>();  // the zero-fill loads past the last tile land before the workgroup ends

    if (MODE == PARTIAL) {
        if (lane == 0) publish_max_u32(absmax, gmax);
    } else if (MODE != REQUANT && absmax) {
        uint32_t amax = vmax >= vmin ? max(abs_u32(vmax), abs_u32(vmin)) : 0u;
        amax = wave_max_u32(amax);
        if (lane == 0) publish_max_u32(absmax, amax);
    }
}

// Finishes a PARTIAL pass: every 16 bytes of the int8 tensor (pixel P,
// channels 16 q4 .. + 15) take their block's shift sb and rounding bits and
// become sat8(rhu(acc, s)) (then max(., 0) with relu), s = the tensor's
// shift from the finished *absmax; block 0 writes s.  In place.  A pixel's
// block is (tile, wavefront) = (n tpi + p / 256, (p / 32) % 8) and its lane
// p % 32 (channels 0-15, 32-47) or p % 32 + 32 (16-31, 48-63).
//
// Per dword of four int8 values f, with d = s - sb:
//  - d = 0: f + bit, bytewise without carries between bytes (the low seven
//    bits added, bit 7 restored by XOR); the only overflow, 127 + 1, shows
//    as a byte whose sign turned on and is set back to 127;
//  - d > 0: rhu(f, d) on int16 pairs (bytes 0, 2 and 1, 3 sign-extended in
//    place), d taken as min(d, 8): for |f| <= 128 and d >= 8,
//    f + 2^(d-1) lies in [0, 2^d), so the result is 0 at d = 8 as at any
//    larger d; the results fit int8, so the low byte of each half is kept.
__global__ __launch_bounds__(256) void conv3x3_requant_fix(int8_t *__restrict__ y8,
                                                           const uint32_t *__restrict__ bits,
                                                           const int32_t *__restrict__ shifts_blk,
                                                           const uint32_t *__restrict__ absmax, int target_bits,
                                                           int relu, uint32_t HW, uint32_t tpi, uint32_t nchunks,
                                                           int32_t *__restrict__ shift_out) {
    typedef short v2s __attribute__((ext_vector_type(2)));
    const int s = niti_shift(*absmax, target_bits);
    if (blockIdx.x == 0 && threadIdx.x == 0 && shift_out) *shift_out = s;
    for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < nchunks; c += gridDim.x * 256u) {
        const uint32_t P = c >> 2, q4 = c & 3u;
        const uint32_t n = P / HW, p = P - n * HW;
        const uint32_t blk = (n * tpi + (p >> 8)) * 8u + ((p >> 5) & 7u);
        const uint32_t w = bits[blk * 64u + (p & 31u) + 32u * (q4 & 1u)] >> (16u * (q4 >> 1));
        const int d = s - shifts_blk[blk];
        v4i v = *reinterpret_cast<const v4i *>(y8 + 16ull * c);
        if (d == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t f = uint32_t(v[q]);
                // bits 4q .. 4q + 3 of w to bit 0 of bytes 0 .. 3
                const uint32_t m = (((w >> (4 * q)) & 15u) * 0x00204081u) & 0x01010101u;
                uint32_t r = ((f & 0x7f7f7f7fu) + m) ^ (f & 0x80808080u);
                r -= (~f & r & 0x80808080u) >> 7;                      // 127 + 1 -> 127
                if (relu) r &= ~(((r >> 7) & 0x01010101u) * 0xffu);   // negative bytes -> 0
                v[q] = int(r);
            }
        } else {
            const short dd = short(d < 8 ? d : 8);
            const v2s dv = {dd, dd}, half = {short(1 << (dd - 1)), short(1 << (dd - 1))}, zero = {0, 0};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t f = uint32_t(v[q]);
                const v2s lo = __builtin_bit_cast(v2s, (f << 8) & 0xff00ff00u) >> v2s{8, 8};  // bytes 0, 2
                const v2s hi = __builtin_bit_cast(v2s, f & 0xff00ff00u) >> v2s{8, 8};         // bytes 1, 3
                v2s rl = (lo + half) >> dv, rh = (hi + half) >> dv;
                if (relu) {
                    rl = __builtin_elementwise_max(rl, zero);
                    rh = __builtin_elementwise_max(rh, zero);
                }
                v[q] = int((__builtin_bit_cast(uint32_t, rl) & 0x00ff00ffu) |
                           ((__builtin_bit_cast(uint32_t, rh) & 0x00ff00ffu) << 8));
            }
        }
        *reinterpret_cast<v4i *>(y8 + 16ull * c) = v;
    }
}

// ---------------------------------------------------------------------------
// Weight gradient, 64 -> 64 channels:
//   G[co][tap*64 + ci] = sum_p dY[p][co] * X[p + off(tap)][ci]
// as C = A B^T with A = dY^T (64 x pixels) and B = im2col(X) (576 x pixels),
// K = pixels.  Persistent workgroups walk the same 256-pixel tiles as the
// forward kernel; each keeps a partial G (64 x 576) in its accumulators over
// all its tiles and writes it once to a workspace row; one pass sums the rows
// into G with the max (wgrad_long.h, no atomics, so the result is
// deterministic; integer sums are exact in any order anyway).
//
// Both operands have their contraction index (pixels) as the outer
// dimension, so fragments come out of LDS with ds_read_b64_tr_b8: lane i of
// each 16-lane group addresses row k0 + i/2 (a pixel), 8 bytes at column
// m0 + 8 (i mod 2), and lane j receives column m0 + j of rows k0..k0+7.  The
// dY tile sits in LDS as [pixel][80 bytes]; the X operand is read from the
// zero-padded halo through a per-tile table of each pixel's slot.
// Eight wavefronts, two per SIMD, so that one's LDS waits overlap the
// other's matrix work.  Wavefront w owns n-blocks [nb0, nb0 + nn) of the 18
// 32-wide blocks of (tap, ci), for both 32-row blocks of co: three blocks
// for w = 0, 1 and two for the others, so the SIMD pairs (w, w + 4) carry
// 5, 5, 4 and 4 blocks.
// ---------------------------------------------------------------------------
constexpr int WNB = 3;                      // n-blocks per wavefront, at most
constexpr int DY_BYTES = TP * SLOT;         // one dY tile in LDS
constexpr int GSZ = 64 * 576;               // elements of G

// Workspace rows of the weight gradient: one partial G per workgroup, at most
// one workgroup per compute unit.
inline int64_t wgrad_rows(int cus) { return cus; }

__device__ __forceinline__ v4i tr_frag(const int8_t *base0, const int8_t *base1) {
    typedef int v2i_ __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i_ lds_v2i_;
    const v2i_ x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ *)(base0));
    const v2i_ y = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ *)(base1));
    return v4i{x.x, x.y, y.x, y.y};
}

__global__ __launch_bounds__(NTF, 1) void conv3x3_wgrad_kernel(const int8_t *__restrict__ dY,
                                                              const int8_t *__restrict__ X,
                                                              int32_t *__restrict__ part, int N,
                                                              int H, int W) {
    __shared__ __attribute__((aligned(16))) int8_t sdy[2][DY_BYTES];
    __shared__ __attribute__((aligned(16))) int8_t halo[2][HALO_BYTES];
    __shared__ int sslot[2][TP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int HW = H * W;
    const int tpi = (HW + TP - 1) / TP;
    const int ntiles = N * tpi;
    const int W2 = W + 2;
    const int nb0 = wave < 2 ? 3 * wave : 6 + 2 * (wave - 2);
    const int nn = wave < 2 ? 3 : 2;

    for (int i = tid; i < 2 * HALO_BYTES / 16; i += NTF)
        reinterpret_cast<v4i *>(&halo[0][0])[i] = v4i{0, 0, 0, 0};

    int hr[HALO_ITF], hw4[HALO_ITF];
#pragma unroll
    for (int i = 0; i < HALO_ITF; ++i) {
        const int q = tid + NTF * i;
        hr[i] = q / (4 * W);
        hw4[i] = q - hr[i] * 4 * W;
    }

    // Registers in flight for the next tile: 2 dY chunks, the halo chunks,
    // and (threads below TP) the slot of pixel tid.
    v4i dv[2], hv[HALO_ITF];
    int myslot = 0;
    auto fetch = [&](int t) __attribute__((always_inline)) {
        const int n = t / tpi, p0 = (t - n * tpi) * TP;
        const int valid = min(TP, HW - p0);
        const int hf = p0 / W, hl = (p0 + valid - 1) / W;
        const int nrows = hl - hf + 3;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + NTF * i, pl = q >> 2, cc = q & 3;
            v4i v = {0, 0, 0, 0};
            if (pl < valid)
                v = *reinterpret_cast<const v4i *>(dY + (int64_t(n) * HW + p0 + pl) * C + 16 * cc);
            dv[i] = v;
        }
#pragma unroll
        for (int i = 0; i < HALO_ITF; ++i) {
            const int h = hf - 1 + hr[i];
            v4i v = {0, 0, 0, 0};
            if (hr[i] < nrows && h >= 0 && h < H)
                v = *reinterpret_cast<const v4i *>(X + ((int64_t(n) * H + h) * W) * C + int64_t(hw4[i]) * 16);
            hv[i] = v;
        }
        if (tid < valid) {
            const int p = p0 + tid, h = p / W, w = p - h * W;
            myslot = (h - hf + 1) * W2 + w + 1;
        } else {
            myslot = W2 + 1;  // any slot whose 3x3 neighbourhood is inside the halo; dY is 0 there
        }
    };
    auto put = [&](int t, int bb) __attribute__((always_inline)) {
        const int n = t / tpi, p0 = (t - n * tpi) * TP;
        const int valid = min(TP, HW - p0);
        const int hf = p0 / W, hl = (p0 + valid - 1) / W;
        const int nrows = hl - hf + 3;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + NTF * i, pl = q >> 2, cc = q & 3;
            *reinterpret_cast<v4i *>(&sdy[bb][pl * SLOT + 16 * cc]) = dv[i];
        }
#pragma unroll
        for (int i = 0; i < HALO_ITF; ++i) {
            if (hr[i] < nrows) {
                const int w = hw4[i] >> 2, cc = hw4[i] & 3;
                *reinterpret_cast<v4i *>(&halo[bb][(hr[i] * W2 + w + 1) * SLOT + cc * 16]) = hv[i];
            }
        }
        if (tid < TP) sslot[bb][tid] = myslot;
    };

    v16i acc[WNB][2];
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[j][cb] = v16i{};

    int t = blockIdx.x;
    if (t < ntiles) fetch(t);
    __syncthreads();
    if (t < ntiles) put(t, 0);
    __syncthreads();

    // lane geometry of the transposing reads
    const int g = lane >> 4, i16 = lane & 15;
    const int prow = 16 * (g >> 1) + (i16 >> 1);     // pixel row within a 32-pixel step, h = 0
    const int mcol = 16 * (g & 1) + 8 * (i16 & 1);   // column within a 32-wide block
    int b = 0;
    for (; t < ntiles; t += gridDim.x, b ^= 1) {
        const int tn = t + gridDim.x;
        if (tn < ntiles) fetch(tn);
        const int8_t *ydb = sdy[b];
        const int8_t *xb = halo[b];
#pragma unroll 2
        for (int kp = 0; kp < TP / 32; ++kp) {
            const int r0 = kp * 32 + prow, r1 = r0 + 8;
            const int s0 = sslot[b][r0], s1 = sslot[b][r1];
            v4i a[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                a[cb] = tr_frag(ydb + r0 * SLOT + cb * 32 + mcol, ydb + r1 * SLOT + cb * 32 + mcol);
#pragma unroll
            for (int j = 0; j < WNB; ++j) {
                if (j < nn) {
                    const int nb = nb0 + j, tap = nb >> 1;
                    const int sh = (tap / 3 - 1) * W2 + (tap % 3 - 1);
                    const int cix = (nb & 1) * 32 + mcol;
                    const v4i bf = tr_frag(xb + (s0 + sh) * SLOT + cix, xb + (s1 + sh) * SLOT + cix);
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        acc[j][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf, a[cb], acc[j][cb], 0, 0, 0);
                }
            }
        }
        if (tn < ntiles) put(tn, b ^ 1);
        __syncthreads();
    }

    // partial G of this workgroup: lane holds co = cb*32 + lane%32 and
    // n = (nb0 + j)*32 + 8 q + 4 (lane / 32) .. +3
    int32_t *row = part + int64_t(blockIdx.x) * GSZ;
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
        if (j < nn) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                int32_t *dst = row + (cb * 32 + (lane & 31)) * 576 + (nb0 + j) * 32 + 4 * (lane >> 5);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<v4i *>(dst + 8 * q) =
                        v4i{acc[j][cb][4 * q], acc[j][cb][4 * q + 1], acc[j][cb][4 * q + 2], acc[j][cb][4 * q + 3]};
            }
        }
    }
}

}  // namespace c3
}  // namespace ionn
