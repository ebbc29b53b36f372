// Software-pipelined fast path of the 3x3 / stride 1 / pad 1 convolution
// contractions for 64 input and 64 output channels ("Integer On-Device
// Training: Overview", section 7: Conv2D layers; NHWC activations and OHWI
// weights as on the TiGrIS "Compilation Pipeline" page), fwd and dgrad,
// with every epilogue mode of conv3x3.h:
//
//   fwd    out[p][co] = sum_{tap, ci} in[p + off(tap)][ci] * W[co][tap][ci]
//   dgrad  out[p][ci] = sum_{tap, co} in[p + off(tap)][co] * W[co][8 - tap][ci]
//
// off(tap) = (kh - 1, kw - 1) for tap = 3 kh + kw, zero outside the image.
//
// Tiles are those of conv3x3_kernel: 256 consecutive output pixels of one
// image, whose input rows (plus one above and one below) are staged in LDS
// as a zero-padded halo, loaded straight from memory two tiles ahead into one
// of three buffers, so every tap of a pixel reads its operand at a fixed
// offset from the pixel's slot.  What differs is the schedule and the
// register layout:
//  - four wavefronts, one per SIMD, each own 64 pixels (two 32-pixel blocks
//    x 64 channels: four 32 x 32 products, 72 v_mfma_i32_32x32x32_i8 per
//    tile), and every other instruction of a tile sits between its MFMAs:
//    the next tile's halo writes to LDS (steps 0..7) and the next-but-one
//    tile's halo loads (steps 8..15), the previous tile's epilogue in
//    pieces on a second accumulator set and its stores (steps 12..15), and
//    the next step's two pixel fragments;
//  - the 64 x 576 weight operand stays in 144 AGPRs (the matrix cores read
//    their operands from AGPRs) and both accumulator sets in VGPRs (this
//    file is built with the VGPR form of the MFMA instructions), so the
//    epilogue reads its values without copies;
//  - the halo holds 8 rows of 64 slots of 64 bytes (a pad slot on each side
//    of the W <= 62 image columns); chunk c of the slot at column position
//    x sits at c ^ ((x >> 2) & 3), which spreads 16 consecutive slots over
//    16 bank groups and depends on the column only, so a tap's fragment
//    address is one of six per-tile column bases plus an immediate row
//    offset;
//  - the halo moves through registers: each wavefront loads its two rows
//    of the next-but-one tile with ordinary 16-byte buffer loads (which do
//    not hold up the instruction stream, unlike loads straight into LDS)
//    and writes them to LDS during the next tile; rows past the tile are
//    skipped and rows outside the image written as zeros.  Two buffers
//    suffice: while one is read, the other receives the next tile;
//  - the weight rows are read in part_row order, so a lane's 16 values of a
//    32-channel block are 16 consecutive channels and leave in 16-byte
//    stores.
#include "conv3x3_common.h"
#include "conv_pipe.h"

namespace ionn {
namespace c3 {
namespace {

constexpr int NTP = 256;                        // threads: four wavefronts, one per SIMD
constexpr int HR = 8;                           // halo rows
constexpr int RS = 64;                          // slots per halo row
constexpr int HROW = RS * C;                    // bytes per halo row (4 KiB)
constexpr int PB = HR * HROW;                   // bytes per halo buffer (32 KiB)
constexpr int NPB = 2;                          // halo buffers
constexpr uint32_t PAD_OFF = 0x40000000u;       // pad slots: past any input, read as zeros

// Max over the 64 lanes of a wavefront with DPP moves (no LDS traffic): row
// shifts fold each row of 16 into its lane 15, the row broadcasts fold rows
// into lane 63, which is read back.  0 is the identity of the unsigned max.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xf, 0xf, true)));   // row_shr:1
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xf, 0xf, true)));   // row_shr:2
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xf, 0xf, true)));   // row_shr:4
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xf, 0xf, true)));   // row_shr:8
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xa, 0xf, false)));  // row_bcast:15
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xc, 0xf, false)));  // row_bcast:31
    return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

#define IONN_CP_FENCE() __builtin_amdgcn_sched_barrier(0)

template <bool DGRAD, int MODE>
__global__ __launch_bounds__(NTP, 1) void conv_pipe_kernel(const int8_t *__restrict__ in,
                                                           const int8_t *__restrict__ wgt,
                                                           void *__restrict__ out_any, int N, int H, int W,
                                                           uint32_t *__restrict__ absmax, int target_bits, int relu,
                                                           int32_t *__restrict__ shift_out,
                                                           uint32_t *__restrict__ bits_out,
                                                           int32_t *__restrict__ shifts_blk) {
    __shared__ __attribute__((aligned(1024))) int8_t halo[NPB][PB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int HW = H * W;
    const int tpi = (HW + TP - 1) / TP;
    const int ntiles = N * tpi;
    const int W2 = W + 2;
    const int G = gridDim.x;

    // ---- weight fragments wf[cb][ks]: row cb*32 + part_row(lane % 32) of
    // B[row][k], k = ks*32 + 16 (lane / 32) .. + 15 (k = tap*64 + channel),
    // held in AGPRs for the whole kernel.
    v4i wf[2][KS];
    if (!DGRAD) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                wf[cb][ks] = *reinterpret_cast<const v4i *>(wgt + (cb * 32 + part_row(lane & 31)) * 576 + ks * 32 +
                                                            16 * (lane >> 5));
    } else {
        // B[ci][tap*64 + co] = W[co][8 - tap][ci], read with ds_read_b64_tr_b8
        // from W staged in LDS with every 32-channel block in part_row order
        // (staged dword b holds channel dword 4 (b & 1) + b / 2): lane i of a
        // 16-lane group addresses co row co0 + i/2 at ci0 + 8 (i mod 2), and
        // lane j receives W[co0 .. co0+7][8 - tap][staged ci0 + j].
        typedef __attribute__((address_space(3))) v2i lds_v2i_t;
        int8_t *stage = &halo[0][0];
        for (int i = tid; i < 64 * 576 / 32; i += NTP) {
            const v4i x = *reinterpret_cast<const v4i *>(wgt + 32 * i);
            const v4i y = *reinterpret_cast<const v4i *>(wgt + 32 * i + 16);
            *reinterpret_cast<v4i *>(stage + 32 * i) = v4i{x[0], y[0], x[1], y[1]};
            *reinterpret_cast<v4i *>(stage + 32 * i + 16) = v4i{x[2], y[2], x[3], y[3]};
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
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(wf[cb][ks]));
    // the weight loads are complete before the halo loads start, so that no
    // wait inside the tile loop has to cover them
    wait_vm<0>();

    // ---- halo.  Wavefront w fills halo rows 2w and 2w + 1 of a buffer, four
    // 1 KiB pieces per row: lane l of piece j covers slot x = 16 j + l / 4
    // (image column x - 1) at position l % 4, which holds channel chunk
    // c = (l % 4) ^ ((x >> 2) & 3).  hc[j] = its byte offset within an
    // image row, or PAD_OFF for the pad slots (read as zeros).
    const __amdgpu_buffer_rsrc_t irsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(in), 0, int(int64_t(N) * HW * C), 0x00020000);
    uint32_t hc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int x = 16 * j + (lane >> 2), c = (lane & 3) ^ ((x >> 2) & 3), w = x - 1;
        hc[j] = (w >= 0 && w < W) ? uint32_t(w * C + 16 * c) : PAD_OFF;
    }
    // halo rows of tile t in the image and in the tile's reach: rb[i] = byte
    // offset of image row hf - 1 + (2 wave + i), or OOB (outside the image:
    // zeros); nrow[i]: whether the row is needed at all
    struct HaloRows {
        uint32_t rb[2];
        bool need[2];
    };
    auto halo_rows = [&](int t) __attribute__((always_inline)) {
        HaloRows g;
        g.rb[0] = g.rb[1] = OOB;
        g.need[0] = g.need[1] = false;
        if (t < ntiles) {
            const int n = t / tpi;
            const int p0 = (t - n * tpi) * TP, valid = min(TP, HW - p0);
            const int hf = p0 / W;
            const int nrows = (p0 + valid - 1) / W - hf + 3;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 2 * wave + i, h = hf - 1 + r;
                g.need[i] = r < nrows;
                g.rb[i] = (h >= 0 && h < H) ? uint32_t((n * H + h) * W * C) : OOB;
            }
        }
        return g;
    };
    v4i hv[2][4];  // the next-but-one tile's halo rows in flight
    auto halo_load = [&](const HaloRows &g, int i, int j) __attribute__((always_inline)) {
        if (g.need[i] && g.rb[i] != OOB)
            hv[i][j] = __builtin_amdgcn_raw_buffer_load_b128(irsrc, int(g.rb[i] + hc[j]), 0, 0);
        else
            hv[i][j] = v4i{0, 0, 0, 0};
    };
    auto halo_write = [&](const HaloRows &g, int bufi, int i, int j) __attribute__((always_inline)) {
        if (g.need[i])
            *reinterpret_cast<v4i *>(&halo[bufi][(2 * wave + i) * HROW + 1024 * j + 16 * lane]) = hv[i][j];
    };

    // ---- outputs through buffer resources (an offset past the end drops
    // the store, so lanes past the valid pixels and the epilogue of the
    // tile before the first store nothing without a branch)
    constexpr int OB = MODE == STORE32 ? 4 : 1;
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        out_any, 0, MODE == MAXONLY ? 0 : int(int64_t(N) * HW * C * OB), 0x00020000);
    const __amdgpu_buffer_rsrc_t brsrc =
        __builtin_amdgcn_make_buffer_rsrc(bits_out, 0, MODE == PARTIAL ? ntiles * 8 * 64 * 4 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t srsrc =
        __builtin_amdgcn_make_buffer_rsrc(shifts_blk, 0, MODE == PARTIAL ? ntiles * 8 * 4 : 0, 0x00020000);
    int rs = 0;
    if (MODE == REQUANT) {
        rs = __builtin_amdgcn_readfirstlane(niti_shift(*absmax, target_bits));
        if (blockIdx.x == 0 && tid == 0 && shift_out) *shift_out = rs;
    }

    // ---- epilogue state of the previous tile (the accumulator set not being
    // written): its index and the output offsets of this lane's pixels
    struct Prev {
        int t;            // tile, -1: none (every store dropped)
        uint32_t ob[2];   // per block: byte offset of pixel, channel 16 (lane / 32); or OOB
    };
    auto prev_of = [&](int t) __attribute__((always_inline)) {
        Prev q;
        q.t = t;
        const int n = t / tpi, p0 = (t - n * tpi) * TP, valid = min(TP, HW - p0);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int pl = 64 * wave + 32 * b + (lane & 31);
            q.ob[b] = pl < valid ? uint32_t((n * HW + p0 + pl) * C + 16 * (lane >> 5)) * uint32_t(OB) : OOB;
        }
        return q;
    };
    Prev none;
    none.t = -1;
    none.ob[0] = none.ob[1] = OOB;

    uint32_t gmax = 0;                 // max |acc| over the finished blocks (this lane)
    uint32_t bm[2] = {0u, 0u};         // per block: max |acc| (this lane, then the wavefront's)
    int sblk[2] = {0, 0};              // PARTIAL: per block shift
    uint32_t bits[2] = {0u, 0u};       // PARTIAL: per block rounding bits
    v4i hold[2][2];                    // REQUANT / PARTIAL: packed int8 per block and channel half

    // compute piece e (0..9) of the previous tile's epilogue on accumulators
    // P: per block b = e / 5, phase e % 5: 0-1 max |acc| of channel half
    // 0-1, 2 the wavefront's max and the block shift, 3-4 the int8 values
    // of channel half 0-1
    auto epi_compute = [&](v16i (&P)[2][2], int e) __attribute__((always_inline)) {
        const int b = e / 5, ph = e % 5;
        if (ph < 2) {
            if (MODE == REQUANT) return;
            int32_t mx = INT32_MIN, mn = INT32_MAX;
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                mx = max(mx, max(P[b][ph][v], P[b][ph][v + 1]));
                mn = min(mn, min(P[b][ph][v], P[b][ph][v + 1]));
            }
            const uint32_t m = max(abs_u32(mx), abs_u32(mn));
            bm[b] = ph == 0 ? m : max(bm[b], m);
        } else if (ph == 2) {
            if (MODE == PARTIAL) {
                bm[b] = wave_max_dpp(bm[b]);
                sblk[b] = __builtin_amdgcn_readfirstlane(niti_shift(bm[b], target_bits));
            }
            if (MODE != REQUANT) gmax = max(gmax, bm[b]);
        } else {
            const int cb = ph - 3;
            if (MODE == REQUANT) {
                auto rq = [&](int32_t v) __attribute__((always_inline)) {
                    const int32_t q8 = sat8(rhu(v, rs));
                    return relu ? max(q8, 0) : q8;
                };
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    hold[b][cb][q] = int(pack4_u8(rq(P[b][cb][4 * q]), rq(P[b][cb][4 * q + 1]), rq(P[b][cb][4 * q + 2]),
                                                  rq(P[b][cb][4 * q + 3])));
            } else if (MODE == PARTIAL) {
                const int sb = sblk[b];
                const uint32_t sh1 = uint32_t(sb > 0 ? sb - 1 : 0);
                const uint32_t one = sb > 0 ? 1u : 0u;
                uint32_t w = cb == 0 ? 0u : bits[b];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    hold[b][cb][q] = int(pack4_u8(P[b][cb][4 * q] >> sb, P[b][cb][4 * q + 1] >> sb,
                                                  P[b][cb][4 * q + 2] >> sb, P[b][cb][4 * q + 3] >> sb));
                    // bit sb - 1 of each value (a field of width 0 when sb = 0)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        w |= __builtin_amdgcn_ubfe(uint32_t(P[b][cb][4 * q + j]), sh1, one) << (16 * cb + 4 * q + j);
                }
                bits[b] = w;
            }
        }
    };
    // store piece e (0..3) of the previous tile's epilogue: block e / 2
    auto epi_store = [&](v16i (&P)[2][2], const Prev &pv, int e) __attribute__((always_inline)) {
        const int b = e >> 1, half = e & 1;
        if (MODE == STORE32) {
            // channels 32 half + 16 (lane / 32) .. + 15: 64 contiguous bytes of int32
#pragma unroll
            for (int q = 0; q < 4; ++q)
                __builtin_amdgcn_raw_buffer_store_b128(
                    v4i{P[b][half][4 * q], P[b][half][4 * q + 1], P[b][half][4 * q + 2], P[b][half][4 * q + 3]}, orsrc,
                    int(pv.ob[b] + uint32_t(128 * half + 16 * q)), 0, 0);
        } else if (MODE == REQUANT) {
            __builtin_amdgcn_raw_buffer_store_b128(hold[b][half], orsrc, int(pv.ob[b] + uint32_t(32 * half)), 0, 0);
        } else if (MODE == PARTIAL) {
            if (half == 0) {
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    __builtin_amdgcn_raw_buffer_store_b128(hold[b][cb], orsrc, int(pv.ob[b] + uint32_t(32 * cb)), 0, 0);
            } else {
                const int blk = pv.t * 8 + 2 * wave + b;
                __builtin_amdgcn_raw_buffer_store_b32(bits[b], brsrc,
                                                      int(pv.t >= 0 ? uint32_t(blk * 64 + lane) * 4u : OOB), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(uint32_t(sblk[b]), srsrc,
                                                      int(pv.t >= 0 && lane == 0 ? uint32_t(blk) * 4u : OOB), 0, 0);
            }
        }
    };

    // One tile into accumulators A while the previous tile's epilogue runs
    // on P.  Per K step: four MFMAs (blocks x channel halves), the next
    // step's two fragment reads, one LDS write of the next tile's halo
    // (steps 0..7) or one load of the next-but-one tile's (steps 8..15), an
    // epilogue piece (steps 0..9) or a store piece (steps 12..15).
    int bf = 0;  // halo buffer of the current tile
    auto tile = [&](int t, v16i (&A)[2][2], v16i (&P)[2][2], const Prev &pv, const HaloRows &nxt,
                    const HaloRows &nxt2) __attribute__((always_inline)) {
        // the current tile's halo is in LDS once every wavefront's writes
        // of it are done and all meet
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int n = t / tpi, p0 = (t - n * tpi) * TP;
        const int valid = min(TP, HW - p0), hf = p0 / W;
        // column bases of this lane's pixels: for dx = -1, 0, 1 the slot
        // column of the neighbour with its chunk swizzle, channel chunk
        // lane / 32 (odd K steps: + 2, i.e. ^ 32 bytes); a pixel past the
        // tile's valid ones reads around an interior slot (never used)
        const int8_t *hb = &halo[bf][0];
        int cbs[2][3], r0[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int pl = 64 * wave + 32 * b + (lane & 31);
            int hr = 1, x = 1;
            if (pl < valid) {
                const int p = p0 + pl, h = p / W, w = p - h * W;
                hr = h - hf + 1;
                x = w + 1;
            }
            r0[b] = (hr - 1) * HROW;
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                const int xx = x + d - 1;
                cbs[b][d] = r0[b] + xx * C + 16 * ((lane >> 5) ^ ((xx >> 2) & 3));
            }
        }
        // fragment of block b at K step ks: tap ks / 2 = 3 row + col, channel
        // chunk 2 (ks & 1) + lane / 32
        auto afrag = [&](int b, int ks) __attribute__((always_inline)) {
            const int tap = ks >> 1, row = tap / 3, col = tap % 3;
            const int off = cbs[b][col] ^ (32 * (ks & 1));
            return *reinterpret_cast<const v4i *>(hb + off + row * HROW);
        };
        v4i a[2][2];
        a[0][0] = afrag(0, 0);
        a[0][1] = afrag(1, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks & 1;
            // the first K step starts from the zero accumulator
            IONN_CP_FENCE();
            A[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[0][ks], a[c][0], ks ? A[0][0] : v16i{}, 0, 0, 0);
            IONN_CP_FENCE();
            if (ks + 1 < KS) a[c ^ 1][0] = afrag(0, ks + 1);
            IONN_CP_FENCE();
            A[0][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[1][ks], a[c][0], ks ? A[0][1] : v16i{}, 0, 0, 0);
            IONN_CP_FENCE();
            if (ks < 8) halo_write(nxt, bf ^ 1, ks >> 2, ks & 3);
            else if (ks < 16) halo_load(nxt2, (ks - 8) >> 2, ks & 3);
            IONN_CP_FENCE();
            A[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[0][ks], a[c][1], ks ? A[1][0] : v16i{}, 0, 0, 0);
            IONN_CP_FENCE();
            if (ks + 1 < KS) a[c ^ 1][1] = afrag(1, ks + 1);
            IONN_CP_FENCE();
            A[1][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[1][ks], a[c][1], ks ? A[1][1] : v16i{}, 0, 0, 0);
            IONN_CP_FENCE();
            if (ks < 10) epi_compute(P, ks);
            else if (ks >= 12 && ks < 16) epi_store(P, pv, ks - 12);
        }
        IONN_CP_FENCE();
        bf ^= 1;
    };

    v16i acc0[2][2], acc1[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc0[b][cb] = acc1[b][cb] = v16i{};

    // prologue: the first tile's halo into buffer 0, the second's into
    // registers
    int t = blockIdx.x;
    {
        const HaloRows g0 = halo_rows(t);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) halo_load(g0, i, j);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) halo_write(g0, 0, i, j);
        const HaloRows g1 = halo_rows(t + G);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) halo_load(g1, i, j);
    }
    // Every prologue load waited for here, once: otherwise registers they
    // fill and the loop reuses carry a pending load into the loop head, and
    // the compiler's wait for it (vmcnt(0), the counter retiring in order)
    // would run in every tile and drain the previous tile's stores.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    Prev pv = none;
    bool last_in_1 = false;  // which set holds the last tile's sums
    while (t < ntiles) {
        tile(t, acc0, acc1, pv, halo_rows(t + G), halo_rows(t + 2 * G));
        pv = prev_of(t);
        t += G;
        last_in_1 = false;
        if (t >= ntiles) break;
        tile(t, acc1, acc0, pv, halo_rows(t + G), halo_rows(t + 2 * G));
        pv = prev_of(t);
        t += G;
        last_in_1 = true;
    }
    // the last tile's epilogue on its own
    if (pv.t >= 0) {
        if (last_in_1) {
#pragma unroll
            for (int e = 0; e < 10; ++e) epi_compute(acc1, e);
#pragma unroll
            for (int e = 0; e < 4; ++e) epi_store(acc1, pv, e);
        } else {
#pragma unroll
            for (int e = 0; e < 10; ++e) epi_compute(acc0, e);
#pragma unroll
            for (int e = 0; e < 4; ++e) epi_store(acc0, pv, e);
        }
    }
    if (MODE != REQUANT && absmax) {
        if (MODE != PARTIAL) gmax = wave_max_dpp(gmax);
        if (lane == 0) publish_max_u32(absmax, gmax);
    }
}

template <bool DGRAD>
void launch_mode(int mode, const int8_t *in, const int8_t *wgt, void *out, int N, int H, int W, uint32_t *absmax,
                 int tb, int relu, int32_t *shift_out, uint32_t *bits, int32_t *sblk, unsigned grid, hipStream_t st) {
    const dim3 g(grid), b(NTP);
    switch (mode) {
    case STORE32:
        conv_pipe_kernel<DGRAD, STORE32><<<g, b, 0, st>>>(in, wgt, out, N, H, W, absmax, tb, relu, shift_out, bits, sblk);
        break;
    case MAXONLY:
        conv_pipe_kernel<DGRAD, MAXONLY><<<g, b, 0, st>>>(in, wgt, out, N, H, W, absmax, tb, relu, shift_out, bits, sblk);
        break;
    case REQUANT:
        conv_pipe_kernel<DGRAD, REQUANT><<<g, b, 0, st>>>(in, wgt, out, N, H, W, absmax, tb, relu, shift_out, bits, sblk);
        break;
    default:
        conv_pipe_kernel<DGRAD, PARTIAL><<<g, b, 0, st>>>(in, wgt, out, N, H, W, absmax, tb, relu, shift_out, bits, sblk);
        break;
    }
}

}  // namespace

bool pipe_fits(int64_t W, int64_t act_bytes) {
    // W + 2 slots per halo row, and the rows a 256-pixel tile touches plus
    // the two around them within the 8 halo rows
    return W >= 1 && W + 2 <= RS && (TP - 1 + W - 1) / W + 3 <= HR && 4 * act_bytes < (int64_t(1) << 31);
}

void launch_pipe(bool dgrad, int mode, const int8_t *in, const int8_t *wgt, void *out, int N, int H, int W,
                 uint32_t *absmax, int target_bits, int relu, int32_t *shift_out, uint32_t *bits_out,
                 int32_t *shifts_blk, unsigned grid, hipStream_t st) {
    if (dgrad)
        launch_mode<true>(mode, in, wgt, out, N, H, W, absmax, target_bits, relu, shift_out, bits_out, shifts_blk,
                          grid, st);
    else
        launch_mode<false>(mode, in, wgt, out, N, H, W, absmax, target_bits, relu, shift_out, bits_out, shifts_blk,
                           grid, st);
}

}  // namespace c3
}  // namespace ionn
