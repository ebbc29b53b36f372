// Shared definitions of the 3x3 / stride 1 / pad 1 convolution fast paths for
// 64 input and 64 output channels (conv3x3.h and conv_pipe.hip): tile and
// halo constants, the halo loads straight into LDS, the epilogue modes and
// the weight-row order of the block-shift form.
#pragma once

#include "common.h"

namespace ionn {
namespace c3 {

typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int C = 64;            // input and output channels of the fast path
constexpr int TP = 256;          // output pixels per tile
constexpr int NTF = 512;         // threads per workgroup (eight wavefronts)
constexpr int SLOT = 80;         // LDS bytes per halo slot
constexpr int HALO_BYTES = 48 * 1024;
constexpr int HALO_CHUNKS = 2560;              // 16-byte halo chunks per tile, at most
constexpr int HALO_ITF = HALO_CHUNKS / NTF;    // the same per thread
constexpr int KS = 18;           // 576 / 32

// Bytes of the halo of a 256-pixel tile: rows touched by 256 consecutive
// pixels (at most ceil(255 / W) + 1) plus one above and one below.
inline int64_t halo_bytes(int64_t W) {
    const int64_t rows = (TP - 1 + W - 1) / W + 1 + 2;
    return rows * (W + 2) * SLOT;
}

inline bool fits(int64_t W) {
    return W >= 1 && halo_bytes(W) <= HALO_BYTES && ((TP - 1 + W - 1) / W + 3) * W * 4 <= HALO_CHUNKS;
}

// ---- fwd / dgrad ---------------------------------------------------------
// The halo of a tile is fetched straight into LDS (buffer_load ... lds, no
// registers in between), two tiles ahead, into one of three buffers.  A halo
// slot is 64 bytes (one pixel); 16-byte chunk c of slot s sits at chunk
// position 4 s + (c ^ ((s >> 2) & 3)), so eight consecutive slots read at
// one channel chunk land in eight distinct bank groups.  The loads go
// through a buffer resource over the activation tensor: pad slots, rows
// outside the image and rows past the tile get an offset beyond the end and
// are filled with zeros by the load itself.
constexpr int NB = 3;                          // halo buffers
constexpr int HBUF = 48 * 1024;                // bytes per buffer
constexpr int NI = HBUF / (NTF / 64) / 1024;   // 1 KiB loads per wavefront per tile (6)
constexpr uint32_t OOB = 0x80000000u;          // an offset past the end of any tensor taken here

// Halo rows of a 256-pixel tile: the rows it touches plus one above and below.
inline int64_t halo_rows(int64_t W) { return (TP - 1 + W - 1) / W + 1 + 2; }

// The fwd / dgrad fast path holds a tile's halo in one buffer and addresses
// the int8 input (act_bytes) and the int32 output with 32-bit offsets.
inline bool fits_fd(int64_t W, int64_t act_bytes) {
    return W >= 1 && halo_rows(W) * (W + 2) * 64 <= HBUF && 4 * act_bytes < (int64_t(1) << 31);
}

__device__ __forceinline__ int chunk_pos(int s, int c) { return 4 * s + (c ^ ((s >> 2) & 3)); }

// 64 lanes x 16 bytes from rsrc.base + voff into LDS at m0 + 16 * lane.  Not
// visible to the compiler: the kernel waits for these loads itself.
__device__ __forceinline__ void dma_lds16(v4i rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(n) alone (expcnt and lgkmcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// What the epilogue does with the int32 accumulators.
enum Mode : int {
    STORE32 = 0,  // store them (int32 out) and max-combine max|acc| into *absmax
    MAXONLY = 1,  // only max-combine max|acc| into *absmax (no output)
    REQUANT = 2,  // store int8 sat8(rhu(acc, s)) (ReLU optional), s from the
                  // finished *absmax and target_bits; block 0 writes s
    PARTIAL = 3,  // one pass of the requantisation (target_bits <= 7): each
                  // wavefront's 32 x 64 block is stored as int8
                  // f = asr(acc, s_b) with its own shift s_b = max(0,
                  // bitlen(max |acc| of the block) - target_bits), which
                  // always fits int8, plus bit s_b - 1 of every acc (the
                  // rounding bit) and s_b; max |acc| is max-combined into
                  // *absmax.  conv3x3_requant_fix then finishes every value
                  // with the tensor's shift s >= s_b:
                  // rhu(acc, s) = f + bit when s = s_b, rhu(f, s - s_b) else.
};

// Weight row loaded by fragment lane i (0..31) of a 32-channel block in
// PARTIAL mode: output row i of the 32 x 32 product is channel
// 16 ((i >> 2) & 1) + 4 (i >> 3) + (i & 3), so the 16 values a lane holds
// (rows 8 q + 4 (lane / 32) + j, q, j = 0..3) are the 16 consecutive
// channels 16 (lane / 32) .. + 15 of the block and leave in one 16-byte store.
__host__ __device__ constexpr int part_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// Vector-memory stores per wavefront and tile of each mode (the halo waits
// count them).
__host__ __device__ constexpr int stores_per_tile(int mode) {
    return mode == MAXONLY ? 0 : (mode == PARTIAL ? 4 : 8);
}

}  // namespace c3
}  // namespace ionn
