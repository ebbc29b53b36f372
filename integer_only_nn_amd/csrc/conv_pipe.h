// Launcher of the software-pipelined 3x3 convolution contraction (64 -> 64
// channels, stride 1, pad 1), compiled in its own translation unit
// (conv_pipe.hip) because its register layout needs a code-generation option
// of its own: the matrix-core accumulators live in VGPRs and the weight
// operand in AGPRs.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ionn {
namespace c3 {

// Whether the pipelined kernel takes this width (its halo of 80-byte slots
// fits one LDS buffer) and activation size (32-bit byte offsets).
bool pipe_fits(int64_t W, int64_t act_bytes);

// Launches fwd (dgrad = false) or dgrad over N x H x W pixels with the
// epilogue `mode` (conv3x3.h Mode: STORE32 int32 out, MAXONLY, REQUANT int8
// out with the shift from *absmax, PARTIAL int8 block-shift form with
// bits_out / shifts_blk) on `grid` persistent workgroups.  The caller has
// checked the geometry and alignment.
void launch_pipe(bool dgrad, int mode, const int8_t *in, const int8_t *wgt, void *out, int N, int H, int W,
                 uint32_t *absmax, int target_bits, int relu, int32_t *shift_out, uint32_t *bits_out,
                 int32_t *shifts_blk, unsigned grid, hipStream_t st);

}  // namespace c3
}  // namespace ionn
