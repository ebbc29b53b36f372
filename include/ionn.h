/*
 * ionn.h -- C ABI of the integer-only training-step library for AMD MI355X
 * (gfx950).  Library file: libionn.so.
 *
 * What the calls compute is defined by these pages (cited by title and
 * section):
 *  [TI]   "Integer On-Device Training: Overview" (TI C2000 MCU-AI guide):
 *         section 3 "The NITI Algorithm" -> "The Solution: Dynamic Shifts"
 *         (steps 1-5, delta propagation with target_bits = 7); section 4
 *         (layers fill an activation buffer and a ReLU mask in the forward
 *         pass; the backward pass reads the loss delta and updates weights);
 *         section 7 (Conv2D, Conv2D+ReLU, Linear, Linear+ReLU layers; grouped
 *         and dilated convolutions are refused).
 *  [DFP]  "Mixed Precision Training of Convolutional Neural Networks using
 *         Integer Operations" (source-linked summary): section 3 (DFP-P
 *         tensor = integers + one shared signed 8-bit exponent), 3.1 (product
 *         exponent Ea+Eb; down-conversion by a right shift Rs), 4 "Handling
 *         overflows" (short int32 partial chains).
 *  [APT]  "Adaptive Precision Training for Resource Constrained Devices"
 *         (quantisation underflow, epsilon; the Gavg metric, Equation 4).
 *  [TGR]  "Compilation Pipeline" (TiGrIS): fully-connected weight index
 *         W[oc*IC + ic]; NHWC activations.
 *
 * Conventions for every call:
 *  - Tensors are DEVICE pointers, allocated and owned by the caller; the
 *    library keeps no pointer after a call returns and allocates nothing.
 *  - Row-major layouts.  Linear: X[B][IN], W[OUT][IN], Y[B][OUT].  Conv:
 *    NHWC activations, OHWI weights W[Cout][KH][KW][Cin], cross-correlation.
 *  - int8 x int8 products accumulate in int32 modulo 2^32 (two's-complement
 *    wrap), so results do not depend on summation order.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call checks
 *    its arguments on the host, then enqueues its kernels on `stream` and
 *    returns without waiting.  On any error nothing is enqueued.
 *  - absmax arguments are device uint32 scalars that the call MAX-COMBINES
 *    into: *absmax = max(*absmax, max |t|) with |INT32_MIN| = 2^31.  Set them
 *    to 0 first (ionn_fill_u32) when a fresh maximum is wanted.  Several
 *    calls may accumulate into one scalar (e.g. a tensor produced in parts).
 *  - Shifts and exponents produced by a call are written to device memory, so
 *    consecutive calls chain on the stream without a host round trip.
 *  - Return value: IONN_OK (0) or one of the IONN_ERR_* codes below;
 *    ionn_last_error() gives a message for the calling thread's last error.
 */
#ifndef IONN_H
#define IONN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    IONN_OK = 0,
    IONN_ERR_ARG = 1,    /* a required pointer is NULL, or a flag is invalid   */
    IONN_ERR_SHAPE = 2,  /* a size is negative, too large, or inconsistent     */
    IONN_ERR_RANGE = 3,  /* target_bits, mu_weight, chunk ... out of range     */
    IONN_ERR_ALIGN = 4,  /* a pointer lacks the alignment the call documents   */
    IONN_ERR_UNSUPPORTED = 5, /* geometry outside what the library implements */
    IONN_ERR_HIP = 6,    /* a HIP runtime call or kernel launch failed         */
    IONN_ERR_WORKSPACE = 7 /* workspace NULL or smaller than required          */
};

/* Message for a status code (static string). */
const char *ionn_status_str(int status);
/* Message describing the calling thread's most recent error ("" if none). */
const char *ionn_last_error(void);
/* Library version, e.g. "ionn 0.1.0 gfx950". */
const char *ionn_version(void);

/* ------------------------------------------------------------------------ */
/* Small helpers.                                                            */
/* ------------------------------------------------------------------------ */

/* dst[0..n) = value.  A kernel, not hipMemset, so it is safe inside captured
 * HIP graphs.  n >= 0. */
int ionn_fill_u32(uint32_t *dst, int64_t n, uint32_t value, void *stream);

/* [TI] step 1, "max_val = max(|G|)": max-combines max |x[j]| over j < n into
 * *absmax.  n >= 0 (n = 0 leaves *absmax unchanged). */
int ionn_absmax_i32(const int32_t *x, int64_t n, uint32_t *absmax, void *stream);

/* ------------------------------------------------------------------------ */
/* Linear layer contractions (int8 x int8 -> int32).                         */
/* Sizes: B, IN, OUT >= 0 and each < 2^31.                                   */
/* ------------------------------------------------------------------------ */

/* Forward product of a Linear layer ([TI] section 7, [TGR] FC index):
 *   Y[b][o] = sum_i X[b][i] * W[o][i].
 * X: int8 [B][IN]; W: int8 [OUT][IN]; Y: int32 [B][OUT] (written).
 * absmax_Y (nullable): max-combined with max |Y|. */
int int_linear_fwd(const int8_t *X, const int8_t *W, int32_t *Y, int64_t B,
                   int64_t IN, int64_t OUT, uint32_t *absmax_Y, void *stream);

/* Delta propagation (dgrad) of a Linear layer ([TI] section 3, delta
 * propagation; section 4, ReLU mask):
 *   dX[b][i] = sum_o dY[b][o] * W[o][i],
 * then, if relu_act is not NULL, dX[b][i] = 0 wherever relu_act[b][i] <= 0
 * (relu_act is the int8 [B][IN] output of the layer below, whose ReLU mask is
 * "activation > 0").  dY: int8 [B][OUT]; W: int8 [OUT][IN]; dX: int32
 * [B][IN] (written).  absmax_dX (nullable) sees the masked values. */
int int_linear_dgrad(const int8_t *dY, const int8_t *W, const int8_t *relu_act,
                     int32_t *dX, int64_t B, int64_t IN, int64_t OUT,
                     uint32_t *absmax_dX, void *stream);

/* Weight gradient of a Linear layer, the tensor G of [TI] section 3:
 *   G[o][i] = sum_b dY[b][o] * X[b][i].
 * dY: int8 [B][OUT]; X: int8 [B][IN]; G: int32 [OUT][IN] (written).
 * absmax_G (nullable): max-combined with max |G|. */
int int_linear_wgrad(const int8_t *dY, const int8_t *X, int32_t *G, int64_t B,
                     int64_t IN, int64_t OUT, uint32_t *absmax_G, void *stream);

/* The same weight gradient with a caller-provided workspace, for a small G
 * over a long batch (G within 32 blocks of 32 x 32, between 2 and 256 per
 * side, B >= 4096): each range of the batch leaves its partial G in the workspace
 * and one pass sums them (modulo 2^32, so the result is the one above bit
 * for bit) and takes the max, instead of adding into a cleared G with
 * atomics.  int_linear_wgrad_workspace_bytes gives the bytes needed (0 when
 * the shape does not take this path; then, or with dY / X not 4-byte
 * aligned, the call is int_linear_wgrad).  workspace: device, 4-byte
 * aligned, at least that many bytes, else IONN_ERR_WORKSPACE. */
size_t int_linear_wgrad_workspace_bytes(int64_t B, int64_t IN, int64_t OUT);
int int_linear_wgrad_ws(const int8_t *dY, const int8_t *X, int32_t *G, int64_t B,
                        int64_t IN, int64_t OUT, uint32_t *absmax_G, void *workspace,
                        size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* NITI quantiser and update ([TI] section 3, steps 1-5).                    */
/* ------------------------------------------------------------------------ */

/* Requantise an int32 tensor to int8 with one dynamic per-tensor shift:
 *   m  = *absmax (device; the caller has max-combined max |acc| into it);
 *   s  = max(0, bitlen(m) - target_bits)            (bitlen = ceil(log2(m+1)))
 *   out[j] = sat8(rhu(acc[j], s)), then max(out, 0) if relu != 0,
 * where rhu(x, s) = floor((x + 2^(s-1)) / 2^s) ("round-half-up", ties toward
 * +infinity) and sat8 clamps to [-128, 127].  target_bits = 7 is the delta
 * propagation setting.  shift_out (nullable, device int32) receives s.
 * n >= 0; target_bits in [1, 31]; relu in {0, 1}. */
int niti_quantize(const int32_t *acc, int64_t n, const uint32_t *absmax,
                  int target_bits, int relu, int8_t *out, int32_t *shift_out,
                  void *stream);

/* NITI weight update, in place on W:
 *   s  = max(0, bitlen(*absmax) - target_bits)
 *   ws = max(0, s - mu_weight)
 *   Gq = rhu(G[j], s)          (int32, not clamped)
 *   d  = rhu(Gq, ws)
 *   W[j] = sat8(W[j] - d)
 * Every W element is rewritten.  shifts_out (nullable, device int32[2])
 * receives {s, ws}.  gq_out (nullable, device int32[n]) receives Gq.
 * n >= 0; target_bits in [1, 31]; mu_weight in [0, 31]. */
int niti_quantize_update(const int32_t *G, int64_t n, const uint32_t *absmax,
                         int target_bits, int mu_weight, int8_t *W,
                         int32_t *shifts_out, int32_t *gq_out, void *stream);

/* One whole NITI step of a small Linear layer in one launch, for layers of
 * microcontroller size ([TI] section 3 "The NITI Algorithm", steps 1-5, and
 * the weight index of the TiGrIS "Compilation Pipeline" page), in this order:
 *   Y[b][o]  = sum_i X[b][i] * W[o][i]                  (int32)
 *   dX[b][i] = sum_o dY[b][o] * W[o][i]                 (int32, W before the update)
 *   delta    = sat8(rhu(dX, s_d)), s_d = max(0, bitlen(max |dX|) - tb_d)
 *   G[o][i]  = sum_b dY[b][o] * X[b][i]                 (int32)
 *   s = max(0, bitlen(max |G|) - tb_w), ws = max(0, s - mu_weight),
 *   Gq = rhu(G, s), W[o][i] = sat8(W[o][i] - rhu(Gq, ws)) (in place).
 * The same results as int_linear_fwd, int_linear_dgrad, niti_quantize,
 * int_linear_wgrad and niti_quantize_update in sequence, from one
 * workgroup.  Device buffers: X int8 [B][IN]; W int8 [OUT][IN] (read, then
 * rewritten); dY int8 [B][OUT]; Y int32 [B][OUT], dX int32 [B][IN], delta
 * int8 [B][IN], G int32 [OUT][IN], gq (nullable) int32 [OUT][IN], all
 * written; maxima uint32[3] receives max |Y|, max |dX|, max |G| (written,
 * not max-combined: nothing needs clearing first); shifts int32[3] receives
 * s_d, s, ws.  Requires int_linear_step_small_fits(B, IN, OUT): X, W and dY
 * together within 32 KiB (IONN_ERR_SHAPE otherwise); tb_w, tb_d in [1, 31];
 * mu_weight in [0, 31]. */
int int_linear_step_small(const int8_t *X, int8_t *W, const int8_t *dY,
                          int64_t B, int64_t IN, int64_t OUT, int tb_w,
                          int mu_weight, int tb_d, int32_t *Y, int32_t *dX,
                          int8_t *delta, int32_t *G, int32_t *gq,
                          uint32_t *maxima, int32_t *shifts, void *stream);

/* 1 when int_linear_step_small takes a layer of this shape (B, IN, OUT >= 1
 * and B*IN + OUT*IN + B*OUT <= 32768), else 0. */
int int_linear_step_small_fits(int64_t B, int64_t IN, int64_t OUT);

/* niti_quantize_update, which also sets clear[0 .. n_clear) to 0 (device
 * uint32, 0 <= n_clear <= 256, must not overlap *absmax).  For a training
 * loop that alternates two sets of max-combined scalars: the update of one
 * step clears the set the next step max-combines into, so no separate fill
 * precedes each step (a HIP graph then captures an even number of steps).
 * Nothing reads clear in the call; the clearing happens before the kernel
 * ends, so the next call on the stream sees zeros. */
int niti_quantize_update_clear(const int32_t *G, int64_t n,
                               const uint32_t *absmax, int target_bits,
                               int mu_weight, int8_t *W, int32_t *shifts_out,
                               int32_t *gq_out, uint32_t *clear,
                               int64_t n_clear, void *stream);

/* Output error of a classifier whose loss pushes the true class toward a
 * target magnitude and the others toward 0 ([TI] sections 4 and 6.2: user
 * loss writes the delta for the backward pass):
 *   e[b][c] = (c == labels[b] ? target_mag : 0) - out[b][c].
 * out: int8 [B][C]; labels: int32 [B] (values outside [0, C) match no class);
 * e: int32 [B][C] (written); absmax_e (nullable) max-combined.
 * target_mag in [-128, 127]. */
int int_output_error(const int8_t *out, const int32_t *labels, int64_t B,
                     int64_t C, int target_mag, int32_t *e, uint32_t *absmax_e,
                     void *stream);

/* ------------------------------------------------------------------------ */
/* Conv2D contractions ([TI] section 7), NHWC / OHWI, cross-correlation.     */
/* Geometry: stride 1, dilation 1, groups 1 (anything else returns           */
/* IONN_ERR_UNSUPPORTED; the page's export refuses grouped and dilated       */
/* convolutions outright); KH, KW in [1, 1024]; zero padding P = pad in     */
/* [0, 1024] (else IONN_ERR_RANGE).  Output Ho = H + 2P - KH + 1,             */
/* Wo = W + 2P - KW + 1.  N, H, W, Cin, Cout >= 0; every tensor must hold    */
/* fewer than 2^31 elements.  3x3 / pad 1 with Cin and Cout multiples of 16  */
/* runs on the matrix cores and needs 16-byte aligned tensors; other         */
/* geometries (e.g. the page's 16 x 2 "valid" filter bank) run on direct     */
/* kernels and need 4-byte aligned int32 tensors only.                       */
/* ------------------------------------------------------------------------ */

typedef struct ionn_conv_desc {
    int64_t N, H, W, Cin, Cout;
    int32_t KH, KW, stride, pad, dilation, groups;
} ionn_conv_desc;

/* Y[n,h,w,co] = sum_{kh,kw,ci} X[n,h+kh-P,w+kw-P,ci] * Wt[co,kh,kw,ci]
 * (zero outside the image).  X: int8 [N][H][W][Cin]; Wt: int8
 * [Cout][KH][KW][Cin]; Y: int32 [N][Ho][Wo][Cout] (written). */
int int_conv_fwd(const int8_t *X, const int8_t *Wt, int32_t *Y,
                 const ionn_conv_desc *desc, uint32_t *absmax_Y, void *stream);

/* dX[n,h,w,ci] = sum_{kh,kw,co} dY[n,h-kh+P,w-kw+P,co] * Wt[co,kh,kw,ci]
 * (terms outside dY dropped).  dY: int8 [N][Ho][Wo][Cout]; dX: int32
 * [N][H][W][Cin] (written). */
int int_conv_dgrad(const int8_t *dY, const int8_t *Wt, int32_t *dX,
                   const ionn_conv_desc *desc, uint32_t *absmax_dX,
                   void *stream);

/* The forward contraction with the NITI requantisation of its result fused
 * in ("Integer On-Device Training: Overview", section 3, steps 1-3 and the
 * ReLU of the Conv2D layer, section 7): Y8 = sat8(rhu(Y, s)), then
 * max(Y8, 0) if relu, with s = max(0, bitlen(max|Y|) - target_bits) and Y
 * the int32 sum of int_conv_fwd.  Y is never stored.
 *  - With a workspace (int_conv_requant_workspace_bytes(desc) bytes, 16-byte
 *    aligned, clobbered; IONN_ERR_WORKSPACE if smaller) and target_bits <= 7:
 *    one contraction pass stores, per block of 32 pixels x 64 channels,
 *    f = asr(Y, s_b) as int8 with the block's own shift s_b (it always fits
 *    int8) and bit s_b - 1 of every Y (its rounding bit) in the workspace;
 *    a streaming pass over Y8 then applies the tensor's shift s >= s_b:
 *    rhu(Y, s) = f + bit when s = s_b, rhu(f, s - s_b) otherwise.  Y8 must
 *    then be 16-byte aligned.
 *  - Without one (workspace NULL), or with target_bits > 7: the contraction
 *    runs twice, first for max|Y| only, then for the int8 output.
 * Same bits either way.  Y8: int8 [N][H][W][Cout] (written).  absmax_Y
 * (device, 4-byte aligned, required): must hold 0 on entry (ionn_fill_u32);
 * receives max|Y|.  shift_out (nullable, device): receives s.  Only 3x3 /
 * stride 1 / pad 1 with 64 input and 64 output channels and a width whose
 * halo fits (as the int32 fast path); other geometries return
 * IONN_ERR_UNSUPPORTED and take int_conv_fwd and niti_quantize.  X and Wt
 * 16-byte aligned, Y8 4-byte aligned. */
size_t int_conv_requant_workspace_bytes(const ionn_conv_desc *desc);
int int_conv_fwd_requant(const int8_t *X, const int8_t *Wt, int8_t *Y8,
                         const ionn_conv_desc *desc, int target_bits, int relu,
                         uint32_t *absmax_Y, int32_t *shift_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/* The same for delta propagation (section 3, the propagated-delta note:
 * target_bits = 7): dX8 = sat8(rhu(dX, s)) with dX the int32 sum of
 * int_conv_dgrad, never stored; one pass plus the streaming pass with a
 * workspace, two contraction passes without. */
int int_conv_dgrad_requant(const int8_t *dY, const int8_t *Wt, int8_t *dX8,
                           const ionn_conv_desc *desc, int target_bits,
                           uint32_t *absmax_dX, int32_t *shift_out,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Device workspace (bytes) that lets int_conv_wgrad take its fast path for
 * this geometry: for 64 input and 64 output channels (3x3, W up to about
 * 100), one partial G per compute unit; for a
 * full-row-window filter (no padding, KW = W, KH*W*Cin a multiple of 4, at
 * most 8 output channels), one partial G per workgroup (at most 1024).  0
 * when the geometry has no fast path (the call then needs no workspace). */
size_t int_conv_wgrad_workspace_bytes(const ionn_conv_desc *desc);

/* G[co,kh,kw,ci] = sum_{n,h,w} dY[n,h,w,co] * X[n,h+kh-P,w+kw-P,ci] over the
 * output positions (h, w) < (Ho, Wo).  G: int32 [Cout][KH][KW][Cin] (written).  workspace (nullable, device,
 * 16-byte aligned, ws_bytes long, owned by the caller, clobbered): with at
 * least int_conv_wgrad_workspace_bytes(desc) bytes, the gradient is
 * computed as per-compute-unit partial sums reduced in two passes; without
 * it, by a split-K product with integer atomics.  Same bits either way. */
int int_conv_wgrad(const int8_t *dY, const int8_t *X, int32_t *G,
                   const ionn_conv_desc *desc, uint32_t *absmax_G,
                   void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* DFP-16 shared-exponent contractions ([DFP] sections 3, 3.1, 4).           */
/*                                                                            */
/* A DFP-16 tensor is int16 mantissas I plus one shared exponent E (value     */
/* I * 2^E); E is a device int32 scalar that must lie in [-128, 127].  Each   */
/* contraction multiplies int16 x int16 -> int32 and sums the reduction in    */
/* chunks of `chunk` terms (the last chunk may be shorter).  Overflow         */
/* management: each chunk's int32 partial p_c is shifted down by              */
/* r = ceil(log2(number of chunks)) (0 for one chunk) with round-half-up      */
/* before the chunks are summed, acc = sum_c rhu(p_c, r) (int32).  Adaptive  */
/* down-conversion: Rs = max(0, bitlen(max |acc|) - 15),                      */
/* out = sat16(rhu(acc, Rs)), E_out = Ea + Eb + r + Rs.  If E_out leaves the  */
/* signed 8-bit range the output exponent is still written and the device     */
/* status word (status_out, nullable int32) is set to 1, else 0.              */
/*                                                                            */
/* Sizes: M, K, N >= 1, every tensor below 2^31 elements; chunk must be 64;  */
/* the int16 output must be 16-byte aligned.  `workspace` is device memory of */
/* at least dfp16_workspace_bytes(M, K, N, which) bytes, 256-byte aligned;    */
/* its contents on entry are ignored (it holds the int32 accumulator, the     */
/* max-abs scalar and, for dgrad/wgrad, K-major copies of the operands).      */
/* ------------------------------------------------------------------------ */

enum { IONN_DFP16_FWD = 0, IONN_DFP16_DGRAD = 1, IONN_DFP16_WGRAD = 2 };

size_t dfp16_workspace_bytes(int64_t M, int64_t K, int64_t N, int which);

/* Y[M][N] = X[M][K] . W[N][K]^T, reduced over K. */
int dfp16_gemm_fwd(const int16_t *X, const int32_t *eX, const int16_t *W,
                   const int32_t *eW, int16_t *Y, int32_t *eY, int64_t M,
                   int64_t K, int64_t N, int chunk, void *workspace,
                   size_t workspace_bytes, int32_t *status_out, void *stream);

/* dX[M][K] = dY[M][N] . W[N][K], reduced over N. */
int dfp16_gemm_dgrad(const int16_t *dY, const int32_t *edY, const int16_t *W,
                     const int32_t *eW, int16_t *dX, int32_t *edX, int64_t M,
                     int64_t K, int64_t N, int chunk, void *workspace,
                     size_t workspace_bytes, int32_t *status_out,
                     void *stream);

/* G[N][K] = dY[M][N]^T . X[M][K], reduced over M. */
int dfp16_gemm_wgrad(const int16_t *dY, const int32_t *edY, const int16_t *X,
                     const int32_t *eX, int16_t *G, int32_t *eG, int64_t M,
                     int64_t K, int64_t N, int chunk, void *workspace,
                     size_t workspace_bytes, int32_t *status_out,
                     void *stream);

/* Gavg of a layer ([APT] Equation 4): the mean gradient magnitude over the
 * layer's n parameters relative to the weights' resolution epsilon = 2^eW:
 *   gavg = (sum_j |G[j]| / n) * 2^(eG - eW),
 * the sum exact in int64, the division and scaling in IEEE double.
 * G: int16 [n]; eG, eW: device int32; gavg_out: device double (written).
 * n >= 1. */
int dfp16_gavg(const int16_t *G, const int32_t *eG, const int32_t *eW,
               int64_t n, double *gavg_out, void *stream);

/* ------------------------------------------------------------------------ */
/* DFP as the DFP page runs it ([DFP] 3.1: float -> DFP conversion with the   */
/* shared exponent from the exponent of the absolute maximum; 4 "Handling    */
/* overflows": int32 partials of short chains converted to FP32, scaled by    */
/* 2^(E_inp + E_wt) and accumulated into an FP32 output, the input shifted by */
/* one bit; 3: Blocked-DFP, several exponents per tensor; 4: the operations   */
/* around the integer kernels, the weight update among them, in floating      */
/* point).  Exponents are device int32.                                       */
/* ------------------------------------------------------------------------ */

/* The FP32-partial contractions: the roles and layouts of dfp16_gemm_*, with
 * an FP32 output instead of the down-converted DFP-16 one.  Per output:
 *   A' = rhu(A, input_shift)   (A is the data operand: X for fwd, dY for
 *                               dgrad and wgrad; input_shift 0 or 1)
 *   p_c = the 64-term chunk partials of A' . B   (int32, modulo 2^32)
 *   the chunks fall into S consecutive ranges, range s covering chunks
 *   [floor(n_c s / S), floor(n_c (s + 1) / S)); each range is summed in FP32
 *   in chunk order starting from 0 (every float(p_c) and every addition
 *   rounded to nearest even), the range sums are added in order to 0, and
 *   out = fl(total * 2^(eA + input_shift + eB)) with one rounding.
 * S = nsplit, or dfp16_f32_splits(M, K, N, which) when nsplit = 0 (a
 * function of the shape alone); 1 <= nsplit <= n_c.  The order is part of
 * the result: the same S gives the same bits on any path.  out: float,
 * 16-byte aligned.  workspace: dfp16_f32_workspace_bytes(M, K, N, which,
 * nsplit) bytes, 256-byte aligned (split partials, operand transposes). */
int dfp16_f32_splits(int64_t M, int64_t K, int64_t N, int which);
size_t dfp16_f32_workspace_bytes(int64_t M, int64_t K, int64_t N, int which,
                                 int nsplit);
int dfp16_gemm_fwd_f32(const int16_t *X, const int32_t *eX, const int16_t *W,
                       const int32_t *eW, float *Y, int64_t M, int64_t K,
                       int64_t N, int input_shift, int nsplit, void *workspace,
                       size_t workspace_bytes, void *stream);
int dfp16_gemm_dgrad_f32(const int16_t *dY, const int32_t *edY,
                         const int16_t *W, const int32_t *eW, float *dX,
                         int64_t M, int64_t K, int64_t N, int input_shift,
                         int nsplit, void *workspace, size_t workspace_bytes,
                         void *stream);
int dfp16_gemm_wgrad_f32(const int16_t *dY, const int32_t *edY,
                         const int16_t *X, const int32_t *eX, float *G,
                         int64_t M, int64_t K, int64_t N, int input_shift,
                         int nsplit, void *workspace, size_t workspace_bytes,
                         void *stream);

/* The forward contraction on Blocked-DFP operands whose blocks are the
 * 64-term chunks: X [M][K] with exponents eX[m * nch + c], W [N][K] with
 * eW[n * nch + c] (device int32, nch = ceil(K / 64); dfp_from_f32_blocked
 * with B = 64 writes this layout).  Each chunk's term is scaled on its own,
 * t_c = fl(float(p_c) * 2^(eX[m][c] + input_shift + eW[n][c])) (one
 * rounding), and the terms are summed in the order of dfp16_gemm_fwd_f32;
 * the output is not scaled again.  Workspace as dfp16_gemm_fwd_f32. */
int dfp16_gemm_fwd_f32_blocked(const int16_t *X, const int32_t *eX,
                               const int16_t *W, const int32_t *eW, float *Y,
                               int64_t M, int64_t K, int64_t N, int input_shift,
                               int nsplit, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Workspace bytes of dfp_from_f32 and dfp16_sgd_update (4-byte aligned). */
size_t dfp_convert_workspace_bytes(void);

/* FP32 -> DFP-P, P in [2, 16]: max |x| = f * 2^q (f in [1, 2)) gives
 * E = q - (P - 2) (0 for an all-zero x) and out = sat_P(round_to_nearest_even
 * (x / 2^E)).  x: float [n], 16-byte aligned; out: int16 [n], 8-byte aligned;
 * e_out: device int32; status_out (nullable): 0, 1 when E leaves the signed
 * 8-bit range (E still written), 2 when x holds a NaN or infinity (outputs
 * then unspecified). */
int dfp_from_f32(const float *x, int64_t n, int P, int16_t *out,
                 int32_t *e_out, int32_t *status_out, void *workspace,
                 size_t workspace_bytes, void *stream);

/* DFP -> FP32: out = fl(I * 2^e), one rounding (exact for normal results). */
int dfp_to_f32(const int16_t *I, int64_t n, const int32_t *e, float *out,
               void *stream);

/* Blocked-DFP: x [rows][K] float; every row is cut into blocks of B values
 * (the last one shorter when B does not divide K) and each block is
 * converted as dfp_from_f32 does with its own exponent,
 * e_out[r * ceil(K / B) + b].  status_out (nullable): the largest status of
 * any block. */
int dfp_from_f32_blocked(const float *x, int64_t rows, int64_t K, int B, int P,
                         int16_t *out, int32_t *e_out, int32_t *status_out,
                         void *stream);

/* The weight update of the DFP pipeline: FP32 master weights
 * W32 = fl(W32 - fl(lr * G32)) (two roundings, never fused), then their
 * DFP-16 copy W16 / eW (as dfp_from_f32 with P = 16) for the next forward.
 * W32, G32: float [n], 16-byte aligned; W16: int16 [n], 8-byte aligned. */
int dfp16_sgd_update(float *W32, const float *G32, int64_t n, float lr,
                     int16_t *W16, int32_t *eW, int32_t *status_out,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Per-channel offsets (bias) and the static OSS requantisation ([TI]        */
/* section 7: every layer carries mutable int32 offsets, updated by the      */
/* backward pass, and per-filter right shifts k with multipliers mult;       */
/* section 8, PC-side Step 2: the chain Add(offset) -> Mul(scale1) ->        */
/* Mul(scale2) -> Floor -> Clip).  Channels are the last dimension: C        */
/* output channels of a Linear layer or of an NHWC convolution output, with  */
/* M = rows (batch, times pixels for a convolution).                         */
/* ------------------------------------------------------------------------ */

/* out[m][c] = clip(floor(t * mult[c] / 2^k[c]), lo, 127),
 *   t = acc[m][c] + offset[c] modulo 2^32 (the int32 accumulator's add),
 *   the product exact in 64 bits, lo = 0 if relu (the *_RELU layer types)
 *   else -128.
 * acc: int32 [M][C]; offset, mult: int32 [C]; k: int8 [C], each in [0, 62]
 * (other values give unspecified outputs, no fault); out: int8 [M][C]
 * (written).  M, C >= 0, M * C < 2^31; relu in {0, 1}. */
int ionn_oss_requant(const int32_t *acc, const int32_t *offset,
                     const int32_t *mult, const int8_t *k, int64_t M,
                     int64_t C, int relu, int8_t *out, void *stream);

/* Forward of a Linear layer with its offsets and static OSS requantisation
 * in one call: Y[b][o] = oss(sum_i X[b][i] * W[o][i]) with the per-output
 * offset, mult and k of ionn_oss_requant (relu selects the *_RELU clip
 * range).  X: int8 [B][IN]; W: int8 [OUT][IN]; Y: int8 [B][OUT] (written).
 * Tile-aligned shapes (B, IN, OUT multiples of 256, IN > 0) with 16-byte
 * aligned X, W, offset, mult and 4-byte aligned k, Y run as one kernel whose
 * epilogue applies the chain to the int32 accumulators (no int32 tensor
 * reaches memory); other shapes or alignments compute the int32 product in
 * `workspace` (16-byte aligned, int_linear_fwd_oss_workspace_bytes bytes;
 * IONN_ERR_WORKSPACE without it) and then run the OSS pass. */
size_t int_linear_fwd_oss_workspace_bytes(int64_t B, int64_t IN, int64_t OUT);
int int_linear_fwd_oss(const int8_t *X, const int8_t *W, const int32_t *offset,
                       const int32_t *mult, const int8_t *k, int relu,
                       int8_t *Y, int64_t B, int64_t IN, int64_t OUT,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Gradient of the offsets: gb[c] = sum_m d[m][c] modulo 2^32, over the int8
 * output error d[M][C] that also feeds dgrad and wgrad.  gb: int32 [C],
 * overwritten.  The row ranges' sums pass through `workspace` (4-byte
 * aligned, ionn_bias_grad_workspace_bytes(M, C) bytes; IONN_ERR_WORKSPACE
 * when NULL or smaller, except for M = 0).  M, C >= 0, M * C < 2^31. */
size_t ionn_bias_grad_workspace_bytes(int64_t M, int64_t C);
int ionn_bias_grad(const int8_t *d, int64_t M, int64_t C, int32_t *gb,
                   void *workspace, size_t workspace_bytes, void *stream);

/* ionn_bias_grad for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same result, with the row-range sums held in a 2 MiB device array of
 * the library instead of a caller workspace.  Allocates nothing and calls
 * no allocating routine; each GPU the library runs on holds one such array
 * until the process ends.  Shapes whose sums need more than 2 MiB
 * (ionn_bias_grad_workspace_bytes(M, C) > 2 MiB) return IONN_ERR_SHAPE and
 * enqueue nothing.  All calls on one GPU share its array: calls that
 * overlap on one GPU (two streams, two threads) race and give unspecified
 * gb; calls ordered on a stream are independent (every entry a call reads
 * it has written first).  The stream's device must be the current device or
 * the stream must belong to it; the array's address is looked up once per
 * device (IONN_ERR_HIP if that lookup fails). */
int ionn_bias_grad_noalloc(const int8_t *d, int64_t M, int64_t C, int32_t *gb,
                           void *stream);

/* NITI update of int32 parameters (the offsets), in place on P: the steps of
 * niti_quantize_update with the last one P[j] = sat32(P[j] - d) (clamped to
 * the int32 range).  *absmax must hold max |G| (e.g. from ionn_absmax_i32).
 * shifts_out (nullable, device int32[2]) receives {s, ws}; gq_out (nullable,
 * device int32[n]) receives Gq.  n >= 0; target_bits in [1, 31]; mu in
 * [0, 31]. */
int niti_quantize_update_i32(const int32_t *G, int64_t n,
                             const uint32_t *absmax, int target_bits, int mu,
                             int32_t *P, int32_t *shifts_out, int32_t *gq_out,
                             void *stream);

/* ------------------------------------------------------------------------ */
/* Model-level driver: the INT_LAYERS forward and backward ([TI] section 7:  */
/* Conv2D, Conv2D+ReLU, Linear and Linear+ReLU layers with int8 weights,     */
/* int32 offsets and per-filter OSS shifts / multipliers; section 8: the OSS */
/* chain and the per-class TARGET_MAG loss; section 3: the NITI updates).    */
/* A sequence of the calls above on one stream; the caller owns the layer    */
/* parameters and one workspace, and the driver allocates nothing.           */
/* ------------------------------------------------------------------------ */

enum {
    IONN_LAYER_CONV2D = 0,
    IONN_LAYER_CONV2D_RELU = 1,
    IONN_LAYER_LINEAR = 2,
    IONN_LAYER_LINEAR_RELU = 3
};
#define IONN_MAX_LAYERS 64

/* One layer.  Per sample it reads H x W x Cin int8 values (NHWC; a Linear
 * layer has H = W = 1 and Cin = its input features) and writes, for a conv,
 * Ho x Wo x Cout (stride 1, zero padding pad, Ho = H + 2 pad - KH + 1,
 * Wo = W + 2 pad - KW + 1), for a Linear, Cout values.  Layer l + 1 must read
 * as many values per sample as layer l writes (a conv output feeds a Linear
 * as one NHWC row).  weight: int8 [Cout][KH][KW][Cin] or [Cout][Cin];
 * offset, mult: int32 [Cout]; k: int8 [Cout] in [0, 62] (the OSS chain of
 * ionn_oss_requant).  weight and offset are device tensors updated in place
 * by ionn_model_backward. */
typedef struct ionn_layer {
    int32_t type;
    int32_t KH, KW, pad;
    int64_t H, W, Cin, Cout;
    int8_t *weight;
    int32_t *offset;
    const int32_t *mult;
    const int8_t *k;
} ionn_layer;

/* Gradient of the MSE loss against per-class target magnitudes ([TI]
 * section 8, PC-side Step 3: TARGET_MAG_CORRECT[c] for the true class,
 * TARGET_MAG_WRONG[c] for the others):
 *   g[b][c] = out[b][c] - (c == labels[b] ? tmc[c] : tmw[c]).
 * out: int8 [B][C]; labels: int32 [B] (values outside [0, C) match no class);
 * tmc, tmw: int8 [C]; g: int32 [B][C] (written); absmax_g (nullable)
 * max-combined. */
int ionn_mse_grad_targets(const int8_t *out, const int32_t *labels, int64_t B,
                          int64_t C, const int8_t *tmc, const int8_t *tmw,
                          int32_t *g, uint32_t *absmax_g, void *stream);

/* d[j] = 0 where act[j] <= 0 (the ReLU mask of [TI] section 4), in place;
 * absmax_d (nullable) is max-combined with the masked values. */
int ionn_relu_mask_i32(int32_t *d, const int8_t *act, int64_t n,
                       uint32_t *absmax_d, void *stream);

/* Device workspace of the driver for this model and batch (0 and an error
 * message on an invalid model).  It holds every layer's activation between
 * ionn_model_forward and ionn_model_backward. */
size_t ionn_model_workspace_bytes(const ionn_layer *layers, int L, int64_t B);

/* Forward of the L layers over the batch X (int8 [B][H0][W0][Cin0]): per
 * layer the int32 contraction, then the OSS chain (ReLU clip for the *_RELU
 * types) into the layer's int8 activation, kept in `workspace` (256-byte
 * aligned, ionn_model_workspace_bytes bytes).  out (nullable): int8
 * [B][last layer's outputs] receives a copy of the last activation. */
int ionn_model_forward(const ionn_layer *layers, int L, const int8_t *X,
                       int64_t B, int8_t *out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Backward of the last ionn_model_forward on the same X and workspace, and
 * the updates: g = the MSE gradient of the last activation against the
 * per-class targets (ionn_mse_grad_targets), delta = niti_quantize(g,
 * tb_delta); for l = L..1: the offset gradient (ionn_bias_grad over the
 * batch and, for a conv, its output pixels), wgrad, and for l > 1 dgrad with
 * the pre-update weights, masked by layer l-1's activation > 0 when layer
 * l-1 has a ReLU, requantised with tb_delta; then niti_quantize_update of the
 * weights and niti_quantize_update_i32 of the offsets (tb_weight, mu).
 * shifts_out (nullable, device int32[1 + 5 L]): [0] the error's shift, then
 * per layer l at 1 + 5 l: the shift of the delta it propagates (-1 for the
 * first layer, which propagates none), {s, ws} of its weight update and
 * {s, ws} of its offset update.
 * Models of at most 8 layers and 2^22 multiply-adds per step whose layers'
 * operands fit in LDS run the forward and the backward as one workgroup each
 * (same bits); others run the sequence above as separate launches.  Either
 * way the calls are stream-ordered and allocate nothing. */
int ionn_model_backward(const ionn_layer *layers, int L, const int8_t *X,
                        int64_t B, const int32_t *labels, const int8_t *tmc,
                        const int8_t *tmw, int tb_delta, int tb_weight, int mu,
                        void *workspace, size_t workspace_bytes,
                        int32_t *shifts_out, void *stream);

/* ------------------------------------------------------------------------ */
/* Adaptive per-layer precision ([APT]: the weight resolution epsilon of a   */
/* k-bit tensor, Equation 2; the update of Equation 1 on that grid,          */
/* Equation 3; Gavg, Equation 4; the policy of Algorithm 1 applied between   */
/* epochs as Algorithm 2 lays out).                                          */
/*                                                                          */
/* Layer l holds k[l]-bit signed weight mantissas W[l] (int16 storage, or   */
/* int8 through the _mixed calls; the k-bit range [-2^(k-1), 2^(k-1) - 1]) */
/* with one shared exponent e_w[l]: a                                       */
/* weight is m * 2^e_w and one grid step is epsilon = 2^e_w.  k, e_w, the   */
/* gradient exponents e_g and the per-epoch Gavg sums are DEVICE int32 /    */
/* double arrays of L entries, so steps and epochs chain on the stream      */
/* without a host synchronisation.  W, G and n are HOST arrays of L device  */
/* pointers and sizes (2-byte aligned; 16-byte aligned tensors take the     */
/* vector path).  1 <= L <= IONN_MAX_LAYERS, 1 <= n[l] <= 2^36.  A k[l]     */
/* outside [2, 16] is read as the nearest bound.                             */
/* ------------------------------------------------------------------------ */

/* Workspace (bytes, 8-byte aligned) a sampling apt_update needs for these
 * layer sizes; 0 on invalid sizes. */
size_t apt_workspace_bytes(int L, const int64_t *n);

/* One step's update of every layer, in place on W:
 *   W[l][j] = sat_k(W[l][j] - c),  c = rhu(G[l][j], sigma) if sigma >= 0,
 *                                  c = G[l][j] * 2^-sigma   otherwise,
 *   sigma = e_w[l] + lr_shift - e_g[l]
 * i.e. W - lr * g with lr = 2^-lr_shift and g = G * 2^e_g, rounded to the
 * layer's grid (a change under half a step is lost: quantisation underflow).
 * G: int16 [n[l]] (a DFP-16 weight gradient, e.g. from dfp16_gemm_wgrad).
 * lr_shift in [0, 62].  Sampling: when gavg_sum (double [L]) and gavg_count
 * (int32 [L]) are given, every layer's Gavg of this gradient,
 * mean(|G|) * 2^(e_g - e_w) (as dfp16_gavg), is added to gavg_sum[l] and
 * gavg_count[l] grows by one; that needs `workspace`
 * (apt_workspace_bytes(L, n) bytes); both NULL: no sampling, no workspace. */
int apt_update(int L, int16_t *const *W, const int16_t *const *G,
               const int64_t *n, const int32_t *k, const int32_t *e_w,
               const int32_t *e_g, int lr_shift, double *gavg_sum,
               int32_t *gavg_count, void *workspace, size_t workspace_bytes,
               void *stream);

/* Between epochs, per layer (Algorithm 1 on the mean of the epoch's
 * samples, gavg_sum[l] / gavg_count[l]; no samples: no change):
 *   mean < t_min and k < k_max:  k += 1, e_w -= 1, m -> 2m
 *   mean > t_max and k > k_min:  k -= 1, e_w += 1, m -> sat_{k-1}(rhu(m, 1))
 * (the range stays, the grid step halves or doubles); then gavg_sum and
 * gavg_count are cleared.  dk_out (nullable, device int32 [L]) receives
 * each layer's change.  2 <= k_min <= k_max <= 16; t_min <= t_max (t_max
 * may be +inf: never lower).  No workspace. */
int apt_adjust(int L, int16_t *const *W, const int64_t *n, int32_t *k,
               int32_t *e_w, double *gavg_sum, int32_t *gavg_count,
               double t_min, double t_max, int k_min, int k_max,
               int32_t *dk_out, void *stream);

/* apt_update and apt_adjust over layers held at their own width, for the
 * memory saving low precision brings ([APT] section on the memory of
 * training): wbytes (HOST int32 [L]) gives each layer's bytes per weight,
 * 2 (int16 mantissas, as above) or 1 (int8 mantissas; W[l] 1-byte aligned,
 * 8-byte aligned for the vector path).  A layer held in int8 reads its k in
 * [2, 8] (a k above 8 as 8) and apt_adjust never raises it past 8, so its
 * mantissas always fit; the arithmetic is that of an int16 layer with the
 * same k, bit for bit.  wbytes NULL: every layer int16.  A wbytes entry other
 * than 1 or 2 is IONN_ERR_ARG. */
int apt_update_mixed(int L, void *const *W, const int32_t *wbytes,
                     const int16_t *const *G, const int64_t *n, const int32_t *k,
                     const int32_t *e_w, const int32_t *e_g, int lr_shift,
                     double *gavg_sum, int32_t *gavg_count, void *workspace,
                     size_t workspace_bytes, void *stream);
int apt_adjust_mixed(int L, void *const *W, const int32_t *wbytes, const int64_t *n,
                     int32_t *k, int32_t *e_w, double *gavg_sum,
                     int32_t *gavg_count, double t_min, double t_max, int k_min,
                     int k_max, int32_t *dk_out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* IONN_H */
