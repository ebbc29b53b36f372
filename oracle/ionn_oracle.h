/*
 * ionn_oracle.h -- CPU oracle for the integer-only training step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the GPU library, and it never calls
 * into it.
 *
 * Sources (cited by page title and section):
 *  [TI]   "Integer On-Device Training: Overview" (TI C2000 MCU-AI user guide),
 *         section 3 "The NITI Algorithm" -> "The Solution: Dynamic Shifts",
 *         steps 1-5, and the note on delta propagation (target_bits = 7).
 *  [APT]  "Adaptive Precision Training for Resource Constrained Devices",
 *         the quantisation-underflow discussion (epsilon, Equations 2-3) and
 *         the Gavg metric (Equation 4).
 *  [DFP]  "Mixed Precision Training of Convolutional Neural Networks using
 *         Integer Operations" (source-linked summary), section 3 "The Dynamic
 *         Fixed Point Format", 3.1 "DFP Tensor Primitives", and section 4
 *         "Handling overflows".
 *  [TGR]  "Compilation Pipeline" (TiGrIS), the fully-connected weight index
 *         W[oc*IC + ic] and the NHWC activation layout.
 *
 * Conventions: row-major everywhere.  Linear: X[B][IN], W[OUT][IN],
 * Y[B][OUT].  Conv: NHWC activations, OHWI weights W[Cout][KH][KW][Cin],
 * cross-correlation (no kernel flip), stride 1, zero padding P.
 *
 * All accumulation is modulo 2^32 (done in uint32_t, then reinterpreted as
 * two's-complement int32).  Functions that accumulate also report how many
 * outputs would differ from the exact (int64) sum, i.e. how many wrapped.
 *
 * Where the pages leave a step open, the reading taken is stated next to the
 * function (ids U1..U22 of the design notes).
 */
#ifndef IONN_ORACLE_H
#define IONN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Thread count used by the parallel loops (OpenMP); returns the count in use. */
int ora_set_threads(int n);
int ora_get_threads(void);

/* ---- primitives ([TI] steps 1-3, 5) ---- */
uint32_t ora_abs_u32(int32_t x);
uint32_t ora_absmax_i32(const int32_t *x, int64_t n);
int      ora_bitlen_u32(uint32_t m);
int      ora_niti_shift(uint32_t max_val, int target_bits);
int32_t  ora_floor_shift(int32_t x, int s);
int32_t  ora_rhu(int32_t x, int s);
void     ora_rhu_array(const int32_t *x, int64_t n, int s, int32_t *out);
int32_t  ora_sat8(int64_t v);
int32_t  ora_sat16(int64_t v);
int      ora_ceil_log2(int64_t n);

/* ---- NITI quantiser and update ([TI] steps 1-5) ---- */
int ora_niti_requant(const int32_t *acc, int64_t n, int target_bits, int relu,
                     int8_t *out);
void ora_niti_update(const int32_t *G, int8_t *W, int64_t n, int target_bits,
                     int mu_weight, int32_t *gq_out, int *shift_out,
                     int *weight_shift_out);

/* ---- linear contractions ---- */
int64_t ora_linear_fwd(const int8_t *X, const int8_t *W, int32_t *Y,
                       int64_t B, int64_t IN, int64_t OUT);
int64_t ora_linear_dgrad(const int8_t *dY, const int8_t *W, int32_t *dX,
                         int64_t B, int64_t IN, int64_t OUT);
int64_t ora_linear_wgrad(const int8_t *dY, const int8_t *X, int32_t *G,
                         int64_t B, int64_t IN, int64_t OUT);
/* One output of each contraction, for sampled checks at full size. */
int32_t ora_linear_fwd_at(const int8_t *X, const int8_t *W, int64_t B,
                          int64_t IN, int64_t OUT, int64_t b, int64_t o);
int32_t ora_linear_dgrad_at(const int8_t *dY, const int8_t *W, int64_t B,
                            int64_t IN, int64_t OUT, int64_t b, int64_t i);
int32_t ora_linear_wgrad_at(const int8_t *dY, const int8_t *X, int64_t B,
                            int64_t IN, int64_t OUT, int64_t o, int64_t i);
/* Elementwise mask: d[j] = (act[j] > 0) ? d[j] : 0 (ReLU backward). */
void ora_relu_mask(int32_t *d, const int8_t *act, int64_t n);
/* Output error e[b][c] = (c == label[b] ? target_mag : 0) - out[b][c]. */
void ora_output_error(const int8_t *out, const int32_t *labels, int64_t B,
                      int64_t C, int target_mag, int32_t *e);

/* ---- convolution, stride 1, zero pad P, NHWC / OHWI ---- */
int64_t ora_conv_fwd(const int8_t *X, const int8_t *W, int32_t *Y, int64_t N,
                     int64_t H, int64_t Wd, int64_t Cin, int64_t Cout, int KH,
                     int KW, int P);
int64_t ora_conv_dgrad(const int8_t *dY, const int8_t *W, int32_t *dX,
                       int64_t N, int64_t H, int64_t Wd, int64_t Cin,
                       int64_t Cout, int KH, int KW, int P);
int64_t ora_conv_wgrad(const int8_t *dY, const int8_t *X, int32_t *G,
                       int64_t N, int64_t H, int64_t Wd, int64_t Cin,
                       int64_t Cout, int KH, int KW, int P);
int32_t ora_conv_fwd_at(const int8_t *X, const int8_t *W, int64_t N, int64_t H,
                        int64_t Wd, int64_t Cin, int64_t Cout, int KH, int KW,
                        int P, int64_t n, int64_t h, int64_t w, int64_t co);
int32_t ora_conv_dgrad_at(const int8_t *dY, const int8_t *W, int64_t N,
                          int64_t H, int64_t Wd, int64_t Cin, int64_t Cout,
                          int KH, int KW, int P, int64_t n, int64_t h,
                          int64_t w, int64_t ci);
int32_t ora_conv_wgrad_at(const int8_t *dY, const int8_t *X, int64_t N,
                          int64_t H, int64_t Wd, int64_t Cin, int64_t Cout,
                          int KH, int KW, int P, int64_t co, int64_t kh,
                          int64_t kw, int64_t ci);

/* ---- DFP16 ([DFP] 3.1 and 4) ---- */
/* Generic chunked contraction with element strides:
 *   acc[m*N + n] = sum_c rhu(p_c, r),  p_c = sum_{k in chunk c} A(m,k)*B(k,n)
 * where A(m,k) = A[m*sam + k*sak], B(k,n) = B[k*sbk + n*sbn], L = reduction
 * length, chunk = chunk length, r = chunk_shift(L, chunk).  Returns the number
 * of chunk partials whose exact value left the int32 range. */
int     ora_dfp_chunk_shift(int64_t L, int chunk);
int64_t ora_dfp_contract(const int16_t *A, int64_t sam, int64_t sak,
                         const int16_t *B, int64_t sbk, int64_t sbn, int64_t M,
                         int64_t N, int64_t L, int chunk, int32_t *acc);
/* Down-conversion: Rs = max(0, bitlen(max|acc|) - 15); out = sat16(rhu(acc, Rs)).
 * Returns Rs. */
int ora_dfp_downconvert(const int32_t *acc, int64_t n, int16_t *out);
/* The three roles; exponents are plain ints; returns 0, or -1 when the
 * output exponent leaves the signed 8-bit range. */
int ora_dfp16_fwd(const int16_t *X, int eX, const int16_t *W, int eW,
                  int16_t *Y, int *eY, int32_t *acc_tmp, int64_t M, int64_t K,
                  int64_t N, int chunk);
int ora_dfp16_dgrad(const int16_t *dY, int edY, const int16_t *W, int eW,
                    int16_t *dX, int *edX, int32_t *acc_tmp, int64_t M,
                    int64_t K, int64_t N, int chunk);
int ora_dfp16_wgrad(const int16_t *dY, int edY, const int16_t *X, int eX,
                    int16_t *G, int *eG, int32_t *acc_tmp, int64_t M,
                    int64_t K, int64_t N, int chunk);
/* Gavg = mean(|g|) * 2^(e_g - e_w)   ([APT] Equation 4, epsilon = 2^e_w). */
double ora_gavg(const int16_t *g, int64_t n, int e_g, int e_w);

/* Gradient of the MSE loss against per-class target magnitudes ([TI]
 * section 8, PC-side Step 3: TARGET_MAG_CORRECT[c] for the true class,
 * TARGET_MAG_WRONG[c] for the others), the loss delta the backward pass
 * reads (reading U27):
 *   g[b][c] = out[b][c] - (c == labels[b] ? tmc[c] : tmw[c]). */
void ora_mse_grad_targets(const int8_t *out, const int32_t *labels, int64_t B, int64_t C,
                          const int8_t *tmc, const int8_t *tmw, int32_t *g);

/* ---- Offsets (bias) and the static OSS forward requantisation ([TI]
 * section 7 "INT_LAYERS": int32 offsets updated by the backward pass, int8
 * per-filter right shifts k and multipliers mult; section 8, "PC-Side Steps",
 * Step 2: the OSS chain Add(offset) -> Mul(scale1) -> Mul(scale2) -> Floor
 * -> Clip) ---- */
/* out[m][c] = clip(floor(t * mult[c] / 2^k[c]), lo, 127) with
 * t = acc[m][c] + offset[c] modulo 2^32 (int32, as the accumulator), the
 * product exact in int64, lo = 0 if relu else -128 (reading U23).
 * k[c] in [0, 62]. */
void ora_oss_requant(const int32_t *acc, const int32_t *offset, const int32_t *mult,
                     const int8_t *k, int64_t M, int64_t C, int relu, int8_t *out);
/* gb[c] = sum_m d[m][c] over the int8 output error rows, modulo 2^32
 * (reading U24: the offset's gradient is the error summed over the batch,
 * as G is summed over it). */
void ora_bias_grad(const int8_t *d, int64_t M, int64_t C, int32_t *gb);
/* NITI update of int32 parameters (the offsets): the steps of
 * ora_niti_update with P = sat32(P - d) (reading U25). */
void ora_niti_update_i32(const int32_t *G, int32_t *P, int64_t n, int target_bits,
                         int mu, int32_t *gq_out, int *shift_out, int *weight_shift_out);

/* ---- Adaptive precision ([APT] Equations 1-4, Algorithms 1 and 2) ---- */
/* k-bit weights m with shared exponent e_w (eps = 2^e_w), k in [2, 16]. */
int32_t ora_sat_bits(int64_t v, int k);
/* W <- sat_k(W - change), change = g_m * 2^(e_g - lr_shift - e_w) rounded
 * half-up to the grid (reading U30).  Returns the underflow count. */
int64_t ora_apt_update(int16_t *W, int64_t n, int k, int e_w, const int16_t *G, int e_g,
                       int lr_shift);
/* Algorithm 1 on the epoch's summed Gavg samples: +1, 0 or -1 (reading U33). */
int ora_apt_decide(double gavg_sum, int32_t count, int k, double t_min, double t_max,
                   int k_min, int k_max);
/* The weights at precision k + dk, dk in {-1, 0, +1}, same range. */
void ora_apt_rescale(int16_t *W, int64_t n, int k, int dk);

/* ---- DFP as the DFP page runs it ([DFP] 3.1 conversions, 4 FP32 partials
 * with the 1-bit input shift, 3 Blocked-DFP; readings U34-U38) ---- */
int     ora_f32_floor_log2(float m);
int     ora_dfp_from_f32(const float *x, int64_t n, int P, int16_t *out, int *e_out);
int     ora_dfp_from_f32_blocked(const float *x, int64_t rows, int64_t K, int B, int P,
                                 int16_t *out, int32_t *e_out);
void    ora_dfp_to_f32(const int16_t *I, int64_t n, int e, float *out);
float   ora_scale_f32(float v, int e);
int64_t ora_dfp_contract_f32(const int16_t *A, int64_t sam, int64_t sak,
                             const int16_t *B, int64_t sbk, int64_t sbn, int64_t M,
                             int64_t N, int64_t L, int input_shift, int eA, int eB,
                             int S, float *out);
int64_t ora_dfp_fwd_f32_blocked(const int16_t *X, const int32_t *eX, const int16_t *W,
                                const int32_t *eW, int64_t M, int64_t K, int64_t N,
                                int input_shift, int S, float *out);
int     ora_dfp16_sgd(float *W32, const float *G32, int64_t n, float lr, int16_t *W16, int *eW);
float   ora_dfp_contract_f32_at(const int16_t *A, int64_t sam, int64_t sak, const int16_t *B,
                                int64_t sbk, int64_t sbn, int64_t L, int input_shift, int eA,
                                int eB, int S, int64_t m, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
