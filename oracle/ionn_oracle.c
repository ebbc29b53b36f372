/*
 * ionn_oracle.c -- CPU oracle for the integer-only training step.
 *
 * TEST INFRASTRUCTURE ONLY (see ionn_oracle.h).  Plain C99, no intrinsics,
 * no blocking or fusion: every function is the definition written out.
 * Parallel loops (OpenMP) split independent outputs only, so results do not
 * depend on the thread count.
 */
#include "ionn_oracle.h"

#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ora_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

int ora_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Reinterpret a 32-bit pattern as two's-complement int32 (defined behaviour). */
static int32_t u32_to_i32(uint32_t u)
{
    if (u <= 0x7fffffffu) return (int32_t)u;
    return -(int32_t)(~u) - 1;
}

static int exact_in_i32(int64_t v)
{
    return v >= -2147483648LL && v <= 2147483647LL;
}

/* ------------------------------------------------------------------------ */
/* Primitives.                                                               */
/* ------------------------------------------------------------------------ */

/* |x| as an unsigned 32-bit value, so |INT32_MIN| = 2^31 is representable
 * (reading U2). */
uint32_t ora_abs_u32(int32_t x)
{
    int64_t v = x;
    return (uint32_t)(v < 0 ? -v : v);
}

/* [TI] step 1: max_val = max(|G|) over the whole tensor; 0 for an empty one. */
uint32_t ora_absmax_i32(const int32_t *x, int64_t n)
{
    uint32_t m = 0;
    for (int64_t j = 0; j < n; ++j) {
        uint32_t a = ora_abs_u32(x[j]);
        if (a > m) m = a;
    }
    return m;
}

/* Number of binary digits of m: 0 for m = 0, else floor(log2 m) + 1.  This is
 * exactly ceil(log2(m + 1)) of [TI] step 2, computed without floating point
 * (reading U1). */
int ora_bitlen_u32(uint32_t m)
{
    int b = 0;
    while (m != 0) {
        ++b;
        m >>= 1;
    }
    return b;
}

/* [TI] step 2: shift = max(0, bits_needed - target_bits). */
int ora_niti_shift(uint32_t max_val, int target_bits)
{
    int s = ora_bitlen_u32(max_val) - target_bits;
    return s > 0 ? s : 0;
}

/* floor(v / 2^s) for a 64-bit value, 0 <= s <= 62. */
static int64_t floor_div_pow2_i64(int64_t v, int s)
{
    int64_t d = (int64_t)1 << s;
    if (v >= 0) return v / d;
    return -((-v + d - 1) / d);
}

/* floor(x / 2^s): an arithmetic right shift, written out because >> on a
 * negative int is implementation-defined in C99. */
int32_t ora_floor_shift(int32_t x, int s)
{
    return (int32_t)floor_div_pow2_i64((int64_t)x, s);
}

/* [TI] step 3 "round-half-up" shift: floor((x + 2^(s-1)) / 2^s) for s >= 1,
 * x for s = 0.  Ties go toward +infinity (reading U3).  The sum is formed in
 * 64 bits, so x near INT32_MAX does not overflow (reading U4). */
int32_t ora_rhu(int32_t x, int s)
{
    if (s <= 0) return x;
    return (int32_t)floor_div_pow2_i64((int64_t)x + ((int64_t)1 << (s - 1)), s);
}

/* rhu applied to every element of x (for exhaustive tests of the primitive). */
void ora_rhu_array(const int32_t *x, int64_t n, int s, int32_t *out)
{
    for (int64_t j = 0; j < n; ++j) out[j] = ora_rhu(x[j], s);
}

/* [TI] step 5: saturate to the int8 range. */
int32_t ora_sat8(int64_t v)
{
    if (v > 127) return 127;
    if (v < -128) return -128;
    return (int32_t)v;
}

/* The same saturation for the int16 mantissas of DFP-16 ([DFP] 3). */
int32_t ora_sat16(int64_t v)
{
    if (v > 32767) return 32767;
    if (v < -32768) return -32768;
    return (int32_t)v;
}

/* Least r with 2^r >= n (0 for n <= 1). */
int ora_ceil_log2(int64_t n)
{
    int r = 0;
    while (((int64_t)1 << r) < n) ++r;
    return r;
}

/* ------------------------------------------------------------------------ */
/* NITI quantiser ([TI] steps 1-3) and update ([TI] steps 1-5).              */
/* ------------------------------------------------------------------------ */

/* Requantise an int32 tensor to int8 with one dynamic per-tensor shift:
 * s = shift(max|acc|, target_bits); out = sat8(rhu(acc, s)); ReLU if asked.
 * target_bits = 7 is the delta-propagation setting of [TI] section 3.  The
 * rounding can reach +2^tb (e.g. 255 >> 1 -> 128); the int8 output saturates
 * it (reading U6).  Returns s. */
int ora_niti_requant(const int32_t *acc, int64_t n, int target_bits, int relu,
                     int8_t *out)
{
    int s = ora_niti_shift(ora_absmax_i32(acc, n), target_bits);
    for (int64_t j = 0; j < n; ++j) {
        int32_t v = ora_sat8(ora_rhu(acc[j], s));
        if (relu && v < 0) v = 0;
        out[j] = (int8_t)v;
    }
    return s;
}

/* NITI weight update, in place on W:
 *   s  = shift(max|G|, target_bits)            steps 1-2
 *   Gq = rhu(G, s)           (kept in int32)   step 3
 *   ws = max(0, s - mu_weight)                 step 4
 *   d  = rhu(Gq, ws)                           step 4 (second rounding, U5)
 *   W  = sat8(W - d)                           step 5
 * gq_out (nullable) receives Gq. */
void ora_niti_update(const int32_t *G, int8_t *W, int64_t n, int target_bits,
                     int mu_weight, int32_t *gq_out, int *shift_out,
                     int *weight_shift_out)
{
    int s = ora_niti_shift(ora_absmax_i32(G, n), target_bits);
    int ws = s - mu_weight;
    if (ws < 0) ws = 0;
    for (int64_t j = 0; j < n; ++j) {
        int32_t gq = ora_rhu(G[j], s);
        int32_t d = ora_rhu(gq, ws);
        if (gq_out) gq_out[j] = gq;
        W[j] = (int8_t)ora_sat8((int64_t)W[j] - (int64_t)d);
    }
    if (shift_out) *shift_out = s;
    if (weight_shift_out) *weight_shift_out = ws;
}

/* ------------------------------------------------------------------------ */
/* Linear layer: Y = X W^T, dX = dY W, G = dY^T X  ([TGR] W[oc*IC+ic]).       */
/* ------------------------------------------------------------------------ */

int32_t ora_linear_fwd_at(const int8_t *X, const int8_t *W, int64_t B,
                          int64_t IN, int64_t OUT, int64_t b, int64_t o)
{
    uint32_t acc = 0;
    (void)B;
    (void)OUT;
    for (int64_t i = 0; i < IN; ++i)
        acc += (uint32_t)((int32_t)X[b * IN + i] * (int32_t)W[o * IN + i]);
    return u32_to_i32(acc);
}

int32_t ora_linear_dgrad_at(const int8_t *dY, const int8_t *W, int64_t B,
                            int64_t IN, int64_t OUT, int64_t b, int64_t i)
{
    uint32_t acc = 0;
    (void)B;
    for (int64_t o = 0; o < OUT; ++o)
        acc += (uint32_t)((int32_t)dY[b * OUT + o] * (int32_t)W[o * IN + i]);
    return u32_to_i32(acc);
}

int32_t ora_linear_wgrad_at(const int8_t *dY, const int8_t *X, int64_t B,
                            int64_t IN, int64_t OUT, int64_t o, int64_t i)
{
    uint32_t acc = 0;
    for (int64_t b = 0; b < B; ++b)
        acc += (uint32_t)((int32_t)dY[b * OUT + o] * (int32_t)X[b * IN + i]);
    return u32_to_i32(acc);
}

/* Y[b][o] = sum_i X[b][i] * W[o][i]. */
int64_t ora_linear_fwd(const int8_t *X, const int8_t *W, int32_t *Y,
                       int64_t B, int64_t IN, int64_t OUT)
{
    int64_t wraps = 0;
#pragma omp parallel for schedule(static) reduction(+ : wraps)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t o = 0; o < OUT; ++o) {
            uint32_t acc = 0;
            int64_t exact = 0;
            for (int64_t i = 0; i < IN; ++i) {
                int32_t p = (int32_t)X[b * IN + i] * (int32_t)W[o * IN + i];
                acc += (uint32_t)p;
                exact += p;
            }
            Y[b * OUT + o] = u32_to_i32(acc);
            wraps += !exact_in_i32(exact);
        }
    }
    return wraps;
}

/* dX[b][i] = sum_o dY[b][o] * W[o][i]. */
int64_t ora_linear_dgrad(const int8_t *dY, const int8_t *W, int32_t *dX,
                         int64_t B, int64_t IN, int64_t OUT)
{
    int64_t wraps = 0;
#pragma omp parallel for schedule(static) reduction(+ : wraps)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < IN; ++i) {
            uint32_t acc = 0;
            int64_t exact = 0;
            for (int64_t o = 0; o < OUT; ++o) {
                int32_t p = (int32_t)dY[b * OUT + o] * (int32_t)W[o * IN + i];
                acc += (uint32_t)p;
                exact += p;
            }
            dX[b * IN + i] = u32_to_i32(acc);
            wraps += !exact_in_i32(exact);
        }
    }
    return wraps;
}

/* G[o][i] = sum_b dY[b][o] * X[b][i]. */
int64_t ora_linear_wgrad(const int8_t *dY, const int8_t *X, int32_t *G,
                         int64_t B, int64_t IN, int64_t OUT)
{
    int64_t wraps = 0;
#pragma omp parallel for schedule(static) reduction(+ : wraps)
    for (int64_t o = 0; o < OUT; ++o) {
        for (int64_t i = 0; i < IN; ++i) {
            uint32_t acc = 0;
            int64_t exact = 0;
            for (int64_t b = 0; b < B; ++b) {
                int32_t p = (int32_t)dY[b * OUT + o] * (int32_t)X[b * IN + i];
                acc += (uint32_t)p;
                exact += p;
            }
            G[o * IN + i] = u32_to_i32(acc);
            wraps += !exact_in_i32(exact);
        }
    }
    return wraps;
}

/* ReLU backward: a delta survives only where the stored activation was
 * positive (the ReLU mask of the forward pass, [TI] section 4.2). */
void ora_relu_mask(int32_t *d, const int8_t *act, int64_t n)
{
    for (int64_t j = 0; j < n; ++j)
        if (!(act[j] > 0)) d[j] = 0;
}

/* Output error of a classifier trained toward a target magnitude for the
 * true class and 0 elsewhere. */
void ora_output_error(const int8_t *out, const int32_t *labels, int64_t B,
                      int64_t C, int target_mag, int32_t *e)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c)
            e[b * C + c] =
                (c == (int64_t)labels[b] ? target_mag : 0) - (int32_t)out[b * C + c];
}

/* ------------------------------------------------------------------------ */
/* Convolution, stride 1, zero padding P, NHWC activations, OHWI weights.    */
/* Output spatial size: Ho = H + 2P - KH + 1, Wo = Wd + 2P - KW + 1.          */
/* ------------------------------------------------------------------------ */

static int64_t conv_out_dim(int64_t in, int k, int p) { return in + 2 * p - k + 1; }

int32_t ora_conv_fwd_at(const int8_t *X, const int8_t *W, int64_t N, int64_t H,
                        int64_t Wd, int64_t Cin, int64_t Cout, int KH, int KW,
                        int P, int64_t n, int64_t h, int64_t w, int64_t co)
{
    uint32_t acc = 0;
    (void)N;
    (void)Cout;
    for (int kh = 0; kh < KH; ++kh) {
        int64_t y = h + kh - P;
        if (y < 0 || y >= H) continue;
        for (int kw = 0; kw < KW; ++kw) {
            int64_t x = w + kw - P;
            if (x < 0 || x >= Wd) continue;
            for (int64_t ci = 0; ci < Cin; ++ci)
                acc += (uint32_t)((int32_t)X[((n * H + y) * Wd + x) * Cin + ci] *
                                  (int32_t)W[((co * KH + kh) * KW + kw) * Cin + ci]);
        }
    }
    return u32_to_i32(acc);
}

int32_t ora_conv_dgrad_at(const int8_t *dY, const int8_t *W, int64_t N,
                          int64_t H, int64_t Wd, int64_t Cin, int64_t Cout,
                          int KH, int KW, int P, int64_t n, int64_t h,
                          int64_t w, int64_t ci)
{
    int64_t Ho = conv_out_dim(H, KH, P), Wo = conv_out_dim(Wd, KW, P);
    uint32_t acc = 0;
    (void)N;
    for (int kh = 0; kh < KH; ++kh) {
        int64_t y = h - kh + P; /* output row that read input row h via tap kh */
        if (y < 0 || y >= Ho) continue;
        for (int kw = 0; kw < KW; ++kw) {
            int64_t x = w - kw + P;
            if (x < 0 || x >= Wo) continue;
            for (int64_t co = 0; co < Cout; ++co)
                acc += (uint32_t)((int32_t)dY[((n * Ho + y) * Wo + x) * Cout + co] *
                                  (int32_t)W[((co * KH + kh) * KW + kw) * Cin + ci]);
        }
    }
    return u32_to_i32(acc);
}

int32_t ora_conv_wgrad_at(const int8_t *dY, const int8_t *X, int64_t N,
                          int64_t H, int64_t Wd, int64_t Cin, int64_t Cout,
                          int KH, int KW, int P, int64_t co, int64_t kh,
                          int64_t kw, int64_t ci)
{
    int64_t Ho = conv_out_dim(H, KH, P), Wo = conv_out_dim(Wd, KW, P);
    uint32_t acc = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t h = 0; h < Ho; ++h) {
            int64_t y = h + kh - P;
            if (y < 0 || y >= H) continue;
            for (int64_t w = 0; w < Wo; ++w) {
                int64_t x = w + kw - P;
                if (x < 0 || x >= Wd) continue;
                acc += (uint32_t)((int32_t)dY[((n * Ho + h) * Wo + w) * Cout + co] *
                                  (int32_t)X[((n * H + y) * Wd + x) * Cin + ci]);
            }
        }
    return u32_to_i32(acc);
}

/* Y[n,h,w,co] = sum_{kh,kw,ci} X[n, h+kh-P, w+kw-P, ci] * W[co,kh,kw,ci]. */
int64_t ora_conv_fwd(const int8_t *X, const int8_t *W, int32_t *Y, int64_t N,
                     int64_t H, int64_t Wd, int64_t Cin, int64_t Cout, int KH,
                     int KW, int P)
{
    int64_t Ho = conv_out_dim(H, KH, P), Wo = conv_out_dim(Wd, KW, P);
    int64_t wraps = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(+ : wraps)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t h = 0; h < Ho; ++h)
            for (int64_t w = 0; w < Wo; ++w)
                for (int64_t co = 0; co < Cout; ++co) {
                    uint32_t acc = 0;
                    int64_t exact = 0;
                    for (int kh = 0; kh < KH; ++kh) {
                        int64_t y = h + kh - P;
                        if (y < 0 || y >= H) continue;
                        for (int kw = 0; kw < KW; ++kw) {
                            int64_t x = w + kw - P;
                            if (x < 0 || x >= Wd) continue;
                            for (int64_t ci = 0; ci < Cin; ++ci) {
                                int32_t p =
                                    (int32_t)X[((n * H + y) * Wd + x) * Cin + ci] *
                                    (int32_t)W[((co * KH + kh) * KW + kw) * Cin + ci];
                                acc += (uint32_t)p;
                                exact += p;
                            }
                        }
                    }
                    Y[((n * Ho + h) * Wo + w) * Cout + co] = u32_to_i32(acc);
                    wraps += !exact_in_i32(exact);
                }
    return wraps;
}

/* dX[n,h,w,ci] = sum_{kh,kw,co} dY[n, h-kh+P, w-kw+P, co] * W[co,kh,kw,ci]
 * (the adjoint of the forward map: every product X*W that fed an output
 * sends dY*W back to the input it read). */
int64_t ora_conv_dgrad(const int8_t *dY, const int8_t *W, int32_t *dX,
                       int64_t N, int64_t H, int64_t Wd, int64_t Cin,
                       int64_t Cout, int KH, int KW, int P)
{
    int64_t Ho = conv_out_dim(H, KH, P), Wo = conv_out_dim(Wd, KW, P);
    int64_t wraps = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(+ : wraps)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t w = 0; w < Wd; ++w)
                for (int64_t ci = 0; ci < Cin; ++ci) {
                    uint32_t acc = 0;
                    int64_t exact = 0;
                    for (int kh = 0; kh < KH; ++kh) {
                        int64_t y = h - kh + P;
                        if (y < 0 || y >= Ho) continue;
                        for (int kw = 0; kw < KW; ++kw) {
                            int64_t x = w - kw + P;
                            if (x < 0 || x >= Wo) continue;
                            for (int64_t co = 0; co < Cout; ++co) {
                                int32_t p =
                                    (int32_t)dY[((n * Ho + y) * Wo + x) * Cout + co] *
                                    (int32_t)W[((co * KH + kh) * KW + kw) * Cin + ci];
                                acc += (uint32_t)p;
                                exact += p;
                            }
                        }
                    }
                    dX[((n * H + h) * Wd + w) * Cin + ci] = u32_to_i32(acc);
                    wraps += !exact_in_i32(exact);
                }
    return wraps;
}

/* G[co,kh,kw,ci] = sum_{n,h,w} dY[n,h,w,co] * X[n, h+kh-P, w+kw-P, ci]. */
int64_t ora_conv_wgrad(const int8_t *dY, const int8_t *X, int32_t *G,
                       int64_t N, int64_t H, int64_t Wd, int64_t Cin,
                       int64_t Cout, int KH, int KW, int P)
{
    int64_t Ho = conv_out_dim(H, KH, P), Wo = conv_out_dim(Wd, KW, P);
    int64_t wraps = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(+ : wraps)
    for (int64_t co = 0; co < Cout; ++co)
        for (int kh = 0; kh < KH; ++kh)
            for (int kw = 0; kw < KW; ++kw)
                for (int64_t ci = 0; ci < Cin; ++ci) {
                    uint32_t acc = 0;
                    int64_t exact = 0;
                    for (int64_t n = 0; n < N; ++n)
                        for (int64_t h = 0; h < Ho; ++h) {
                            int64_t y = h + kh - P;
                            if (y < 0 || y >= H) continue;
                            for (int64_t w = 0; w < Wo; ++w) {
                                int64_t x = w + kw - P;
                                if (x < 0 || x >= Wd) continue;
                                int32_t p =
                                    (int32_t)dY[((n * Ho + h) * Wo + w) * Cout + co] *
                                    (int32_t)X[((n * H + y) * Wd + x) * Cin + ci];
                                acc += (uint32_t)p;
                                exact += p;
                            }
                        }
                    G[((co * KH + kh) * KW + kw) * Cin + ci] = u32_to_i32(acc);
                    wraps += !exact_in_i32(exact);
                }
    return wraps;
}

/* ------------------------------------------------------------------------ */
/* DFP-16 ([DFP] sections 3, 3.1, 4).                                        */
/*                                                                            */
/* A DFP tensor is an integer tensor I plus one shared exponent E, value       */
/* I * 2^E.  A product of two DFP-16 tensors is a 32-bit tensor with exponent */
/* Ea + Eb.  Overflow management: the reduction is split into chunks of       */
/* `chunk` terms; each chunk's int32 partial is right-shifted (round-half-up)  */
/* by r = ceil(log2(number of chunks)) before the chunks are summed, so the    */
/* sum of chunk results stays in int32 (readings U17, U18, U22).  The result  */
/* then has exponent Ea + Eb + r.  Down-conversion right-shifts the int32      */
/* tensor by Rs = max(0, bitlen(max|acc|) - 15) so it fits 16 bits (U19).      */
/* ------------------------------------------------------------------------ */

int ora_dfp_chunk_shift(int64_t L, int chunk)
{
    int64_t nc = (L + chunk - 1) / chunk;
    return nc <= 1 ? 0 : ora_ceil_log2(nc);
}

int64_t ora_dfp_contract(const int16_t *A, int64_t sam, int64_t sak,
                         const int16_t *B, int64_t sbk, int64_t sbn, int64_t M,
                         int64_t N, int64_t L, int chunk, int32_t *acc_out)
{
    int r = ora_dfp_chunk_shift(L, chunk);
    int64_t wraps = 0;
#pragma omp parallel for schedule(static) reduction(+ : wraps)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            uint32_t acc = 0;
            for (int64_t k0 = 0; k0 < L; k0 += chunk) {
                uint32_t p = 0;
                int64_t exact = 0;
                for (int64_t k = k0; k < k0 + chunk && k < L; ++k) {
                    int32_t a = A[m * sam + k * sak], b = B[k * sbk + n * sbn];
                    p += (uint32_t)(a * b);
                    exact += (int64_t)a * b;
                }
                wraps += !exact_in_i32(exact);
                acc += (uint32_t)ora_rhu(u32_to_i32(p), r);
            }
            acc_out[m * N + n] = u32_to_i32(acc);
        }
    }
    return wraps;
}

int ora_dfp_downconvert(const int32_t *acc, int64_t n, int16_t *out)
{
    int rs = ora_niti_shift(ora_absmax_i32(acc, n), 15);
    for (int64_t j = 0; j < n; ++j)
        out[j] = (int16_t)ora_sat16(ora_rhu(acc[j], rs));
    return rs;
}

static int dfp_finish(const int32_t *acc, int64_t n, int16_t *out, int e_in,
                      int r, int *e_out)
{
    int rs = ora_dfp_downconvert(acc, n, out);
    int e = e_in + r + rs;
    *e_out = e;
    /* One signed 8-bit shared exponent per tensor ([DFP] 3). */
    return (e < -128 || e > 127) ? -1 : 0;
}

/* Forward: Y[M][N] = X[M][K] . W[N][K]^T, reduced over K. */
int ora_dfp16_fwd(const int16_t *X, int eX, const int16_t *W, int eW,
                  int16_t *Y, int *eY, int32_t *acc, int64_t M, int64_t K,
                  int64_t N, int chunk)
{
    ora_dfp_contract(X, K, 1, W, 1, K, M, N, K, chunk, acc);
    return dfp_finish(acc, M * N, Y, eX + eW, ora_dfp_chunk_shift(K, chunk), eY);
}

/* Backward data: dX[M][K] = dY[M][N] . W[N][K], reduced over N. */
int ora_dfp16_dgrad(const int16_t *dY, int edY, const int16_t *W, int eW,
                    int16_t *dX, int *edX, int32_t *acc, int64_t M, int64_t K,
                    int64_t N, int chunk)
{
    ora_dfp_contract(dY, N, 1, W, K, 1, M, K, N, chunk, acc);
    return dfp_finish(acc, M * K, dX, edY + eW, ora_dfp_chunk_shift(N, chunk), edX);
}

/* Weight gradient: G[N][K] = dY[M][N]^T . X[M][K], reduced over M. */
int ora_dfp16_wgrad(const int16_t *dY, int edY, const int16_t *X, int eX,
                    int16_t *G, int *eG, int32_t *acc, int64_t M, int64_t K,
                    int64_t N, int chunk)
{
    ora_dfp_contract(dY, 1, N, X, K, 1, N, K, M, chunk, acc);
    return dfp_finish(acc, N * K, G, edY + eX, ora_dfp_chunk_shift(M, chunk), eG);
}

/* [APT] Equation 4 as the text describes it: the mean magnitude of a layer's
 * gradient over its N parameters, divided by the layer's minimum weight
 * resolution epsilon.  With the gradient stored as DFP (g * 2^e_g) and
 * epsilon = 2^e_w (one step of the weight mantissa, reading U20):
 *   Gavg = (sum |g| / N) * 2^(e_g - e_w).
 * The sum is exact in int64; the scaling by a power of two is exact. */
double ora_gavg(const int16_t *g, int64_t n, int e_g, int e_w)
{
    int64_t sum = 0;
    if (n <= 0) return 0.0;
    for (int64_t j = 0; j < n; ++j) sum += g[j] < 0 ? -(int64_t)g[j] : (int64_t)g[j];
    double v = (double)sum / (double)n;
    int e = e_g - e_w;
    for (; e > 0; --e) v *= 2.0;
    for (; e < 0; ++e) v *= 0.5;
    return v;
}

/* ------------------------------------------------------------------------ */
/* Offsets (bias) and the static OSS forward requantisation.                 */
/* ------------------------------------------------------------------------ */

/* floor(v / 2^k) for k in [0, 62], written with non-negative shifts only. */
static int64_t floor_div_pow2(int64_t v, int k)
{
    const int64_t d = (int64_t)1 << k;
    if (v >= 0) return v / d;
    return -((-v + d - 1) / d);
}

/* [TI] section 8, Step 2: Add(offset) -> Mul(scale1 = mult) -> Mul(scale2 =
 * 2^-k) -> Floor -> Clip, on the int32 accumulator of output channel c. */
void ora_oss_requant(const int32_t *acc, const int32_t *offset, const int32_t *mult,
                     const int8_t *k, int64_t M, int64_t C, int relu, int8_t *out)
{
    const int64_t lo = relu ? 0 : -128;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < C; ++c) {
            const int32_t t = u32_to_i32((uint32_t)acc[m * C + c] + (uint32_t)offset[c]);
            int64_t y = floor_div_pow2((int64_t)t * (int64_t)mult[c], k[c]);
            if (y < lo) y = lo;
            if (y > 127) y = 127;
            out[m * C + c] = (int8_t)y;
        }
}

/* The offset's gradient: the output error summed over the rows (batch, and
 * pixels for a convolution). */
void ora_bias_grad(const int8_t *d, int64_t M, int64_t C, int32_t *gb)
{
    for (int64_t c = 0; c < C; ++c) {
        uint32_t s = 0;
        for (int64_t m = 0; m < M; ++m) s += (uint32_t)(int32_t)d[m * C + c];
        gb[c] = u32_to_i32(s);
    }
}

/* [TI] section 3 steps 1-5 on int32 parameters; the final clamp is to the
 * int32 range instead of int8. */
void ora_niti_update_i32(const int32_t *G, int32_t *P, int64_t n, int target_bits,
                         int mu, int32_t *gq_out, int *shift_out, int *weight_shift_out)
{
    int s = ora_niti_shift(ora_absmax_i32(G, n), target_bits);
    int ws = s - mu;
    if (ws < 0) ws = 0;
    for (int64_t j = 0; j < n; ++j) {
        int32_t gq = ora_rhu(G[j], s);
        int32_t d = ora_rhu(gq, ws);
        int64_t v = (int64_t)P[j] - (int64_t)d;
        if (v < -2147483648LL) v = -2147483648LL;
        if (v > 2147483647LL) v = 2147483647LL;
        if (gq_out) gq_out[j] = gq;
        P[j] = (int32_t)v;
    }
    if (shift_out) *shift_out = s;
    if (weight_shift_out) *weight_shift_out = ws;
}

/* [TI] section 8, Step 3: the MSE loss against per-class target magnitudes;
 * its gradient with respect to the output. */
void ora_mse_grad_targets(const int8_t *out, const int32_t *labels, int64_t B, int64_t C,
                          const int8_t *tmc, const int8_t *tmw, int32_t *g)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c) {
            const int32_t t = (c == (int64_t)labels[b]) ? (int32_t)tmc[c] : (int32_t)tmw[c];
            g[b * C + c] = (int32_t)out[b * C + c] - t;
        }
}

/* ------------------------------------------------------------------------ */
/* Adaptive precision ([APT]): a layer's weights are k-bit signed integers    */
/* m with one shared exponent e, so one step of the grid is eps = 2^e         */
/* (Equation 2, reading U29); the update of Equation 1 lands on that grid     */
/* (Equation 3, reading U30); Algorithm 1 moves k by one bit per epoch.       */
/* ------------------------------------------------------------------------ */

/* Saturate to the signed k-bit range [-2^(k-1), 2^(k-1) - 1], k in [1, 32]. */
int32_t ora_sat_bits(int64_t v, int k)
{
    const int64_t hi = ((int64_t)1 << (k - 1)) - 1;
    const int64_t lo = -((int64_t)1 << (k - 1));
    if (v > hi) return (int32_t)hi;
    if (v < lo) return (int32_t)lo;
    return (int32_t)v;
}

/* The change of one weight in units of eps for W <- W - lr * g, with
 * lr = 2^-lr_shift, g = g_m * 2^e_g and eps = 2^e_w:  g_m * 2^-sigma,
 * sigma = e_w + lr_shift - e_g.  When sigma > 0 the change is rounded to
 * the grid half-up (a change under half a step is lost: quantisation
 * underflow); when sigma < 0 it is exact.  |g_m| < 2^15, so a shift past 40
 * either way gives the same final weight as any larger one. */
static int64_t apt_change(int32_t g, int64_t sigma)
{
    if (sigma >= 0) return sigma > 40 ? 0 : (int64_t)ora_rhu(g, (int)sigma);
    if (sigma < -40) sigma = -40;
    return (int64_t)g * ((int64_t)1 << (-sigma));
}

/* In place: W[j] = sat_k(W[j] - change(G[j])).  Returns how many nonzero
 * gradients changed nothing (underflowed). */
int64_t ora_apt_update(int16_t *W, int64_t n, int k, int e_w, const int16_t *G, int e_g,
                       int lr_shift)
{
    const int64_t sigma = (int64_t)e_w + (int64_t)lr_shift - (int64_t)e_g;
    int64_t under = 0;
    for (int64_t j = 0; j < n; ++j) {
        const int64_t u = apt_change(G[j], sigma);
        if (u == 0 && G[j] != 0) ++under;
        W[j] = (int16_t)ora_sat_bits((int64_t)W[j] - u, k);
    }
    return under;
}

/* Algorithm 1 for one layer (reading U33): the mean of the epoch's Gavg
 * samples against the limits; +1 raises k, -1 lowers it, 0 keeps it.  A
 * layer without samples keeps its precision. */
int ora_apt_decide(double gavg_sum, int32_t count, int k, double t_min, double t_max,
                   int k_min, int k_max)
{
    if (count <= 0) return 0;
    const double mean = gavg_sum / (double)count;
    if (mean < t_min && k < k_max) return 1;
    if (mean > t_max && k > k_min) return -1;
    return 0;
}

/* The weights at the new precision, same range (reading U33): one more bit
 * halves eps, so m -> 2m (exact) and e -> e - 1; one bit less doubles it,
 * so m -> sat_{k-1}(rhu(m, 1)) and e -> e + 1. */
void ora_apt_rescale(int16_t *W, int64_t n, int k, int dk)
{
    for (int64_t j = 0; j < n; ++j) {
        if (dk > 0) W[j] = (int16_t)ora_sat_bits(2 * (int64_t)W[j], k + 1);
        else if (dk < 0) W[j] = (int16_t)ora_sat_bits(ora_rhu(W[j], 1), k - 1);
    }
}

/* ------------------------------------------------------------------------ */
/* DFP as the DFP page runs it ([DFP] 3.1: float -> DFP conversion by the    */
/* exponent of the absolute maximum, and back; 4 "Handling overflows": int32 */
/* chunk partials converted to FP32, scaled by 2^(E_inp + E_wt) and summed   */
/* into an FP32 output, with the input shifted by one bit; 3: Blocked-DFP,   */
/* several exponents per tensor).  Readings U34-U38.                         */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x)
{
    union { float f; uint32_t u; } v;
    v.f = x;
    return v.u;
}

/* 2^e as a double, e in [-1022, 1023], by repeated exact doubling/halving. */
static double pow2d(int e)
{
    double v = 1.0;
    for (; e > 0; --e) v *= 2.0;
    for (; e < 0; ++e) v *= 0.5;
    return v;
}

/* floor(log2 m) of a finite m > 0, read from the IEEE single fields. */
int ora_f32_floor_log2(float m)
{
    const uint32_t u = f32_bits(m) & 0x7fffffffu;
    const int ex = (int)(u >> 23);
    if (ex > 0) return ex - 127;
    return -150 + ora_bitlen_u32(u & 0x7fffffu);   /* subnormal: mantissa * 2^-149 */
}

/* Round a double with |v| < 2^52 to the nearest integer, ties to even. */
static int64_t rne_i64(double v)
{
    int64_t t = (int64_t)v;            /* toward zero, exact for |v| < 2^52 */
    double f = v - (double)t;          /* exact: the fraction, sign of v */
    if (f > 0.5 || (f == 0.5 && (t & 1))) ++t;
    else if (f < -0.5 || (f == -0.5 && (t & 1))) --t;
    return t;
}

/* One element of a P-bit DFP tensor with shared exponent E:
 * sat_P(round_to_nearest_even(x / 2^E)), the division exact in double. */
static int32_t dfp_elem(float x, int E, int P)
{
    const double v = (double)x * pow2d(-E);
    return ora_sat_bits(rne_i64(v), P);
}

/* Shared exponent of a P-bit tensor whose max |x| is m (reading U34):
 * m = f * 2^q with f in [1, 2) gives E = q - (P - 2), so that m / 2^E lies in
 * [2^(P-2), 2^(P-1)); 0 for m = 0. */
static int dfp_exponent(float m, int P)
{
    return m > 0.0f ? ora_f32_floor_log2(m) - (P - 2) : 0;
}

/* Float -> DFP-P (P in [2, 16]) over n values with one exponent.  Returns 0,
 * 1 when the exponent leaves the signed 8-bit range (still written), 2 when
 * a value is not finite (outputs then unspecified). */
int ora_dfp_from_f32(const float *x, int64_t n, int P, int16_t *out, int *e_out)
{
    float m = 0.0f;
    for (int64_t j = 0; j < n; ++j) {
        const float a = x[j] < 0.0f ? -x[j] : x[j];
        if (!(a <= 3.402823466e38f)) return 2;       /* inf or NaN */
        if (a > m) m = a;
    }
    const int E = dfp_exponent(m, P);
    for (int64_t j = 0; j < n; ++j) out[j] = (int16_t)dfp_elem(x[j], E, P);
    *e_out = E;
    return (E < -128 || E > 127) ? 1 : 0;
}

/* Blocked-DFP: rows of K values, each split into blocks of B consecutive
 * values (the last one shorter when B does not divide K), one exponent per
 * block: e_out[r * nb + b], nb = ceil(K / B).  Returns as ora_dfp_from_f32
 * (1 when any exponent leaves the 8-bit range). */
int ora_dfp_from_f32_blocked(const float *x, int64_t rows, int64_t K, int B, int P,
                             int16_t *out, int32_t *e_out)
{
    const int64_t nb = (K + B - 1) / B;
    int st = 0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t k0 = b * B, k1 = (k0 + B < K) ? k0 + B : K;
            int e = 0;
            const int s = ora_dfp_from_f32(x + r * K + k0, k1 - k0, P, out + r * K + k0, &e);
            if (s == 2) return 2;
            if (s == 1) st = 1;
            e_out[r * nb + b] = e;
        }
    return st;
}

/* Exponent sums beyond the double range: clamped to [-1022, 1023], where
 * every single-precision result is already 0 or infinite (reading U35). */
static int clamp_exp(int e)
{
    return e < -1022 ? -1022 : (e > 1023 ? 1023 : e);
}

/* DFP -> float: out = I * 2^e rounded once to single (exact whenever the
 * value is a normal single). */
void ora_dfp_to_f32(const int16_t *I, int64_t n, int e, float *out)
{
    const double s = pow2d(clamp_exp(e));
    for (int64_t j = 0; j < n; ++j) out[j] = (float)((double)I[j] * s);
}

/* fl(v * 2^e): the exact product in double, rounded once to single. */
float ora_scale_f32(float v, int e)
{
    return (float)((double)v * pow2d(clamp_exp(e)));
}

/* Chunk ranges of the FP32 accumulation: range s of S covers chunks
 * [floor(nch * s / S), floor(nch * (s + 1) / S)). */
static int64_t range_start(int64_t nch, int S, int s)
{
    return nch * s / S;
}

/* The FP32-partial contraction (reading U35), per output (m, n):
 *   A'(m,k) = rhu(A(m,k), input_shift)   (the input shifted by one bit)
 *   p_c     = sum over chunk c of A'(m,k) * B(k,n)     (int32, modulo 2^32)
 *   part_s  = 0 + float(p_c0) + float(p_c0+1) + ...    (single, in order)
 *   total   = 0 + part_0 + part_1 + ... + part_{S-1}   (single, in order)
 *   out     = fl(total * 2^(eA + input_shift + eB))
 * with A(m,k) = A[m*sam + k*sak], B(k,n) = B[k*sbk + n*sbn], 64-term chunks.
 * Returns the number of chunk partials whose exact value left int32. */
int64_t ora_dfp_contract_f32(const int16_t *A, int64_t sam, int64_t sak,
                             const int16_t *B, int64_t sbk, int64_t sbn, int64_t M,
                             int64_t N, int64_t L, int input_shift, int eA, int eB,
                             int S, float *out)
{
    const int64_t nch = (L + 63) / 64;
    const int e = eA + input_shift + eB;
    int64_t wraps = 0;
#pragma omp parallel for schedule(static) reduction(+ : wraps)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float total = 0.0f;
            for (int s = 0; s < S; ++s) {
                float part = 0.0f;
                for (int64_t c = range_start(nch, S, s); c < range_start(nch, S, s + 1); ++c) {
                    uint32_t p = 0;
                    int64_t exact = 0;
                    for (int64_t k = 64 * c; k < 64 * c + 64 && k < L; ++k) {
                        const int32_t a = ora_rhu(A[m * sam + k * sak], input_shift);
                        const int32_t b = B[k * sbk + n * sbn];
                        p += (uint32_t)(a * b);
                        exact += (int64_t)a * b;
                    }
                    wraps += !exact_in_i32(exact);
                    part = part + (float)u32_to_i32(p);
                }
                total = total + part;
            }
            out[m * N + n] = ora_scale_f32(total, e);
        }
    return wraps;
}

/* The forward contraction on Blocked-DFP operands whose blocks are the
 * 64-term chunks (reading U37): X [M][K] with exponents eX[m][c], W [N][K]
 * with eW[n][c]; every chunk's term is scaled on its own,
 *   t_c = fl(float(p_c) * 2^(eX[m][c] + input_shift + eW[n][c])),
 * and the terms are summed as in ora_dfp_contract_f32 (S ranges in order). */
int64_t ora_dfp_fwd_f32_blocked(const int16_t *X, const int32_t *eX, const int16_t *W,
                                const int32_t *eW, int64_t M, int64_t K, int64_t N,
                                int input_shift, int S, float *out)
{
    const int64_t nch = (K + 63) / 64;
    int64_t wraps = 0;
#pragma omp parallel for schedule(static) reduction(+ : wraps)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float total = 0.0f;
            for (int s = 0; s < S; ++s) {
                float part = 0.0f;
                for (int64_t c = range_start(nch, S, s); c < range_start(nch, S, s + 1); ++c) {
                    uint32_t p = 0;
                    int64_t exact = 0;
                    for (int64_t k = 64 * c; k < 64 * c + 64 && k < K; ++k) {
                        const int32_t a = ora_rhu(X[m * K + k], input_shift);
                        const int32_t b = W[n * K + k];
                        p += (uint32_t)(a * b);
                        exact += (int64_t)a * b;
                    }
                    wraps += !exact_in_i32(exact);
                    const int e = eX[m * nch + c] + input_shift + eW[n * nch + c];
                    part = part + ora_scale_f32((float)u32_to_i32(p), e);
                }
                total = total + part;
            }
            out[m * N + n] = total;
        }
    return wraps;
}

/* The weight update of the DFP pipeline (reading U38): FP32 master weights
 * W32[j] = fl(W32[j] - fl(lr * G32[j])) (two roundings, no fused multiply-
 * add), then the DFP-16 copy the next forward reads. */
int ora_dfp16_sgd(float *W32, const float *G32, int64_t n, float lr, int16_t *W16, int *eW)
{
    for (int64_t j = 0; j < n; ++j) {
        const float t = lr * G32[j];
        W32[j] = W32[j] - t;
    }
    return ora_dfp_from_f32(W32, n, 16, W16, eW);
}

/* One output of ora_dfp_contract_f32 (for sampled checks at full size). */
float ora_dfp_contract_f32_at(const int16_t *A, int64_t sam, int64_t sak, const int16_t *B,
                              int64_t sbk, int64_t sbn, int64_t L, int input_shift, int eA,
                              int eB, int S, int64_t m, int64_t n)
{
    const int64_t nch = (L + 63) / 64;
    float total = 0.0f;
    for (int s = 0; s < S; ++s) {
        float part = 0.0f;
        for (int64_t c = range_start(nch, S, s); c < range_start(nch, S, s + 1); ++c) {
            uint32_t p = 0;
            for (int64_t k = 64 * c; k < 64 * c + 64 && k < L; ++k)
                p += (uint32_t)(ora_rhu(A[m * sam + k * sak], input_shift) * (int32_t)B[k * sbk + n * sbn]);
            part = part + (float)u32_to_i32(p);
        }
        total = total + part;
    }
    return ora_scale_f32(total, eA + input_shift + eB);
}
