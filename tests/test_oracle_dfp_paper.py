"""Pins of the oracle's DFP steps as the DFP page runs them ("Mixed Precision
Training of Convolutional Neural Networks using Integer Operations": 3.1,
float -> DFP conversion by the exponent of the absolute maximum and back;
4 "Handling overflows", int32 chunk partials converted to FP32, scaled by
2^(E_inp + E_wt) and summed into an FP32 output, with the input shifted by
one bit; 3, Blocked-DFP), checked against exact rational and big-integer
arithmetic, Python's own frexp and round-half-even, hand-worked rounding-
order cases and the textbook error bound of recursive summation."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rhu1(a):
    return (a + 1) >> 1   # floor((a + 1) / 2): rhu by one bit, Python big ints


def _rne(fr):
    """Round a Fraction to the nearest integer, ties to even (Python's round)."""
    return round(fr)


def _f32(v):
    return float(np.float32(v))


# ---- conversion -------------------------------------------------------------

def test_floor_log2_against_frexp():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                           [1.0, 2.0, 3.0, 0.75, 2 ** -126, 2 ** -149, 3 * 2 ** -149, 3.4e38]])
    for v in np.abs(vals).astype(np.float32):
        if v == 0:
            continue
        m, e = math.frexp(float(v))   # v = m * 2^e, m in [0.5, 1)
        assert oracle.f32_floor_log2(v) == e - 1, v


def test_conversion_hand_worked():
    # max |x| = 1.0 = 1 * 2^0 -> E = 0 - 14; mantissas x * 2^14 rounded to even
    I, e, st = oracle.dfp_from_f32(np.array([1.0, -0.75, 0.3], np.float32))
    assert (I.tolist(), e, st) == ([16384, -12288, 4915], -14, 0)   # 0.3f * 16384 = 4915.2
    # ties go to even: 2.5 and -2.5 grid steps -> 2 and -2; 3.5 -> 4
    x = np.array([1.0, 2.5 * 2 ** -14, -2.5 * 2 ** -14, 3.5 * 2 ** -14], np.float32)
    assert oracle.dfp_from_f32(x)[0].tolist() == [16384, 2, -2, 4]
    # the maximum rounds up to 2^15 and saturates to 32767
    I, e, _ = oracle.dfp_from_f32(np.array([np.float32(2.0) - np.float32(2 ** -23)], np.float32))
    assert I.tolist() == [32767] and e == -14
    # -2^15 fits: the negative maximum of magnitude 2^q maps to -16384 * ... exactly
    I, e, _ = oracle.dfp_from_f32(np.array([-4.0, 1.0], np.float32))
    assert I.tolist() == [-16384, 4096] and e == 2 - 14
    # all zeros: exponent 0, mantissas 0
    assert oracle.dfp_from_f32(np.zeros(5, np.float32))[:2][1] == 0


@pytest.mark.parametrize("P", [2, 4, 8, 12, 15, 16])
def test_conversion_against_exact_rounding(P):
    rng = np.random.default_rng(P)
    for scale in (1e-30, 1e-3, 1.0, 7.0, 1e30, 1e-44):
        x = (rng.standard_normal(300) * scale).astype(np.float32)
        I, e, st = oracle.dfp_from_f32(x, P)
        m = float(np.max(np.abs(x)))
        if m == 0:
            continue
        q = math.frexp(m)[1] - 1
        assert e == q - (P - 2)
        lim = 1 << (P - 1)
        want = [max(-lim, min(lim - 1, _rne(Fraction(float(v)) / Fraction(2) ** e))) for v in x]
        assert I.tolist() == want
        assert st == (0 if -128 <= e <= 127 else 1)
        # back to float: within half a grid step, exact on the grid
        back = oracle.dfp_to_f32(I, e).astype(np.float64)
        err = np.abs(back - x.astype(np.float64))
        sat = np.abs(I.astype(np.int64)) >= lim - 1
        assert (err[~sat] <= 2.0 ** (e - 1) * (1 + 1e-12) + 2.0 ** -149).all()


def test_non_finite_input_is_refused():
    for bad in (np.inf, -np.inf, np.nan):
        assert oracle.dfp_from_f32(np.array([1.0, bad], np.float32))[2] == 2


def test_blocked_conversion_blocks_are_independent():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((5, 150)) * np.array([1e-3, 1.0, 1e3])[rng.integers(0, 3, (5, 1))]).astype(np.float32)
    x[2, 64:128] *= 1e6          # one block far larger than its neighbours
    I, E, st = oracle.dfp_from_f32_blocked(x, B=64)
    assert E.shape == (5, 3) and st == 0
    for r in range(5):
        for b in range(3):
            blk = x[r, 64 * b:64 * b + 64]
            q = math.frexp(float(np.max(np.abs(blk))))[1] - 1
            assert E[r, b] == q - 14
            want = [max(-32768, min(32767, _rne(Fraction(float(v)) / Fraction(2) ** int(E[r, b])))) for v in blk]
            assert I[r, 64 * b:64 * b + 64].tolist() == want
    # a large block does not cost the small blocks their precision
    assert E[2, 1] > E[2, 0] + 15


def test_scale_rounds_once():
    assert oracle.scale_f32(3.0, 4) == 48.0
    # into the subnormal range: 3 * 2^-150 = 1.5 * 2^-149 -> ties to even 2 * 2^-149
    assert oracle.scale_f32(3.0, -150) == _f32(2 * 2.0 ** -149)
    assert oracle.scale_f32(5.0, -151) == _f32(2.0 ** -149)        # 1.25 ulp -> 1
    assert oracle.scale_f32(1.0, 128) == float("inf")


# ---- FP32-partial contraction -------------------------------------------------

def _exact_terms(A, B, input_shift):
    """Exact chunk partials (Python ints, wrapped to int32) per output."""
    M, K = A.shape
    N = B.shape[0]
    nch = (K + 63) // 64
    out = {}
    for m in range(M):
        for n in range(N):
            ps = []
            for c in range(nch):
                p = sum((_rhu1(int(A[m, k])) if input_shift else int(A[m, k])) * int(B[n, k])
                        for k in range(64 * c, min(64 * c + 64, K)))
                p = (p + 2 ** 31) % 2 ** 32 - 2 ** 31
                ps.append(p)
            out[(m, n)] = ps
    return out


def test_f32_contract_exact_when_no_rounding():
    """Small mantissas: every partial and every running sum is an integer
    below 2^24, so the FP32 result is the exact sum times 2^e."""
    rng = np.random.default_rng(1)
    X = rng.integers(-40, 41, (5, 200)).astype(np.int16)
    W = rng.integers(-40, 41, (7, 200)).astype(np.int16)
    for shift in (0, 1):
        for S in (1, 2, 4):
            Y, wr = oracle.dfp16_fwd_f32(X, -9, W, -3, S=S, input_shift=shift)
            assert wr == 0
            terms = _exact_terms(X, W, shift)
            for (m, n), ps in terms.items():
                want = Fraction(sum(ps)) * Fraction(2) ** (-9 + shift - 3)
                assert Fraction(float(Y[m, n])) == want


def _one_term_operands(partials):
    """Operands whose chunk partials (no input shift) are exactly `partials`:
    one nonzero product per chunk, a * b with b = 1."""
    K = 64 * len(partials)
    A = np.zeros((1, K), np.int16)
    B = np.zeros((1, K), np.int16)
    for c, p in enumerate(partials):
        # p = a * b with |a|, |b| < 2^15
        b = 1
        while abs(p) // b >= 2 ** 15:
            b *= 2
        assert p % b == 0
        A[0, 64 * c] = p // b
        B[0, 64 * c] = b
    return A, B


def test_f32_contract_order_hand_worked():
    """The accumulation order decides the rounding: chunk partials
    2^24, 1, 1 sum to 2^24 in order (each +1 is a tie that rounds to even),
    not to the exact 2^24 + 2; and 1, 1, 2^24, 1 give 2^24 + 4 in one range
    (2 + 2^24 = 2^24 + 2, then + 1 ties to even 2^24 + 4) but 2^24 + 2 in two
    ranges (2, then 2^24 + 1 -> 2^24, then 2 + 2^24)."""
    A, B = _one_term_operands([2 ** 24, 1, 1])
    assert oracle.dfp16_fwd_f32(A, 0, B, 0, S=1, input_shift=0)[0][0, 0] == 2.0 ** 24
    assert oracle.dfp16_fwd_f32(A, 0, B, 0, S=3, input_shift=0)[0][0, 0] == 2.0 ** 24
    A, B = _one_term_operands([1, 1, 2 ** 24, 1])
    assert oracle.dfp16_fwd_f32(A, 0, B, 0, S=1, input_shift=0)[0][0, 0] == 2.0 ** 24 + 4
    assert oracle.dfp16_fwd_f32(A, 0, B, 0, S=2, input_shift=0)[0][0, 0] == 2.0 ** 24 + 2
    # the exponents scale the whole sum: eA + shift + eB = -20
    assert oracle.dfp16_fwd_f32(A, -7, B, -13, S=2, input_shift=0)[0][0, 0] == (2.0 ** 24 + 2) * 2.0 ** -20


def test_f32_contract_input_shift_is_rhu():
    # one term: a = 3 -> rhu(3, 1) = 2; a = -3 -> -1; a = 32767 -> 16384
    A = np.array([[3, -3, 32767, -32768] + [0] * 60], np.int16)
    for j, want in enumerate([2, -1, 16384, -16384]):
        B = np.zeros((1, 64), np.int16)
        B[0, j] = 1
        Y, _ = oracle.dfp16_fwd_f32(A, 0, B, 0, S=1, input_shift=1)
        assert Y[0, 0] == want * 2.0   # exponent grows by the shift


@pytest.mark.parametrize("S", [1, 3, 8])
def test_f32_contract_error_bound(S):
    """Recursive FP32 summation of n terms in any bracketing stays within
    (n - 1) u sum|t| of the exact sum (u = 2^-24; the final scaling is exact
    here), with the int32-to-FP32 conversion adding u |p| per term."""
    rng = np.random.default_rng(S)
    X = rng.integers(-32768, 32768, (3, 64 * 40)).astype(np.int16)
    W = rng.integers(-32768, 32768, (4, 64 * 40)).astype(np.int16)
    Y, _ = oracle.dfp16_fwd_f32(X, -20, W, -18, S=S, input_shift=1)
    terms = _exact_terms(X, W, 1)
    u = 2.0 ** -24
    for (m, n), ps in terms.items():
        exact = Fraction(sum(ps)) * Fraction(2) ** (-20 + 1 - 18)
        bound = (len(ps) + 1) * u * sum(abs(p) for p in ps) * 2.0 ** (-37)
        assert abs(Fraction(float(Y[m, n])) - exact) <= Fraction(bound)


def test_f32_roles_are_the_same_contraction():
    """dgrad and wgrad are the forward contraction on rearranged operands:
    dX = dY . W is fwd(dY, W^T), G = dY^T . X is fwd(dY^T, X^T)."""
    rng = np.random.default_rng(5)
    M, K, N = 70, 130, 90
    dY = rng.integers(-3000, 3000, (M, N)).astype(np.int16)
    W = rng.integers(-3000, 3000, (N, K)).astype(np.int16)
    X = rng.integers(-3000, 3000, (M, K)).astype(np.int16)
    for S in (1, 2):
        a, _ = oracle.dfp16_dgrad_f32(dY, -5, W, -6, S=S)
        b, _ = oracle.dfp16_fwd_f32(dY, -5, np.ascontiguousarray(W.T), -6, S=S)
        assert np.array_equal(a, b)
        a, _ = oracle.dfp16_wgrad_f32(dY, -5, X, -7, S=S)
        b, _ = oracle.dfp16_fwd_f32(np.ascontiguousarray(dY.T), -5, np.ascontiguousarray(X.T), -7, S=S)
        assert np.array_equal(a, b)


def test_blocked_fwd_reduces_to_per_tensor_and_is_exact_when_small():
    rng = np.random.default_rng(6)
    X = rng.integers(-30, 31, (4, 256)).astype(np.int16)
    W = rng.integers(-30, 31, (6, 256)).astype(np.int16)
    eX = np.full((4, 4), -8, np.int32)
    eW = np.full((6, 4), -5, np.int32)
    for S in (1, 2):
        a, _ = oracle.dfp16_fwd_f32_blocked(X, eX, W, eW, S=S)
        b, _ = oracle.dfp16_fwd_f32(X, -8, W, -5, S=S)
        assert np.array_equal(a, b)
    # block exponents that differ: each chunk's term carries its own scale,
    # and with small values every sum is exact
    eX = rng.integers(-6, 2, (4, 4)).astype(np.int32)
    eW = rng.integers(-6, 2, (6, 4)).astype(np.int32)
    Y, _ = oracle.dfp16_fwd_f32_blocked(X, eX, W, eW, S=1)
    terms = _exact_terms(X, W, 1)
    for (m, n), ps in terms.items():
        want = sum(Fraction(p) * Fraction(2) ** int(eX[m, c] + 1 + eW[n, c]) for c, p in enumerate(ps))
        assert Fraction(float(Y[m, n])) == want


def test_sgd_update_and_copy():
    W = np.array([1.0, -0.5, 3.0, 0.25], np.float32)
    G = np.array([0.5, 0.25, -1.0, 0.0], np.float32)
    W2, W16, e, st = oracle.dfp16_sgd(W, G, 0.5)
    assert W2.tolist() == [0.75, -0.625, 3.5, 0.25]      # exact in binary
    assert e == 1 - 14 and st == 0                        # max 3.5 = 1.75 * 2^1
    assert W16.tolist() == [6144, -5120, 28672, 2048]     # W2 * 2^13
    # two roundings, not one: lr * g rounds first
    lr = np.float32(0.1)
    g = np.float32(3.0)
    w = np.float32(1.0)
    W2, _, _, _ = oracle.dfp16_sgd(np.array([w]), np.array([g]), float(lr))
    t = Fraction(float(lr)) * Fraction(float(g))
    t32 = Fraction(_f32(float(t)))
    assert Fraction(float(W2[0])) == Fraction(_f32(float(Fraction(float(w)) - t32)))


# ---- the single-output form and the default order ---------------------------

@pytest.mark.parametrize("role", ["fwd", "dgrad", "wgrad"])
def test_f32_single_output_equals_full_contraction(role):
    """dfp16_f32_at (the full-size sampled checker) against the whole-tensor
    contraction, every output of ragged shapes, for several range counts and
    both input shifts: a wrong stride, operand role or range bound in either
    fails here."""
    rng = np.random.default_rng({"fwd": 1, "dgrad": 2, "wgrad": 3}[role])
    full = {"fwd": oracle.dfp16_fwd_f32, "dgrad": oracle.dfp16_dgrad_f32, "wgrad": oracle.dfp16_wgrad_f32}[role]
    for M, K, N in ((37, 200, 29), (5, 64, 3), (70, 131, 66)):
        X = rng.integers(-32768, 32768, (M, K)).astype(np.int16)
        W = rng.integers(-32768, 32768, (N, K)).astype(np.int16)
        dY = rng.integers(-32768, 32768, (M, N)).astype(np.int16)
        A, B = {"fwd": (X, W), "dgrad": (dY, W), "wgrad": (dY, X)}[role]
        L = {"fwd": K, "dgrad": N, "wgrad": M}[role]
        nch = -(-L // 64)
        for S in sorted({1, 2, 3, nch} & set(range(1, nch + 1))):
            for shift in (0, 1):
                want, _ = full(A, -30, B, -21, S=S, input_shift=shift)
                R, C = want.shape
                got = np.array([[oracle.dfp16_f32_at(role, A, -30, B, -21, r, c, S=S, input_shift=shift)
                                 for c in range(C)] for r in range(R)], np.float32)
                np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32),
                                              err_msg=f"{role} {M}x{K}x{N} S={S} shift={shift}")


def test_default_split_rule_hand_worked():
    """The default range count (a function of the shape, reading U35) on
    hand-worked shapes: the DFP-16 layer M 25088, K 256, N 1024 has 1568
    forward tiles and 392 dgrad tiles (S = 1) and 16 wgrad tiles over 392
    chunks (S = min(ceil(256 / 16), 392 // 4) = 16)."""
    rule = oracle.dfp16_default_splits
    assert [rule(25088, 256, 1024, r) for r in ("fwd", "dgrad", "wgrad")] == [1, 1, 16]
    assert rule(128, 64, 128, "wgrad") == 1                 # one chunk: nothing to split
    assert rule(640, 1024, 128, "fwd") == 4                 # 5 tiles, 16 chunks: min(52, 4)
    assert rule(64, 4096, 64, "fwd") == 16                  # 1 tile, 64 chunks: min(256, 16)
    assert rule(256, 512, 384, "fwd") == 2                  # 6 tiles, 8 chunks: min(43, 2)
    assert rule(256, 512, 384, "dgrad") == 1                # 8 tiles, 6 chunks (< 8)
