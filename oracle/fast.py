"""Full-size oracle contractions with a matrix product as the primitive step.

TEST INFRASTRUCTURE ONLY.  Same definitions as the plain-C loops in
ionn_oracle.c, evaluated with numpy's float64 matrix product so that the
large workloads finish in seconds.  float64 is exact here: each function
asserts that the largest possible |partial sum| (reduction length x max|a| x
max|b|) is below 2^53, so every product and sum is an exact integer.  The
exact sums are then reduced modulo 2^32 to int32, as the C oracle does.
These functions are pinned against the C loops in tests/test_oracle_fast.py.

Sources: Linear and Conv2D layers of "Integer On-Device Training: Overview"
(section 7); FC weight index W[oc*IC + ic] and NHWC layout of the TiGrIS
"Compilation Pipeline"; DFP-16 chunked accumulation of "Mixed Precision
Training of CNNs using Integer Operations" (sections 3.1 and 4).
"""
import numpy as np

from . import dfp_chunk_shift, dfp_downconvert

_EXACT = float(2 ** 53)


def _mm(a, b):
    """Exact integer product of two integer matrices via float64 BLAS."""
    k = a.shape[1]
    bound = float(k) * float(np.abs(a.astype(np.int64)).max(initial=0)) * \
        float(np.abs(b.astype(np.int64)).max(initial=0))
    assert bound < _EXACT, "float64 would not be exact for this product"
    return (a.astype(np.float64) @ b.astype(np.float64)).astype(np.int64)


def wrap32(x):
    """int64 -> int32 modulo 2^32 (two's complement)."""
    return ((x.astype(np.int64) + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int32)


# ---- Linear: Y = X W^T, dX = dY W, G = dY^T X --------------------------------

def linear_fwd(X, W):
    return wrap32(_mm(X, W.T))


def linear_dgrad(dY, W):
    return wrap32(_mm(dY, W))


def linear_wgrad(dY, X):
    return wrap32(_mm(dY.T, X))


# ---- Conv 3x3 / stride 1 / pad P, NHWC / OHWI: one product per tap ------------

def _pad(img, P):
    return np.pad(img, ((0, 0), (P, P), (P, P), (0, 0)))


def conv_fwd(X, W, P=1):
    """Y[n,h,w,co] = sum_{kh,kw} sum_ci X[n,h+kh-P,w+kw-P,ci] W[co,kh,kw,ci]."""
    N, H, Wd, Cin = X.shape
    Cout, KH, KW, _ = W.shape
    Ho, Wo = H + 2 * P - KH + 1, Wd + 2 * P - KW + 1
    Xp = _pad(X, P)
    Y = np.zeros((N * Ho * Wo, Cout), np.int64)
    for kh in range(KH):
        for kw in range(KW):
            win = Xp[:, kh:kh + Ho, kw:kw + Wo, :].reshape(-1, Cin)
            Y += _mm(win, W[:, kh, kw, :].T)
    return wrap32(Y).reshape(N, Ho, Wo, Cout)


def conv_dgrad(dY, W, X_shape, P=1):
    """dX[n,h,w,ci] = sum_{kh,kw} sum_co dY[n,h-kh+P,w-kw+P,co] W[co,kh,kw,ci]."""
    N, H, Wd, Cin = X_shape
    Cout, KH, KW, _ = W.shape
    Ho, Wo = dY.shape[1], dY.shape[2]
    # dY padded by KH-1 / KW-1 so every tap's window is a plain slice
    dYp = np.pad(dY, ((0, 0), (KH - 1, KH - 1), (KW - 1, KW - 1), (0, 0)))
    dX = np.zeros((N * H * Wd, Cin), np.int64)
    for kh in range(KH):
        for kw in range(KW):
            # input h reads dY row y = h - kh + P  ->  padded index h - kh + P + KH - 1
            r0, c0 = P - kh + KH - 1, P - kw + KW - 1
            win = dYp[:, r0:r0 + H, c0:c0 + Wd, :].reshape(-1, Cout)
            dX += _mm(win, W[:, kh, kw, :])
    return wrap32(dX).reshape(N, H, Wd, Cin)


def conv_wgrad(dY, X, KH=3, KW=3, P=1):
    """G[co,kh,kw,ci] = sum_{n,h,w} dY[n,h,w,co] X[n,h+kh-P,w+kw-P,ci]."""
    N, H, Wd, Cin = X.shape
    Cout = dY.shape[3]
    Ho, Wo = dY.shape[1], dY.shape[2]
    Xp = _pad(X, P)
    d2 = dY.reshape(-1, Cout)
    G = np.zeros((Cout, KH, KW, Cin), np.int64)
    for kh in range(KH):
        for kw in range(KW):
            win = Xp[:, kh:kh + Ho, kw:kw + Wo, :].reshape(-1, Cin)
            G[:, kh, kw, :] = _mm(d2.T, win)
    return wrap32(G)


# ---- DFP-16 chunked contraction ----------------------------------------------

def _rhu64(x, s):
    return x if s == 0 else (x + (1 << (s - 1))) >> s


def dfp_contract(A, B, chunk=64):
    """acc[m][n] = sum_c rhu(p_c, r) with p_c = A[m, chunk c] . B[chunk c, n]
    taken modulo 2^32 as int32, r = ceil(log2(#chunks)); the sum modulo 2^32.
    A: [M][L], B: [L][N] (any strides: numpy handles the layout)."""
    L = A.shape[1]
    r = dfp_chunk_shift(L, chunk)
    acc = np.zeros((A.shape[0], B.shape[1]), np.int64)
    for k0 in range(0, L, chunk):
        p = wrap32(_mm(A[:, k0:k0 + chunk], B[k0:k0 + chunk, :])).astype(np.int64)
        acc = (acc + _rhu64(p, r)) % 2 ** 32
    return wrap32(acc)


def _dfp_role(acc, e_in, r):
    out, rs = dfp_downconvert(np.ascontiguousarray(acc))
    return out, e_in + r + rs, acc


def dfp16_fwd(X, eX, W, eW, chunk=64):
    return _dfp_role(dfp_contract(X, W.T, chunk), eX + eW, dfp_chunk_shift(X.shape[1], chunk))


def dfp16_dgrad(dY, edY, W, eW, chunk=64):
    return _dfp_role(dfp_contract(dY, W, chunk), edY + eW, dfp_chunk_shift(dY.shape[1], chunk))


def dfp16_wgrad(dY, edY, X, eX, chunk=64):
    return _dfp_role(dfp_contract(dY.T, X, chunk), edY + eX, dfp_chunk_shift(dY.shape[0], chunk))
