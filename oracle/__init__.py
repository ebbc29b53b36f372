"""CPU oracle for the integer-only training step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps the plain-C oracle in
``ionn_oracle.c`` (built by ``oracle/build.py``) with numpy marshalling; all
arithmetic happens in that C file.  It shares nothing with the GPU library.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_lib = None


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int


def _declare(L):
    sig = {
        "ora_set_threads": (_I, [_I]),
        "ora_get_threads": (_I, []),
        "ora_abs_u32": (ctypes.c_uint32, [ctypes.c_int32]),
        "ora_absmax_i32": (ctypes.c_uint32, [_P, _I64]),
        "ora_bitlen_u32": (_I, [ctypes.c_uint32]),
        "ora_niti_shift": (_I, [ctypes.c_uint32, _I]),
        "ora_floor_shift": (ctypes.c_int32, [ctypes.c_int32, _I]),
        "ora_rhu": (ctypes.c_int32, [ctypes.c_int32, _I]),
        "ora_rhu_array": (None, [_P, _I64, _I, _P]),
        "ora_sat8": (ctypes.c_int32, [_I64]),
        "ora_sat16": (ctypes.c_int32, [_I64]),
        "ora_ceil_log2": (_I, [_I64]),
        "ora_niti_requant": (_I, [_P, _I64, _I, _I, _P]),
        "ora_niti_update": (None, [_P, _P, _I64, _I, _I, _P, _P, _P]),
        "ora_linear_fwd": (_I64, [_P, _P, _P, _I64, _I64, _I64]),
        "ora_linear_dgrad": (_I64, [_P, _P, _P, _I64, _I64, _I64]),
        "ora_linear_wgrad": (_I64, [_P, _P, _P, _I64, _I64, _I64]),
        "ora_linear_fwd_at": (ctypes.c_int32, [_P, _P, _I64, _I64, _I64, _I64, _I64]),
        "ora_linear_dgrad_at": (ctypes.c_int32, [_P, _P, _I64, _I64, _I64, _I64, _I64]),
        "ora_linear_wgrad_at": (ctypes.c_int32, [_P, _P, _I64, _I64, _I64, _I64, _I64]),
        "ora_relu_mask": (None, [_P, _P, _I64]),
        "ora_output_error": (None, [_P, _P, _I64, _I64, _I, _P]),
        "ora_oss_requant": (None, [_P, _P, _P, _P, _I64, _I64, _I, _P]),
        "ora_mse_grad_targets": (None, [_P, _P, _I64, _I64, _P, _P, _P]),
        "ora_bias_grad": (None, [_P, _I64, _I64, _P]),
        "ora_niti_update_i32": (None, [_P, _P, _I64, _I, _I, _P, _P, _P]),
        "ora_conv_fwd": (_I64, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _I]),
        "ora_conv_dgrad": (_I64, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _I]),
        "ora_conv_wgrad": (_I64, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _I]),
        "ora_conv_fwd_at": (ctypes.c_int32, [_P, _P] + [_I64] * 5 + [_I] * 3 + [_I64] * 4),
        "ora_conv_dgrad_at": (ctypes.c_int32, [_P, _P] + [_I64] * 5 + [_I] * 3 + [_I64] * 4),
        "ora_conv_wgrad_at": (ctypes.c_int32, [_P, _P] + [_I64] * 5 + [_I] * 3 + [_I64] * 4),
        "ora_dfp_chunk_shift": (_I, [_I64, _I]),
        "ora_dfp_contract": (_I64, [_P, _I64, _I64, _P, _I64, _I64, _I64, _I64, _I64, _I, _P]),
        "ora_dfp_downconvert": (_I, [_P, _I64, _P]),
        "ora_dfp16_fwd": (_I, [_P, _I, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I]),
        "ora_dfp16_dgrad": (_I, [_P, _I, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I]),
        "ora_dfp16_wgrad": (_I, [_P, _I, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I]),
        "ora_gavg": (ctypes.c_double, [_P, _I64, _I, _I]),
        "ora_sat_bits": (ctypes.c_int32, [_I64, _I]),
        "ora_apt_update": (_I64, [_P, _I64, _I, _I, _P, _I, _I]),
        "ora_apt_decide": (_I, [ctypes.c_double, ctypes.c_int32, _I, ctypes.c_double,
                                ctypes.c_double, _I, _I]),
        "ora_apt_rescale": (None, [_P, _I64, _I, _I]),
        "ora_f32_floor_log2": (_I, [ctypes.c_float]),
        "ora_dfp_from_f32": (_I, [_P, _I64, _I, _P, _P]),
        "ora_dfp_from_f32_blocked": (_I, [_P, _I64, _I64, _I, _I, _P, _P]),
        "ora_dfp_to_f32": (None, [_P, _I64, _I, _P]),
        "ora_scale_f32": (ctypes.c_float, [ctypes.c_float, _I]),
        "ora_dfp_contract_f32": (_I64, [_P, _I64, _I64, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _I, _I, _P]),
        "ora_dfp_fwd_f32_blocked": (_I64, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P]),
        "ora_dfp16_sgd": (_I, [_P, _P, _I64, ctypes.c_float, _P, _P]),
        "ora_dfp_contract_f32_at": (ctypes.c_float, [_P, _I64, _I64, _P, _I64, _I64, _I64, _I, _I, _I, _I,
                                                     _I64, _I64]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _c(a, dtype):
    """Check dtype/contiguity (no silent conversion) and return the pointer."""
    if not isinstance(a, np.ndarray) or a.dtype != np.dtype(dtype):
        raise TypeError(f"expected numpy {np.dtype(dtype)}, got {getattr(a, 'dtype', type(a))}")
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("array must be C-contiguous")
    return a.ctypes.data


def set_threads(n: int) -> int:
    return lib().ora_set_threads(int(n))


def get_threads() -> int:
    return lib().ora_get_threads()


# ---- primitives ---------------------------------------------------------

def abs_u32(x: int) -> int:
    return lib().ora_abs_u32(int(x))


def absmax(x: np.ndarray) -> int:
    return lib().ora_absmax_i32(_c(x, np.int32), x.size)


def bitlen(m: int) -> int:
    return lib().ora_bitlen_u32(int(m))


def niti_shift(max_val: int, target_bits: int) -> int:
    return lib().ora_niti_shift(int(max_val), int(target_bits))


def floor_shift(x: int, s: int) -> int:
    return lib().ora_floor_shift(int(x), int(s))


def rhu(x: int, s: int) -> int:
    return lib().ora_rhu(int(x), int(s))


def rhu_array(x: np.ndarray, s: int) -> np.ndarray:
    out = np.empty(x.shape, np.int32)
    lib().ora_rhu_array(_c(x, np.int32), x.size, int(s), _c(out, np.int32))
    return out


def sat8(v: int) -> int:
    return lib().ora_sat8(int(v))


def sat16(v: int) -> int:
    return lib().ora_sat16(int(v))


def ceil_log2(n: int) -> int:
    return lib().ora_ceil_log2(int(n))


# ---- NITI ---------------------------------------------------------------

def niti_requant(acc: np.ndarray, target_bits: int, relu: bool = False):
    """Return (int8 out, shift)."""
    out = np.empty(acc.shape, np.int8)
    s = lib().ora_niti_requant(_c(acc, np.int32), acc.size, int(target_bits), int(bool(relu)),
                               _c(out, np.int8))
    return out, s


def niti_update(G: np.ndarray, W: np.ndarray, target_bits: int, mu_weight: int):
    """Return (W_new, Gq, shift, weight_shift); W is not modified."""
    if G.shape != W.shape:
        raise ValueError("G and W shapes differ")
    Wn = np.ascontiguousarray(W, dtype=np.int8).copy()
    gq = np.empty(G.shape, np.int32)
    s = ctypes.c_int()
    ws = ctypes.c_int()
    lib().ora_niti_update(_c(G, np.int32), _c(Wn, np.int8), G.size, int(target_bits),
                          int(mu_weight), _c(gq, np.int32), ctypes.byref(s), ctypes.byref(ws))
    return Wn, gq, s.value, ws.value


# ---- offsets (bias) and OSS requantisation -------------------------------

def oss_requant(acc, offset, mult, k, relu=False):
    """int8 [M][C] = clip(floor(((acc + offset) mod 2^32) * mult / 2^k)) per channel."""
    M, C = acc.shape
    assert offset.shape == (C,) and mult.shape == (C,) and k.shape == (C,)
    out = np.empty((M, C), np.int8)
    lib().ora_oss_requant(_c(acc, np.int32), _c(offset, np.int32), _c(mult, np.int32),
                          _c(k, np.int8), M, C, int(bool(relu)), _c(out, np.int8))
    return out


def mse_grad_targets(out, labels, tmc, tmw):
    """int32 [B][C] = out - (c == label ? tmc[c] : tmw[c])."""
    B, C = out.shape
    g = np.empty((B, C), np.int32)
    lib().ora_mse_grad_targets(_c(out, np.int8), _c(labels, np.int32), B, C, _c(tmc, np.int8),
                               _c(tmw, np.int8), _c(g, np.int32))
    return g


def bias_grad(d):
    """int32 [C] column sums of the int8 error rows d [M][C]."""
    M, C = d.shape
    gb = np.empty(C, np.int32)
    lib().ora_bias_grad(_c(d, np.int8), M, C, _c(gb, np.int32))
    return gb


def niti_update_i32(G, P, target_bits, mu):
    """Return (P_new, Gq, shift, weight_shift); P is not modified."""
    if G.shape != P.shape:
        raise ValueError("G and P shapes differ")
    Pn = np.ascontiguousarray(P, dtype=np.int32).copy()
    gq = np.empty(G.shape, np.int32)
    s = ctypes.c_int()
    ws = ctypes.c_int()
    lib().ora_niti_update_i32(_c(G, np.int32), _c(Pn, np.int32), G.size, int(target_bits),
                              int(mu), _c(gq, np.int32), ctypes.byref(s), ctypes.byref(ws))
    return Pn, gq, s.value, ws.value


# ---- linear -------------------------------------------------------------

def linear_fwd(X, W, return_wraps=False):
    B, IN = X.shape
    OUT = W.shape[0]
    assert W.shape == (OUT, IN)
    Y = np.empty((B, OUT), np.int32)
    w = lib().ora_linear_fwd(_c(X, np.int8), _c(W, np.int8), _c(Y, np.int32), B, IN, OUT)
    return (Y, w) if return_wraps else Y


def linear_dgrad(dY, W, return_wraps=False):
    B, OUT = dY.shape
    IN = W.shape[1]
    assert W.shape == (OUT, IN)
    dX = np.empty((B, IN), np.int32)
    w = lib().ora_linear_dgrad(_c(dY, np.int8), _c(W, np.int8), _c(dX, np.int32), B, IN, OUT)
    return (dX, w) if return_wraps else dX


def linear_wgrad(dY, X, return_wraps=False):
    B, OUT = dY.shape
    IN = X.shape[1]
    assert X.shape == (B, IN)
    G = np.empty((OUT, IN), np.int32)
    w = lib().ora_linear_wgrad(_c(dY, np.int8), _c(X, np.int8), _c(G, np.int32), B, IN, OUT)
    return (G, w) if return_wraps else G


def linear_fwd_at(X, W, b, o):
    B, IN = X.shape
    return lib().ora_linear_fwd_at(_c(X, np.int8), _c(W, np.int8), B, IN, W.shape[0], int(b), int(o))


def linear_dgrad_at(dY, W, b, i):
    B, OUT = dY.shape
    return lib().ora_linear_dgrad_at(_c(dY, np.int8), _c(W, np.int8), B, W.shape[1], OUT,
                                     int(b), int(i))


def linear_wgrad_at(dY, X, o, i):
    B, OUT = dY.shape
    return lib().ora_linear_wgrad_at(_c(dY, np.int8), _c(X, np.int8), B, X.shape[1], OUT,
                                     int(o), int(i))


def relu_mask(d: np.ndarray, act: np.ndarray) -> np.ndarray:
    out = np.array(d, dtype=np.int32, copy=True)
    assert out.shape == act.shape
    lib().ora_relu_mask(_c(out, np.int32), _c(act, np.int8), out.size)
    return out


def output_error(out, labels, target_mag=127):
    B, C = out.shape
    e = np.empty((B, C), np.int32)
    lib().ora_output_error(_c(out, np.int8), _c(labels, np.int32), B, C, int(target_mag),
                           _c(e, np.int32))
    return e


# ---- conv (stride 1, zero pad P, NHWC / OHWI) ---------------------------

def _conv_dims(X_shape, W_shape, P):
    N, H, Wd, Cin = X_shape
    Cout, KH, KW, Cin2 = W_shape
    assert Cin == Cin2
    return N, H, Wd, Cin, Cout, KH, KW, H + 2 * P - KH + 1, Wd + 2 * P - KW + 1


def conv_fwd(X, W, P=1, return_wraps=False):
    N, H, Wd, Cin, Cout, KH, KW, Ho, Wo = _conv_dims(X.shape, W.shape, P)
    Y = np.empty((N, Ho, Wo, Cout), np.int32)
    w = lib().ora_conv_fwd(_c(X, np.int8), _c(W, np.int8), _c(Y, np.int32), N, H, Wd, Cin, Cout,
                           KH, KW, P)
    return (Y, w) if return_wraps else Y


def conv_dgrad(dY, W, X_shape, P=1, return_wraps=False):
    N, H, Wd, Cin, Cout, KH, KW, Ho, Wo = _conv_dims(X_shape, W.shape, P)
    assert dY.shape == (N, Ho, Wo, Cout)
    dX = np.empty((N, H, Wd, Cin), np.int32)
    w = lib().ora_conv_dgrad(_c(dY, np.int8), _c(W, np.int8), _c(dX, np.int32), N, H, Wd, Cin,
                             Cout, KH, KW, P)
    return (dX, w) if return_wraps else dX


def conv_wgrad(dY, X, KH=3, KW=3, P=1, return_wraps=False):
    N, H, Wd, Cin = X.shape
    Cout = dY.shape[3]
    G = np.empty((Cout, KH, KW, Cin), np.int32)
    w = lib().ora_conv_wgrad(_c(dY, np.int8), _c(X, np.int8), _c(G, np.int32), N, H, Wd, Cin,
                             Cout, KH, KW, P)
    return (G, w) if return_wraps else G


def conv_fwd_at(X, W, P, n, h, w, co):
    N, H, Wd, Cin, Cout, KH, KW, _, _ = _conv_dims(X.shape, W.shape, P)
    return lib().ora_conv_fwd_at(_c(X, np.int8), _c(W, np.int8), N, H, Wd, Cin, Cout, KH, KW, P,
                                 n, h, w, co)


def conv_dgrad_at(dY, W, X_shape, P, n, h, w, ci):
    N, H, Wd, Cin, Cout, KH, KW, _, _ = _conv_dims(X_shape, W.shape, P)
    return lib().ora_conv_dgrad_at(_c(dY, np.int8), _c(W, np.int8), N, H, Wd, Cin, Cout, KH, KW,
                                   P, n, h, w, ci)


def conv_wgrad_at(dY, X, KH, KW, P, co, kh, kw, ci):
    N, H, Wd, Cin = X.shape
    Cout = dY.shape[3]
    return lib().ora_conv_wgrad_at(_c(dY, np.int8), _c(X, np.int8), N, H, Wd, Cin, Cout, KH, KW,
                                   P, co, kh, kw, ci)


# ---- DFP16 --------------------------------------------------------------

def dfp_chunk_shift(L, chunk=64):
    return lib().ora_dfp_chunk_shift(int(L), int(chunk))


def dfp_contract(A, sam, sak, B, sbk, sbn, M, N, L, chunk=64, return_wraps=False):
    acc = np.empty((M, N), np.int32)
    w = lib().ora_dfp_contract(_c(A, np.int16), sam, sak, _c(B, np.int16), sbk, sbn, M, N, L,
                               int(chunk), _c(acc, np.int32))
    return (acc, w) if return_wraps else acc


def dfp_downconvert(acc):
    out = np.empty(acc.shape, np.int16)
    rs = lib().ora_dfp_downconvert(_c(acc, np.int32), acc.size, _c(out, np.int16))
    return out, rs


def _dfp_role(fn, A, eA, B, eB, out_shape, M, K, N, chunk):
    out = np.empty(out_shape, np.int16)
    acc = np.empty(out_shape, np.int32)
    e = ctypes.c_int()
    rc = fn(_c(A, np.int16), int(eA), _c(B, np.int16), int(eB), _c(out, np.int16),
            ctypes.byref(e), _c(acc, np.int32), M, K, N, int(chunk))
    if rc != 0:
        raise OverflowError(f"DFP output exponent {e.value} outside the signed 8-bit range")
    return out, e.value, acc


def dfp16_fwd(X, eX, W, eW, chunk=64):
    """Return (Y int16 [M][N], eY, acc int32)."""
    M, K = X.shape
    N = W.shape[0]
    return _dfp_role(lib().ora_dfp16_fwd, X, eX, W, eW, (M, N), M, K, N, chunk)


def dfp16_dgrad(dY, edY, W, eW, chunk=64):
    """Return (dX int16 [M][K], edX, acc int32)."""
    M, N = dY.shape
    K = W.shape[1]
    return _dfp_role(lib().ora_dfp16_dgrad, dY, edY, W, eW, (M, K), M, K, N, chunk)


def dfp16_wgrad(dY, edY, X, eX, chunk=64):
    """Return (G int16 [N][K], eG, acc int32)."""
    M, N = dY.shape
    K = X.shape[1]
    return _dfp_role(lib().ora_dfp16_wgrad, dY, edY, X, eX, (N, K), M, K, N, chunk)


def gavg(g, e_g, e_w):
    return lib().ora_gavg(_c(g, np.int16), g.size, int(e_g), int(e_w))


# ---- adaptive precision ([APT]) -------------------------------------------

def sat_bits(v, k):
    return lib().ora_sat_bits(int(v), int(k))


def apt_update(W, k, e_w, G, e_g, lr_shift):
    """k-bit weight update on the grid of eps = 2^e_w; returns (W', underflows)."""
    if W.shape != G.shape:
        raise ValueError("W and G must have the same shape")
    out = np.array(W, dtype=np.int16, order="C", copy=True)
    under = lib().ora_apt_update(_c(out, np.int16), out.size, int(k), int(e_w),
                                 _c(G, np.int16), int(e_g), int(lr_shift))
    return out, int(under)


def apt_decide(gavg_sum, count, k, t_min, t_max, k_min, k_max):
    return lib().ora_apt_decide(float(gavg_sum), int(count), int(k), float(t_min),
                                float(t_max), int(k_min), int(k_max))


def apt_rescale(W, k, dk):
    out = np.array(W, dtype=np.int16, order="C", copy=True)
    lib().ora_apt_rescale(_c(out, np.int16), out.size, int(k), int(dk))
    return out


# ---- DFP as the DFP page runs it (FP32 partials, conversions, Blocked-DFP) ----

def f32_floor_log2(m):
    return lib().ora_f32_floor_log2(float(m))


def dfp_from_f32(x, P=16):
    """float32 array -> (int16 mantissas, exponent, status)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.int16)
    e = ctypes.c_int()
    st = lib().ora_dfp_from_f32(_c(x, np.float32), x.size, int(P), _c(out, np.int16), ctypes.byref(e))
    return out, e.value, st


def dfp_from_f32_blocked(x, B=64, P=16):
    """float32 [rows][K] -> (int16 [rows][K], int32 exponents [rows][ceil(K/B)], status)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    nb = (K + B - 1) // B
    out = np.empty(x.shape, np.int16)
    e = np.empty((rows, nb), np.int32)
    st = lib().ora_dfp_from_f32_blocked(_c(x, np.float32), rows, K, int(B), int(P), _c(out, np.int16),
                                        _c(e, np.int32))
    return out, e, st


def dfp_to_f32(I, e):
    out = np.empty(I.shape, np.float32)
    lib().ora_dfp_to_f32(_c(I, np.int16), I.size, int(e), _c(out, np.float32))
    return out


def scale_f32(v, e):
    return lib().ora_scale_f32(float(v), int(e))


def _f32_role(A, sam, sak, B, sbk, sbn, M, N, L, input_shift, eA, eB, S):
    out = np.empty((M, N), np.float32)
    w = lib().ora_dfp_contract_f32(_c(A, np.int16), sam, sak, _c(B, np.int16), sbk, sbn, M, N, L,
                                   int(input_shift), int(eA), int(eB), int(S), _c(out, np.float32))
    return out, int(w)


def dfp16_fwd_f32(X, eX, W, eW, S=1, input_shift=1):
    """Y [M][N] float32 = X [M][K] . W [N][K]^T with FP32 chunk partials; returns (Y, wraps)."""
    M, K = X.shape
    N = W.shape[0]
    return _f32_role(X, K, 1, W, 1, K, M, N, K, input_shift, eX, eW, S)


def dfp16_dgrad_f32(dY, edY, W, eW, S=1, input_shift=1):
    """dX [M][K] float32 = dY [M][N] . W [N][K]."""
    M, N = dY.shape
    K = W.shape[1]
    return _f32_role(dY, N, 1, W, K, 1, M, K, N, input_shift, edY, eW, S)


def dfp16_wgrad_f32(dY, edY, X, eX, S=1, input_shift=1):
    """G [N][K] float32 = dY [M][N]^T . X [M][K]."""
    M, N = dY.shape
    K = X.shape[1]
    return _f32_role(dY, 1, N, X, K, 1, N, K, M, input_shift, edY, eX, S)


def dfp16_fwd_f32_blocked(X, eX, W, eW, S=1, input_shift=1):
    """Y [M][N] float32 from Blocked-DFP X (exponents [M][K/64]) and W ([N][K/64])."""
    M, K = X.shape
    N = W.shape[0]
    out = np.empty((M, N), np.float32)
    w = lib().ora_dfp_fwd_f32_blocked(_c(X, np.int16), _c(eX, np.int32), _c(W, np.int16), _c(eW, np.int32),
                                      M, K, N, int(input_shift), int(S), _c(out, np.float32))
    return out, int(w)


def dfp16_sgd(W32, G32, lr):
    """FP32 master update and its DFP-16 copy: returns (W32', W16, eW, status)."""
    W = np.array(W32, dtype=np.float32, copy=True)
    G = np.ascontiguousarray(G32, dtype=np.float32)
    W16 = np.empty(W.shape, np.int16)
    e = ctypes.c_int()
    st = lib().ora_dfp16_sgd(_c(W, np.float32), _c(G, np.float32), W.size, float(lr), _c(W16, np.int16),
                             ctypes.byref(e))
    return W, W16, e.value, st


def dfp16_default_splits(M, K, N, role):
    """The default number S of chunk ranges of the FP32 accumulation for a
    shape (reading U35 of the design notes: the order is a function of the
    shape alone).  With R x C outputs of the role in 128 x 128 tiles and n_c
    chunks of 64 along its reduction: S = 1 when there are at least 256 tiles
    or fewer than 8 chunks; otherwise S = min(ceil(256 / tiles),
    floor(n_c / 4)), at least 1."""
    R, C, L = {"fwd": (M, N, K), "dgrad": (M, K, N), "wgrad": (N, K, M)}[role]
    tiles = -(-R // 128) * -(-C // 128)
    nch = -(-L // 64)
    if tiles >= 256 or nch < 8:
        return 1
    return max(1, min(-(-256 // tiles), nch // 4))


def dfp16_f32_at(role, A, eA, B, eB, m, n, S=1, input_shift=1):
    """One output (row m, column n) of dfp16_{fwd,dgrad,wgrad}_f32."""
    if role == "fwd":      # A = X [M][K], B = W [N][K]
        K = A.shape[1]
        args = (A, K, 1, B, 1, K, K)
    elif role == "dgrad":  # A = dY [M][N], B = W [N][K]
        N, K = B.shape
        args = (A, N, 1, B, K, 1, N)
    else:                  # A = dY [M][N], B = X [M][K]; output [N][K]
        M, N = A.shape
        K = B.shape[1]
        args = (A, 1, N, B, K, 1, M)
    a, sam, sak, b, sbk, sbn, L = args
    return lib().ora_dfp_contract_f32_at(_c(a, np.int16), sam, sak, _c(b, np.int16), sbk, sbn, L,
                                         int(input_shift), int(eA), int(eB), int(S), int(m), int(n))
