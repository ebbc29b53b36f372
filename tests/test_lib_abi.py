"""The C-ABI library loads and exports every function include/ionn.h
declares, and its host-side argument checks reject bad calls before touching
the GPU (these calls return without any HIP call, so they run without one)."""
import ctypes

import pytest

from integer_only_nn_amd import _lib

lib = _lib.lib()
OK, ARG, SHAPE, RANGE, ALIGN, UNSUP, HIP, WS = range(8)


def test_exports_every_header_function():
    names = _lib.header_functions()
    assert len(names) >= 19
    for n in names:
        assert hasattr(lib, n), f"libionn.so does not export {n}"
        assert n in _lib.SIGNATURES, f"no ctypes signature for {n}"
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings_and_version():
    assert lib.ionn_status_str(0) == b"ok"
    assert b"workspace" in lib.ionn_status_str(WS)
    assert lib.ionn_version().startswith(b"ionn")


P = ctypes.c_void_p
FAKE = P(0x1000)        # never dereferenced: every call below fails validation first
FAKE_ODD = P(0x1001)


def _err():
    return lib.ionn_last_error().decode()


def test_linear_validation():
    assert lib.int_linear_fwd(FAKE, FAKE, FAKE, -1, 4, 4, None, None) == SHAPE
    assert lib.int_linear_fwd(FAKE, FAKE, FAKE, 1 << 31, 4, 4, None, None) == SHAPE
    assert lib.int_linear_fwd(None, FAKE, FAKE, 2, 4, 4, None, None) == ARG
    assert "NULL" in _err()
    assert lib.int_linear_fwd(FAKE, FAKE, FAKE_ODD, 2, 4, 4, None, None) == ALIGN
    assert lib.int_linear_dgrad(FAKE, None, None, FAKE, 2, 4, 4, None, None) == ARG
    assert lib.int_linear_wgrad(FAKE, FAKE, None, 2, 4, 4, None, None) == ARG
    # empty outputs are a no-op, even with NULL tensors
    assert lib.int_linear_fwd(None, None, None, 0, 4, 4, None, None) == OK
    assert lib.int_linear_wgrad(None, None, None, 4, 0, 4, None, None) == OK


def test_linear_wgrad_workspace_query_and_checks():
    # a small G over a long batch takes the partial-sums path: groups of at
    # least 256 rows, at most 256, times the G size, or times its 32 x 32
    # blocks (1024 values each) when they pad G by at most a quarter
    need = lib.int_linear_wgrad_workspace_bytes(65536, 147, 160)
    assert need == 256 * 25 * 1024 * 4
    assert lib.int_linear_wgrad_workspace_bytes(65536, 160, 2) == 256 * 160 * 2 * 4
    assert lib.int_linear_wgrad_workspace_bytes(5000, 33, 7) == 20 * 33 * 7 * 4
    assert lib.int_linear_wgrad_workspace_bytes(200000, 33, 7) == 256 * 33 * 7 * 4
    # short batches, large G, bad sizes: no workspace (the call is int_linear_wgrad)
    assert lib.int_linear_wgrad_workspace_bytes(100, 64, 32) == 0
    assert lib.int_linear_wgrad_workspace_bytes(65536, 512, 512) == 0
    assert lib.int_linear_wgrad_workspace_bytes(-1, 4, 4) == 0
    f = lib.int_linear_wgrad_ws
    assert f(FAKE, FAKE, FAKE, 65536, 147, 160, None, None, need - 4, None) == WS
    assert "workspace" in _err()
    assert f(FAKE, FAKE, FAKE, 65536, 147, 160, None, FAKE_ODD, need, None) == WS
    assert f(FAKE, FAKE, None, 65536, 147, 160, None, FAKE, need, None) == ARG
    assert f(FAKE, FAKE, FAKE_ODD, 65536, 147, 160, None, FAKE, need, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, -1, 147, 160, None, FAKE, need, None) == SHAPE


def test_niti_validation():
    assert lib.niti_quantize(FAKE, 8, None, 7, 0, FAKE, None, None) == ARG
    assert lib.niti_quantize(FAKE, 8, FAKE, 0, 0, FAKE, None, None) == RANGE
    assert lib.niti_quantize(FAKE, 8, FAKE, 32, 0, FAKE, None, None) == RANGE
    assert lib.niti_quantize(FAKE, 8, FAKE, 7, 2, FAKE, None, None) == ARG
    assert lib.niti_quantize(FAKE, -1, FAKE, 7, 0, FAKE, None, None) == SHAPE
    assert lib.niti_quantize_update(FAKE, 8, FAKE, 8, -1, FAKE, None, None, None) == RANGE
    assert lib.niti_quantize_update(FAKE, 8, FAKE, 8, 32, FAKE, None, None, None) == RANGE
    assert lib.niti_quantize_update(FAKE_ODD, 8, FAKE, 8, 2, FAKE, None, None, None) == ALIGN
    assert lib.int_output_error(FAKE, FAKE, 4, 10, 200, FAKE, None, None) == RANGE
    assert lib.ionn_fill_u32(None, 4, 0, None) == ARG
    assert lib.ionn_absmax_i32(FAKE, 4, None, None) == ARG


def _desc(**kw):
    d = dict(N=1, H=8, W=8, Cin=16, Cout=16, KH=3, KW=3, stride=1, pad=1, dilation=1, groups=1)
    d.update(kw)
    return _lib.ConvDesc(**d)


@pytest.mark.parametrize("kw", [dict(stride=2), dict(dilation=2), dict(groups=2)])
def test_conv_refuses_unsupported_geometry(kw):
    d = _desc(**kw)
    for f in (lib.int_conv_fwd, lib.int_conv_dgrad):
        assert f(FAKE, FAKE, FAKE, ctypes.byref(d), None, None) == UNSUP
    assert lib.int_conv_wgrad(FAKE, FAKE, FAKE, ctypes.byref(d), None, None, 0, None) == UNSUP
    assert "stride 1" in _err()


@pytest.mark.parametrize("kw", [dict(KH=0), dict(KW=0), dict(pad=2000), dict(pad=-1), dict(KH=2000)])
def test_conv_refuses_bad_kernel_or_pad(kw):
    d = _desc(**kw)
    for f in (lib.int_conv_fwd, lib.int_conv_dgrad):
        assert f(FAKE, FAKE, FAKE, ctypes.byref(d), None, None) == RANGE
    assert lib.int_conv_wgrad(FAKE, FAKE, FAKE, ctypes.byref(d), None, None, 0, None) == RANGE


def test_conv_wgrad_workspace_query():
    """Workspace for the 64-channel fast path (one partial G per compute
    unit, 64*576 int32 each) and for full-row-window
    filters; 0 otherwise."""
    big = lib.int_conv_wgrad_workspace_bytes(ctypes.byref(_desc(Cin=64, Cout=64, W=56, H=56, N=128)))
    assert big > 0 and big % (64 * 576 * 4) == 0
    assert lib.int_conv_wgrad_workspace_bytes(ctypes.byref(_desc(Cin=64, Cout=32))) == 0
    assert lib.int_conv_wgrad_workspace_bytes(ctypes.byref(_desc(Cin=64, Cout=64, W=4000))) == 0
    assert lib.int_conv_wgrad_workspace_bytes(ctypes.byref(_desc(Cin=64, Cout=64, KH=5, KW=5, pad=2))) == 0
    assert lib.int_conv_wgrad_workspace_bytes(None) == 0
    # full-row-window filters (no padding, KW = W): one partial G per
    # workgroup of up to 64 staged samples, at most 1024 workgroups
    ex = _desc(N=65536, H=64, W=2, Cin=1, Cout=3, KH=16, KW=2, pad=0)
    assert lib.int_conv_wgrad_workspace_bytes(ctypes.byref(ex)) == 1024 * 3 * 32 * 4
    few = _desc(N=100, H=64, W=2, Cin=1, Cout=3, KH=16, KW=2, pad=0)
    assert lib.int_conv_wgrad_workspace_bytes(ctypes.byref(few)) == 2 * 3 * 32 * 4
    assert lib.int_conv_wgrad_workspace_bytes(ctypes.byref(_desc(N=100, H=64, W=2, Cin=1, Cout=9, KH=16, KW=2,
                                                                 pad=0))) == 0


def test_conv_validation():
    assert lib.int_conv_fwd(FAKE, FAKE, FAKE, None, None, None) == ARG
    d = _desc(N=-1)
    assert lib.int_conv_fwd(FAKE, FAKE, FAKE, ctypes.byref(d), None, None) == SHAPE
    d = _desc()
    assert lib.int_conv_fwd(FAKE_ODD, FAKE, FAKE, ctypes.byref(d), None, None) == ALIGN
    # descriptors whose element counts overflow 64 bits when multiplied out
    # (2^20 x 2^20 x 2^20 x 2^20) or wrap to a small value are refused, not
    # accepted as empty
    for kw in (dict(N=1 << 20, H=1 << 20, W=1 << 20, Cin=1 << 20, Cout=16),
               dict(N=1 << 40, H=1 << 24, W=1 << 24, Cin=16, Cout=16),
               dict(N=1 << 31, H=1, W=1, Cin=1, Cout=1),
               dict(N=1 << 16, H=1 << 16, W=1, Cin=16, Cout=16)):
        d = _desc(**kw)
        for f in (lib.int_conv_fwd, lib.int_conv_dgrad):
            assert f(FAKE, FAKE, FAKE, ctypes.byref(d), None, None) == SHAPE, kw


def test_dfp16_validation():
    need = lib.dfp16_workspace_bytes(100, 64, 32, 0)
    assert need >= 100 * 32 * 4
    assert lib.dfp16_workspace_bytes(0, 64, 32, 0) == 0
    assert lib.dfp16_workspace_bytes(4, 4, 4, 3) == 0
    assert lib.dfp16_workspace_bytes(100, 64, 32, 2) > lib.dfp16_workspace_bytes(100, 64, 32, 0)
    f = lib.dfp16_gemm_fwd
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 64, 32, 32, FAKE, need, None, None) == RANGE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 32, 64, FAKE, need, None, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 64, 32, 64, FAKE, need - 1, None, None) == WS
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 64, 32, 64, P(0x1010), need, None, None) == WS
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 64, 32, 64, FAKE, need, None, None) == ARG
    assert lib.dfp16_gavg(FAKE, FAKE, FAKE, 0, FAKE, None) == SHAPE


def test_apt_validation():
    arrP = lambda *ps: (ctypes.c_void_p * len(ps))(*ps)
    arrN = lambda *ns: (ctypes.c_int64 * len(ns))(*ns)
    W, G, N = arrP(0x1000, 0x2000), arrP(0x3000, 0x4000), arrN(100, 9000)
    # apt_update(L, W, G, n, k, e_w, e_g, lr_shift, gsum, gcnt, ws, ws_bytes, stream)
    assert lib.apt_update(0, W, G, N, FAKE, FAKE, FAKE, 3, None, None, None, 0, None) == SHAPE
    assert lib.apt_update(65, W, G, N, FAKE, FAKE, FAKE, 3, None, None, None, 0, None) == SHAPE
    assert lib.apt_update(2, W, None, N, FAKE, FAKE, FAKE, 3, None, None, None, 0, None) == ARG
    assert lib.apt_update(2, W, G, arrN(100, 0), FAKE, FAKE, FAKE, 3, None, None, None, 0, None) == SHAPE
    assert lib.apt_update(2, W, G, arrN(100, 1 << 37), FAKE, FAKE, FAKE, 3, None, None, None, 0, None) == SHAPE
    assert lib.apt_update(2, arrP(0x1000, None), G, N, FAKE, FAKE, FAKE, 3, None, None, None, 0, None) == ARG
    assert lib.apt_update(2, arrP(0x1000, 0x2001), G, N, FAKE, FAKE, FAKE, 3, None, None, None, 0, None) == ALIGN
    assert lib.apt_update(2, W, G, N, None, FAKE, FAKE, 3, None, None, None, 0, None) == ARG
    assert lib.apt_update(2, W, G, N, FAKE_ODD, FAKE, FAKE, 3, None, None, None, 0, None) == ALIGN
    assert lib.apt_update(2, W, G, N, FAKE, FAKE, FAKE, -1, None, None, None, 0, None) == RANGE
    assert lib.apt_update(2, W, G, N, FAKE, FAKE, FAKE, 63, None, None, None, 0, None) == RANGE
    assert lib.apt_update(2, W, G, N, FAKE, FAKE, FAKE, 3, FAKE, None, None, 0, None) == ARG
    need = lib.apt_workspace_bytes(2, N)
    assert need == 8 * (1 + 5)   # 2048 weights per workgroup: one for 100, five for 9000
    assert lib.apt_update(2, W, G, N, FAKE, FAKE, FAKE, 3, FAKE, FAKE, None, 0, None) == WS
    assert lib.apt_update(2, W, G, N, FAKE, FAKE, FAKE, 3, FAKE, FAKE, FAKE, need - 8, None) == WS
    assert "workspace" in _err()
    assert lib.apt_workspace_bytes(0, N) == 0 and lib.apt_workspace_bytes(2, arrN(1, -1)) == 0
    # apt_adjust(L, W, n, k, e_w, gsum, gcnt, t_min, t_max, k_min, k_max, dk_out, stream)
    adj = lambda L=2, w=W, n=N, k=FAKE, tmin=1.0, tmax=2.0, kmin=2, kmax=16, dk=None: lib.apt_adjust(
        L, w, n, k, FAKE, FAKE, FAKE, tmin, tmax, kmin, kmax, dk, None)
    assert adj(L=0) == SHAPE
    assert adj(k=None) == ARG
    assert adj(k=FAKE_ODD) == ALIGN
    assert adj(dk=FAKE_ODD) == ALIGN
    assert adj(kmin=1) == RANGE and adj(kmax=17) == RANGE and adj(kmin=9, kmax=8) == RANGE
    assert adj(tmin=3.0, tmax=2.0) == RANGE
    assert adj(tmin=float("nan")) == RANGE
    assert adj(n=arrN(5, 0)) == SHAPE


def test_apt_mixed_width_validation():
    arrP = lambda *ps: (ctypes.c_void_p * len(ps))(*ps)
    arrN = lambda *ns: (ctypes.c_int64 * len(ns))(*ns)
    arrB = lambda *bs: (ctypes.c_int32 * len(bs))(*bs)
    W, G, N = arrP(0x1000, 0x2001), arrP(0x3000, 0x4000), arrN(100, 9000)
    upd = lambda W_, wb: lib.apt_update_mixed(2, W_, wb, G, N, FAKE, FAKE, FAKE, 3, None, None, None, 0, None)
    # bytes per weight must be 1 or 2
    assert upd(W, arrB(2, 3)) == ARG and "bytes per weight" in _err()
    assert upd(W, arrB(0, 1)) == ARG
    # an int8 layer may sit at any byte; an int16 one needs 2-byte alignment
    assert upd(arrP(0x1000, 0x2001), arrB(2, 2)) == ALIGN
    assert upd(arrP(0x1001, 0x2001), arrB(1, 2)) == ALIGN
    adj = lambda W_, wb: lib.apt_adjust_mixed(2, W_, wb, N, FAKE, FAKE, FAKE, FAKE, 1.0, 2.0, 2, 16, None, None)
    assert adj(W, arrB(1, 4)) == ARG
    assert adj(W, arrB(2, 2)) == ALIGN


def test_dfp_paper_form_validation():
    ws = lib.dfp16_f32_workspace_bytes(256, 256, 256, 0, 0)
    assert ws >= 256 and lib.dfp16_f32_workspace_bytes(0, 1, 1, 0, 0) == 0
    # the default range count depends on the shape only
    assert lib.dfp16_f32_splits(25088, 256, 1024, 0) == 1
    assert lib.dfp16_f32_splits(25088, 256, 1024, 2) > 1        # wgrad: 8 tiles over 392 chunks
    assert lib.dfp16_f32_splits(0, 256, 1024, 2) == 0
    call = lambda M=256, K=256, N=256, shift=1, ns=0, w=ws, out=FAKE: lib.dfp16_gemm_fwd_f32(
        FAKE, FAKE, FAKE, FAKE, out, M, K, N, shift, ns, FAKE, w, None)
    assert call(M=0) == SHAPE
    assert call(shift=2) == RANGE
    assert call(ns=-1) == RANGE and call(ns=5) == RANGE          # 4 chunks
    assert call(ns=4, w=0) == WS
    assert call(out=P(0x1008)) == ALIGN
    assert lib.dfp16_gemm_dgrad_f32(None, FAKE, FAKE, FAKE, FAKE, 8, 8, 8, 1, 0, FAKE, 1 << 20, None) == ARG
    assert lib.dfp16_gemm_wgrad_f32(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 8, 1, 0, FAKE, 10, None) == WS
    cw = lib.dfp_convert_workspace_bytes()
    assert lib.dfp_from_f32(FAKE, 0, 16, FAKE, FAKE, None, FAKE, cw, None) == SHAPE
    assert lib.dfp_from_f32(FAKE, 8, 1, FAKE, FAKE, None, FAKE, cw, None) == RANGE
    assert lib.dfp_from_f32(FAKE, 8, 17, FAKE, FAKE, None, FAKE, cw, None) == RANGE
    assert lib.dfp_from_f32(P(0x1004), 8, 16, FAKE, FAKE, None, FAKE, cw, None) == ALIGN
    assert lib.dfp_from_f32(FAKE, 8, 16, FAKE, FAKE, None, None, cw, None) == WS
    assert lib.dfp_to_f32(FAKE, 8, None, FAKE, None) == ARG
    assert lib.dfp_from_f32_blocked(FAKE, 4, 100, 0, 16, FAKE, FAKE, None, None) == RANGE
    assert lib.dfp_from_f32_blocked(FAKE, 0, 100, 64, 16, FAKE, FAKE, None, None) == SHAPE
    assert lib.dfp16_sgd_update(FAKE, P(0x1004), 8, ctypes.c_float(0.1), FAKE, FAKE, None, FAKE, cw, None) == ALIGN
    assert lib.dfp16_sgd_update(FAKE, FAKE, 8, ctypes.c_float(0.1), FAKE, FAKE, None, FAKE, 0, None) == WS


def test_bias_grad_noalloc_refuses_sizes_beyond_its_scratch():
    # 64 rows x 2^20 columns need 4 MiB of row-range sums, over the 2 MiB
    # device scratch: refused before any HIP call
    assert lib.ionn_bias_grad_workspace_bytes(64, 1 << 20) > 2 << 20
    assert lib.ionn_bias_grad_noalloc(FAKE, 64, 1 << 20, FAKE, None) == SHAPE
    assert "scratch" in _err()
    assert lib.ionn_bias_grad_noalloc(FAKE, -1, 16, FAKE, None) == SHAPE
    assert lib.ionn_bias_grad_noalloc(None, 4, 16, FAKE, None) == ARG
    assert lib.ionn_bias_grad_noalloc(FAKE, 4, 16, FAKE_ODD, None) == ALIGN
    assert lib.ionn_bias_grad_noalloc(None, 4, 0, None, None) == OK


def test_update_clear_validation():
    f = lib.niti_quantize_update_clear
    # clear overlapping absmax, n_clear out of range, NULL clear with a count
    assert f(FAKE, 8, P(0x2000), 8, 2, FAKE, None, None, P(0x2000), 3, None) == ARG
    assert f(FAKE, 8, P(0x2004), 8, 2, FAKE, None, None, P(0x2000), 3, None) == ARG
    assert f(FAKE, 8, P(0x2000), 8, 2, FAKE, None, None, P(0x3000), 257, None) == ARG
    assert f(FAKE, 8, P(0x2000), 8, 2, FAKE, None, None, None, 2, None) == ARG
    assert f(FAKE, 8, P(0x2000), 8, 2, FAKE, None, None, P(0x3002), 2, None) == ALIGN
    assert f(FAKE, 8, P(0x2000), 0, 2, FAKE, None, None, P(0x3000), 2, None) == RANGE


def test_linear_step_small_validation():
    fits = lib.int_linear_step_small_fits
    assert fits(16, 64, 32) == 1 and fits(128, 128, 64) == 1
    assert fits(128, 128, 65) == 0 and fits(0, 4, 4) == 0 and fits(4, -1, 4) == 0
    step = lib.int_linear_step_small
    args = lambda B, IN, OUT, tbw=8, mu=2, tbd=7, Y=FAKE: (FAKE, FAKE, FAKE, B, IN, OUT, tbw, mu, tbd, Y, FAKE,
                                                          FAKE, FAKE, None, FAKE, FAKE, None)
    assert step(*args(256, 784, 256)) == SHAPE
    assert "32768" in _err()
    assert step(*args(16, 64, 32, Y=None)) == ARG
    assert step(*args(16, 64, 32, tbw=0)) == RANGE
    assert step(*args(16, 64, 32, mu=32)) == RANGE
    assert step(*args(16, 64, 32, Y=FAKE_ODD)) == ALIGN
