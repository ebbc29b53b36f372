"""Thin Python binding of libionn.so: one function per C entry point, same
names, same argument order.  Arguments are torch tensors on a ROCm device
(PyTorch is used only for device memory and streams); this module only
checks dtypes/shapes and passes raw pointers.  Every computation runs in the
library's HIP kernels.  Outputs are caller-provided, as in the C ABI.
"""
import ctypes

import torch

from ._lib import ConvDesc, check, lib


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _p(t, dtype=None, numel=None, name="tensor"):
    """Device pointer of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor (no CPU path exists)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


i8, i16, i32, u32 = torch.int8, torch.int16, torch.int32, torch.int32  # uint32 scalars held as int32


def ionn_fill_u32(dst, value=0, stream=None):
    check(lib().ionn_fill_u32(_p(dst, torch.int32, name="dst"), dst.numel(), value & 0xFFFFFFFF,
                              _stream(stream)), "ionn_fill_u32")


def ionn_absmax_i32(x, absmax, stream=None):
    check(lib().ionn_absmax_i32(_p(x, i32, name="x"), x.numel(), _p(absmax, u32, 1, "absmax"),
                                _stream(stream)), "ionn_absmax_i32")


def int_linear_fwd(X, W, Y, absmax_Y=None, stream=None):
    B, IN = X.shape
    OUT = W.shape[0]
    assert tuple(W.shape) == (OUT, IN) and tuple(Y.shape) == (B, OUT), "shape mismatch"
    check(lib().int_linear_fwd(_p(X, i8, name="X"), _p(W, i8, name="W"), _p(Y, i32, name="Y"),
                               B, IN, OUT, _p(absmax_Y, u32, 1, "absmax_Y"), _stream(stream)),
          "int_linear_fwd")


def int_linear_dgrad(dY, W, dX, relu_act=None, absmax_dX=None, stream=None):
    B, OUT = dY.shape
    IN = W.shape[1]
    assert tuple(W.shape) == (OUT, IN) and tuple(dX.shape) == (B, IN), "shape mismatch"
    if relu_act is not None:
        assert tuple(relu_act.shape) == (B, IN), "relu_act shape mismatch"
    check(lib().int_linear_dgrad(_p(dY, i8, name="dY"), _p(W, i8, name="W"),
                                 _p(relu_act, i8, name="relu_act"), _p(dX, i32, name="dX"), B, IN,
                                 OUT, _p(absmax_dX, u32, 1, "absmax_dX"), _stream(stream)),
          "int_linear_dgrad")


def int_linear_wgrad(dY, X, G, absmax_G=None, stream=None):
    B, OUT = dY.shape
    IN = X.shape[1]
    assert tuple(X.shape) == (B, IN) and tuple(G.shape) == (OUT, IN), "shape mismatch"
    check(lib().int_linear_wgrad(_p(dY, i8, name="dY"), _p(X, i8, name="X"), _p(G, i32, name="G"),
                                 B, IN, OUT, _p(absmax_G, u32, 1, "absmax_G"), _stream(stream)),
          "int_linear_wgrad")


def int_linear_wgrad_workspace_bytes(B, IN, OUT):
    return int(lib().int_linear_wgrad_workspace_bytes(int(B), int(IN), int(OUT)))


def int_linear_wgrad_ws(dY, X, G, workspace, absmax_G=None, stream=None):
    B, OUT = dY.shape
    IN = X.shape[1]
    assert tuple(X.shape) == (B, IN) and tuple(G.shape) == (OUT, IN), "shape mismatch"
    check(lib().int_linear_wgrad_ws(_p(dY, i8, name="dY"), _p(X, i8, name="X"), _p(G, i32, name="G"),
                                    B, IN, OUT, _p(absmax_G, u32, 1, "absmax_G"),
                                    _p(workspace, None, name="workspace"),
                                    workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                    _stream(stream)), "int_linear_wgrad_ws")


def niti_quantize(acc, absmax, target_bits, relu, out, shift_out=None, stream=None):
    assert acc.numel() == out.numel()
    check(lib().niti_quantize(_p(acc, i32, name="acc"), acc.numel(), _p(absmax, u32, 1, "absmax"),
                              int(target_bits), int(bool(relu)), _p(out, i8, name="out"),
                              _p(shift_out, i32, 1, "shift_out"), _stream(stream)),
          "niti_quantize")


def niti_quantize_update(G, absmax, target_bits, mu_weight, W, shifts_out=None, gq_out=None,
                         stream=None):
    assert G.numel() == W.numel()
    check(lib().niti_quantize_update(_p(G, i32, name="G"), G.numel(), _p(absmax, u32, 1, "absmax"),
                                     int(target_bits), int(mu_weight), _p(W, i8, name="W"),
                                     _p(shifts_out, i32, 2, "shifts_out"),
                                     _p(gq_out, i32, G.numel(), "gq_out"), _stream(stream)),
          "niti_quantize_update")


def int_linear_step_small_fits(B, IN, OUT):
    return bool(lib().int_linear_step_small_fits(int(B), int(IN), int(OUT)))


def int_linear_step_small(X, W, dY, tb_w, mu_weight, tb_d, Y, dX, delta, G, maxima, shifts, gq=None,
                          stream=None):
    B, IN = X.shape
    OUT = W.shape[0]
    assert tuple(W.shape) == (OUT, IN) and tuple(dY.shape) == (B, OUT), "shape mismatch"
    assert tuple(Y.shape) == (B, OUT) and tuple(dX.shape) == (B, IN) and tuple(delta.shape) == (B, IN)
    assert tuple(G.shape) == (OUT, IN) and (gq is None or tuple(gq.shape) == (OUT, IN))
    check(lib().int_linear_step_small(_p(X, i8, name="X"), _p(W, i8, name="W"), _p(dY, i8, name="dY"), B, IN,
                                      OUT, int(tb_w), int(mu_weight), int(tb_d), _p(Y, i32, name="Y"),
                                      _p(dX, i32, name="dX"), _p(delta, i8, name="delta"), _p(G, i32, name="G"),
                                      _p(gq, i32, OUT * IN, "gq"), _p(maxima, u32, 3, "maxima"),
                                      _p(shifts, i32, 3, "shifts"), _stream(stream)),
          "int_linear_step_small")


def niti_quantize_update_clear(G, absmax, target_bits, mu_weight, W, clear, shifts_out=None, gq_out=None,
                               stream=None):
    assert G.numel() == W.numel()
    check(lib().niti_quantize_update_clear(_p(G, i32, name="G"), G.numel(), _p(absmax, u32, 1, "absmax"),
                                           int(target_bits), int(mu_weight), _p(W, i8, name="W"),
                                           _p(shifts_out, i32, 2, "shifts_out"),
                                           _p(gq_out, i32, G.numel(), "gq_out"),
                                           _p(clear, u32, None, "clear"), clear.numel() if clear is not None else 0,
                                           _stream(stream)),
          "niti_quantize_update_clear")


def ionn_oss_requant(acc, offset, mult, k, out, relu=False, stream=None):
    M, C = acc.shape
    assert tuple(out.shape) == (M, C) and offset.numel() == C and mult.numel() == C and k.numel() == C
    check(lib().ionn_oss_requant(_p(acc, i32, name="acc"), _p(offset, i32, name="offset"),
                                 _p(mult, i32, name="mult"), _p(k, i8, name="k"), M, C, int(bool(relu)),
                                 _p(out, i8, name="out"), _stream(stream)), "ionn_oss_requant")


def int_linear_fwd_oss_workspace_bytes(B, IN, OUT):
    return int(lib().int_linear_fwd_oss_workspace_bytes(int(B), int(IN), int(OUT)))


def int_linear_fwd_oss(X, W, offset, mult, k, Y, relu=False, workspace=None, stream=None):
    B, IN = X.shape
    OUT = W.shape[0]
    assert tuple(W.shape) == (OUT, IN) and tuple(Y.shape) == (B, OUT), "shape mismatch"
    assert offset.numel() == OUT and mult.numel() == OUT and k.numel() == OUT
    check(lib().int_linear_fwd_oss(_p(X, i8, name="X"), _p(W, i8, name="W"), _p(offset, i32, name="offset"),
                                   _p(mult, i32, name="mult"), _p(k, i8, name="k"), int(bool(relu)),
                                   _p(Y, i8, name="Y"), B, IN, OUT, _p(workspace, None, name="workspace"),
                                   workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                   _stream(stream)), "int_linear_fwd_oss")


def ionn_bias_grad_workspace_bytes(M, C):
    return int(lib().ionn_bias_grad_workspace_bytes(int(M), int(C)))


def ionn_bias_grad_noalloc(d, gb, stream=None):
    M, C = d.shape
    assert gb.numel() == C
    check(lib().ionn_bias_grad_noalloc(_p(d, i8, name="d"), M, C, _p(gb, i32, name="gb"), _stream(stream)),
          "ionn_bias_grad_noalloc")


def ionn_bias_grad(d, gb, workspace, stream=None):
    M, C = d.shape
    assert gb.numel() == C
    check(lib().ionn_bias_grad(_p(d, i8, name="d"), M, C, _p(gb, i32, name="gb"),
                               _p(workspace, None, name="workspace"),
                               workspace.numel() * workspace.element_size() if workspace is not None else 0,
                               _stream(stream)), "ionn_bias_grad")


def niti_quantize_update_i32(G, absmax, target_bits, mu, P, shifts_out=None, gq_out=None, stream=None):
    assert G.numel() == P.numel()
    check(lib().niti_quantize_update_i32(_p(G, i32, name="G"), G.numel(), _p(absmax, u32, 1, "absmax"),
                                         int(target_bits), int(mu), _p(P, i32, name="P"),
                                         _p(shifts_out, i32, 2, "shifts_out"),
                                         _p(gq_out, i32, G.numel(), "gq_out"), _stream(stream)),
          "niti_quantize_update_i32")


def ionn_mse_grad_targets(out, labels, tmc, tmw, g, absmax_g=None, stream=None):
    B, C = out.shape
    assert tuple(g.shape) == (B, C) and labels.numel() == B and tmc.numel() == C and tmw.numel() == C
    check(lib().ionn_mse_grad_targets(_p(out, i8, name="out"), _p(labels, i32, name="labels"), B, C,
                                      _p(tmc, i8, name="tmc"), _p(tmw, i8, name="tmw"), _p(g, i32, name="g"),
                                      _p(absmax_g, u32, 1, "absmax_g"), _stream(stream)), "ionn_mse_grad_targets")


def ionn_relu_mask_i32(d, act, absmax_d=None, stream=None):
    assert d.numel() == act.numel()
    check(lib().ionn_relu_mask_i32(_p(d, i32, name="d"), _p(act, i8, name="act"), d.numel(),
                                   _p(absmax_d, u32, 1, "absmax_d"), _stream(stream)), "ionn_relu_mask_i32")


def layer_array(layers):
    """ctypes array of ionn_layer from dicts with type, KH, KW, pad, H, W, Cin,
    Cout and device tensors weight (int8), offset (int32), mult (int32), k (int8)."""
    from ._lib import Layer
    arr = (Layer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = Layer(int(L["type"]), int(L.get("KH", 1)), int(L.get("KW", 1)), int(L.get("pad", 0)),
                       int(L["H"]), int(L["W"]), int(L["Cin"]), int(L["Cout"]),
                       _p(L["weight"], i8, name="weight"), _p(L["offset"], i32, name="offset"),
                       _p(L["mult"], i32, name="mult"), _p(L["k"], i8, name="k"))
    return arr


def ionn_model_workspace_bytes(larr, B):
    n = int(lib().ionn_model_workspace_bytes(larr, len(larr), int(B)))
    if n == 0:
        check(2, "ionn_model_workspace_bytes")
    return n


def ionn_model_forward(larr, X, workspace, out=None, stream=None):
    check(lib().ionn_model_forward(larr, len(larr), _p(X, i8, name="X"), X.shape[0], _p(out, i8, name="out"),
                                   _p(workspace, None, name="workspace"), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "ionn_model_forward")


def ionn_model_backward(larr, X, labels, tmc, tmw, workspace, tb_delta=7, tb_weight=8, mu=2, shifts_out=None,
                        stream=None):
    check(lib().ionn_model_backward(larr, len(larr), _p(X, i8, name="X"), X.shape[0],
                                    _p(labels, i32, name="labels"), _p(tmc, i8, name="tmc"), _p(tmw, i8, name="tmw"),
                                    int(tb_delta), int(tb_weight), int(mu), _p(workspace, None, name="workspace"),
                                    workspace.numel() * workspace.element_size(),
                                    _p(shifts_out, i32, 1 + 5 * len(larr), "shifts_out"), _stream(stream)),
          "ionn_model_backward")


def int_output_error(out, labels, target_mag, e, absmax_e=None, stream=None):
    B, C = out.shape
    assert tuple(e.shape) == (B, C) and labels.numel() == B
    check(lib().int_output_error(_p(out, i8, name="out"), _p(labels, i32, name="labels"), B, C,
                                 int(target_mag), _p(e, i32, name="e"),
                                 _p(absmax_e, u32, 1, "absmax_e"), _stream(stream)),
          "int_output_error")


def conv_desc(N, H, W, Cin, Cout, KH=3, KW=3, stride=1, pad=1, dilation=1, groups=1):
    return ConvDesc(N, H, W, Cin, Cout, KH, KW, stride, pad, dilation, groups)


def _conv_numels(desc):
    """Elements of X [N][H][W][Cin], W [Cout][KH][KW][Cin] and the output
    [N][Ho][Wo][Cout] (Ho = H + 2 pad - KH + 1, stride 1) that a call with
    this descriptor touches."""
    ho = max(desc.H + 2 * desc.pad - desc.KH + 1, 0)
    wo = max(desc.W + 2 * desc.pad - desc.KW + 1, 0)
    return (desc.N * desc.H * desc.W * desc.Cin, desc.Cout * desc.KH * desc.KW * desc.Cin,
            desc.N * ho * wo * desc.Cout)


def int_conv_fwd(X, Wt, Y, desc, absmax_Y=None, stream=None):
    nx, nw, ny = _conv_numels(desc)
    check(lib().int_conv_fwd(_p(X, i8, nx, "X"), _p(Wt, i8, nw, "W"), _p(Y, i32, ny, "Y"),
                             ctypes.byref(desc), _p(absmax_Y, u32, 1, "absmax_Y"), _stream(stream)),
          "int_conv_fwd")


def int_conv_dgrad(dY, Wt, dX, desc, absmax_dX=None, stream=None):
    nx, nw, ny = _conv_numels(desc)
    check(lib().int_conv_dgrad(_p(dY, i8, ny, "dY"), _p(Wt, i8, nw, "W"), _p(dX, i32, nx, "dX"),
                               ctypes.byref(desc), _p(absmax_dX, u32, 1, "absmax_dX"),
                               _stream(stream)), "int_conv_dgrad")




def int_conv_requant_workspace_bytes(desc):
    return int(lib().int_conv_requant_workspace_bytes(ctypes.byref(desc)))


def _ws(workspace):
    return (_p(workspace, None, name="workspace"),
            workspace.numel() * workspace.element_size() if workspace is not None else 0)


def int_conv_fwd_requant(X, Wt, Y8, desc, target_bits, relu, absmax_Y, shift_out=None, workspace=None,
                         stream=None):
    nx, nw, ny = _conv_numels(desc)
    check(lib().int_conv_fwd_requant(_p(X, i8, nx, "X"), _p(Wt, i8, nw, "W"), _p(Y8, i8, ny, "Y8"),
                                     ctypes.byref(desc), int(target_bits), int(bool(relu)),
                                     _p(absmax_Y, u32, 1, "absmax_Y"), _p(shift_out, i32, 1, "shift_out"),
                                     *_ws(workspace), _stream(stream)), "int_conv_fwd_requant")


def int_conv_dgrad_requant(dY, Wt, dX8, desc, target_bits, absmax_dX, shift_out=None, workspace=None,
                           stream=None):
    nx, nw, ny = _conv_numels(desc)
    check(lib().int_conv_dgrad_requant(_p(dY, i8, ny, "dY"), _p(Wt, i8, nw, "W"), _p(dX8, i8, nx, "dX8"),
                                       ctypes.byref(desc), int(target_bits), _p(absmax_dX, u32, 1, "absmax_dX"),
                                       _p(shift_out, i32, 1, "shift_out"), *_ws(workspace), _stream(stream)),
          "int_conv_dgrad_requant")


def int_conv_wgrad_workspace_bytes(desc):
    return int(lib().int_conv_wgrad_workspace_bytes(ctypes.byref(desc)))


def int_conv_wgrad(dY, X, G, desc, absmax_G=None, workspace=None, stream=None):
    nx, nw, ny = _conv_numels(desc)
    check(lib().int_conv_wgrad(_p(dY, i8, ny, "dY"), _p(X, i8, nx, "X"), _p(G, i32, nw, "G"),
                               ctypes.byref(desc), _p(absmax_G, u32, 1, "absmax_G"),
                               _p(workspace, None, name="workspace"),
                               workspace.numel() * workspace.element_size() if workspace is not None else 0,
                               _stream(stream)), "int_conv_wgrad")


def dfp16_workspace_bytes(M, K, N, which):
    return int(lib().dfp16_workspace_bytes(M, K, N, which))


def _dfp(fn, name, A, eA, B, eB, out, eout, M, K, N, chunk, workspace, status_out, stream):
    check(fn(_p(A, i16, name="A"), _p(eA, i32, 1, "eA"), _p(B, i16, name="B"),
             _p(eB, i32, 1, "eB"), _p(out, i16, name="out"), _p(eout, i32, 1, "e_out"), M, K, N,
             int(chunk), _p(workspace, None, name="workspace"),
             workspace.numel() * workspace.element_size() if workspace is not None else 0,
             _p(status_out, i32, 1, "status_out"), _stream(stream)), name)


def dfp16_gemm_fwd(X, eX, W, eW, Y, eY, workspace, chunk=64, status_out=None, stream=None):
    M, K = X.shape
    N = W.shape[0]
    assert tuple(W.shape) == (N, K) and tuple(Y.shape) == (M, N)
    _dfp(lib().dfp16_gemm_fwd, "dfp16_gemm_fwd", X, eX, W, eW, Y, eY, M, K, N, chunk, workspace,
         status_out, stream)


def dfp16_gemm_dgrad(dY, edY, W, eW, dX, edX, workspace, chunk=64, status_out=None, stream=None):
    M, N = dY.shape
    K = W.shape[1]
    assert tuple(W.shape) == (N, K) and tuple(dX.shape) == (M, K)
    _dfp(lib().dfp16_gemm_dgrad, "dfp16_gemm_dgrad", dY, edY, W, eW, dX, edX, M, K, N, chunk,
         workspace, status_out, stream)


def dfp16_gemm_wgrad(dY, edY, X, eX, G, eG, workspace, chunk=64, status_out=None, stream=None):
    M, N = dY.shape
    K = X.shape[1]
    assert tuple(X.shape) == (M, K) and tuple(G.shape) == (N, K)
    _dfp(lib().dfp16_gemm_wgrad, "dfp16_gemm_wgrad", dY, edY, X, eX, G, eG, M, K, N, chunk,
         workspace, status_out, stream)


# ---- DFP as the DFP page runs it: FP32 partials, conversions, SGD -----------

f32 = torch.float32


def dfp16_f32_splits(M, K, N, which):
    return int(lib().dfp16_f32_splits(M, K, N, which))


def dfp16_f32_workspace_bytes(M, K, N, which, nsplit=0):
    return int(lib().dfp16_f32_workspace_bytes(M, K, N, which, nsplit))


def _dfp_f32(fn, name, A, eA, B, eB, out, M, K, N, input_shift, nsplit, workspace, stream):
    check(fn(_p(A, i16, name="A"), _p(eA, i32, 1, "eA"), _p(B, i16, name="B"), _p(eB, i32, 1, "eB"),
             _p(out, f32, name="out"), M, K, N, int(input_shift), int(nsplit), _p(workspace, None, name="workspace"),
             workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream)), name)


def dfp16_gemm_fwd_f32(X, eX, W, eW, Y, workspace, input_shift=1, nsplit=0, stream=None):
    M, K = X.shape
    N = W.shape[0]
    assert tuple(W.shape) == (N, K) and tuple(Y.shape) == (M, N)
    _dfp_f32(lib().dfp16_gemm_fwd_f32, "dfp16_gemm_fwd_f32", X, eX, W, eW, Y, M, K, N, input_shift, nsplit,
             workspace, stream)


def dfp16_gemm_dgrad_f32(dY, edY, W, eW, dX, workspace, input_shift=1, nsplit=0, stream=None):
    M, N = dY.shape
    K = W.shape[1]
    assert tuple(W.shape) == (N, K) and tuple(dX.shape) == (M, K)
    _dfp_f32(lib().dfp16_gemm_dgrad_f32, "dfp16_gemm_dgrad_f32", dY, edY, W, eW, dX, M, K, N, input_shift, nsplit,
             workspace, stream)


def dfp16_gemm_wgrad_f32(dY, edY, X, eX, G, workspace, input_shift=1, nsplit=0, stream=None):
    M, N = dY.shape
    K = X.shape[1]
    assert tuple(X.shape) == (M, K) and tuple(G.shape) == (N, K)
    _dfp_f32(lib().dfp16_gemm_wgrad_f32, "dfp16_gemm_wgrad_f32", dY, edY, X, eX, G, M, K, N, input_shift, nsplit,
             workspace, stream)


def dfp16_gemm_fwd_f32_blocked(X, eX, W, eW, Y, workspace, input_shift=1, nsplit=0, stream=None):
    """eX: int32 [M][ceil(K/64)], eW: int32 [N][ceil(K/64)] (device)."""
    M, K = X.shape
    N = W.shape[0]
    nch = (K + 63) // 64
    assert tuple(W.shape) == (N, K) and tuple(Y.shape) == (M, N)
    check(lib().dfp16_gemm_fwd_f32_blocked(
        _p(X, i16, name="X"), _p(eX, i32, M * nch, "eX"), _p(W, i16, name="W"), _p(eW, i32, N * nch, "eW"),
        _p(Y, f32, name="Y"), M, K, N, int(input_shift), int(nsplit), _p(workspace, None, name="workspace"),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream)),
        "dfp16_gemm_fwd_f32_blocked")


def dfp_convert_workspace_bytes():
    return int(lib().dfp_convert_workspace_bytes())


def dfp_from_f32(x, out, e_out, workspace, P=16, status_out=None, stream=None):
    assert x.numel() == out.numel()
    check(lib().dfp_from_f32(_p(x, f32, name="x"), x.numel(), int(P), _p(out, i16, name="out"),
                             _p(e_out, i32, 1, "e_out"), _p(status_out, i32, 1, "status_out"),
                             _p(workspace, None, name="workspace"),
                             workspace.numel() * workspace.element_size(), _stream(stream)), "dfp_from_f32")


def dfp_to_f32(I, e, out, stream=None):
    assert I.numel() == out.numel()
    check(lib().dfp_to_f32(_p(I, i16, name="I"), I.numel(), _p(e, i32, 1, "e"), _p(out, f32, name="out"),
                           _stream(stream)), "dfp_to_f32")


def dfp_from_f32_blocked(x, out, e_out, B=64, P=16, status_out=None, stream=None):
    rows, K = x.shape
    nb = (K + B - 1) // B
    assert tuple(out.shape) == (rows, K) and e_out.numel() >= rows * nb
    check(lib().dfp_from_f32_blocked(_p(x, f32, name="x"), rows, K, int(B), int(P), _p(out, i16, name="out"),
                                     _p(e_out, i32, rows * nb, "e_out"), _p(status_out, i32, 1, "status_out"),
                                     _stream(stream)), "dfp_from_f32_blocked")


def dfp16_sgd_update(W32, G32, lr, W16, eW, workspace, status_out=None, stream=None):
    n = W32.numel()
    assert G32.numel() == n and W16.numel() == n
    check(lib().dfp16_sgd_update(_p(W32, f32, name="W32"), _p(G32, f32, name="G32"), n, float(lr),
                                 _p(W16, i16, name="W16"), _p(eW, i32, 1, "eW"), _p(status_out, i32, 1, "status_out"),
                                 _p(workspace, None, name="workspace"), workspace.numel() * workspace.element_size(),
                                 _stream(stream)), "dfp16_sgd_update")


def dfp16_gavg(G, eG, eW, gavg_out, stream=None):
    check(lib().dfp16_gavg(_p(G, i16, name="G"), _p(eG, i32, 1, "eG"), _p(eW, i32, 1, "eW"),
                           G.numel(), _p(gavg_out, torch.float64, 1, "gavg_out"), _stream(stream)),
          "dfp16_gavg")


# ---- adaptive per-layer precision -------------------------------------------

def _ptr_array(ts, dtype, name):
    return (ctypes.c_void_p * len(ts))(*[_p(t, dtype, name=f"{name}[{l}]").value for l, t in enumerate(ts)])


def _sizes(ts):
    return (ctypes.c_int64 * len(ts))(*[t.numel() for t in ts])


def apt_workspace_bytes(sizes):
    return lib().apt_workspace_bytes(len(sizes), (ctypes.c_int64 * len(sizes))(*[int(n) for n in sizes]))


def apt_update(Ws, Gs, k, e_w, e_g, lr_shift, gavg_sum=None, gavg_count=None, workspace=None, stream=None):
    """One step's k-bit update of every layer (lists of int16 device tensors);
    k, e_w, e_g: int32 [L]; gavg_sum (float64 [L]) and gavg_count (int32 [L])
    given together make it a sampling step."""
    L = len(Ws)
    if len(Gs) != L or any(w.numel() != g.numel() for w, g in zip(Ws, Gs)):
        raise ValueError("Ws and Gs must pair up with equal sizes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().apt_update(L, _ptr_array(Ws, i16, "W"), _ptr_array(Gs, i16, "G"), _sizes(Ws),
                           _p(k, i32, L, "k"), _p(e_w, i32, L, "e_w"), _p(e_g, i32, L, "e_g"), int(lr_shift),
                           _p(gavg_sum, torch.float64, L, "gavg_sum"), _p(gavg_count, i32, L, "gavg_count"),
                           _p(workspace, name="workspace"), ws_bytes, _stream(stream)), "apt_update")


def _wbytes(Ws):
    """Host int32 array of bytes per weight (1 for int8 tensors, 2 for int16)."""
    out = []
    for l, w in enumerate(Ws):
        if w.dtype not in (torch.int8, torch.int16):
            raise TypeError(f"W[{l}] must be int8 or int16, not {w.dtype}")
        out.append(1 if w.dtype == torch.int8 else 2)
    return (ctypes.c_int32 * len(Ws))(*out)


def apt_update_mixed(Ws, Gs, k, e_w, e_g, lr_shift, gavg_sum=None, gavg_count=None, workspace=None, stream=None):
    """apt_update over layers held in int8 (k in [2, 8]) or int16."""
    L = len(Ws)
    if len(Gs) != L or any(w.numel() != g.numel() for w, g in zip(Ws, Gs)):
        raise ValueError("Ws and Gs must pair up with equal sizes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().apt_update_mixed(L, _ptr_array(Ws, None, "W"), _wbytes(Ws), _ptr_array(Gs, i16, "G"), _sizes(Ws),
                                 _p(k, i32, L, "k"), _p(e_w, i32, L, "e_w"), _p(e_g, i32, L, "e_g"), int(lr_shift),
                                 _p(gavg_sum, torch.float64, L, "gavg_sum"), _p(gavg_count, i32, L, "gavg_count"),
                                 _p(workspace, name="workspace"), ws_bytes, _stream(stream)), "apt_update_mixed")


def apt_adjust_mixed(Ws, k, e_w, gavg_sum, gavg_count, t_min, t_max, k_min=2, k_max=16, dk_out=None, stream=None):
    """apt_adjust over layers held in int8 (never raised past 8 bits) or int16."""
    L = len(Ws)
    check(lib().apt_adjust_mixed(L, _ptr_array(Ws, None, "W"), _wbytes(Ws), _sizes(Ws), _p(k, i32, L, "k"),
                                 _p(e_w, i32, L, "e_w"), _p(gavg_sum, torch.float64, L, "gavg_sum"),
                                 _p(gavg_count, i32, L, "gavg_count"), float(t_min), float(t_max), int(k_min),
                                 int(k_max), _p(dk_out, i32, L, "dk_out"), _stream(stream)), "apt_adjust_mixed")


def apt_adjust(Ws, k, e_w, gavg_sum, gavg_count, t_min, t_max, k_min=2, k_max=16, dk_out=None, stream=None):
    """Between epochs: one bit more or less per layer on its mean Gavg."""
    L = len(Ws)
    check(lib().apt_adjust(L, _ptr_array(Ws, i16, "W"), _sizes(Ws), _p(k, i32, L, "k"), _p(e_w, i32, L, "e_w"),
                           _p(gavg_sum, torch.float64, L, "gavg_sum"), _p(gavg_count, i32, L, "gavg_count"),
                           float(t_min), float(t_max), int(k_min), int(k_max), _p(dk_out, i32, L, "dk_out"),
                           _stream(stream)), "apt_adjust")
