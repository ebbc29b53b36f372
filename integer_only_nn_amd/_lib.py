"""ctypes loader for libionn.so (the HIP library built by build.py).

The product path has no fallback: if the library is missing or fails to
load, every call raises.
"""
import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libionn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "ionn.h")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int

# Argument/return types of every entry point declared in include/ionn.h.
SIGNATURES = {
    "ionn_status_str": (ctypes.c_char_p, [_I]),
    "ionn_last_error": (ctypes.c_char_p, []),
    "ionn_version": (ctypes.c_char_p, []),
    "ionn_fill_u32": (_I, [_P, _I64, ctypes.c_uint32, _P]),
    "ionn_absmax_i32": (_I, [_P, _I64, _P, _P]),
    "int_linear_fwd": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "int_linear_dgrad": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "int_linear_wgrad": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "int_linear_wgrad_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "int_linear_wgrad_ws": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P, ctypes.c_size_t, _P]),
    "niti_quantize": (_I, [_P, _I64, _P, _I, _I, _P, _P, _P]),
    "niti_quantize_update": (_I, [_P, _I64, _P, _I, _I, _P, _P, _P, _P]),
    "niti_quantize_update_clear": (_I, [_P, _I64, _P, _I, _I, _P, _P, _P, _P, _I64, _P]),
    "int_linear_step_small": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "int_linear_step_small_fits": (_I, [_I64, _I64, _I64]),
    "int_output_error": (_I, [_P, _P, _I64, _I64, _I, _P, _P, _P]),
    "int_conv_fwd": (_I, [_P, _P, _P, _P, _P, _P]),
    "int_conv_dgrad": (_I, [_P, _P, _P, _P, _P, _P]),
    "int_conv_requant_workspace_bytes": (ctypes.c_size_t, [_P]),
    "int_conv_fwd_requant": (_I, [_P, _P, _P, _P, _I, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    "int_conv_dgrad_requant": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    "int_conv_wgrad_workspace_bytes": (ctypes.c_size_t, [_P]),
    "int_conv_wgrad": (_I, [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "dfp16_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I]),
    "dfp16_gemm_fwd": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, ctypes.c_size_t, _P, _P]),
    "dfp16_gemm_dgrad": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, ctypes.c_size_t, _P, _P]),
    "dfp16_gemm_wgrad": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, ctypes.c_size_t, _P, _P]),
    "dfp16_gavg": (_I, [_P, _P, _P, _I64, _P, _P]),
    "dfp16_f32_splits": (_I, [_I64, _I64, _I64, _I]),
    "dfp16_f32_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I, _I]),
    "dfp16_gemm_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P, ctypes.c_size_t, _P]),
    "dfp16_gemm_dgrad_f32": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P, ctypes.c_size_t, _P]),
    "dfp16_gemm_wgrad_f32": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P, ctypes.c_size_t, _P]),
    "dfp16_gemm_fwd_f32_blocked": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P, ctypes.c_size_t, _P]),
    "dfp_convert_workspace_bytes": (ctypes.c_size_t, []),
    "dfp_from_f32": (_I, [_P, _I64, _I, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "dfp_to_f32": (_I, [_P, _I64, _P, _P, _P]),
    "dfp_from_f32_blocked": (_I, [_P, _I64, _I64, _I, _I, _P, _P, _P, _P]),
    "dfp16_sgd_update": (_I, [_P, _P, _I64, ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "apt_workspace_bytes": (ctypes.c_size_t, [_I, _P]),
    "apt_update": (_I, [_I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    "apt_adjust": (_I, [_I, _P, _P, _P, _P, _P, _P, ctypes.c_double, ctypes.c_double, _I, _I, _P, _P]),
    "apt_update_mixed": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    "apt_adjust_mixed": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, ctypes.c_double, ctypes.c_double, _I, _I, _P, _P]),
    "ionn_oss_requant": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _P, _P]),
    "ionn_bias_grad_workspace_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "ionn_bias_grad": (_I, [_P, _I64, _I64, _P, _P, ctypes.c_size_t, _P]),
    "ionn_bias_grad_noalloc": (_I, [_P, _I64, _I64, _P, _P]),
    "int_linear_fwd_oss_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "int_linear_fwd_oss": (_I, [_P, _P, _P, _P, _P, _I, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "niti_quantize_update_i32": (_I, [_P, _I64, _P, _I, _I, _P, _P, _P, _P]),
    "ionn_mse_grad_targets": (_I, [_P, _P, _I64, _I64, _P, _P, _P, _P, _P]),
    "ionn_relu_mask_i32": (_I, [_P, _P, _I64, _P, _P]),
    "ionn_model_workspace_bytes": (ctypes.c_size_t, [_P, _I, _I64]),
    "ionn_model_forward": (_I, [_P, _I, _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "ionn_model_backward": (_I, [_P, _I, _P, _I64, _P, _P, _P, _I, _I, _I, _P, ctypes.c_size_t, _P, _P]),
}


class ConvDesc(ctypes.Structure):
    """Mirror of ionn_conv_desc."""
    _fields_ = [("N", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
                ("Cin", ctypes.c_int64), ("Cout", ctypes.c_int64),
                ("KH", ctypes.c_int32), ("KW", ctypes.c_int32), ("stride", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("dilation", ctypes.c_int32), ("groups", ctypes.c_int32)]


class Layer(ctypes.Structure):
    """Mirror of ionn_layer."""
    _fields_ = [("type", ctypes.c_int32), ("KH", ctypes.c_int32), ("KW", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
                ("Cin", ctypes.c_int64), ("Cout", ctypes.c_int64), ("weight", ctypes.c_void_p),
                ("offset", ctypes.c_void_p), ("mult", ctypes.c_void_p), ("k", ctypes.c_void_p)]


LAYER_CONV2D, LAYER_CONV2D_RELU, LAYER_LINEAR, LAYER_LINEAR_RELU = 0, 1, 2, 3


class IonnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"[{status}] {message}")
        self.status = status


def header_functions():
    """Names of the functions declared in include/ionn.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) -
                  {"sizeof", "defined", "if", "while", "for", "return", "switch"})


_lib = None


def lib():
    """Load libionn.so once; raise if it is missing (no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} not found: build it with `python -m integer_only_nn_amd.build` "
                "(or __graft_entry__.build()); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status, what=""):
    if status != 0:
        L = lib()
        msg = L.ionn_last_error().decode() or L.ionn_status_str(status).decode()
        raise IonnError(status, f"{what}: {msg}" if what else msg)
    return status
