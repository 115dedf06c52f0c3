"""ctypes view of libqws.so (the C ABI declared in include/qws.h). Loading fails loudly."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqws.so")

QWS_OK = 0
QWS_ERR_ARG = -1
QWS_ERR_SHAPE = -2
QWS_ERR_ALIGN = -3
QWS_ERR_FORMAT = -4
QWS_ERR_WORKSPACE = -5
QWS_ERR_DEVICE = -6
QWS_ERR_SELFCHECK = -7
QWS_ERR_COMPILE = -8

QWS_FMT_MXFP4_E2M1_E8M0_B32 = 0x4D584634
QWS_FMT_FP8_E4M3FN_ROWSCALE = 0x46503845
QWS_FMT_BF16 = 0x42463136
QWS_FMT_MXFP4_E2M1_E8M0_B32_TASKMAJOR = 0x4D584655
QWS_FMT_FP8_E4M3FN_ROWSCALE_T16 = 0x46503854
QWS_TASK_BYTES = 131072


class MxFp4Experts(C.Structure):
    _fields_ = [("format", C.c_uint), ("n_routed", C.c_int), ("has_shared", C.c_int), ("hidden", C.c_int),
                ("inter", C.c_int), ("gate_up_q", C.c_void_p), ("gate_up_s", C.c_void_p), ("down_q", C.c_void_p),
                ("down_s", C.c_void_p)]


class MoeLayerDesc(C.Structure):
    _fields_ = [("x_bf16", C.c_void_p), ("w_router_bf16", C.c_void_p), ("bias", C.c_void_p),
                ("bias_row_stride", C.c_longlong), ("experts", MxFp4Experts), ("topk_idx", C.c_void_p),
                ("topk_w", C.c_void_p), ("logits_out", C.c_void_p), ("y_bf16", C.c_void_p), ("y_f32", C.c_void_p)]


class LMHeadDesc(C.Structure):
    _fields_ = [("format", C.c_uint), ("rows", C.c_longlong), ("cols", C.c_longlong), ("w", C.c_void_p),
                ("row_scale", C.c_void_p)]


class RtcStats(C.Structure):
    _fields_ = [("compiles", C.c_ulonglong), ("disk_hits", C.c_ulonglong), ("memory_hits", C.c_ulonglong),
                ("compile_ms", C.c_double), ("load_ms", C.c_double)]


_P = C.c_void_p
_I = C.c_int
_LL = C.c_longlong
_SZ = C.c_size_t

# name -> (restype, argtypes); every entry point of include/qws.h
SIGNATURES = {
    "qws_strerror": (C.c_char_p, [_I]),
    "qws_abi_version": (_I, []),
    "qws_selfcheck": (_I, [_P]),
    "moe_route_workspace_bytes": (_SZ, [_I, _I]),
    "moe_route_topk": (_I, [_P, _I, _I, _P, _I, _P, _LL, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "moe_expert_gemv_mxfp4": (_I, [C.POINTER(MxFp4Experts), _P, _I, _P, _P, _I, _P, _P, _P, _SZ, _P]),
    "moe_pack_mxfp4_bytes": (_SZ, [_I, _I, _I]),
    "moe_pack_mxfp4": (_I, [C.POINTER(MxFp4Experts), _P, _SZ, C.POINTER(MxFp4Experts), _P]),
    "moe_layer_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_layer_mxfp4": (_I, [C.POINTER(MoeLayerDesc), _I, _I, _P, _SZ, _P]),
    "moe_layers_mxfp4": (_I, [C.POINTER(MoeLayerDesc), _P, _I, _I, _I, _P, _SZ, _P]),
    "moe_layer_w4a8": (_I, [C.POINTER(MoeLayerDesc), _I, _I, _P, _SZ, _P]),
    "moe_layers_w4a8": (_I, [C.POINTER(MoeLayerDesc), _P, _I, _I, _I, _P, _SZ, _P]),
    "moe_workspace_errors": (_I, [_P, _I, _I, _I, _I, C.POINTER(C.c_uint), _P]),
    "lmhead_bf16_desc": (_I, [_P, _LL, _LL, C.POINTER(LMHeadDesc)]),
    "lmhead_quantize_fp8": (_I, [_P, _LL, _LL, _P, _P, C.POINTER(LMHeadDesc), _P]),
    "lmhead_fp8_codes_bytes": (_SZ, [_LL, _LL]),
    "lmhead_fp8_tile_major": (_I, [C.POINTER(LMHeadDesc), _P, _SZ, C.POINTER(LMHeadDesc), _P]),
    "lmhead_gemv_fp8": (_I, [C.POINTER(LMHeadDesc), _P, _I, _P, _P]),
    "lmhead_verify_workspace_bytes": (_SZ, [_I]),
    "lmhead_verify_greedy_fp8": (_I, [C.POINTER(LMHeadDesc), _P, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "lmhead_verify_greedy_fp8_noalloc": (_I, [C.POINTER(LMHeadDesc), _P, _I, _P, _P, _P, _P, _P, _P]),
    "lmhead_verify_sample_fp8": (_I, [C.POINTER(LMHeadDesc), _P, _I, _P, C.c_float, _I, C.c_float, _P, _P, _P, _P,
                                      _P, _P, _P, _SZ, _P]),
    "lmhead_gemv_bf16": (_I, [C.POINTER(LMHeadDesc), _P, _I, _P, _P]),
    "lmhead_gemv_fp8_rtc": (_I, [C.POINTER(LMHeadDesc), _P, _I, _P, C.c_char_p, _P]),
    "qws_rtc_compile_head_fp8": (_I, [_I, _LL, _LL, C.c_char_p, C.c_char_p]),
    "moe_layers_rtc": (_I, [C.POINTER(MoeLayerDesc), _P, _I, _I, _I, _I, _P, _SZ, C.c_char_p, _P]),
    "qws_rtc_compile_moe": (_I, [_I, _I, _I, _I, _I, _I, _I, C.c_char_p, C.c_char_p]),
    "qws_rtc_stats_get": (_I, [C.POINTER(RtcStats)]),
    "qws_rtc_reset": (_I, []),
    "qws_debug_dequant_mxfp4": (_I, [_P, _P, _LL, _I, _I, _P, _P]),
    "qws_debug_dequant_fp8": (_I, [C.POINTER(LMHeadDesc), _P, _P]),
    "qws_probe_read": (_I, [_P, _SZ, _P, _I, _P]),
    "qws_probe_read_nt": (_I, [_P, _SZ, _P, _I, _P]),
    "qws_probe_copy": (_I, [_P, _P, _SZ, _I, _P]),
    "qws_debug_trace_buffer": (_I, [_P, _SZ]),
    "qws_debug_w4a8_act_buffer": (_I, [_P, _SZ]),
}

_lib = None


_lib_path = None


def load(path: str | None = None) -> C.CDLL:
    """The loaded libqws: the in-tree build unless `path` names another build, which then replaces
    it for every later call. Raises if it has not been built: there is no fallback path."""
    global _lib, _lib_path
    if _lib is None or (path is not None and os.path.realpath(path) != _lib_path):
        path = path or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"libqws.so not built at {path}; run quantized_weight_streaming_amd/build.py "
                               "(hipcc --offload-arch=gfx950). There is no CPU fallback.")
        lib = C.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib, _lib_path = lib, os.path.realpath(path)
    return _lib


class QwsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().qws_strerror(status).decode(errors="replace")
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != QWS_OK:
        raise QwsError(fn, status)
