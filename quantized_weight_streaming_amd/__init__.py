"""Batch-size-1 MoE decode-step weight streaming on MI355X (gfx950).

Python binding of libqws (include/qws.h): the same entry points, taking torch device tensors and
the current HIP stream. Argument marshalling only -- every step runs in the library's HIP kernels;
if libqws.so is missing, the first call raises (there is no CPU fallback).

    route  = moe_route_topk(x, w_router, K)               # router GEMV + top-K + softmax
    y      = moe_expert_gemv_mxfp4(bank, x, idx, w)       # union of experts, SwiGLU, combine
    packed = moe_pack_mxfp4(bank)                         # task-major copy, once per bank
    layer  = moe_layer_mxfp4(MoeLayer(x, w_router, packed, K))   # the whole layer, one launch
    layer  = moe_layer_w4a8(MoeLayer(x, w_router, packed, K))    # the same with MXFP8 activations
    head   = lmhead_quantize_fp8(w_head_bf16)             # online FP8 head, once
    logits = lmhead_gemv_fp8(head, x)
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (QWS_FMT_BF16, QWS_FMT_FP8_E4M3FN_ROWSCALE, QWS_FMT_MXFP4_E2M1_E8M0_B32,  # noqa: F401
                   QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, QWS_FMT_MXFP4_E2M1_E8M0_B32_TASKMAJOR, QWS_TASK_BYTES, LMHeadDesc, MoeLayerDesc, MxFp4Experts,
                   QwsError, check)

__all__ = ["selfcheck", "moe_route_topk", "moe_expert_gemv_mxfp4", "ExpertBank", "moe_pack_mxfp4", "LMHead",
           "lmhead_bf16",
           "moe_layer_mxfp4", "moe_layers_mxfp4", "moe_layer_w4a8", "moe_layers_w4a8", "MoeLayer", "moe_layer_workspace", "moe_workspace_errors",
           "lmhead_quantize_fp8", "lmhead_fp8_codes_bytes", "fp8_codes_rowmajor", "lmhead_gemv_fp8", "lmhead_gemv_bf16",
           "lmhead_verify_greedy_fp8", "lmhead_verify_sample_fp8", "lmhead_gemv_fp8_rtc", "rtc_compile_head_fp8", "rtc_compile_moe",
           "rtc_stats", "rtc_reset",
           "verify_workspace", "debug_dequant_mxfp4", "debug_dequant_fp8",
           "probe_read", "probe_read_nt", "probe_copy", "route_workspace", "expert_workspace", "QwsError", "lib"]


def lib():
    return _lib.load()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def selfcheck(device=None) -> None:
    """Device format self-check against host tables; raises QwsError on any mismatch."""
    check("qws_selfcheck", lib().qws_selfcheck(_stream(device)))


# ----------------------------------------------------------------------------------- router
def route_workspace(M: int, E: int, device) -> torch.Tensor:
    n = lib().moe_route_workspace_bytes(M, E)
    if n == 0:
        raise ValueError(f"unsupported router shape M={M} E={E}")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_route_topk(x: torch.Tensor, w_router: torch.Tensor, K: int, bias: torch.Tensor | None = None,
                   topk_idx=None, topk_w=None, logits_out=None, workspace=None):
    """(topk_idx int32 [M, K], topk_w fp32 [M, K]); logits_out (fp32 [M, E]) is filled if given."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_router, "w_router", torch.bfloat16, 2)
    M, H = x.shape
    E = w_router.shape[0]
    stride = 0
    if bias is not None:
        _need(bias, "bias", torch.float32)
        stride = 0 if bias.dim() == 1 else bias.shape[-1]
    if topk_idx is None:
        topk_idx = torch.empty((M, K), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((M, K), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = route_workspace(M, E, x.device)
    st = lib().moe_route_topk(_p(x), M, H, _p(w_router), E, _p(bias), stride, K, _p(topk_idx), _p(topk_w),
                              _p(logits_out), _p(workspace), workspace.numel(), _stream(x.device))
    check("moe_route_topk", st)
    return topk_idx, topk_w


# ----------------------------------------------------------------------------------- experts
@dataclass
class ExpertBank:
    """MXFP4 experts (uint8 tensors); the shared expert, if any, is the last one.

    layout "canonical": gate_up_q [n, 2I, H/2], gate_up_s [n, 2I, H/32], down_q [n, H, I/2],
    down_s [n, H, I/32] (row-major per expert).
    layout "task_major" (from moe_pack_mxfp4): gate_up_q holds the task records [n, I/32,
    QWS_TASK_BYTES] (the layout is stated with moe_pack_mxfp4 in include/qws.h); the other three
    are None and `hidden` must be given."""
    gate_up_q: torch.Tensor
    gate_up_s: Optional[torch.Tensor]
    down_q: Optional[torch.Tensor]
    down_s: Optional[torch.Tensor]
    n_routed: int
    has_shared: bool = True
    layout: str = "canonical"
    hidden: int = 0

    def __post_init__(self):
        n = self.n_routed + int(self.has_shared)
        if self.layout == "canonical":
            two_i, hb = self.gate_up_q.shape[1:]
            H, I = hb * 2, two_i // 2
            checks = (("gate_up_q", self.gate_up_q, (n, two_i, hb)), ("gate_up_s", self.gate_up_s, (n, two_i, H // 32)),
                      ("down_q", self.down_q, (n, H, I // 2)), ("down_s", self.down_s, (n, H, I // 32)))
            fmt = QWS_FMT_MXFP4_E2M1_E8M0_B32
            ptrs = [t.data_ptr() for t in (self.gate_up_q, self.gate_up_s, self.down_q, self.down_s)]
        elif self.layout == "task_major":
            H, I = self.hidden, self.gate_up_q.shape[1] * 32
            checks = (("records", self.gate_up_q, (n, I // 32, QWS_TASK_BYTES)),)
            fmt = QWS_FMT_MXFP4_E2M1_E8M0_B32_TASKMAJOR
            ptrs = [self.gate_up_q.data_ptr(), None, None, None]
        else:
            raise ValueError(f"unknown layout {self.layout!r}")
        for name, t, shape in checks:
            _need(t, name, torch.uint8, 3)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        self.hidden = H
        self.inter = I
        self.desc = MxFp4Experts(fmt, self.n_routed, int(self.has_shared), self.hidden, self.inter, *ptrs)

    @classmethod
    def from_dict(cls, d: dict, n_routed: int, has_shared: bool = True):
        return cls(d["gate_up_q"], d["gate_up_s"], d["down_q"], d["down_s"], n_routed, has_shared)


def moe_pack_mxfp4(bank: ExpertBank) -> ExpertBank:
    """A task-major copy of the bank for the fused entry points (new record tensor; `bank` is not
    referenced afterwards and may be freed)."""
    if bank.layout != "canonical":
        raise ValueError("moe_pack_mxfp4 needs a canonical bank")
    n = bank.n_routed + int(bank.has_shared)
    dev = bank.gate_up_q.device
    nbytes = lib().moe_pack_mxfp4_bytes(n, bank.hidden, bank.inter)
    if nbytes == 0:
        raise ValueError("unsupported expert shape for the task-major pack")
    rec = torch.empty((n, bank.inter // 32, QWS_TASK_BYTES), dtype=torch.uint8, device=dev)
    out = MxFp4Experts()
    st = lib().moe_pack_mxfp4(C.byref(bank.desc), _p(rec), rec.numel(), C.byref(out), _stream(dev))
    check("moe_pack_mxfp4", st)
    return ExpertBank(rec, None, None, None, bank.n_routed, bank.has_shared, "task_major", hidden=bank.hidden)


def expert_workspace(M: int, K: int, hidden: int, inter: int, device) -> torch.Tensor:
    n = lib().moe_expert_workspace_bytes(M, K, hidden, inter)
    if n == 0:
        raise ValueError("unsupported expert shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_expert_gemv_mxfp4(bank: ExpertBank, x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                          y_bf16=None, y_f32=None, workspace=None, want_bf16=True, want_f32=True):
    """(y_bf16, y_f32) for the window x [M, H]; either output may be skipped."""
    _need(x, "x", torch.bfloat16, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    M, H = x.shape
    K = topk_idx.shape[1]
    if H != bank.hidden or tuple(topk_w.shape) != (M, K) or topk_idx.shape[0] != M:
        raise ValueError("x / routing shapes do not match the bank")
    if y_bf16 is None and want_bf16:
        y_bf16 = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    if y_f32 is None and want_f32:
        y_f32 = torch.empty((M, H), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = expert_workspace(M, K, bank.hidden, bank.inter, x.device)
    st = lib().moe_expert_gemv_mxfp4(C.byref(bank.desc), _p(x), M, _p(topk_idx), _p(topk_w), K, _p(y_bf16),
                                     _p(y_f32), _p(workspace), workspace.numel(), _stream(x.device))
    check("moe_expert_gemv_mxfp4", st)
    return y_bf16, y_f32


# ----------------------------------------------------------------------------------- fused layer(s)
def moe_layer_workspace(M: int, K: int, E: int, hidden: int, inter: int, device) -> torch.Tensor:
    n = lib().moe_layer_workspace_bytes(M, K, E, hidden, inter)
    if n == 0:
        raise ValueError("unsupported fused-layer shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


class MoeLayer:
    """Tensors and the qws_moe_layer descriptor of one layer for the fused entry points. The bank
    must be packed (moe_pack_mxfp4). Passing the previous layer's y_bf16 as x chains the layers."""

    def __init__(self, x, w_router, bank: ExpertBank, K: int, bias=None, y_bf16=None, y_f32=None,
                 topk_idx=None, topk_w=None, logits_out=None, want_bf16=True, want_f32=True):
        if bank.layout != "task_major":
            raise ValueError("the fused entry points need a bank packed by moe_pack_mxfp4")
        _need(x, "x", torch.bfloat16, 2)
        _need(w_router, "w_router", torch.bfloat16, 2)
        M, H = x.shape
        dev = x.device
        if bias is not None:
            _need(bias, "bias", torch.float32)
        if y_bf16 is None and want_bf16:
            y_bf16 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        if y_f32 is None and want_f32:
            y_f32 = torch.empty((M, H), dtype=torch.float32, device=dev)
        if topk_idx is None:
            topk_idx = torch.empty((M, K), dtype=torch.int32, device=dev)
        if topk_w is None:
            topk_w = torch.empty((M, K), dtype=torch.float32, device=dev)
        self.x, self.w_router, self.bank, self.bias = x, w_router, bank, bias
        self.y_bf16, self.y_f32, self.topk_idx, self.topk_w, self.logits_out = y_bf16, y_f32, topk_idx, topk_w, logits_out
        self.M, self.K = M, K
        stride = 0 if bias is None or bias.dim() == 1 else bias.shape[-1]
        self.desc = MoeLayerDesc(x.data_ptr(), w_router.data_ptr(), None if bias is None else bias.data_ptr(), stride,
                                 bank.desc, topk_idx.data_ptr(), topk_w.data_ptr(),
                                 None if logits_out is None else logits_out.data_ptr(),
                                 None if y_bf16 is None else y_bf16.data_ptr(),
                                 None if y_f32 is None else y_f32.data_ptr())


def _run_layer(name: str, layer: MoeLayer, workspace) -> MoeLayer:
    b = layer.bank
    if workspace is None:
        workspace = moe_layer_workspace(layer.M, layer.K, b.n_routed, b.hidden, b.inter, layer.x.device)
    st = getattr(lib(), name)(C.byref(layer.desc), layer.M, layer.K, _p(workspace), workspace.numel(),
                              _stream(layer.x.device))
    check(name, st)
    return layer


def moe_layer_mxfp4(layer: MoeLayer, workspace=None) -> MoeLayer:
    """Router + top-K + experts of one layer in one launch; fills the layer's output tensors."""
    return _run_layer("moe_layer_mxfp4", layer, workspace)


def moe_layer_w4a8(layer: MoeLayer, workspace=None) -> MoeLayer:
    """moe_layer_mxfp4 with MXFP8 activations: x and each expert's SwiGLU output quantised per 32
    elements (E4M3 codes, E8M0 scale) before they meet the MXFP4 weights."""
    return _run_layer("moe_layer_w4a8", layer, workspace)


class MoeLayers:
    """A sequence of layers run by moe_layers_mxfp4 in one launch (descriptors copied to the device once)."""

    def __init__(self, layers: list):
        self.layers = layers
        n = len(layers)
        self.host = (MoeLayerDesc * n)(*[L.desc for L in layers])
        raw = torch.frombuffer(bytearray(C.string_at(C.addressof(self.host), C.sizeof(self.host))), dtype=torch.uint8)
        self.dev = raw.to(layers[0].x.device)

    def run(self, workspace, w4a8: bool = False, rtc: bool = False, cache_dir=None) -> None:
        """One launch of all the layers: moe_layers_mxfp4 (or _w4a8); with rtc, the kernel compiled
        at run time for this shape (moe_layers_rtc; code objects cached in `cache_dir`)."""
        L0 = self.layers[0]
        if rtc:
            st = lib().moe_layers_rtc(self.host, _p(self.dev), len(self.layers), L0.M, L0.K, int(w4a8), _p(workspace),
                                      workspace.numel(), _enc(cache_dir), _stream(L0.x.device))
            check("moe_layers_rtc", st)
            return
        name = "moe_layers_w4a8" if w4a8 else "moe_layers_mxfp4"
        st = getattr(lib(), name)(self.host, _p(self.dev), len(self.layers), L0.M, L0.K, _p(workspace),
                                  workspace.numel(), _stream(L0.x.device))
        check(name, st)


def moe_layers_mxfp4(layers: MoeLayers, workspace) -> None:
    layers.run(workspace)


def moe_layers_w4a8(layers: MoeLayers, workspace) -> None:
    layers.run(workspace, w4a8=True)


def moe_workspace_errors(workspace: torch.Tensor, M: int, K: int, E: int, inter: int) -> int:
    out = C.c_uint(0)
    check("moe_workspace_errors", lib().moe_workspace_errors(_p(workspace), M, K, E, inter, C.byref(out),
                                                             _stream(workspace.device)))
    return int(out.value)


# ----------------------------------------------------------------------------------- LM head
@dataclass
class LMHead:
    """A vocabulary head and its descriptor: bf16 weights, or E4M3 codes with fp32 row scales."""
    w: torch.Tensor
    row_scale: torch.Tensor | None
    desc: LMHeadDesc

    @property
    def format(self) -> int:
        return self.desc.format

    @property
    def rows(self) -> int:
        return self.desc.rows


def lmhead_bf16(w: torch.Tensor) -> LMHead:
    _need(w, "w", torch.bfloat16, 2)
    d = LMHeadDesc()
    check("lmhead_bf16_desc", lib().lmhead_bf16_desc(_p(w), w.shape[0], w.shape[1], C.byref(d)))
    return LMHead(w, None, d)


def lmhead_fp8_codes_bytes(rows: int, cols: int) -> int:
    """Bytes of the tile-major FP8 codes of a rows x cols head (rows padded to a multiple of 16)."""
    n = int(lib().lmhead_fp8_codes_bytes(rows, cols))
    if n == 0:
        raise QwsError("lmhead_fp8_codes_bytes", _lib.QWS_ERR_SHAPE)
    return n


def lmhead_quantize_fp8(w: torch.Tensor, codes=None, row_scale=None) -> LMHead:
    """Online per-row FP8 quantisation of a bf16 head (done once, at construction). The codes are
    a flat uint8 tensor in the tile-major layout of the library (fp8_codes_rowmajor undoes it)."""
    _need(w, "w", torch.bfloat16, 2)
    rows, cols = w.shape
    n = lmhead_fp8_codes_bytes(rows, cols)
    if codes is None:
        codes = torch.empty(n, dtype=torch.uint8, device=w.device)
    elif codes.dtype != torch.uint8 or not codes.is_contiguous() or codes.numel() < n:
        raise ValueError(f"codes must be contiguous uint8 with at least {n} elements")
    if row_scale is None:
        row_scale = torch.empty(rows, dtype=torch.float32, device=w.device)
    d = LMHeadDesc()
    st = lib().lmhead_quantize_fp8(_p(w), rows, cols, _p(codes), _p(row_scale), C.byref(d), _stream(w.device))
    check("lmhead_quantize_fp8", st)
    return LMHead(codes, row_scale, d)


def lmhead_fp8_tile_major(codes_rowmajor: torch.Tensor, row_scale: torch.Tensor, codes=None) -> LMHead:
    """An FP8 head from row-major E4M3 codes uint8 [rows, cols] and fp32 row scales [rows]: the
    codes are moved into the library's tile-major layout (lmhead_fp8_tile_major)."""
    _need(codes_rowmajor, "codes_rowmajor", torch.uint8, 2)
    _need(row_scale, "row_scale", torch.float32, 1)
    rows, cols = codes_rowmajor.shape
    n = lmhead_fp8_codes_bytes(rows, cols)
    if codes is None:
        codes = torch.empty(n, dtype=torch.uint8, device=codes_rowmajor.device)
    src = LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE, rows, cols, _p(codes_rowmajor), _p(row_scale))
    d = LMHeadDesc()
    st = lib().lmhead_fp8_tile_major(C.byref(src), _p(codes), codes.numel(), C.byref(d),
                                     _stream(codes_rowmajor.device))
    check("lmhead_fp8_tile_major", st)
    return LMHead(codes, row_scale, d)


def fp8_codes_rowmajor(head: LMHead) -> torch.Tensor:
    """The E4M3 codes of an FP8 head as uint8 [rows, cols], row-major (a copy, on the head's
    device): tile t of 16 rows starts at byte 16 t cols and holds chunk c (16 codes) of its row i
    at byte 16 (16 c + i)."""
    rows, cols = head.desc.rows, head.desc.cols
    tiles = (rows + 15) // 16
    t = head.w[:tiles * 16 * cols].view(tiles, cols // 16, 16, 16)   # tile, chunk, row, byte
    return t.permute(0, 2, 1, 3).reshape(tiles * 16, cols)[:rows].contiguous()


def _gemv(fn: str, head: LMHead, x: torch.Tensor, out):
    _need(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, head.rows), dtype=torch.float32, device=x.device)
    st = getattr(lib(), fn)(C.byref(head.desc), _p(x), M, _p(out), _stream(x.device))
    check(fn, st)
    return out


def lmhead_gemv_fp8(head: LMHead, x: torch.Tensor, out=None) -> torch.Tensor:
    return _gemv("lmhead_gemv_fp8", head, x, out)


def lmhead_gemv_bf16(head: LMHead, x: torch.Tensor, out=None) -> torch.Tensor:
    return _gemv("lmhead_gemv_bf16", head, x, out)


# ----------------------------------------------------------------------------------- run-time specialisation
def _enc(path):
    return None if path is None else os.fsencode(path)


def lmhead_gemv_fp8_rtc(head: LMHead, x: torch.Tensor, out=None, cache_dir=None) -> torch.Tensor:
    """lmhead_gemv_fp8 compiled at run time for this head's shape, M and the device (hipRTC), with
    the code object cached in `cache_dir` ($QWS_RTC_CACHE or ~/.cache/qws_rtc when None)."""
    _need(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, head.rows), dtype=torch.float32, device=x.device)
    st = lib().lmhead_gemv_fp8_rtc(C.byref(head.desc), _p(x), M, _p(out), _enc(cache_dir), _stream(x.device))
    check("lmhead_gemv_fp8_rtc", st)
    return out


def rtc_compile_head_fp8(M: int, rows: int, cols: int, arch: str = "gfx950", cache_dir=None) -> None:
    """Compile (or find cached) the run-time-specialised FP8 head GEMV without a device."""
    check("qws_rtc_compile_head_fp8", lib().qws_rtc_compile_head_fp8(M, rows, cols, arch.encode(), _enc(cache_dir)))


def rtc_compile_moe(M: int, K: int, E: int, hidden: int, inter: int, has_shared: bool = True, w4a8: bool = False,
                    arch: str = "gfx950", cache_dir=None) -> None:
    """Compile (or find in the disk cache) the fused MoE kernel for a shape; needs no GPU."""
    check("qws_rtc_compile_moe", lib().qws_rtc_compile_moe(M, K, E, hidden, inter, int(has_shared), int(w4a8),
                                                           arch.encode(), _enc(cache_dir)))


def rtc_stats() -> dict:
    s = _lib.RtcStats()
    check("qws_rtc_stats_get", lib().qws_rtc_stats_get(C.byref(s)))
    return {k: getattr(s, k) for k, _ in _lib.RtcStats._fields_}


def rtc_reset() -> None:
    """Unload the run-time-compiled modules and zero the counters (the disk cache stays)."""
    check("qws_rtc_reset", lib().qws_rtc_reset())


def verify_workspace(M: int, device) -> torch.Tensor:
    """Zero-filled workspace of lmhead_verify_greedy_fp8 for windows of up to M positions."""
    n = int(lib().lmhead_verify_workspace_bytes(M))
    if n == 0:
        raise QwsError("lmhead_verify_workspace_bytes", _lib.QWS_ERR_SHAPE)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def lmhead_verify_greedy_fp8(head: LMHead, x: torch.Tensor, draft: torch.Tensor | None, workspace: torch.Tensor,
                             logits: torch.Tensor | None = None, out: dict | None = None) -> dict:
    """Greedy verification of an M-position window: {"target": int32 [M], "emitted": int32 [M],
    "n": int32 [1]} (device tensors; reused from `out` when given), logits into `logits` if given."""
    _need(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    dev = x.device
    if out is None:
        out = {k: torch.empty(n, dtype=torch.int32, device=dev) for k, n in (("target", M), ("emitted", M), ("n", 1))}
    if draft is not None and (draft.dtype != torch.int32 or draft.numel() != M - 1 or draft.device != dev):
        raise ValueError("draft: int32 [M - 1] on the device of x")
    st = lib().lmhead_verify_greedy_fp8(C.byref(head.desc), _p(x), M, None if draft is None else _p(draft),
                                        None if logits is None else _p(logits), _p(out["target"]), _p(out["emitted"]),
                                        _p(out["n"]), _p(workspace), workspace.numel(), _stream(dev))
    check("lmhead_verify_greedy_fp8", st)
    return out


def lmhead_verify_greedy_fp8_noalloc(head: LMHead, x: torch.Tensor, draft: torch.Tensor | None,
                                     logits: torch.Tensor | None = None, out: dict | None = None) -> dict:
    """lmhead_verify_greedy_fp8 with the library's own device scratch instead of a workspace: no
    allocation on the library's side (outputs come from `out` when given, else are allocated here
    by torch). Calls that overlap in time on one GPU race."""
    _need(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    dev = x.device
    if out is None:
        out = {k: torch.empty(n, dtype=torch.int32, device=dev) for k, n in (("target", M), ("emitted", M), ("n", 1))}
    if draft is not None and (draft.dtype != torch.int32 or draft.numel() != M - 1 or draft.device != dev):
        raise ValueError("draft: int32 [M - 1] on the device of x")
    st = lib().lmhead_verify_greedy_fp8_noalloc(C.byref(head.desc), _p(x), M, None if draft is None else _p(draft),
                                                None if logits is None else _p(logits), _p(out["target"]),
                                                _p(out["emitted"]), _p(out["n"]), _stream(dev))
    check("lmhead_verify_greedy_fp8_noalloc", st)
    return out


def lmhead_verify_sample_fp8(head: LMHead, x: torch.Tensor, draft: torch.Tensor | None, u: torch.Tensor,
                             workspace: torch.Tensor, temperature: float = 0.6, top_k: int = 29, top_p: float = 0.95,
                             logits: torch.Tensor | None = None, topk: bool = False, out: dict | None = None) -> dict:
    """Sampled verification of an M-position window with one uniform u[m] in [0, 1) per position:
    {"token": int32 [M], "emitted": int32 [M], "n": int32 [1], "logits": fp32 [M, rows] and, with
    topk=True, "topk": int32 [M, top_k] (rows in order)} (device tensors; reused from `out`)."""
    _need(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    dev = x.device
    if out is None:
        out = {k: torch.empty(n, dtype=torch.int32, device=dev) for k, n in (("token", M), ("emitted", M), ("n", 1))}
        if topk:
            out["topk"] = torch.empty((M, top_k), dtype=torch.int32, device=dev)
    if logits is None:
        logits = out.get("logits")
    if logits is None:
        logits = torch.empty((M, head.rows), dtype=torch.float32, device=dev)
    out["logits"] = logits
    if draft is not None and (draft.dtype != torch.int32 or draft.numel() != M - 1 or draft.device != dev):
        raise ValueError("draft: int32 [M - 1] on the device of x")
    if u.dtype != torch.float32 or u.numel() != M or u.device != dev:
        raise ValueError("u: float32 [M] on the device of x")
    tk = out.get("topk")
    st = lib().lmhead_verify_sample_fp8(C.byref(head.desc), _p(x), M, None if draft is None else _p(draft),
                                        float(temperature), int(top_k), float(top_p), _p(u), _p(logits),
                                        _p(out["token"]), None if tk is None else _p(tk), _p(out["emitted"]),
                                        _p(out["n"]), _p(workspace), workspace.numel(), _stream(dev))
    check("lmhead_verify_sample_fp8", st)
    return out


# ----------------------------------------------------------------------------------- diagnostics
def debug_dequant_mxfp4(q: torch.Tensor, s: torch.Tensor, path: int = 0) -> torch.Tensor:
    _need(q, "q", torch.uint8, 2)
    _need(s, "s", torch.uint8, 2)
    rows, cols = q.shape[0], q.shape[1] * 2
    out = torch.empty((rows, cols), dtype=torch.float32, device=q.device)
    check("qws_debug_dequant_mxfp4", lib().qws_debug_dequant_mxfp4(_p(q), _p(s), rows, cols, path, _p(out),
                                                                    _stream(q.device)))
    return out


def debug_dequant_fp8(head: LMHead) -> torch.Tensor:
    out = torch.empty((head.desc.rows, head.desc.cols), dtype=torch.float32, device=head.w.device)
    check("qws_debug_dequant_fp8", lib().qws_debug_dequant_fp8(C.byref(head.desc), _p(out), _stream(head.w.device)))
    return out


def debug_w4a8_act_buffer(buf) -> None:
    """Register (or, with None, unregister) a uint8 device buffer for the W4A8 layer's activations,
    codes and scales (layout in include/qws.h); diagnostics only."""
    check("qws_debug_w4a8_act_buffer",
          lib().qws_debug_w4a8_act_buffer(_p(buf), 0 if buf is None else buf.numel() * buf.element_size()))


def debug_trace_buffer(buf) -> None:
    """Register (or, with None, unregister) a device buffer for fused-launch phase timestamps."""
    check("qws_debug_trace_buffer", lib().qws_debug_trace_buffer(_p(buf), 0 if buf is None else buf.numel() * buf.element_size()))


def probe_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    check("qws_probe_read", lib().qws_probe_read(_p(buf), buf.numel() * buf.element_size(), _p(sink), blocks,
                                                 _stream(buf.device)))


def probe_read_nt(buf: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    check("qws_probe_read_nt", lib().qws_probe_read_nt(_p(buf), buf.numel() * buf.element_size(), _p(sink), blocks,
                                                       _stream(buf.device)))


def probe_copy(src: torch.Tensor, dst: torch.Tensor, blocks: int) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("probe_copy: dst smaller than src")
    check("qws_probe_copy", lib().qws_probe_copy(_p(src), _p(dst), nbytes, blocks, _stream(src.device)))
