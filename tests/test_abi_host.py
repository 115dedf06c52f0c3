"""The C-ABI library without a GPU: it loads, exports every entry point include/qws.h declares,
and its host-side validation returns the documented status before anything is enqueued. All
pointers here are fake; every call below is refused by validation, so none reaches HIP."""
import ctypes as C
import os
import re

import pytest

from quantized_weight_streaming_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qws.h")

A = 0x10000          # a fake, 16-byte aligned device address (never dereferenced)
MIS = 0x10008        # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\*|int|size_t)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqws.so not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strerror(lib):
    assert lib.qws_abi_version() == 1
    for st in range(0, -8, -1):
        assert lib.qws_strerror(st)
    assert b"format" in lib.qws_strerror(_lib.QWS_ERR_FORMAT)


def test_workspace_sizes(lib):
    assert lib.moe_route_workspace_bytes(1, 512) >= 512 * 4
    assert lib.moe_route_workspace_bytes(0, 512) == 0
    assert lib.moe_route_workspace_bytes(5, 512) == 0
    assert lib.moe_route_workspace_bytes(1, 1025) == 0
    w1 = lib.moe_expert_workspace_bytes(1, 8, 2560, 768)
    w4 = lib.moe_expert_workspace_bytes(4, 8, 2560, 768)
    assert 0 < w1 < w4
    assert w4 >= 33 * 4 * (2560 + 768) * 4
    assert lib.moe_expert_workspace_bytes(1, 9, 2560, 768) == 0
    assert lib.moe_expert_workspace_bytes(1, 8, 4096, 768) == 0


def _route(lib, **kw):
    a = dict(x=A, M=1, H=2560, w=A, E=512, bias=None, stride=0, K=8, idx=A, tw=A, logits=None, ws=A,
             wsb=lib.moe_route_workspace_bytes(1, 512), stream=None)
    a.update(kw)
    return lib.moe_route_topk(a["x"], a["M"], a["H"], a["w"], a["E"], a["bias"], a["stride"], a["K"], a["idx"],
                              a["tw"], a["logits"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.QWS_ERR_ARG), (dict(idx=None), _lib.QWS_ERR_ARG),
    (dict(M=0), _lib.QWS_ERR_SHAPE), (dict(M=5), _lib.QWS_ERR_SHAPE), (dict(H=2568), _lib.QWS_ERR_SHAPE),
    (dict(H=100), _lib.QWS_ERR_SHAPE), (dict(E=0), _lib.QWS_ERR_SHAPE), (dict(E=1025), _lib.QWS_ERR_SHAPE),
    (dict(K=0), _lib.QWS_ERR_SHAPE), (dict(K=9), _lib.QWS_ERR_SHAPE), (dict(E=4, K=5), _lib.QWS_ERR_SHAPE),
    (dict(bias=A, stride=7), _lib.QWS_ERR_SHAPE), (dict(x=MIS), _lib.QWS_ERR_ALIGN),
    (dict(w=MIS), _lib.QWS_ERR_ALIGN), (dict(ws=None), _lib.QWS_ERR_WORKSPACE), (dict(wsb=16), _lib.QWS_ERR_WORKSPACE),
])
def test_route_validation(lib, kw, status):
    assert _route(lib, **kw) == status


def _bank(**kw):
    d = dict(format=_lib.QWS_FMT_MXFP4_E2M1_E8M0_B32, n_routed=512, has_shared=1, hidden=2560, inter=768,
             gate_up_q=A, gate_up_s=A, down_q=A, down_s=A)
    d.update(kw)
    return _lib.MxFp4Experts(**d)


def _experts(lib, bank=None, **kw):
    a = dict(x=A, M=1, idx=A, tw=A, K=8, y16=A, y32=A, ws=A, wsb=lib.moe_expert_workspace_bytes(1, 8, 2560, 768))
    a.update(kw)
    b = bank if bank is not None else _bank()
    return lib.moe_expert_gemv_mxfp4(C.byref(b), a["x"], a["M"], a["idx"], a["tw"], a["K"], a["y16"], a["y32"],
                                     a["ws"], a["wsb"], None)


@pytest.mark.parametrize("bank_kw,kw,status", [
    (dict(format=_lib.QWS_FMT_BF16), {}, _lib.QWS_ERR_FORMAT),
    (dict(format=_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE), {}, _lib.QWS_ERR_FORMAT),
    (dict(down_s=None), {}, _lib.QWS_ERR_ARG), (dict(has_shared=2), {}, _lib.QWS_ERR_ARG),
    ({}, dict(y16=None, y32=None), _lib.QWS_ERR_ARG), ({}, dict(idx=None), _lib.QWS_ERR_ARG),
    (dict(hidden=2592), {}, _lib.QWS_ERR_SHAPE), (dict(hidden=48), {}, _lib.QWS_ERR_SHAPE),
    (dict(inter=1056), {}, _lib.QWS_ERR_SHAPE), (dict(n_routed=0), {}, _lib.QWS_ERR_SHAPE),
    ({}, dict(M=5), _lib.QWS_ERR_SHAPE), ({}, dict(K=9), _lib.QWS_ERR_SHAPE),
    (dict(gate_up_q=MIS), {}, _lib.QWS_ERR_ALIGN), ({}, dict(x=MIS), _lib.QWS_ERR_ALIGN),
    ({}, dict(wsb=1024), _lib.QWS_ERR_WORKSPACE), ({}, dict(ws=None), _lib.QWS_ERR_WORKSPACE),
])
def test_expert_validation(lib, bank_kw, kw, status):
    assert _experts(lib, _bank(**bank_kw), **kw) == status


def test_expert_workspace_for_larger_window_is_required(lib):
    # a workspace sized for M = 1 is refused for M = 4
    assert _experts(lib, M=4) == _lib.QWS_ERR_WORKSPACE


def test_lmhead_format_tags_refuse_mismatched_heads(lib):
    fp8 = _lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, 157184, 2560, A, A)
    bf16 = _lib.LMHeadDesc(_lib.QWS_FMT_BF16, 157184, 2560, A, None)
    # an FP8 head handed to the bf16 GEMV is refused instead of being read as bf16, and vice versa
    assert lib.lmhead_gemv_bf16(C.byref(fp8), A, 1, A, None) == _lib.QWS_ERR_FORMAT
    assert lib.lmhead_gemv_fp8(C.byref(bf16), A, 1, A, None) == _lib.QWS_ERR_FORMAT
    assert lib.qws_debug_dequant_fp8(C.byref(bf16), A, None) == _lib.QWS_ERR_FORMAT
    nos = _lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, 157184, 2560, A, None)
    assert lib.lmhead_gemv_fp8(C.byref(nos), A, 1, A, None) == _lib.QWS_ERR_ARG


def test_row_major_fp8_head_is_refused_by_every_tile_major_reader(lib):
    """The tile layout is part of the format tag: a head whose descriptor says its E4M3 codes are
    row-major is refused by every entry point that reads tiles, instead of giving wrong logits."""
    rm = C.byref(_lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE, 157184, 2560, A, A))
    wsb = lib.lmhead_verify_workspace_bytes(4)
    assert lib.lmhead_gemv_fp8(rm, A, 1, A, None) == _lib.QWS_ERR_FORMAT
    assert lib.lmhead_gemv_fp8_rtc(rm, A, 1, A, None, None) == _lib.QWS_ERR_FORMAT
    assert lib.qws_debug_dequant_fp8(rm, A, None) == _lib.QWS_ERR_FORMAT
    assert lib.lmhead_verify_greedy_fp8(rm, A, 4, A, None, A, A, A, A, wsb, None) == _lib.QWS_ERR_FORMAT
    assert lib.lmhead_verify_sample_fp8(rm, A, 4, A, 0.6, 29, 0.95, A, A, A, None, A, A, A, wsb,
                                        None) == _lib.QWS_ERR_FORMAT
    assert lib.lmhead_gemv_bf16(rm, A, 1, A, None) == _lib.QWS_ERR_FORMAT


def test_fp8_tile_major_validation(lib):
    rows, cols = 100, 64
    need = lib.lmhead_fp8_codes_bytes(rows, cols)
    out = _lib.LMHeadDesc()
    src = _lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE, rows, cols, A, A)
    far = A + (1 << 24)
    call = lambda s, o=far, n=need, d=C.byref(out): lib.lmhead_fp8_tile_major(C.byref(s), o, n, d, None)  # noqa: E731
    # only row-major FP8 is converted: tile-major or bf16 sources are refused
    assert call(_lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, rows, cols, A, A)) == _lib.QWS_ERR_FORMAT
    assert call(_lib.LMHeadDesc(_lib.QWS_FMT_BF16, rows, cols, A, None)) == _lib.QWS_ERR_FORMAT
    assert call(_lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE, rows, cols, A, None)) == _lib.QWS_ERR_ARG
    assert call(_lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE, rows, 48, A, A)) == _lib.QWS_ERR_SHAPE
    assert call(src, n=need - 1) == _lib.QWS_ERR_WORKSPACE
    assert call(src, o=far + 8) == _lib.QWS_ERR_ALIGN
    assert call(src, o=A + 16 * cols) == _lib.QWS_ERR_ARG            # overlaps the source codes
    assert call(src, o=None) == _lib.QWS_ERR_ARG
    assert call(src, d=None) == _lib.QWS_ERR_ARG


@pytest.mark.parametrize("rows,cols,x,M,status", [
    (0, 2560, A, 1, _lib.QWS_ERR_SHAPE), (10, 2592, A, 1, _lib.QWS_ERR_SHAPE), (10, 48, A, 1, _lib.QWS_ERR_SHAPE),
    (10, 2560, A, 0, _lib.QWS_ERR_SHAPE), (10, 2560, A, 5, _lib.QWS_ERR_SHAPE), (10, 2560, MIS, 1, _lib.QWS_ERR_ALIGN),
    (10, 2560, None, 1, _lib.QWS_ERR_ARG),
])
def test_lmhead_gemv_validation(lib, rows, cols, x, M, status):
    d = _lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, rows, cols, A, A)
    assert lib.lmhead_gemv_fp8(C.byref(d), x, M, A, None) == status


def test_lmhead_desc_and_quantize_validation(lib):
    d = _lib.LMHeadDesc()
    assert lib.lmhead_bf16_desc(A, 157184, 2560, C.byref(d)) == _lib.QWS_OK
    assert d.format == _lib.QWS_FMT_BF16 and d.rows == 157184 and d.cols == 2560
    assert lib.lmhead_bf16_desc(MIS, 10, 64, C.byref(d)) == _lib.QWS_ERR_ALIGN
    assert lib.lmhead_bf16_desc(A, 10, 63, C.byref(d)) == _lib.QWS_ERR_SHAPE
    assert lib.lmhead_quantize_fp8(A, 10, 64, A, A, None, None) == _lib.QWS_ERR_ARG
    assert lib.lmhead_quantize_fp8(A, 10, 2600, A, A, C.byref(d), None) == _lib.QWS_ERR_SHAPE
    assert lib.lmhead_quantize_fp8(A, 10, 64, MIS, A, C.byref(d), None) == _lib.QWS_ERR_ALIGN


def test_fp8_codes_bytes(lib):
    # rows padded to whole 16-row tiles; 0 for shapes the head refuses
    assert lib.lmhead_fp8_codes_bytes(157184, 2560) == 157184 * 2560
    assert lib.lmhead_fp8_codes_bytes(1, 32) == 16 * 32
    assert lib.lmhead_fp8_codes_bytes(17, 96) == 32 * 96
    assert lib.lmhead_fp8_codes_bytes(0, 2560) == 0
    assert lib.lmhead_fp8_codes_bytes(10, 48) == 0
    assert lib.lmhead_fp8_codes_bytes(10, 2592) == 0


def test_verify_validation(lib):
    bf = C.byref(_lib.LMHeadDesc(_lib.QWS_FMT_BF16, 100, 64, A, None))
    fp8 = C.byref(_lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, 100, 64, A, A))
    wsb = lib.lmhead_verify_workspace_bytes(4)
    assert wsb > 0 and lib.lmhead_verify_workspace_bytes(0) == 0 and lib.lmhead_verify_workspace_bytes(5) == 0
    ok = dict(head=fp8, x=A, M=4, draft=A, lg=None, t=A, e=A, n=A, ws=A, wsb=wsb)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.lmhead_verify_greedy_fp8(a["head"], a["x"], a["M"], a["draft"], a["lg"], a["t"], a["e"], a["n"],
                                            a["ws"], a["wsb"], None)
    assert call(head=bf) == _lib.QWS_ERR_FORMAT
    assert call(x=None) == _lib.QWS_ERR_ARG
    assert call(draft=None) == _lib.QWS_ERR_ARG
    assert call(t=None) == _lib.QWS_ERR_ARG
    assert call(n=None) == _lib.QWS_ERR_ARG
    assert call(M=0) == _lib.QWS_ERR_SHAPE
    assert call(M=5) == _lib.QWS_ERR_SHAPE
    assert call(x=MIS) == _lib.QWS_ERR_ALIGN
    assert call(ws=MIS) == _lib.QWS_ERR_ALIGN
    assert call(wsb=wsb - 1) == _lib.QWS_ERR_WORKSPACE
    assert call(ws=None) == _lib.QWS_ERR_WORKSPACE


def test_sample_validation(lib):
    bf = C.byref(_lib.LMHeadDesc(_lib.QWS_FMT_BF16, 100, 64, A, None))
    fp8 = C.byref(_lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, 100, 64, A, A))
    big = C.byref(_lib.LMHeadDesc(_lib.QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, 262145, 64, A, A))
    wsb = lib.lmhead_verify_workspace_bytes(4)
    ok = dict(head=fp8, x=A, M=4, draft=A, T=0.6, k=29, p=0.95, u=A, lg=A, tok=A, tk=None, e=A, n=A, ws=A, wsb=wsb)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.lmhead_verify_sample_fp8(a["head"], a["x"], a["M"], a["draft"], a["T"], a["k"], a["p"], a["u"],
                                            a["lg"], a["tok"], a["tk"], a["e"], a["n"], a["ws"], a["wsb"], None)
    assert call(head=bf) == _lib.QWS_ERR_FORMAT
    for name in ("x", "draft", "u", "lg", "tok", "e", "n"):
        assert call(**{name: None}) == _lib.QWS_ERR_ARG, name
    for T in (0.0, -1.0, float("inf"), float("nan")):
        assert call(T=T) == _lib.QWS_ERR_ARG, T
    for p in (0.0, -0.5, 1.5, float("nan")):
        assert call(p=p) == _lib.QWS_ERR_ARG, p
    assert call(k=0) == _lib.QWS_ERR_SHAPE and call(k=33) == _lib.QWS_ERR_SHAPE
    assert call(M=0) == _lib.QWS_ERR_SHAPE and call(M=5) == _lib.QWS_ERR_SHAPE
    assert call(head=big) == _lib.QWS_ERR_SHAPE   # more than 2,048 x 16 x 8 rows
    assert call(x=MIS) == _lib.QWS_ERR_ALIGN and call(ws=MIS) == _lib.QWS_ERR_ALIGN
    assert call(wsb=wsb - 1) == _lib.QWS_ERR_WORKSPACE and call(ws=None) == _lib.QWS_ERR_WORKSPACE


def test_diagnostics_validation(lib):
    assert lib.qws_debug_dequant_mxfp4(A, A, 4, 64, 2, A, None) == _lib.QWS_ERR_ARG
    assert lib.qws_debug_dequant_mxfp4(A, A, 4, 48, 0, A, None) == _lib.QWS_ERR_SHAPE
    assert lib.qws_debug_dequant_mxfp4(MIS, A, 4, 64, 0, A, None) == _lib.QWS_ERR_ALIGN
    assert lib.qws_probe_read(A, 100, A, 4, None) == _lib.QWS_ERR_SHAPE
    assert lib.qws_probe_read(A, 1024, A, 0, None) == _lib.QWS_ERR_SHAPE
    assert lib.qws_probe_read(None, 1024, A, 4, None) == _lib.QWS_ERR_ARG
    assert lib.qws_probe_read_nt(A, 100, A, 4, None) == _lib.QWS_ERR_SHAPE
    assert lib.qws_probe_read_nt(A, 1024, A, 70000, None) == _lib.QWS_ERR_SHAPE
    assert lib.qws_probe_read_nt(None, 1024, A, 4, None) == _lib.QWS_ERR_ARG
    assert lib.qws_probe_read_nt(MIS, 1024, A, 4, None) == _lib.QWS_ERR_ALIGN


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load(str(tmp_path / "missing.so"))


def _packed(**kw):
    return _bank(**{"format": _lib.QWS_FMT_MXFP4_E2M1_E8M0_B32_TASKMAJOR, "gate_up_s": None, "down_q": None,
                    "down_s": None, **kw})


def _layer_desc(**kw):
    d = dict(x_bf16=A, w_router_bf16=A, bias=None, bias_row_stride=0, experts=_packed(), topk_idx=A, topk_w=A,
             logits_out=None, y_bf16=A, y_f32=A)
    d.update(kw)
    return _lib.MoeLayerDesc(**d)


@pytest.mark.parametrize("kw,M,K,wsb,status", [
    (dict(x_bf16=None), 1, 8, None, _lib.QWS_ERR_ARG),
    (dict(y_bf16=None, y_f32=None), 1, 8, None, _lib.QWS_ERR_ARG),
    (dict(experts=_bank(format=_lib.QWS_FMT_BF16)), 1, 8, None, _lib.QWS_ERR_FORMAT),
    (dict(experts=_bank()), 1, 8, None, _lib.QWS_ERR_FORMAT),               # canonical: not packed
    (dict(experts=_packed(gate_up_q=None)), 1, 8, None, _lib.QWS_ERR_ARG),
    ({}, 5, 8, None, _lib.QWS_ERR_SHAPE), ({}, 1, 9, None, _lib.QWS_ERR_SHAPE),
    (dict(experts=_packed(hidden=2592)), 1, 8, None, _lib.QWS_ERR_SHAPE),
    (dict(experts=_packed(n_routed=4)), 1, 8, None, _lib.QWS_ERR_SHAPE),       # E < K
    (dict(bias=A, bias_row_stride=3), 1, 8, None, _lib.QWS_ERR_SHAPE),
    (dict(x_bf16=MIS), 1, 8, None, _lib.QWS_ERR_ALIGN),
    (dict(experts=_packed(gate_up_q=MIS)), 1, 8, None, _lib.QWS_ERR_ALIGN),
    ({}, 1, 8, 64, _lib.QWS_ERR_WORKSPACE),
])
def test_fused_layer_validation(lib, kw, M, K, wsb, status):
    d = _layer_desc(**kw)
    n = lib.moe_layer_workspace_bytes(M, K, 512, 2560, 768) if wsb is None else wsb
    assert lib.moe_layer_mxfp4(C.byref(d), M, K, A, n if n else 1 << 20, None) == status


def test_fused_layers_validation(lib):
    good = _layer_desc()
    bad = _layer_desc(experts=_packed(inter=512))                                 # shapes differ across layers
    arr = (_lib.MoeLayerDesc * 2)(good, bad)
    n = lib.moe_layer_workspace_bytes(1, 8, 512, 2560, 768)
    assert lib.moe_layers_mxfp4(arr, A, 2, 1, 8, A, n, None) == _lib.QWS_ERR_SHAPE
    arr2 = (_lib.MoeLayerDesc * 2)(good, good)
    assert lib.moe_layers_mxfp4(arr2, None, 2, 1, 8, A, n, None) == _lib.QWS_ERR_ARG  # no device copy
    assert lib.moe_layers_mxfp4(arr2, A, 0, 1, 8, A, n, None) == _lib.QWS_ERR_ARG
    # tagged logits, tagged y and the tagged partial sums of M * (K + 1) pairs x I/32 blocks x H rows
    assert lib.moe_layer_workspace_bytes(1, 8, 512, 2560, 768) >= 512 * 8 + 2560 * 4 + 9 * 24 * 2560 * 8
    assert lib.moe_layer_workspace_bytes(5, 8, 512, 2560, 768) == 0
    arr3 = (_lib.MoeLayerDesc * 1025)(*([good] * 1025))
    assert lib.moe_layers_mxfp4(arr3, A, 1025, 1, 8, A, n, None) == _lib.QWS_ERR_SHAPE   # > 1024 layers


def test_expert_gemv_refuses_packed_bank(lib):
    # the two-call path reads the canonical layout only
    assert _experts(lib, _packed()) == _lib.QWS_ERR_FORMAT


def _pack(lib, src=None, dst=A, nbytes=None, out=True):
    o = _lib.MxFp4Experts()
    if nbytes is None:
        nbytes = lib.moe_pack_mxfp4_bytes(513, 2560, 768)
    return lib.moe_pack_mxfp4(C.byref(src if src is not None else _bank()), dst, nbytes, C.byref(o) if out else None,
                              None)


def test_pack_bytes(lib):
    # one 128 KB record per (expert, 32-activation block)
    assert lib.moe_pack_mxfp4_bytes(513, 2560, 768) == 513 * 24 * _lib.QWS_TASK_BYTES == 513 * 24 * 131072
    assert lib.moe_pack_mxfp4_bytes(65, 2560, 768) == 65 * 24 * 131072
    for bad in ((0, 2560, 768), (1026, 2560, 768), (513, 2592, 768), (513, 2560, 48), (513, 48, 768)):
        assert lib.moe_pack_mxfp4_bytes(*bad) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(src=_packed()), _lib.QWS_ERR_FORMAT), (dict(src=_bank(format=_lib.QWS_FMT_BF16)), _lib.QWS_ERR_FORMAT),
    (dict(dst=None), _lib.QWS_ERR_ARG), (dict(out=False), _lib.QWS_ERR_ARG),
    (dict(src=_bank(down_s=None)), _lib.QWS_ERR_ARG), (dict(src=_bank(has_shared=3)), _lib.QWS_ERR_ARG),
    (dict(src=_bank(n_routed=0)), _lib.QWS_ERR_SHAPE), (dict(src=_bank(hidden=2592)), _lib.QWS_ERR_SHAPE),
    (dict(src=_bank(inter=48)), _lib.QWS_ERR_SHAPE), (dict(dst=MIS), _lib.QWS_ERR_ALIGN),
    (dict(nbytes=513 * 24 * 131072 - 16), _lib.QWS_ERR_WORKSPACE),
])
def test_pack_validation(lib, kw, status):
    assert _pack(lib, **kw) == status



def test_load_switches_to_another_build(tmp_path):
    import shutil
    default = _lib.load()
    assert _lib.load() is default and _lib.load(_lib.LIB_PATH) is default
    copy = str(tmp_path / "libqws_copy.so")
    shutil.copy(_lib.LIB_PATH, copy)
    try:
        other = _lib.load(copy)
        assert other is not default and _lib.load() is other      # later calls use the named build
        assert other.qws_abi_version() == default.qws_abi_version()
    finally:
        _lib.load(_lib.LIB_PATH)
    assert _lib.load() is not other


def test_header_is_plain_c(tmp_path):
    """include/qws.h compiles as C99 (no C++ or HIP types in the boundary) and as C++17."""
    import shutil
    import subprocess
    src = tmp_path / "use.c"
    src.write_text('#include "qws.h"\nint main(void) { qws_lmhead h; qws_rtc_stats s; (void)h; (void)s;'
                   ' return qws_abi_version() == 0; }\n')
    inc = os.path.join(ROOT, "include")
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not installed")
        lang = ["-x", "c++"] if cc == "g++" else []
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", inc, *lang, str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
