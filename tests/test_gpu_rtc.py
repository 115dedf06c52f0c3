"""GPU parity of the run-time-specialised FP8 head GEMV (lmhead_gemv_fp8_rtc): against the oracle
(max|err|/max|ref| <= 2e-3 and the argmax rule), and the same logits as the library's template
build, bit for bit, for ragged small heads, every M and the full 157,184 x 2,560 head; the
code-object cache is used as stated (compile once, then the loaded module, then the disk after the
modules are dropped)."""
import numpy as np
import pytest
import torch

import quantized_weight_streaming_amd as qws
import synth
from quantized_weight_streaming_amd import _lib

from oracle import lmhead as OL

from .helpers import assert_close, bf16, check_argmax, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(1, 32), (999, 96), (5000, 544), (2049, 2560)])
def test_rtc_equals_template(tmp_path, rows, cols):
    say("rtc small", rows, cols)
    w = synth.bf16_normal(14, 0, synth.HEAD, rows + cols, (rows, cols), 0.02)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    codes, scales = OL.fp8_rowquant(w)
    for M in (1, 2, 3, 4):
        x = synth.token_vectors(14, M, M, cols)
        xt = bf16(x)
        a = qws.lmhead_gemv_fp8(h8, xt).cpu().numpy()
        b = qws.lmhead_gemv_fp8_rtc(h8, xt, cache_dir=str(tmp_path)).cpu().numpy()
        assert_close(b, OL.lmhead_fp8(codes, scales, x), what=f"rtc head {rows}x{cols} M={M}")
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"M = {M}"


def test_rtc_cache_levels(tmp_path):
    say("rtc cache levels")
    rows, cols = 3001, 256
    h8 = qws.lmhead_quantize_fp8(bf16(synth.bf16_normal(15, 0, synth.HEAD, 0, (rows, cols), 0.02)))
    xt = bf16(synth.token_vectors(15, 0, 2, cols))
    d = str(tmp_path)
    qws.rtc_reset()
    want = qws.lmhead_gemv_fp8(h8, xt)
    for expect in (dict(compiles=1, disk_hits=0, memory_hits=0), dict(compiles=1, disk_hits=0, memory_hits=1)):
        got = qws.lmhead_gemv_fp8_rtc(h8, xt, cache_dir=d)
        torch.cuda.synchronize()
        s = qws.rtc_stats()
        assert {k: s[k] for k in expect} == expect
        assert torch.equal(got, want)
    qws.rtc_reset()   # modules dropped: the next call reads the disk cache
    got = qws.lmhead_gemv_fp8_rtc(h8, xt, cache_dir=d)
    torch.cuda.synchronize()
    s = qws.rtc_stats()
    assert (s["compiles"], s["disk_hits"], s["memory_hits"]) == (0, 1, 0)
    assert torch.equal(got, want)


def test_rtc_full_head(tmp_path):
    say("rtc full head")
    w = synth.head_weights(0)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    codes, scales = OL.fp8_rowquant(w)
    for M in (1, 4):
        x = synth.token_vectors(0, 20 + M, M)
        xt = bf16(x)
        a = qws.lmhead_gemv_fp8(h8, xt).cpu().numpy()
        b = qws.lmhead_gemv_fp8_rtc(h8, xt, cache_dir=str(tmp_path)).cpu().numpy()
        ref = OL.lmhead_fp8(codes, scales, x)
        assert_close(b, ref, what=f"rtc full head M={M}")
        assert check_argmax(b, ref) > 0
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"M = {M}"


def test_rtc_refuses_a_bf16_head():
    w = bf16(synth.bf16_normal(16, 0, synth.HEAD, 0, (64, 64), 0.02))
    hb = qws.lmhead_bf16(w)
    with pytest.raises(qws.QwsError) as e:
        qws.lmhead_gemv_fp8_rtc(hb, bf16(synth.token_vectors(16, 0, 1, 64)))
    assert e.value.status == _lib.QWS_ERR_FORMAT


# ------------------------------------------------------------------------------ fused MoE layers
def _rtc_layers(M, shape, seed, n=3):
    from .helpers import Layer
    from .test_gpu_fused import _packed
    layers = [Layer(seed, l, shape, M) for l in range(n)]
    return layers, [qws.MoeLayer(t.x_t, t.wr_t, _packed(t), shape.topk) for t in layers]


@pytest.mark.parametrize("M,w4a8", [(1, False), (1, True), (4, False), (4, True), (2, False)])
def test_moe_rtc_equals_template(tmp_path, M, w4a8):
    """The run-time-compiled fused kernel (shape as constants) gives the template build's outputs
    bit for bit, three layers in one launch; its first layer also against the oracle."""
    from .test_gpu_fused import _check_layer
    from .test_gpu_w4a8 import _act_buffer, _check_w4a8
    say("rtc moe M", M, "w4a8", w4a8)
    shape = synth.LayerShape()
    layers, Ls = _rtc_layers(M, shape, 60 + M)
    _, Lt = _rtc_layers(M, shape, 60 + M)
    ws = qws.moe_layer_workspace(M, 8, 512, 2560, 768, "cuda")
    qws.MoeLayers(Lt).run(ws, w4a8=w4a8)
    qws.MoeLayers(Ls).run(ws, w4a8=w4a8, rtc=True, cache_dir=str(tmp_path))
    torch.cuda.synchronize()
    for a, b in zip(Lt, Ls):
        assert np.array_equal(a.y_f32.cpu().numpy().view(np.uint32), b.y_f32.cpu().numpy().view(np.uint32))
        assert np.array_equal(a.topk_idx.cpu().numpy(), b.topk_idx.cpu().numpy())
        assert np.array_equal(a.topk_w.cpu().numpy().view(np.uint32), b.topk_w.cpu().numpy().view(np.uint32))
    assert qws.moe_workspace_errors(ws, M, 8, 512, 768) == 0
    # the first layer alone through the run-time path, against the oracle (W4A8: with the
    # activation record, as in the template tests)
    L0 = qws.MoeLayer(layers[0].x_t, layers[0].wr_t, Ls[0].bank, 8,
                      logits_out=torch.empty((M, 512), dtype=torch.float32, device="cuda"))
    buf = _act_buffer(shape, M) if w4a8 else None
    qws.debug_w4a8_act_buffer(buf)
    try:
        qws.MoeLayers([L0]).run(ws, w4a8=w4a8, rtc=True, cache_dir=str(tmp_path))
        torch.cuda.synchronize()
    finally:
        qws.debug_w4a8_act_buffer(None)
    if w4a8:
        _check_w4a8(layers[0], L0, buf.cpu().numpy())
    else:
        _check_layer(layers[0], L0)


def test_moe_rtc_small_shape_and_cache_levels(tmp_path):
    """A small shape (64 experts, H 544, I 1024, top-8) through the run-time path: oracle parity,
    then the loaded module serves the next call, and after the modules are dropped the disk."""
    from .test_gpu_fused import _check_layer
    say("rtc moe small shape, cache levels")
    shape = synth.LayerShape(hidden=544, inter=1024, n_routed=64)
    layers, Ls = _rtc_layers(2, shape, 70, n=1)
    ws = qws.moe_layer_workspace(2, 8, 64, 544, 1024, "cuda")
    qws.rtc_reset()
    seq = qws.MoeLayers(Ls)
    for expect in ((1, 0, 0), (1, 0, 1)):
        seq.run(ws, rtc=True, cache_dir=str(tmp_path))
        torch.cuda.synchronize()
        s = qws.rtc_stats()
        assert (s["compiles"], s["disk_hits"], s["memory_hits"]) == expect
    qws.rtc_reset()
    L1 = qws.MoeLayer(layers[0].x_t, layers[0].wr_t, Ls[0].bank, 8,
                      logits_out=torch.empty((2, 64), dtype=torch.float32, device="cuda"))
    qws.MoeLayers([L1]).run(ws, rtc=True, cache_dir=str(tmp_path))
    torch.cuda.synchronize()
    s = qws.rtc_stats()
    assert (s["compiles"], s["disk_hits"], s["memory_hits"]) == (0, 1, 0)
    _check_layer(layers[0], L1)
    assert qws.moe_workspace_errors(ws, 2, 8, 64, 1024) == 0
