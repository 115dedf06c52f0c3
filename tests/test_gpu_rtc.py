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
