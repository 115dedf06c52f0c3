"""Pins for oracle.lmhead: one-hot inputs give the dequantised column exactly, exactly rounded
bf16 dot products (math.fsum), quantiser invariants and error bounds, a pure-Python quantiser at
a tiny shape, and the pages' printed head sizes."""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import lmhead


def _head(rows, cols, seed=0, sigma=0.02):
    return synth.bf16_normal(seed, 0, synth.HEAD, 0, (rows, cols), sigma)


def test_quantiser_pure_python_tiny():
    w = _head(7, 64, seed=2)
    codes, scales = lmhead.fp8_rowquant(w)
    wf = F.bf16_to_f32(w)
    for r in range(7):
        a = max(abs(float(v)) for v in wf[r])
        s = np.float32(np.float32(a) / np.float32(448.0))
        assert scales[r] == s
        for k in range(64):
            v = float(np.float32(wf[r, k]) / s)
            assert codes[r, k] == F.e4m3_encode_scalar(v)


def test_quantiser_invariants():
    w = _head(300, 256, seed=4)
    codes, scales = lmhead.fp8_rowquant(w)
    wf = F.bf16_to_f64(w)
    am = np.argmax(np.abs(wf), axis=1)
    top = codes[np.arange(300), am]
    assert np.all((top & 0x7F) == 0x7E)                       # each row's absmax element -> +-448
    deq = F.e4m3_table()[codes] * scales[:, None].astype(np.float64)
    v = wf / scales[:, None].astype(np.float64)
    nrm = np.abs(v) >= 2.0 ** -6
    err = np.abs(deq - wf)
    # half an E4M3 step, plus the two float32 roundings (division, scale) around it
    slack = 2.0 ** -22 * np.abs(wf)
    assert np.all(err[nrm] <= 2.0 ** -4 * np.abs(wf[nrm]) + slack[nrm])
    sub_bound = (2.0 ** -10) * np.broadcast_to(scales[:, None].astype(np.float64), wf.shape)
    assert np.all(err[~nrm] <= sub_bound[~nrm] + slack[~nrm])


def test_zero_row_and_tiny_row():
    w = np.zeros((3, 32), dtype=np.uint16)
    w[1, 5] = synth.f32_to_bf16_bits(np.array([3.0e-38], dtype=np.float32))[0]
    w[2] = synth.f32_to_bf16_bits(np.linspace(-1, 1, 32).astype(np.float32))
    codes, scales = lmhead.fp8_rowquant(w)
    assert scales[0] == 1.0 and np.all(codes[0] == 0)
    assert scales[1] > 0 and codes[1, 5] == 0x7E and np.all(np.delete(codes[1], 5) == 0)
    assert codes[2, 0] == 0xFE and codes[2, 31] == 0x7E


def test_one_hot_input_gives_dequantised_column():
    w = _head(500, 128, seed=6)
    codes, scales = lmhead.fp8_rowquant(w)
    for k in (0, 17, 127):
        x = np.zeros((1, 128), dtype=np.uint16)
        x[0, k] = 0x3F80                                       # bf16 1.0
        got = lmhead.lmhead_fp8(codes, scales, x)[0]
        want = F.e4m3_table()[codes[:, k]] * scales.astype(np.float64)
        assert np.array_equal(got, want)
        assert np.array_equal(lmhead.lmhead_bf16(w, x)[0], F.bf16_to_f64(w[:, k]))


def test_bf16_head_is_exactly_rounded_dot():
    w = _head(20, 96, seed=7)
    x = synth.token_vectors(7, 0, 2, 96)
    got = lmhead.lmhead_bf16(w, x)
    wf, xf = F.bf16_to_f64(w), F.bf16_to_f64(x)
    for m in range(2):
        for r in range(20):
            want = math.fsum(float(wf[r, k]) * float(xf[m, k]) for k in range(96))
            assert abs(got[m, r] - want) <= 4e-16 * math.fsum(abs(float(wf[r, k]) * float(xf[m, k])) for k in range(96))


def test_fp8_head_brute_force_and_row_subset():
    w = _head(40, 64, seed=8)
    codes, scales = lmhead.fp8_rowquant(w)
    x = synth.token_vectors(8, 0, 3, 64)
    got = lmhead.lmhead_fp8(codes, scales, x)
    xf = F.bf16_to_f64(x)
    for m in range(3):
        for r in range(40):
            want = float(scales[r]) * math.fsum(F.e4m3_value(int(codes[r, k])) * float(xf[m, k]) for k in range(64))
            assert abs(got[m, r] - want) <= 1e-14 * max(1e-30, abs(want)) + 1e-300
    rows = np.array([39, 2, 17])
    assert np.array_equal(lmhead.lmhead_fp8(codes, scales, x, rows), got[:, rows])


def test_head_is_linear_in_x():
    w = _head(64, 64, seed=9)
    codes, scales = lmhead.fp8_rowquant(w)
    x1 = np.zeros((1, 64), dtype=np.uint16)
    x2 = np.zeros((1, 64), dtype=np.uint16)
    x1[0, :32] = synth.token_vectors(9, 0, 1, 32)[0]
    x2[0, 32:] = synth.token_vectors(9, 1, 1, 32)[0]
    x12 = x1 | x2                                               # disjoint supports: exact sum
    l1, l2, l12 = (lmhead.lmhead_fp8(codes, scales, x) for x in (x1, x2, x12))
    assert np.allclose(l12, l1 + l2, rtol=1e-13, atol=1e-15)


def test_fp8_dequant_is_float32_product():
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    scales = np.array([0.013, 3.7e-5], dtype=np.float32)
    d = lmhead.fp8_dequant(codes, scales)
    assert d.dtype == np.float32
    want = np.array([[np.float32(F.e4m3_value(int(c))) * scales[r] for c in codes[r]] for r in range(2)], dtype=np.float32)
    assert np.array_equal(d, want)


def test_agreement_metric():
    a = np.array([[0.0, 3.0, 1.0, 2.0], [5.0, 1.0, 1.0, 0.0]])
    b = np.array([[0.0, 2.0, 1.0, 3.0], [5.0, 0.0, 2.0, 1.0]])
    r = lmhead.topk_agreement(a, b, k=2)
    assert r["top1"] == 0.5 and r["topk_overlap"] == 0.75 and r["top1_in_topk"] == 1.0


def test_page_head_figures(golden_dir):
    with open(os.path.join(golden_dir, "page_figures.json")) as f:
        fig = {d["what"]: d for d in json.load(f)["figures"]}
    v, h = synth.VOCAB, synth.HIDDEN
    assert v == fig["vocabulary"]["value"] and h == fig["hidden size"]["value"]
    for what, got in (("LM-head weights, 'roughly 402 million'", v * h),
                      ("LM-head bf16 bytes per token, 'about 805 MB'", 2 * v * h),
                      ("LM-head FP8 bytes per token, 'roughly 400 MB'", v * h)):
        d = fig[what]
        assert abs(got - d["approx"]) <= d["rel_tol"] * d["approx"], what
    assert synth.INTER == fig["moe_intermediate_size"]["value"]
    assert synth.TOPK == fig["routed experts per token"]["value"]
    assert synth.N_LAYERS == fig["layers"]["value"]
    assert synth.TOPK * 4 == fig["experts a four-position verification pass can touch"]["value"]
    assert synth.LayerShape().n_routed == fig["routed experts per layer"]["value"]
