"""Pins of the W4A8 oracle (oracle/w4a8.py) against what the MX and E4M3 definitions fix: hand-worked
MXFP8 blocks, exact round trips of representable blocks, the round-to-nearest error bound, a
brute-force scalar layer at a tiny shape, and closeness to the bf16 layer."""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import moe as OM
from oracle import w4a8 as W


def _blocks(golden_dir):
    with open(os.path.join(golden_dir, "mxfp8_blocks.json")) as f:
        return json.load(f)["blocks"]


def test_mxfp8_worked_blocks(golden_dir):
    blocks = _blocks(golden_dir)
    v = np.zeros((len(blocks), 32))
    for b, blk in enumerate(blocks):
        for k, (val, _, _) in blk["elements"].items():
            v[b, int(k)] = float.fromhex(val)
    codes, scales = W.mxfp8_quantize(v.reshape(-1))
    codes = codes.reshape(len(blocks), 32)
    for b, blk in enumerate(blocks):
        assert int(scales[b]) == blk["scale_byte"], blk["why"]
        want = np.zeros(32, np.uint8)
        for k, (_, code, _) in blk["elements"].items():
            want[int(k)] = int(code, 16)
        assert list(codes[b]) == list(want), blk["why"]


def test_mxfp8_roundtrip_of_representable_blocks():
    """A block whose largest code has exponent field 15 (values 256 .. 448) and any scale byte
    re-quantises to the same codes and scale: the conversion picks floor(log2 max) - 8."""
    rng = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    for _ in range(200):
        codes = rng.choice(finite, 32)
        top = rng.integers(0, 32)
        codes[top] = (rng.integers(0, 2) << 7) | (15 << 3) | rng.integers(0, 7)   # 256 .. 448 in magnitude
        s = np.array([rng.integers(1, 255)], np.uint8)
        v = W.mxfp8_dequant(codes, s)
        c2, s2 = W.mxfp8_quantize(v)
        assert int(s2[0]) == int(s[0])
        assert np.array_equal(W.mxfp8_dequant(c2, s2), v)   # equal values (+0 and -0 may swap codes)


@pytest.mark.parametrize("spread", [1.0, 8.0])
def test_mxfp8_rounding_error_bound(spread):
    """Round to nearest: within half an E4M3 step of v / X, the step being 2^(floor(log2|v/X|) - 3)
    for normals and 2^-9 below 2^-6; only magnitudes past 448 (clamped) may be further."""
    rng = np.random.default_rng(int(spread))
    v = rng.standard_normal((64, 256)) * np.exp(spread * rng.standard_normal((64, 256)))
    q = W.mxfp8_round(v)
    X = np.repeat(np.ldexp(1.0, W.mxfp8_scale_exponents(v)), 32, axis=-1)
    a = np.abs(v) / X
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, np.floor(np.log2(np.maximum(a, 2.0 ** -6))).astype(int) - 3))
    unclamped = a <= 448
    assert np.all(np.abs(q - v)[unclamped] <= 0.5 * step[unclamped] * X[unclamped])
    assert np.all(np.abs(q[~unclamped]) == 448 * X[~unclamped])
    assert np.all(a < 512)                   # the scale keeps every element below 2^9
    assert np.all(np.sign(q) * np.sign(v) >= 0)


def test_mxfp8_blocks_are_independent_and_along_the_last_axis():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((3, 128))
    c, s = W.mxfp8_quantize(v)
    assert c.shape == (3, 128) and s.shape == (3, 4)
    v2 = v.copy()
    v2[1, 32:64] *= 1000.0
    c2, s2 = W.mxfp8_quantize(v2)
    assert np.array_equal(c2[0], c[0]) and np.array_equal(c2[2], c[2])
    assert np.array_equal(c2[1, :32], c[1, :32]) and np.array_equal(c2[1, 64:], c[1, 64:])
    assert int(s2[1, 1]) == int(s[1, 1]) + 10 or int(s2[1, 1]) == int(s[1, 1]) + 9
    with pytest.raises(ValueError):
        W.mxfp8_quantize(np.ones(40))


# ----------------------------------------------------------------------------- brute force
_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP MX v1.0 FP4 (E2M1) magnitudes, codes 0 .. 7


def _e4m3_rne(t: float) -> float:
    """Nearest E4M3 value of t (ties to even mantissa), 448 past the top: by enumerating the
    positive E4M3 values (exponent fields 0 .. 15, mantissas 0 .. 7, S.1111.111 excluded)."""
    vals = sorted({(m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
                   for e in range(16) for m in range(8) if not (e == 15 and m == 7)})
    a = abs(t)
    if a >= 448:
        return math.copysign(448.0, t)
    best = min(vals, key=lambda q: (abs(q - a), 0))
    ties = [q for q in vals if abs(q - a) == abs(best - a)]
    if len(ties) > 1:   # the even mantissa: of two neighbours, the one whose code is even
        codes = {q: i for i, q in enumerate(vals)}
        best = [q for q in ties if codes[q] % 2 == 0][0]
    return math.copysign(best, t)


def _mx8_scalar(v: list) -> list:
    out = []
    for b in range(0, len(v), 32):
        blk = v[b:b + 32]
        amax = max(abs(t) for t in blk)
        e = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
        out += [_e4m3_rne(t / 2.0 ** e) * 2.0 ** e for t in blk]
    return out


def _mxfp4_row(q: np.ndarray, s: np.ndarray) -> list:
    """One MXFP4 row by hand: byte j holds elements 2j (low nibble) and 2j + 1 (high nibble), bit 3
    the sign; element k scaled by 2^(s[k // 32] - 127)."""
    row = []
    for j, byte in enumerate(q.tolist()):
        for nib in (byte & 15, byte >> 4):
            k = len(row)
            val = _E2M1[nib & 7] * (-1.0 if nib & 8 else 1.0)
            row.append(val * 2.0 ** (int(s[k // 32]) - 127))
    return row


def test_w4a8_layer_brute_force_tiny():
    """Scalar loops over a tiny layer (H 64, I 64, 4 routed + shared, top-2, 2 tokens) with their own
    FP4 and MXFP8 conversions, against the numpy oracle."""
    shape = synth.LayerShape(hidden=64, inter=64, n_routed=4, topk=2)
    experts = {e: synth.expert_np(5, 0, e, shape) for e in range(5)}
    x_bits = synth.token_vectors(5, 0, 2, 64)
    idx = np.array([[2, 0], [1, 3]])
    wts = np.array([[0.7, 0.3], [0.55, 0.45]])
    got = W.moe_layer_w4a8(x_bits, idx, wts, experts, 4)
    for m in range(2):
        x = [float(np.frombuffer(np.uint32(int(b) << 16).tobytes(), np.float32)[0]) for b in x_bits[m]]
        xh = _mx8_scalar(x)
        y = [0.0] * 64
        for e, we in [(4, 1.0), (int(idx[m, 0]), wts[m, 0]), (int(idx[m, 1]), wts[m, 1])]:
            t = experts[e]
            h = []
            for r in range(128):
                wrow = _mxfp4_row(t["gate_up_q"][r], t["gate_up_s"][r])
                h.append(sum(wrow[k] * xh[k] for k in range(64)))
            a = [(g / (1.0 + math.exp(-g))) * u for g, u in zip(h[:64], h[64:])]
            ah = _mx8_scalar(a)
            for r in range(64):
                drow = _mxfp4_row(t["down_q"][r], t["down_s"][r])
                y[r] += we * sum(drow[k] * ah[k] for k in range(64))
        np.testing.assert_allclose(got[m], y, rtol=1e-12, atol=1e-12 * max(abs(v) for v in y))


def test_w4a8_close_to_the_bf16_layer_and_different():
    """8-bit activations move the output, but by less than 0.15 of its largest magnitude: E4M3 keeps
    three fraction bits (each rounding within 2^-4 relative), and the two roundings (x, then a) move
    each product sum by ~3-5 % rms on these inputs."""
    shape = synth.LayerShape(hidden=256, inter=128, n_routed=8, topk=2)
    experts = {e: synth.expert_np(9, 1, e, shape) for e in range(9)}
    x_bits = synth.token_vectors(9, 1, 3, 256)
    wr = synth.router_weights(9, 1, 8, 256)
    idx, w, _ = OM.route(x_bits, wr, 2)
    y16 = OM.moe_layer(x_bits, idx, w, experts, 8)
    y8 = W.moe_layer_w4a8(x_bits, idx, w, experts, 8)
    d = np.max(np.abs(y8 - y16)) / np.max(np.abs(y16))
    assert 1e-3 < d < 0.15, d


def test_w4a8_degenerate_inputs():
    shape = synth.LayerShape(hidden=64, inter=32, n_routed=4, topk=2)
    experts = {e: synth.expert_np(2, 0, e, shape) for e in range(5)}
    zero = np.zeros((1, 64), np.uint16)
    assert np.array_equal(W.moe_layer_w4a8(zero, np.array([[0, 1]]), np.array([[0.5, 0.5]]), experts, 4),
                          np.zeros((1, 64)))
    x = synth.token_vectors(2, 0, 2, 64)
    y = W.moe_layer_w4a8(x, np.array([[0, 1], [4, 1]]), np.array([[0.5, 0.5], [0.5, 0.5]]), experts, 4)
    assert np.all(np.isfinite(y[0])) and np.all(np.isnan(y[1]))
