"""Pins for oracle.formats: spec tables, a hand-worked MXFP4 example, exhaustive FP8 checks
against torch's float8_e4m3fn (a library routine), and brute force at tiny shapes."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- e2m1 / E8M0
def test_e2m1_table_matches_spec(golden_dir):
    want = _load(golden_dir, "e2m1_values.json")["values"]
    got = F.e2m1_table()
    for c in range(16):
        assert got[c] == want[c]
        assert math.copysign(1.0, got[c]) == math.copysign(1.0, want[c]), c  # -0.0 for code 8


def test_e2m1_is_symmetric_and_monotone():
    t = F.e2m1_table()
    assert np.all(np.diff(t[:8]) > 0)
    assert np.array_equal(t[8:], -t[:8])


def test_e8m0_closed_form():
    assert F.e8m0_value(127) == 1.0
    assert F.e8m0_value(0) == 2.0 ** -127
    assert F.e8m0_value(254) == 2.0 ** 127
    t = F.e8m0_table()
    assert np.all(t[1:255] == 2.0 * t[0:254])
    assert math.isnan(t[255])
    with pytest.raises(ValueError):
        F.e8m0_value(255)


def test_mxfp4_worked_example(golden_dir):
    ex = _load(golden_dir, "mxfp4_worked_example.json")
    q = np.frombuffer(bytes.fromhex(ex["row_bytes_hex"]), dtype=np.uint8)[None, :]
    s = np.array([ex["scale_bytes"]], dtype=np.uint8)
    w = F.mxfp4_dequant(q, s)
    assert w.shape == (1, ex["cols"])
    for k, v in ex["expected"].items():
        assert w[0, int(k)] == v and math.copysign(1, w[0, int(k)]) == math.copysign(1, v), k
    b = ex["block1_case"]
    q2 = np.zeros((1, 32), dtype=np.uint8)
    q2[0, b["byte_index"]] = int(b["byte_value"], 16)
    w2 = F.mxfp4_dequant(q2, np.array([b["scale_bytes"]], dtype=np.uint8))
    for k, v in b["expected"].items():
        assert w2[0, int(k)] == v


def test_mxfp4_brute_force_tiny(golden_dir):
    """Per-element pure-Python decode using the spec table (not the oracle's decoder)."""
    table = _load(golden_dir, "e2m1_values.json")["values"]
    rng = np.random.default_rng(7)
    rows, cols = 5, 96
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    s = rng.integers(100, 150, (rows, cols // 32), dtype=np.uint8)
    w = F.mxfp4_dequant(q, s)
    for r in range(rows):
        for k in range(cols):
            byte = int(q[r, k // 2])
            code = (byte >> 4) if k % 2 else (byte & 15)
            want = table[code] * 2.0 ** (int(s[r, k // 32]) - 127)
            assert w[r, k] == want


def test_mxfp4_block_scale_doubles_only_its_block():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, (3, 64), dtype=np.uint8)
    s = rng.integers(110, 130, (3, 4), dtype=np.uint8)
    w0 = F.mxfp4_dequant(q, s)
    s1 = s.copy()
    s1[1, 2] += 1
    w1 = F.mxfp4_dequant(q, s1)
    d = np.zeros_like(w0, dtype=bool)
    d[1, 64:96] = True
    assert np.array_equal(w1[d], 2 * w0[d])
    assert np.array_equal(w1[~d], w0[~d])


# ----------------------------------------------------------------------------- E4M3
def _torch_e4m3_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes_vs_torch():
    want = _torch_e4m3_decode_all()
    got = F.e4m3_table()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}


def test_e4m3_spec_points(golden_dir):
    g = _load(golden_dir, "e4m3_points.json")
    for p in g["points"]:
        c = int(p["code"], 16)
        assert F.e4m3_value(c) == p["value"] and math.copysign(1, F.e4m3_value(c)) == math.copysign(1, p["value"])
        assert F.e4m3_encode_scalar(p["value"]) == c
    for c in g["nan_codes"]:
        assert math.isnan(F.e4m3_value(int(c, 16)))
    for r in g["rounding_cases"]:
        assert F.e4m3_encode_scalar(r["in"]) == int(r["code"], 16), r
        assert int(F.e4m3_encode(np.array([r["in"]]))[0]) == int(r["code"], 16), r


def test_e4m3_roundtrip_every_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        v = F.e4m3_value(c)
        assert F.e4m3_encode_scalar(v) == c
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(F.e4m3_encode(F.e4m3_table()[codes]), codes.astype(np.uint8))


def _all_bf16_finite_as_f32():
    u = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    v = u.view(np.float32)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -20, 2.0 ** 7, 0.0137, 311.7])
def test_e4m3_encode_vs_torch_all_bf16(scale):
    """Every finite bf16 value times a scale, clamped into the finite range, against torch's
    float32 -> float8_e4m3fn cast (round to nearest even)."""
    with np.errstate(over="ignore"):
        v = (_all_bf16_finite_as_f32().astype(np.float64) * scale).astype(np.float32)
    v = v[np.isfinite(v)]
    clamped = np.clip(v, -448.0, 448.0).astype(np.float32)
    want = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(v)
    assert np.array_equal(got, want)


def test_e4m3_encode_random_vs_scalar_and_torch():
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 7, 20000))).astype(np.float32)
    got = F.e4m3_encode(v)
    for i in range(0, 20000, 37):
        assert got[i] == F.e4m3_encode_scalar(float(v[i]))
    want = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_encode_error_bound():
    rng = np.random.default_rng(5)
    v = rng.uniform(-448, 448, 50000)
    d = F.e4m3_table()[F.e4m3_encode(v)]
    nrm = np.abs(v) >= 2.0 ** -6
    assert np.all(np.abs(d[nrm] - v[nrm]) <= 2.0 ** -4 * np.abs(v[nrm]))
    assert np.all(np.abs(d[~nrm] - v[~nrm]) <= 2.0 ** -10)


def test_bf16_decode_vs_torch():
    u = np.arange(65536, dtype=np.uint16)
    want = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_to_f64(u)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
