"""Number formats: MXFP4 (e2m1 elements, E8M0 block-of-32 scales) and FP8 E4M3 (the "FN" variant).

The pages call the expert weights "MXFP4" (runbyai.xyz/posts/593 paragraph 4; Netics post,
"Humming MXFP4 kernels compile at run time ...") and the quantised head "FP8" (posts/593
paragraph 3; Netics, "Online FP8 quantization halves the LM head weight reads"), without bit
layouts. The definitions below are the public OCP Microscaling (MX) v1.0 and OCP 8-bit Floating
Point specifications, written from their field definitions.

Container layout of an MXFP4 matrix [rows, cols] (a reading; the pages are silent): nibbles
row-major, byte j of a row holds element 2j in bits 3:0 and element 2j+1 in bits 7:4; one E8M0
byte per 32 consecutive elements of a row, stored row-major as [rows, cols/32].
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------- e2m1
def e2m1_value(code: int) -> float:
    """Value of a 4-bit e2m1 code: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0.

    Exponent field 0 is subnormal: magnitude = mantissa * 2^(1-1) * 1/2. Otherwise magnitude =
    2^(exponent-1) * (1 + mantissa/2). No infinities or NaN.
    """
    if not 0 <= code <= 15:
        raise ValueError("e2m1 code out of range")
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else math.ldexp(1.0 + m / 2.0, e - 1)
    return -mag if s else mag


def e2m1_table() -> np.ndarray:
    """float64 [16]: value of every code (code 8 is -0.0)."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


# ----------------------------------------------------------------------------- E8M0
def e8m0_value(s: int) -> float:
    """Scale 2^(s-127) of an E8M0 byte; byte 255 is NaN and is rejected."""
    if not 0 <= s <= 254:
        raise ValueError("E8M0 byte 255 is NaN; only 0..254 are scales")
    return math.ldexp(1.0, s - 127)


def e8m0_table() -> np.ndarray:
    """float64 [256]; entry 255 is NaN."""
    t = np.array([math.ldexp(1.0, s - 127) for s in range(256)], dtype=np.float64)
    t[255] = np.nan
    return t


# ----------------------------------------------------------------------------- MXFP4 matrices
def mxfp4_codes(q: np.ndarray) -> np.ndarray:
    """Unpack nibble bytes [rows, cols/2] into codes [rows, cols] (low nibble first)."""
    q = np.asarray(q, dtype=np.uint8)
    codes = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = q & 0x0F
    codes[:, 1::2] = q >> 4
    return codes


def mxfp4_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W[r, k] = e2m1(code[r, k]) * 2^(S[r, k // 32] - 127), float64 [rows, cols] (exact)."""
    codes = mxfp4_codes(q)
    s = np.asarray(s, dtype=np.uint8)
    rows, cols = codes.shape
    if s.shape != (rows, cols // 32) or cols % 32:
        raise ValueError("scale shape must be [rows, cols/32]")
    if np.any(s == 255):
        raise ValueError("E8M0 byte 255 (NaN) in scales")
    vals = e2m1_table()[codes]
    scale = e8m0_table()[s]
    return vals * np.repeat(scale, 32, axis=1)


# ----------------------------------------------------------------------------- bf16
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


# ----------------------------------------------------------------------------- E4M3 (FN)
E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of an E4M3 code: sign bit 7, exponent bits 6:3 (bias 7), mantissa bits 2:0.

    Exponent 0 is subnormal: 2^-6 * m/8. S.1111.111 is NaN; there are no infinities, so the
    largest finite magnitude is S.1111.110 = 448.
    """
    if not 0 <= code <= 255:
        raise ValueError("E4M3 code out of range")
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return math.nan
    mag = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -mag if s else mag


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode_scalar(v: float) -> int:
    """Round-to-nearest-even, saturating E4M3 encode of one finite value (pure Python).

    Magnitudes at or above 448 give 448 (nothing above it is finite). Below 2^-6 the result is a
    subnormal, m = RNE(|v| / 2^-9), where m = 8 carries into the smallest normal. Otherwise
    e = floor(log2 |v|), m = RNE((|v| / 2^e - 1) * 8), where m = 8 carries into e + 1.
    """
    if math.isnan(v) or math.isinf(v):
        raise ValueError("only finite values are encoded")
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a >= E4M3_MAX:
        return sign | 0x7E
    if a < 2.0 ** -6:
        m = round(a / 2.0 ** -9)  # Python round: half to even; exact for dyadic a
        return sign | m           # m == 8 is 0x08, the smallest normal
    e = math.floor(math.log2(a))
    if 2.0 ** e > a:              # guard log2 rounding at exact powers of two
        e -= 1
    elif 2.0 ** (e + 1) <= a:
        e += 1
    m = round((a / 2.0 ** e - 1.0) * 8.0)
    if m == 8:
        e, m = e + 1, 0
    return sign | ((e + 7) << 3) | m


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Vectorised twin of :func:`e4m3_encode_scalar` for finite float32/float64 arrays -> uint8."""
    v = np.asarray(v)
    if not np.all(np.isfinite(v)):
        raise ValueError("only finite values are encoded")
    a = np.abs(v.astype(np.float64))
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)       # np.rint: half to even
    nrm = ~sub
    f, ex = np.frexp(a[nrm])                                    # a = f * 2^ex, f in [0.5, 1)
    m = np.rint(16.0 * f - 8.0).astype(np.int64)                # (a / 2^e - 1) * 8, e = ex - 1
    code[nrm] = ((ex.astype(np.int64) - 1 + 7) << 3) + m       # m == 8 carries into the exponent
    code[a >= E4M3_MAX] = 0x7E
    code |= np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)
