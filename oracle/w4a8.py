"""W4A8 MoE layer at decode time: MXFP4 weights x 8-bit activations, float64.

Test infrastructure: only tests, the smoke check and the benchmark's CPU baseline use this module.

The Netics post, section "Humming MXFP4 kernels compile at run time for the model's real shapes",
names the baseline's MoE recipe W4A8 (MXFP4 weights, 8-bit activations) and says nothing more of
the activation format. Readings (each listed in the design notes):
* the 8-bit activation format is MXFP8 from the same OCP Microscaling family as the weights:
  E4M3 elements (bias 7, no infinities, largest finite 448) sharing one E8M0 power-of-two scale
  per 32 consecutive elements;
* the scale of a block follows the OCP MX v1.0 conversion: X = 2^(floor(log2 max|v|) - 8), 8
  being the exponent of E4M3's largest normal; each element is v / X rounded to the nearest E4M3
  value (ties to even), magnitudes past 448 saturating to 448; the scale exponent is clamped to
  E8M0's range [-127, 127] (an all-zero block gets 2^-127 and zero codes);
* both activation operands of an expert are quantised on the fly ("dynamic"): the token vector x
  before gate_up (blocks of 32 along the hidden dimension) and the SwiGLU output a before down
  (blocks of 32 along the intermediate dimension, the down projection's own MX blocks);
* the router stays in bf16 (the recipe names the MoE kernels, and routing precedes them), as do
  the gate weights, the combine and the shared expert's weight 1; the shared expert is an expert
  like the routed ones and runs W4A8 too.
Everything after the two quantisations is exact float64 arithmetic, as in the bf16 layer.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e4m3_encode, e4m3_table, mxfp4_dequant
from .moe import silu

MX_BLOCK = 32
E4M3_EMAX = 8   # exponent of E4M3's largest normal, 448 = 1.75 * 2^8


def scale_exponent_of_max(amax: np.ndarray) -> np.ndarray:
    """floor(log2 amax) - 8, clamped to [-127, 127]; -127 for amax = 0 (int64)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                      # amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1
    s = np.where(amax > 0, ex.astype(np.int64) - 1 - E4M3_EMAX, -127)
    return np.clip(s, -127, 127)


def mxfp8_scale_exponents(v: np.ndarray) -> np.ndarray:
    """Per block of 32 along the last axis: the scale exponent of the block's max|v| (int64
    [..., n / 32])."""
    v = np.asarray(v, dtype=np.float64)
    if v.shape[-1] % MX_BLOCK:
        raise ValueError("the last dimension must be a multiple of 32")
    return scale_exponent_of_max(np.max(np.abs(v.reshape(*v.shape[:-1], -1, MX_BLOCK)), axis=-1))


def mxfp8_quantize(v: np.ndarray) -> tuple:
    """(E4M3 codes uint8 [..., n], E8M0 scale bytes uint8 [..., n / 32]) of v, blocks of 32 along
    the last axis, by the conversion above."""
    v = np.asarray(v, dtype=np.float64)
    s = mxfp8_scale_exponents(v)
    scaled = v / np.repeat(np.ldexp(1.0, s), MX_BLOCK, axis=-1)
    return e4m3_encode(scaled), (s + 127).astype(np.uint8)


def mxfp8_dequant(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """value = E4M3(code) * 2^(scale byte - 127), float64."""
    s = np.asarray(scale_bytes).astype(np.int64) - 127
    return e4m3_table()[np.asarray(codes)] * np.repeat(np.ldexp(1.0, s), MX_BLOCK, axis=-1)


def mxfp8_round(v: np.ndarray) -> np.ndarray:
    """v after MXFP8 quantisation and dequantisation."""
    return mxfp8_dequant(*mxfp8_quantize(v))


def expert_ffn_w4a8(gate_up: np.ndarray, down: np.ndarray, x_hat: np.ndarray) -> tuple:
    """One expert on one token whose x is already MXFP8-rounded: h = W_gu x_hat; a = silu(h[:I]) *
    h[I:]; out = W_d mxfp8(a). Returns (out, a) in float64 (a before its rounding)."""
    inter = down.shape[1]
    h = gate_up @ x_hat
    a = silu(h[:inter]) * h[inter:]
    return down @ mxfp8_round(a), a


def _dequant(t):
    return t if isinstance(t, tuple) else (mxfp4_dequant(t["gate_up_q"], t["gate_up_s"]),
                                           mxfp4_dequant(t["down_q"], t["down_s"]))


def moe_layer_w4a8(x_bits: np.ndarray, idx: np.ndarray, w: np.ndarray, experts, n_routed: int,
                   has_shared: bool = True, detail: bool = False):
    """y[m] = shared(x_hat[m]) + sum_i w[m, i] * expert_{idx[m, i]}(x_hat[m]), float64 [M, H],
    with x_hat = mxfp8(x) and each expert's a rounded by mxfp8 before down.

    ``experts`` maps an expert id (n_routed = the shared expert) to its canonical byte tensors or
    to a dequantised (gate_up, down) pair. A token whose idx holds an id outside [0, n_routed) has
    no defined output: its row is NaN. With detail=True, also returns {(m, e): (weight, a)} for
    every (token, expert) product, a being the float64 SwiGLU output before its rounding."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    idx = np.atleast_2d(idx)
    w = np.atleast_2d(np.asarray(w, dtype=np.float64))
    cache = {}

    def weights_of(e):
        if e not in cache:
            cache[e] = _dequant(experts[e])
        return cache[e]

    x_hat = mxfp8_round(x)
    y = np.zeros_like(x)
    acts = {}
    for m in range(x.shape[0]):
        if np.any((idx[m] < 0) | (idx[m] >= n_routed)):
            y[m] = np.nan
            continue
        terms = ([(n_routed, 1.0)] if has_shared else []) + [(int(idx[m, i]), w[m, i]) for i in range(idx.shape[1])]
        for e, we in terms:
            out, a = expert_ffn_w4a8(*weights_of(e), x_hat[m])
            y[m] += we * out
            acts[(m, e)] = (we, a)
    return (y, acts) if detail else y

