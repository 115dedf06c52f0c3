"""Routed-expert MoE layer at decode time, float64.

Follows runbyai.xyz/posts/593 paragraph 2 (each MoE layer routes a token to eight of 512 routed
experts plus one shared expert), paragraph 4 (moe_intermediate_size 768, experts in MXFP4) and
paragraph 5 (a verification pass over four positions touches the union of their experts, up to
32); the Netics post's section "Decoding was memory-bound on a 124-billion-parameter model at
batch size 1" gives the same routing and hidden size 2560.

Readings where the pages are silent (each is listed in the design notes):
* the router scores by logits = x . W_r (+ an optional bias); the top-k are taken on those
  logits, ordered by (logit descending, expert index ascending), so ties go to the lower index,
  and the gate weights are a softmax over the k selected logits (equal to a full softmax
  renormalised over the selection);
* SwiGLU on gate_up rows [0, I) = gate and [I, 2I) = up: a = silu(gate) * up,
  silu(g) = g / (1 + e^-g);
* the shared expert is always on with weight 1 and no routed scaling factor.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, mxfp4_dequant


def router_logits(x_bits: np.ndarray, w_router_bits: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """logits[m, e] = sum_k x[m, k] * W_r[e, k] + bias[(m,) e], float64 [M, E]."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    w = bf16_to_f64(w_router_bits)
    logits = x @ w.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)  # [E] or [M, E] broadcast
    return logits


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """The k largest logits per row, ordered by (value desc, index asc). int64 [M, k].

    NaN logits rank below every number; -0.0 and +0.0 compare equal.
    """
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    m, e = logits.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= k <= number of experts")
    out = np.empty((m, k), dtype=np.int64)
    idx = np.arange(e)
    for r in range(m):
        key = np.where(np.isnan(logits[r]), -np.inf, logits[r]) + 0.0  # + 0.0 turns -0 into +0
        order = np.lexsort((idx, -key))  # primary: -value ascending; secondary: index ascending
        out[r] = order[:k]
    return out


def route_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[m, i] = exp(l_i - l_max) / sum_j exp(l_j - l_max) over the selected logits. float64."""
    logits = np.atleast_2d(logits)
    sel = np.take_along_axis(logits, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route(x_bits, w_router_bits, k: int, bias=None):
    """Router step: (idx int64 [M, k], w float64 [M, k], logits float64 [M, E])."""
    logits = router_logits(x_bits, w_router_bits, bias)
    idx = topk_select(logits, k)
    return idx, route_weights(logits, idx), logits


def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(gate_up: np.ndarray, down: np.ndarray, x: np.ndarray) -> np.ndarray:
    """One expert on one token: h = W_gu x; a = silu(h[:I]) * h[I:]; out = W_d a (float64)."""
    inter = down.shape[1]
    h = gate_up @ x
    a = silu(h[:inter]) * h[inter:]
    return down @ a


def dequant_expert(tensors: dict) -> tuple:
    """(gate_up float64 [2I, H], down float64 [H, I]) from one expert's canonical MXFP4 bytes."""
    return (mxfp4_dequant(tensors["gate_up_q"], tensors["gate_up_s"]),
            mxfp4_dequant(tensors["down_q"], tensors["down_s"]))


def moe_layer(x_bits: np.ndarray, idx: np.ndarray, w: np.ndarray, experts, n_routed: int,
              has_shared: bool = True) -> np.ndarray:
    """y[m] = shared(x[m]) + sum_i w[m, i] * expert_{idx[m, i]}(x[m]), float64 [M, H].

    ``experts`` maps an expert id (n_routed = the shared expert) to its canonical byte tensors,
    or to an already dequantised (gate_up, down) pair. A token whose idx holds an id outside
    [0, n_routed) has no defined output: its row is NaN.
    """
    x = bf16_to_f64(np.atleast_2d(x_bits))
    idx = np.atleast_2d(idx)
    w = np.atleast_2d(np.asarray(w, dtype=np.float64))
    cache = {}

    def weights_of(e):
        if e not in cache:
            t = experts[e]
            cache[e] = t if isinstance(t, tuple) else dequant_expert(t)
        return cache[e]

    y = np.zeros_like(x)
    for m in range(x.shape[0]):
        if np.any((idx[m] < 0) | (idx[m] >= n_routed)):
            y[m] = np.nan
            continue
        if has_shared:
            y[m] += expert_ffn(*weights_of(n_routed), x[m])
        for i in range(idx.shape[1]):
            y[m] += w[m, i] * expert_ffn(*weights_of(int(idx[m, i])), x[m])
    return y


def expert_union(idx: np.ndarray, n_routed: int) -> list:
    """Sorted distinct valid routed expert ids selected by any token of the window."""
    v = np.unique(np.asarray(idx).reshape(-1))
    return [int(e) for e in v if 0 <= e < n_routed]
