"""Vocabulary LM head: online per-row FP8 quantisation and the head GEMV, FP8 and bf16.

The head projects a 2,560-wide hidden state onto 157,184 tokens; every token reads all of it,
~805 MB in bf16, halved by FP8 (runbyai.xyz/posts/593 paragraph 3). The FP8 configuration is
applied when the head is constructed, from the bf16 weights (Netics post, "Online FP8
quantization halves the LM head weight reads"). Logits are float32 in the product, float64 here.

Readings where the pages are silent: per-row scale s_r = fl32(max_k |W[r, k]| / 448) and codes
q = E4M3_RNE_saturating(fl32(W[r, k] / s_r)) -- both steps in IEEE float32 as the product does
them, so codes compare bit for bit; an all-zero row takes s_r = 1. The activation stays bf16.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, bf16_to_f64, e4m3_encode, e4m3_table

CHUNK_ROWS = 8192


def fp8_rowquant(w_bits: np.ndarray) -> tuple:
    """(codes uint8 [R, C], scales float32 [R]) for a bf16 weight [R, C]."""
    w_bits = np.atleast_2d(w_bits)
    rows = w_bits.shape[0]
    codes = np.empty(w_bits.shape, dtype=np.uint8)
    scales = np.empty(rows, dtype=np.float32)
    for r0 in range(0, rows, CHUNK_ROWS):
        w = bf16_to_f32(w_bits[r0:r0 + CHUNK_ROWS])
        amax = np.abs(w).max(axis=1)
        s = amax / np.float32(448.0)              # float32 IEEE division
        s[amax == 0] = np.float32(1.0)
        v = w / s[:, None]                        # float32 IEEE division, elementwise
        codes[r0:r0 + CHUNK_ROWS] = e4m3_encode(v)
        scales[r0:r0 + CHUNK_ROWS] = s
    return codes, scales


def fp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float32 [R, C]: fl32(e4m3(q) * s_r), one IEEE float32 product per element."""
    vals = e4m3_table()[np.asarray(codes)].astype(np.float32)
    return vals * np.asarray(scales, dtype=np.float32)[:, None]


def lmhead_fp8(codes: np.ndarray, scales: np.ndarray, x_bits: np.ndarray, rows=None) -> np.ndarray:
    """logits[m, r] = s_r * sum_k e4m3(q[r, k]) * x[m, k], float64 [M, R'] (R' = len(rows))."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    table = e4m3_table()
    sel = np.arange(codes.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((x.shape[0], sel.size), dtype=np.float64)
    for j0 in range(0, sel.size, CHUNK_ROWS):
        r = sel[j0:j0 + CHUNK_ROWS]
        deq = table[codes[r]]
        out[:, j0:j0 + r.size] = (deq @ x.T).T * scales[r].astype(np.float64)
    return out


def lmhead_bf16(w_bits: np.ndarray, x_bits: np.ndarray, rows=None) -> np.ndarray:
    """logits[m, r] = sum_k W[r, k] * x[m, k], float64 [M, R']."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    sel = np.arange(w_bits.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((x.shape[0], sel.size), dtype=np.float64)
    for j0 in range(0, sel.size, CHUNK_ROWS):
        r = sel[j0:j0 + CHUNK_ROWS]
        out[:, j0:j0 + r.size] = (bf16_to_f64(w_bits[r]) @ x.T).T
    return out


def topk_indices(logits: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k largest entries ordered (value desc, index asc). int64 [M, k]."""
    logits = np.atleast_2d(logits)
    out = np.empty((logits.shape[0], k), dtype=np.int64)
    idx = np.arange(logits.shape[1])
    for m in range(logits.shape[0]):
        out[m] = np.lexsort((idx, -(logits[m] + 0.0)))[:k]
    return out


def topk_agreement(a: np.ndarray, b: np.ndarray, k: int = 10) -> dict:
    """Agreement of head A against head B over the rows (x vectors) of two logit matrices.

    top1: fraction with equal argmax; topk_overlap: mean |topk_A & topk_B| / k;
    top1_in_topk: fraction where A's argmax is among B's top k. Ties go to the lower index.
    """
    ta, tb = topk_indices(a, k), topk_indices(b, k)
    top1 = float(np.mean(ta[:, 0] == tb[:, 0]))
    overlap = float(np.mean([len(set(ta[i]) & set(tb[i])) / k for i in range(ta.shape[0])]))
    in_k = float(np.mean([ta[i, 0] in set(tb[i]) for i in range(ta.shape[0])]))
    return {"top1": top1, "topk_overlap": overlap, "top1_in_topk": in_k, "k": k, "n": int(ta.shape[0])}
