"""Verification epilogue of a speculative-decoding window, after the LM head -- TEST INFRASTRUCTURE.

The configuration drafts three tokens and verifies a four-position window at once, accepting the
correct prefix (runbyai.xyz/signal/190, paragraph on speculative decoding; Netics post, "Speculative
decoding reduces the number of steps"). The synthetic run decodes greedily; the GSM8K run samples
at temperature 0.6, top_p 0.95, top_k 29 (Netics post, "GSM8K measured a 42.5% throughput gain").

Readings where the pages are silent:
* the target token of a position (greedy) is the argmax of its logits, ties to the lower index,
  NaN below every number, -0 equal to +0;
* greedy acceptance: draft token i (i < M - 1) is accepted while it equals the target token of
  position i; a round emits the accepted drafts and then the target token of the first position
  whose draft was not accepted (the last position when all were), so it emits 1 .. M tokens;
* sampling: the logits divided by the temperature, then the top_k largest (ties to the lower
  index) in that order, their softmax, then the shortest prefix of that order whose probability
  reaches top_p (at least one token), and the token is the first of the prefix whose cumulative
  probability exceeds u times the prefix's total, for a uniform u in [0, 1) that the caller draws
  and passes in.
"""
from __future__ import annotations

import numpy as np


def _keys(logits: np.ndarray) -> np.ndarray:
    """float64 copy with NaN -> -inf and -0 -> +0."""
    x = np.asarray(logits, dtype=np.float64)
    return np.where(np.isnan(x), -np.inf, x) + 0.0


def ranked(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of a 1-D vector, ordered (value desc, index asc)."""
    key = _keys(logits)
    return np.lexsort((np.arange(key.size), -key))[:k]


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Per row: the index of the largest logit, ties to the lower index. int64 [M]."""
    rows = np.atleast_2d(logits)
    return np.array([int(ranked(r, 1)[0]) for r in rows], dtype=np.int64)


def greedy_accept(target: np.ndarray, draft: np.ndarray) -> tuple:
    """(emitted count n in 1 .. M, the n emitted tokens) for target tokens [M] and drafts [M-1]."""
    target = np.asarray(target, dtype=np.int64).reshape(-1)
    draft = np.asarray(draft, dtype=np.int64).reshape(-1)
    if draft.size != target.size - 1:
        raise ValueError("a window of M positions verifies M - 1 drafts")
    a = 0
    while a < draft.size and draft[a] == target[a]:
        a += 1
    return a + 1, np.concatenate([draft[:a], target[a:a + 1]])


def sample_probs(logits: np.ndarray, temperature: float, top_k: int, top_p: float) -> tuple:
    """(token order, probabilities) of the kept prefix of one position: float64, summing to 1."""
    if not (temperature > 0.0 and 1 <= top_k and 0.0 < top_p <= 1.0):
        raise ValueError("need temperature > 0, top_k >= 1, 0 < top_p <= 1")
    key = _keys(logits)
    order = ranked(key, min(top_k, key.size))
    z = key[order] / temperature
    p = np.exp(z - z[0])
    p = p / p.sum()
    c = np.cumsum(p)
    keep = int(np.searchsorted(c, top_p) + 1)   # shortest prefix whose cumulative probability reaches top_p
    keep = min(max(keep, 1), order.size)
    q = p[:keep] / p[:keep].sum()
    return order[:keep], q


def sample_token(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float) -> int:
    """The sampled token of one position for a uniform u in [0, 1)."""
    order, q = sample_probs(logits, temperature, top_k, top_p)
    c = np.cumsum(q)
    j = int(np.searchsorted(c, u * c[-1], side="right"))   # first cumulative value > u * total
    return int(order[min(j, order.size - 1)])


def sample_tokens(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u) -> np.ndarray:
    """Per row of logits [M, V], one sampled token for u[m]. int64 [M]."""
    rows = np.atleast_2d(logits)
    u = np.asarray(u, dtype=np.float64).reshape(-1)
    return np.array([sample_token(r, temperature, top_k, top_p, float(u[m])) for m, r in enumerate(rows)],
                    dtype=np.int64)
