"""Pins of the verification-epilogue oracle (oracle/verify.py): hand-worked windows, closed forms of
the sampling distribution, brute force on tiny inputs, and the inversion checked by frequency."""
import math

import numpy as np
import pytest

from oracle import verify as OV


def test_argmax_ties_nan_and_signed_zero():
    assert OV.argmax_first(np.array([1.0, 3.0, 3.0, 2.0])).tolist() == [1]
    assert OV.argmax_first(np.array([np.nan, 1.0, -5.0])).tolist() == [1]
    assert OV.argmax_first(np.array([-0.0, 0.0, -1.0])).tolist() == [0]
    assert OV.argmax_first(np.array([-np.inf, -np.inf])).tolist() == [0]
    assert OV.argmax_first(np.array([[0.0, 1.0], [2.0, 1.0]])).tolist() == [1, 0]


def test_argmax_matches_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(200):
        v = rng.integers(-3, 4, 9).astype(np.float64)     # small integers: many exact ties
        best = max(range(v.size), key=lambda i: (v[i], -i))
        assert OV.argmax_first(v)[0] == best


@pytest.mark.parametrize("target,draft,n,emitted", [
    ([5, 6, 7, 8], [5, 6, 7], 4, [5, 6, 7, 8]),       # every draft accepted, plus the last target
    ([5, 6, 7, 8], [5, 9, 7], 2, [5, 6]),             # second draft rejected: the target replaces it
    ([5, 6, 7, 8], [1, 6, 7], 1, [5]),                # nothing accepted: one token per round
    ([5, 6, 7, 8], [5, 6, 9], 3, [5, 6, 7]),
    ([3], [], 1, [3]),                                # a window of one position is a plain step
    ([4, 4], [4], 2, [4, 4]),
])
def test_greedy_acceptance_worked_windows(target, draft, n, emitted):
    got_n, got = OV.greedy_accept(np.array(target), np.array(draft, dtype=np.int64))
    assert got_n == n and got.tolist() == emitted


def test_greedy_acceptance_rejects_a_malformed_window():
    with pytest.raises(ValueError):
        OV.greedy_accept(np.array([1, 2, 3]), np.array([1, 2, 3]))


def test_sampling_distribution_closed_form():
    # p proportional to 1, 2, 4 (logits 0, ln 2, ln 4 at temperature 1)
    logits = np.array([0.0, math.log(2.0), math.log(4.0)])
    order, q = OV.sample_probs(logits, 1.0, 3, 1.0)
    assert order.tolist() == [2, 1, 0]
    np.testing.assert_allclose(q, [4 / 7, 2 / 7, 1 / 7], rtol=1e-12)
    # top_p 0.5: the first token alone reaches it
    order, q = OV.sample_probs(logits, 1.0, 3, 0.5)
    assert order.tolist() == [2] and q.tolist() == [1.0]
    # top_p 0.8: 4/7 < 0.8 <= 6/7, two tokens, renormalised
    order, q = OV.sample_probs(logits, 1.0, 3, 0.8)
    assert order.tolist() == [2, 1]
    np.testing.assert_allclose(q, [2 / 3, 1 / 3], rtol=1e-12)
    # top_k 2 before top_p
    order, q = OV.sample_probs(logits, 1.0, 2, 1.0)
    assert order.tolist() == [2, 1]
    np.testing.assert_allclose(q, [2 / 3, 1 / 3], rtol=1e-12)
    # temperature 0.5 squares the ratios: 1 : 4 : 16
    order, q = OV.sample_probs(logits, 0.5, 3, 1.0)
    np.testing.assert_allclose(q, np.array([16, 4, 1]) / 21, rtol=1e-12)


def test_top_p_boundary_is_inclusive():
    # two equal tokens: the first reaches exactly one half
    order, q = OV.sample_probs(np.array([1.0, 1.0]), 1.0, 2, 0.5)
    assert order.tolist() == [0] and q.tolist() == [1.0]


def test_sample_token_inverts_the_cumulative_distribution():
    logits = np.array([0.0, math.log(2.0), math.log(4.0)])
    for u, tok in ((0.0, 2), (0.5, 2), (4 / 7 - 1e-9, 2), (0.6, 1), (6 / 7 - 1e-9, 1), (0.9, 0), (1 - 1e-12, 0)):
        assert OV.sample_token(logits, 1.0, 3, 1.0, u) == tok, u
    # top_k 1 is the argmax whatever u is
    rng = np.random.default_rng(1)
    v = rng.standard_normal(50)
    for u in rng.random(20):
        assert OV.sample_token(v, 0.6, 1, 0.95, float(u)) == int(np.argmax(v))


def test_sampling_frequencies_follow_the_kept_distribution():
    """u on an even grid of [0, 1): the token frequencies equal the kept probabilities to 1/n."""
    rng = np.random.default_rng(2)
    v = rng.standard_normal(40) * 2.0
    order, q = OV.sample_probs(v, 0.6, 29, 0.95)
    n = 20000
    toks = [OV.sample_token(v, 0.6, 29, 0.95, (i + 0.5) / n) for i in range(n)]
    freq = np.array([toks.count(int(t)) for t in order]) / n
    np.testing.assert_allclose(freq, q, atol=2.0 / n)
    assert set(toks) <= set(order.tolist())


def test_kept_set_is_the_top_k_by_brute_force_sort():
    rng = np.random.default_rng(3)
    for _ in range(50):
        v = np.round(rng.standard_normal(30), 1)                # ties
        order, _ = OV.sample_probs(v, 0.6, 29, 1.0)
        want = sorted(range(v.size), key=lambda i: (-v[i], i))[:29]
        assert order.tolist() == want
