"""The speculation cost model of bench.py (host arithmetic, no GPU): its invariants, and the pages'
own figures run through it (verification-cost ratio 2.26 with accept lengths 3.90 and 2.68,
Netics post and runbyai.xyz signal/190)."""
import pytest

import bench


def test_pages_figures_without_draft_cost():
    m = bench.speculation_model(1.0, 2.26, 0.0)
    assert m["verify_cost_ratio"] == pytest.approx(2.26)
    # a round of cost 2.26 steps emitting 3.90 tokens: 1.73x plain decoding; 2.68 tokens: 1.19x
    assert m["by_accept"]["3.90"]["speedup"] == pytest.approx(3.90 / 2.26, abs=1e-3)
    assert m["by_accept"]["2.68"]["speedup"] == pytest.approx(2.68 / 2.26, abs=1e-3)
    assert m["break_even_accept"] == pytest.approx(2.26)


def test_silent_fallback_is_slower_than_plain_decoding():
    # accept length 1.00 (the draft reading FP8 weights as bf16): every round pays verification for
    # one token, so the stack runs below plain decoding whenever a round costs more than a step
    for t4, d in ((2.26, 0.0), (1.2, 0.05), (1.01, 0.0)):
        m = bench.speculation_model(1.0, t4, d)
        assert m["by_accept"]["1.00"]["speedup"] < 1.0


def test_throughput_is_linear_in_accept_length_and_units():
    m = bench.speculation_model(0.5, 1.25, 0.1, drafts=3, accepts=(1.0, 2.0, 4.0))
    assert m["round_ms"] == pytest.approx(1.25 + 0.3)
    assert m["plain_tokens_per_s"] == pytest.approx(2000.0)
    t = [m["by_accept"][k]["tokens_per_s"] for k in ("1.00", "2.00", "4.00")]
    assert t[1] == pytest.approx(2 * t[0], rel=1e-3) and t[2] == pytest.approx(4 * t[0], rel=1e-3)
    assert t[0] == pytest.approx(1e3 / 1.55, rel=1e-3)
