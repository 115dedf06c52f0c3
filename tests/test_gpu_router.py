"""GPU parity of moe_route_topk: logits, top-K (with the near-tie rule), gate weights; closed-form
and exact-tie cases; bias shapes; the Zipf-concentrated and regime routings at full shape."""
import numpy as np
import pytest
import torch

import quantized_weight_streaming_amd as qws
import synth
from oracle import moe as OM

from .helpers import assert_close, bf16, check_topk, f32, say

pytestmark = pytest.mark.gpu


def _run(x, wr, K, bias=None):
    M, E = x.shape[0], wr.shape[0]
    logits = torch.empty((M, E), dtype=torch.float32, device="cuda")
    bt = None if bias is None else f32(bias)
    idx, w = qws.moe_route_topk(bf16(x), bf16(wr), K, bt, logits_out=logits)
    return idx.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()


def _check(x, wr, K, bias=None):
    idx, w, lg = _run(x, wr, K, bias)
    ridx, rw, rlg = OM.route(x, wr, K, bias)
    assert_close(lg, rlg, tol=1e-5, what="logits")
    near = check_topk(idx, lg, rlg, K, gpu_w=w)
    if near == 0:
        assert_close(w, rw, tol=1e-5, what="gate weights")
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    return idx, w, near


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("E,H,K", [(64, 2560, 8), (512, 2560, 8), (37, 136, 5), (1024, 2560, 8), (3, 8, 3), (512, 64, 1)])
def test_route_matches_oracle(M, E, H, K):
    say("route", M, E, H, K)
    wr = synth.router_weights(E + H, M, E, H)
    x = synth.token_vectors(E + H, M, M, H)
    _check(x, wr, K)


@pytest.mark.parametrize("shape", ["vector", "matrix"])
def test_route_bias(shape):
    say("route bias", shape)
    wr = synth.router_weights(4, 0, 512)
    x = synth.token_vectors(4, 0, 4)
    if shape == "vector":
        bias = synth.zipf_bias(1, 0, 512)
    else:
        bias = synth.regime_bias(synth.regime_sets(0, 0, "half", 4, 512), 512)
    _check(x, wr, 8, bias)


def test_zero_input_closed_form():
    say("route x=0")
    wr = synth.router_weights(0, 0, 512)
    idx, w, lg = _run(np.zeros((2, 2560), dtype=np.uint16), wr, 8)
    assert np.all(lg == 0.0)
    assert idx.tolist() == [list(range(8))] * 2
    assert np.all(w == np.float32(0.125))


def test_exact_ties_go_to_lower_index():
    say("route ties")
    wr = synth.router_weights(0, 0, 512).copy()
    for dup, src in ((300, 5), (17, 5), (480, 200)):
        wr[dup] = wr[src]
    x = synth.token_vectors(0, 0, 1)
    bias = np.zeros(512, dtype=np.float32)
    bias[[5, 17, 300, 200, 480]] = 50.0        # make the tied rows the top of the ranking
    idx, _, lg = _run(x, wr, 8, bias)
    assert lg[0, 5] == lg[0, 17] == lg[0, 300] and lg[0, 200] == lg[0, 480]
    top = idx[0, :5].tolist()
    a, b = (5, 17, 300), (200, 480)
    want = list(a) + list(b) if lg[0, 5] > lg[0, 200] else list(b) + list(a)
    assert top == want


def test_negative_and_positive_zero_tie():
    say("route signed zeros")
    wr = np.zeros((6, 64), dtype=np.uint16)
    x = np.zeros((1, 64), dtype=np.uint16)
    bias = np.array([-1.0, -0.0, 0.0, -2.0, -0.0, -3.0], dtype=np.float32)
    idx, w, _ = _run(x, wr, 3, bias)
    assert idx[0].tolist() == [1, 2, 4]


def test_zipf_concentrated_full_shape():
    say("route zipf")
    bias = synth.zipf_bias(1, 0, 512)
    wr = synth.router_weights(1, 0, 512)
    x = synth.token_vectors(1, 0, 4)
    idx, _, _ = _check(x, wr, 8, bias)
    assert np.mean(idx < 512) == 1.0


@pytest.mark.parametrize("regime,union", [("same", 8), ("half", 20), ("disjoint", 32)])
def test_regimes(regime, union):
    say("route regime", regime)
    sets = synth.regime_sets(0, 0, regime, 4, 512)
    bias = synth.regime_bias(sets, 512)
    idx, _, _ = _check(synth.token_vectors(0, 0, 4), synth.router_weights(0, 0, 512), 8, bias)
    assert [sorted(r) for r in idx.tolist()] == sets
    assert len(set(idx.reshape(-1).tolist())) == union


def test_workspace_left_zero_and_reusable():
    say("route workspace reuse")
    wr = bf16(synth.router_weights(0, 0, 512))
    x = bf16(synth.token_vectors(0, 0, 2))
    ws = qws.route_workspace(2, 512, "cuda")
    a = qws.moe_route_topk(x, wr, 8, workspace=ws)
    b = qws.moe_route_topk(x, wr, 8, workspace=ws)
    torch.cuda.synchronize()
    counter_off = ((2 * 512 * 4 + 255) // 256) * 256
    counters = ws[counter_off:].cpu().view(torch.int32).numpy()
    assert counters.size >= 17 * 32 and np.all(counters == 0)   # 17 arrival counters, 128 B apart
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
