"""Pins for oracle.moe: closed-form routing cases, exact ties, library top-k/softmax, pure-Python
brute force of the SwiGLU experts at tiny shapes, the one-hot routing that reduces the layer to
shared + one dense FFN (checked against torch's float64 silu/matmul), linearity in the gates."""
import math

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import formats as F
from oracle import moe

TINY = synth.LayerShape(hidden=64, inter=32, n_routed=6, topk=2, has_shared=True)


def _bits(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _tiny_bank(seed=0, shape=TINY, layer=0):
    return {e: synth.expert_np(seed, layer, e, shape) for e in range(shape.n_experts)}


# ----------------------------------------------------------------------------- router
def test_zero_input_routes_to_first_k_with_uniform_weights():
    wr = synth.router_weights(0, 0, 64, 256)
    x = np.zeros((1, 256), dtype=np.uint16)
    idx, w, logits = moe.route(x, wr, 8)
    assert np.all(logits == 0.0)
    assert idx.tolist() == [list(range(8))]
    assert np.all(w == 0.125)


def test_exact_tie_goes_to_lower_index():
    rng = np.random.default_rng(1)
    wr = _bits(rng.standard_normal((16, 64)) * 0.01)
    x = _bits(np.abs(rng.standard_normal((1, 64))))
    wr[11] = _bits(np.full(64, 0.5))   # the two largest rows are identical
    wr[4] = wr[11]
    idx, _, logits = moe.route(x, wr, 3)
    assert logits[0, 4] == logits[0, 11]
    assert idx[0, :2].tolist() == [4, 11]


def test_negative_zero_ties_with_positive_zero():
    logits = np.array([[-1.0, -0.0, 0.0, -2.0]])
    assert moe.topk_select(logits, 2).tolist() == [[1, 2]]


def test_nan_ranks_as_minus_infinity_and_ties_with_it_by_index():
    """A NaN logit ranks below every number and ties with -inf by index (the selection's reading
    of NaN, stated with the router's entry point), written out by hand for a small row."""
    nan, inf = np.nan, np.inf
    logits = np.array([[nan, -inf, 1.0, nan, -inf, -3.0, 0.0]])
    # numbers first (1.0 @2, 0.0 @6, -3.0 @5), then the five -inf/NaN entries in index order
    assert moe.topk_select(logits, 7).tolist() == [[2, 6, 5, 0, 1, 3, 4]]
    assert moe.topk_select(logits, 4).tolist() == [[2, 6, 5, 0]]
    # a row of NaN only: index order, like an all-equal row
    assert moe.topk_select(np.full((1, 5), nan), 3).tolist() == [[0, 1, 2]]
    # brute force: a pure-Python insertion of each index behind every key that beats it
    rng = np.random.default_rng(9)
    row = rng.choice(np.array([nan, -inf, inf, -0.0, 0.0, 1.0, -1.0]), size=40)
    key = [(-inf if math.isnan(v) else float(v)) for v in row]
    order = []
    for i in range(len(row)):
        pos = 0
        while pos < len(order) and (key[order[pos]] > key[i] or key[order[pos]] == key[i]):
            pos += 1
        order.insert(pos, i)
    assert moe.topk_select(row[None], 40)[0].tolist() == order


def test_topk_matches_torch_on_distinct_values():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((5, 512))
    idx = moe.topk_select(logits, 8)
    ref = torch.topk(torch.from_numpy(logits), 8, dim=1, sorted=True).indices.numpy()
    assert np.array_equal(idx, ref)


def test_weights_are_softmax_over_selection_and_sum_to_one():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((4, 64)) * 3
    idx = moe.topk_select(logits, 8)
    w = moe.route_weights(logits, idx)
    sel = np.take_along_axis(logits, idx, 1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
    full = scipy.special.softmax(logits, axis=1)           # full softmax, then renormalise
    ren = np.take_along_axis(full, idx, 1)
    assert np.allclose(w, ren / ren.sum(1, keepdims=True), rtol=1e-12, atol=0)


def test_router_logits_brute_force():
    rng = np.random.default_rng(4)
    wr = _bits(rng.standard_normal((6, 32)) * 0.02)
    x = _bits(rng.standard_normal((2, 32)))
    bias = rng.standard_normal(6).astype(np.float32)
    got = moe.router_logits(x, wr, bias)
    xf, wf = F.bf16_to_f64(x), F.bf16_to_f64(wr)
    for m in range(2):
        for e in range(6):
            want = math.fsum(float(xf[m, k]) * float(wf[e, k]) for k in range(32)) + float(bias[e])
            assert abs(got[m, e] - want) <= 1e-15 * max(1.0, abs(want))


def test_router_permutation_equivariance():
    rng = np.random.default_rng(5)
    wr = _bits(rng.standard_normal((32, 64)) * 0.02)
    x = _bits(rng.standard_normal((3, 64)))
    perm = rng.permutation(32)
    idx, w, _ = moe.route(x, wr, 8)
    idx_p, w_p, _ = moe.route(x, wr[perm], 8)
    assert np.array_equal(perm[idx_p], idx)
    assert np.array_equal(w_p, w)


def test_bias_forces_designated_sets():
    wr = synth.router_weights(0, 0, 512)
    x = synth.token_vectors(0, 0, 4)
    for regime, union in (("same", 8), ("half", 20), ("disjoint", 32)):
        sets = synth.regime_sets(0, 0, regime, 4, 512)
        idx, _, _ = moe.route(x, wr, 8, synth.regime_bias(sets, 512))
        for m in range(4):
            assert sorted(idx[m].tolist()) == sets[m]
        assert len(moe.expert_union(idx, 512)) == union


# ----------------------------------------------------------------------------- experts
def _brute_expert(t, x):
    """Pure-Python SwiGLU expert: bit-level decode, math.fsum dot products, math.exp."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]

    def w(q, s, r, k):
        b = int(q[r][k // 2])
        c = (b >> 4) if k & 1 else (b & 15)
        v = table[c & 7] * (-1.0 if c & 8 else 1.0)
        return v * 2.0 ** (int(s[r][k // 32]) - 127)

    gq, gs, dq, ds = t["gate_up_q"], t["gate_up_s"], t["down_q"], t["down_s"]
    two_i, h = gq.shape[0], gq.shape[1] * 2
    inter = two_i // 2
    hv = [math.fsum(w(gq, gs, r, k) * x[k] for k in range(h)) for r in range(two_i)]
    a = [hv[i] / (1.0 + math.exp(-hv[i])) * hv[inter + i] for i in range(inter)]
    return [math.fsum(w(dq, ds, r, k) * a[k] for k in range(inter)) for r in range(h)]


def test_expert_ffn_brute_force_tiny():
    bank = _tiny_bank()
    x_bits = synth.token_vectors(0, 0, 1, TINY.hidden)
    x = F.bf16_to_f64(x_bits)[0]
    for e in (0, 3, TINY.n_routed):
        got = moe.expert_ffn(*moe.dequant_expert(bank[e]), x)
        want = np.array(_brute_expert(bank[e], list(x)))
        assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_layer_brute_force_tiny():
    bank = _tiny_bank(seed=3)
    x = synth.token_vectors(3, 0, 2, TINY.hidden)
    wr = synth.router_weights(3, 0, TINY.n_routed, TINY.hidden)
    idx, w, _ = moe.route(x, wr, TINY.topk)
    got = moe.moe_layer(x, idx, w, bank, TINY.n_routed)
    xf = F.bf16_to_f64(x)
    for m in range(2):
        want = np.array(_brute_expert(bank[TINY.n_routed], list(xf[m])))
        for i in range(TINY.topk):
            want = want + w[m, i] * np.array(_brute_expert(bank[int(idx[m, i])], list(xf[m])))
        assert np.max(np.abs(got[m] - want)) <= 1e-12 * np.max(np.abs(want))


def _torch_dense_ffn(gate_up, down, x):
    g = torch.from_numpy(gate_up)
    d = torch.from_numpy(down)
    xv = torch.from_numpy(x)
    inter = d.shape[1]
    h = g @ xv
    return (d @ (torch.nn.functional.silu(h[:inter]) * h[inter:])).numpy()


def test_one_hot_routing_is_shared_plus_one_dense_ffn():
    shape = synth.LayerShape(hidden=128, inter=64, n_routed=8, topk=4, has_shared=True)
    bank = {e: synth.expert_np(1, 0, e, shape) for e in range(shape.n_experts)}
    wr = synth.router_weights(1, 0, 8, 128)
    x = synth.token_vectors(1, 0, 1, 128)
    bias = np.full(8, -1000.0, dtype=np.float32)
    bias[5] = 0.0
    idx, w, _ = moe.route(x, wr, 4, bias)
    assert idx[0, 0] == 5 and w[0, 0] == 1.0 and np.all(w[0, 1:] == 0.0)
    y = moe.moe_layer(x, idx, w, bank, 8)
    xf = F.bf16_to_f64(x)[0]
    want = _torch_dense_ffn(*moe.dequant_expert(bank[8]), xf) + _torch_dense_ffn(*moe.dequant_expert(bank[5]), xf)
    assert np.max(np.abs(y[0] - want)) <= 1e-12 * np.max(np.abs(want))
    # K = 1 gives the same layer
    idx1, w1, _ = moe.route(x, wr, 1, bias)
    assert np.array_equal(moe.moe_layer(x, idx1, w1, bank, 8), y)


def test_zero_routed_down_weights_leave_the_shared_expert():
    bank = _tiny_bank(seed=5)
    for e in range(TINY.n_routed):
        bank[e] = dict(bank[e])
        bank[e]["down_q"] = np.zeros_like(bank[e]["down_q"])
    x = synth.token_vectors(5, 0, 1, TINY.hidden)
    idx = np.array([[1, 4]])
    y = moe.moe_layer(x, idx, np.array([[0.7, 0.3]]), bank, TINY.n_routed)
    want = moe.expert_ffn(*moe.dequant_expert(bank[TINY.n_routed]), F.bf16_to_f64(x)[0])
    assert np.array_equal(y[0], want)


def test_layer_is_linear_in_the_gate_weights():
    bank = _tiny_bank(seed=6)
    x = synth.token_vectors(6, 0, 1, TINY.hidden)
    idx = np.array([[2, 5]])
    sh = moe.moe_layer(x, idx, np.zeros((1, 2)), bank, TINY.n_routed)
    y1 = moe.moe_layer(x, idx, np.array([[1.0, 0.0]]), bank, TINY.n_routed) - sh
    y2 = moe.moe_layer(x, idx, np.array([[0.0, 1.0]]), bank, TINY.n_routed) - sh
    y = moe.moe_layer(x, idx, np.array([[0.25, 0.75]]), bank, TINY.n_routed) - sh
    assert np.allclose(y, 0.25 * y1 + 0.75 * y2, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_invalid_expert_id_gives_nan_row():
    bank = _tiny_bank()
    x = synth.token_vectors(0, 0, 2, TINY.hidden)
    y = moe.moe_layer(x, np.array([[0, 1], [2, 99]]), np.full((2, 2), 0.5), bank, TINY.n_routed)
    assert np.all(np.isfinite(y[0])) and np.all(np.isnan(y[1]))


def test_union_of_a_window():
    idx = np.array([[3, 1, 7], [7, 9, 1], [2, 3, 9], [1, 1, 3]])
    assert moe.expert_union(idx, 10) == [1, 2, 3, 7, 9]
    assert moe.expert_union(np.array([[0, 12, -1]]), 10) == [0]


@pytest.mark.parametrize("bad", [[[0, 1, 255]], [[255, 0, 0]]])
def test_dequant_rejects_nan_scales(bad):
    with pytest.raises(ValueError):
        F.mxfp4_dequant(np.zeros((1, 48), dtype=np.uint8), np.array(bad, dtype=np.uint8))
