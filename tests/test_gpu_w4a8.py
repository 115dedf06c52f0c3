"""GPU parity of the W4A8 MoE layer (moe_layer_w4a8 / moe_layers_w4a8: MXFP4 weights x MXFP8
activations) against the W4A8 oracle.

The float32 SwiGLU output a decides its own E4M3 codes, so parity is taken in three parts, each
against the oracle (the S3 pattern of the router's top-k):
(i) the GPU's a of every (token, expert) matches the oracle's float64 a within the float tolerance;
(ii) the GPU's codes and scale bytes are, bit for bit, the oracle's MXFP8 conversion of the GPU's
     own float32 a;
(iii) the GPU's y matches the oracle's down projection and combine applied to those codes.
End to end, y also stays within 5e-3 of the float64 oracle, well apart from the bf16 layer's
(~5e-2 here). Tolerances (max|err| / max|ref|): 5e-4 for (i) and (iii), from the scaled matrix
instruction's internal accumulation (~1e-4 of an op's largest output) with margin; measured
~3e-5 and ~8e-5; end to end 5e-3, the codes that float32 rounds the other way adding up to
~4e-4 measured."""
import numpy as np
import pytest
import torch

import quantized_weight_streaming_amd as qws
import synth
from oracle import formats as OF
from oracle import moe as OM
from oracle import w4a8 as OW

from .helpers import Layer, assert_close, check_topk, rel_err, say
from .test_gpu_experts import TINY, _assert_bf16_is_rne_of_f32
from .test_gpu_fused import _packed

pytestmark = pytest.mark.gpu

TOL_A8 = 5e-4


def _act_buffer(shape, M):
    na = (shape.n_routed + 1) * M * shape.inter
    return torch.zeros(na * 5 + na // 32, dtype=torch.uint8, device="cuda")


def _w4a8(layer: Layer, ws=None):
    lg = torch.empty((layer.M, layer.shape.n_routed), dtype=torch.float32, device="cuda")
    L = qws.MoeLayer(layer.x_t, layer.wr_t, _packed(layer), layer.shape.topk, bias=layer.bias_t, logits_out=lg)
    buf = _act_buffer(layer.shape, layer.M)
    qws.debug_w4a8_act_buffer(buf)
    try:
        qws.moe_layer_w4a8(L, workspace=ws)
        torch.cuda.synchronize()
    finally:
        qws.debug_w4a8_act_buffer(None)
    return L, buf.cpu().numpy()


def _check_w4a8(layer: Layer, L, buf):
    shape, M = layer.shape, layer.M
    E, I = shape.n_routed, shape.inter
    ridx, rw, rlg = layer.oracle_route()
    assert check_topk(L.topk_idx.cpu().numpy(), L.logits_out.cpu().numpy(), rlg, shape.topk,
                      gpu_w=L.topk_w.cpu().numpy()) == 0
    experts = {e: layer.expert(e) for e in set(ridx.reshape(-1).tolist()) | {E} if 0 <= e <= E}
    y_ref, acts = OW.moe_layer_w4a8(layer.x, ridx, rw, experts, E, shape.has_shared, detail=True)
    na = (E + 1) * M * I
    a_gpu = buf[:na * 4].view(np.float32).reshape(E + 1, M, I)
    c_gpu = buf[na * 4:na * 5].reshape(E + 1, M, I)
    s_gpu = buf[na * 5:na * 5 + na // 32].reshape(E + 1, M, I // 32)
    y_codes = np.zeros((M, shape.hidden))
    worst_a = 0.0
    for (m, e), (we, a_ref) in acts.items():
        a = a_gpu[e, m].astype(np.float64)
        # (i) the activations themselves, float32 against float64
        worst_a = max(worst_a, assert_close(a, a_ref, tol=TOL_A8, what=f"a of token {m}, expert {e}"))
        # (ii) the quantisation decision, taken on the GPU's own values
        c_want, s_want = OW.mxfp8_quantize(a)
        assert np.array_equal(c_gpu[e, m], c_want), f"codes of token {m}, expert {e}"
        assert np.array_equal(s_gpu[e, m], s_want), f"scales of token {m}, expert {e}"
        # (iii) down + combine of those codes
        dn = OF.mxfp4_dequant(experts[e]["down_q"], experts[e]["down_s"])
        y_codes[m] += we * (dn @ OW.mxfp8_dequant(c_gpu[e, m], s_gpu[e, m]))
    y = L.y_f32.cpu().numpy()
    e3 = assert_close(y, y_codes, tol=TOL_A8, what=f"y from the GPU's codes, seed={layer.seed} M={M}")
    _assert_bf16_is_rne_of_f32(L.y_bf16, L.y_f32)
    e_end = rel_err(y, y_ref)
    y16 = OM.moe_layer(layer.x, ridx, rw, experts, E, shape.has_shared)
    e_bf16 = rel_err(y, y16)
    say(f"w4a8 seed={layer.seed} M={M}: a {worst_a:.2e}, y(codes) {e3:.2e}, y(oracle) {e_end:.2e}, "
        f"y(bf16 oracle) {e_bf16:.2e}")
    assert e_end <= 5e-3 and e_end < e_bf16
    return e3


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("si", range(len(TINY)))
def test_w4a8_small_layers(M, si):
    shape = TINY[si]
    say("w4a8 small", M, shape)
    layer = Layer(40 + si, M, shape, M)
    _check_w4a8(layer, *_w4a8(layer))


@pytest.mark.parametrize("E", [64, 512])
def test_w4a8_layer_m1(E):
    say("w4a8 layer M=1 E", E)
    layer = Layer(0, 0, synth.LayerShape(n_routed=E), 1)
    _check_w4a8(layer, *_w4a8(layer))


@pytest.mark.parametrize("regime", ["same", "half", "disjoint", "natural"])
def test_w4a8_window_m4(regime):
    say("w4a8 M=4", regime)
    bias = None if regime == "natural" else synth.regime_bias(synth.regime_sets(0, 0, regime, 4, 512), 512)
    layer = Layer(0, 0, synth.LayerShape(), 4, bias=bias)
    _check_w4a8(layer, *_w4a8(layer))


def test_w4a8_routing_equals_the_bf16_layer():
    """Same router, top-K and gate weights as the bf16 layer, bit for bit; different y."""
    say("w4a8 vs bf16 layer routing")
    layer = Layer(2, 0, synth.LayerShape(), 2)
    L8, _ = _w4a8(layer)
    L16 = qws.moe_layer_mxfp4(qws.MoeLayer(layer.x_t, layer.wr_t, _packed(layer), 8,
                                           logits_out=torch.empty((2, 512), dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    assert np.array_equal(L8.topk_idx.cpu().numpy(), L16.topk_idx.cpu().numpy())
    assert np.array_equal(L8.topk_w.cpu().numpy().view(np.uint32), L16.topk_w.cpu().numpy().view(np.uint32))
    assert np.array_equal(L8.logits_out.cpu().numpy().view(np.uint32), L16.logits_out.cpu().numpy().view(np.uint32))
    assert rel_err(L8.y_f32.cpu().numpy(), L16.y_f32.cpu().numpy()) > 1e-3


@pytest.mark.parametrize("M", [1, 4])
def test_w4a8_multi_layer_launch(M):
    """Three layers in one launch equal three one-layer launches bit for bit, and the workspace
    stays healthy."""
    say("w4a8 multi-layer launch M", M)
    shape = synth.LayerShape()
    layers = [Layer(50, l, shape, M) for l in range(3)]
    Ls = [qws.MoeLayer(t.x_t, t.wr_t, _packed(t), 8) for t in layers]
    ws = qws.moe_layer_workspace(M, 8, 512, 2560, 768, "cuda")
    qws.moe_layers_w4a8(qws.MoeLayers(Ls), ws)
    torch.cuda.synchronize()
    for t, L in zip(layers, Ls):
        single = qws.moe_layer_w4a8(qws.MoeLayer(t.x_t, t.wr_t, _packed(t), 8), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(single.y_f32.cpu().numpy().view(np.uint32), L.y_f32.cpu().numpy().view(np.uint32))
        assert np.array_equal(single.topk_idx.cpu().numpy(), L.topk_idx.cpu().numpy())
    assert qws.moe_workspace_errors(ws, M, 8, 512, 768) == 0
    # the first layer against the oracle as well
    L0, buf = _w4a8(layers[0], ws)
    _check_w4a8(layers[0], L0, buf)
