"""GPU parity of the fused one-launch MoE layer (moe_layer_mxfp4) and of the multi-layer launch
(moe_layers_mxfp4) against the oracle and against the two-call path; the task-major pack; chained
sequences (x of layer l+1 = y of layer l) against an oracle chain; graph replay; the full 42-layer
decode step."""
import numpy as np
import pytest
import torch

import quantized_weight_streaming_amd as qws
import synth

from .helpers import Layer, assert_close, check_topk, say
from .test_gpu_experts import TINY, _assert_bf16_is_rne_of_f32, _bank

pytestmark = pytest.mark.gpu


def _packed(layer: Layer):
    if not hasattr(layer, "_packed"):
        layer._packed = qws.moe_pack_mxfp4(_bank(layer))
    return layer._packed


def _fused(layer: Layer, ws=None, logits=True):
    lg = torch.empty((layer.M, layer.shape.n_routed), dtype=torch.float32, device="cuda") if logits else None
    L = qws.MoeLayer(layer.x_t, layer.wr_t, _packed(layer), layer.shape.topk, bias=layer.bias_t, logits_out=lg)
    qws.moe_layer_mxfp4(L, workspace=ws)
    return L


def _check_layer(layer: Layer, L):
    ridx, rw, rlg = layer.oracle_route()
    near = check_topk(L.topk_idx.cpu().numpy(), L.logits_out.cpu().numpy(), rlg, layer.shape.topk,
                      gpu_w=L.topk_w.cpu().numpy())
    assert near == 0
    e = assert_close(L.y_f32.cpu().numpy(), layer.oracle_y(ridx, rw), what=f"fused layer seed={layer.seed} M={layer.M}")
    _assert_bf16_is_rne_of_f32(L.y_bf16, L.y_f32)
    assert_close(L.topk_w.cpu().numpy(), rw, tol=1e-5, what="gate weights")
    return e


def _task_major(bank: dict, n: int, H: int, I: int) -> np.ndarray:
    """The task-major records, built by moving bytes of the canonical bank as the header states
    (piece p of lane l = 16 g + i of wave w = 4 rg + ks in record (e, j))."""
    J, nch = I // 32, H // 32
    gq, gs, dq, ds = (bank[k].reshape(n, -1, bank[k].shape[-1]) for k in ("gate_up_q", "gate_up_s", "down_q", "down_s"))
    w = np.arange(16)[:, None]
    lane = np.arange(64)[None, :]
    g, i, rg, ks = lane >> 4, lane & 15, w >> 2, w & 3
    out = np.zeros((n, J, 8, 16, 64, 16), np.uint8)
    b16 = np.arange(16)
    for e in range(n):
        for j in range(J):
            grow = np.where(rg >= 2, I, 0) + 32 * j + 16 * (rg & 1) + i            # [16, 64]
            for t in range(5):
                c = 20 * ks + 4 * t + g
                ok = c < nch
                cc = np.minimum(c, nch - 1)
                out[e, j, 1 + t] = np.where(ok[..., None], gq[e][grow[..., None], 16 * cc[..., None] + b16], 0)
                out[e, j, 0, :, :, 8 + t] = np.where(ok, gs[e][grow, cc], 0)
            def tile_row(q):   # [16, 64, 16] bytes: row i of tile q of wave w (zero past H or q > 9)
                row = 16 * (w + 16 * q) + i
                ok = (q < 10) & (row < H)
                rr = np.minimum(row, H - 1)
                return np.where(ok[..., None], dq[e][rr[..., None], 16 * j + b16], 0)
            for p in (6, 7):
                out[e, j, p] = tile_row(4 * (p - 6) + g)
            half = tile_row(8 + (g & 1))                                          # tiles 8, 9
            out[e, j, 0, :, :, :8] = np.take_along_axis(half, 8 * (g[..., None] >> 1) + np.arange(8), axis=-1)
            for Q in range(3):
                q = 4 * Q + g
                row = 16 * (w + 16 * q) + i
                ok = (q < 10) & (row < H)
                out[e, j, 0, :, :, 13 + Q] = np.where(ok, ds[e][np.minimum(row, H - 1), j], 0)
    return out.reshape(n, J, 8 * 16 * 64 * 16)


@pytest.mark.parametrize("si", range(len(TINY)))
def test_pack_is_the_task_major_relayout(si):
    """moe_pack_mxfp4 moves bytes only, to the places the header states (zeros past H)."""
    shape = TINY[si]
    say("pack", shape)
    layer = Layer(40 + si, 0, shape, 1)
    pk = _packed(layer)
    torch.cuda.synchronize()
    n, H, I = shape.n_routed + int(shape.has_shared), shape.hidden, shape.inter
    bank = {k: layer.bank_t[k].cpu().numpy() for k in ("gate_up_q", "gate_up_s", "down_q", "down_s")}
    assert np.array_equal(pk.gate_up_q.cpu().numpy(), _task_major(bank, n, H, I))
    assert pk.layout == "task_major" and pk.gate_up_s is None


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("si", range(len(TINY)))
def test_fused_small_layers(M, si):
    shape = TINY[si]
    say("fused small", M, shape)
    layer = Layer(20 + si, M, shape, M)
    _check_layer(layer, _fused(layer))


@pytest.mark.parametrize("E", [64, 512])
def test_fused_layer_m1(E):
    say("fused layer M=1 E", E)
    _check_layer(Layer(0, 0, synth.LayerShape(n_routed=E), 1), _fused(Layer(0, 0, synth.LayerShape(n_routed=E), 1)))


@pytest.mark.parametrize("M", [1, 2, 4])
def test_fused_layer_1024_experts(M):
    """More than 512 routed experts: a lane holds 16 logits in the selection and a workgroup
    computes four router rows."""
    say("fused layer E=1024 M", M)
    layer = Layer(3, 0, synth.LayerShape(hidden=256, inter=64, n_routed=1024), M)
    _check_layer(layer, _fused(layer))


def test_fused_layer_zipf():
    say("fused layer zipf")
    layer = Layer(1, 0, synth.LayerShape(), 1, bias=synth.zipf_bias(1, 0, 512))
    _check_layer(layer, _fused(layer))


@pytest.mark.parametrize("regime,union", [("same", 8), ("half", 20), ("disjoint", 32), ("natural", None)])
def test_fused_window_m4(regime, union):
    say("fused M=4", regime)
    bias = None if regime == "natural" else synth.regime_bias(synth.regime_sets(0, 0, regime, 4, 512), 512)
    layer = Layer(0, 0, synth.LayerShape(), 4, bias=bias)
    L = _fused(layer)
    _check_layer(layer, L)
    if union:
        assert len(set(L.topk_idx.cpu().numpy().reshape(-1).tolist())) == union


def _zero_router(layer: Layer) -> Layer:
    layer.wr = np.zeros_like(layer.wr)
    layer.wr_t = torch.zeros_like(layer.wr_t)
    return layer


@pytest.mark.parametrize("M", [1, 4])
def test_fused_all_logits_tied(M):
    """Zero router weights: every logit is 0.0 and all 512 experts tie (far more candidates than
    one wave holds), so the selection is experts 0 .. K-1 (ties go to the lower index) with
    weights 1/K, and y follows the oracle."""
    say("fused all tied", M)
    layer = _zero_router(Layer(0, 0, synth.LayerShape(), M))
    L = _fused(layer)
    K = layer.shape.topk
    ridx, rw, _ = layer.oracle_route()
    assert np.array_equal(ridx, np.tile(np.arange(K), (M, 1)))
    assert L.topk_idx.cpu().numpy().tolist() == ridx.tolist()
    assert np.all(L.topk_w.cpu().numpy() == np.float32(1.0 / K))
    assert_close(L.y_f32.cpu().numpy(), layer.oracle_y(ridx, rw), what=f"all tied M={M}")


@pytest.mark.parametrize("n_tied", [40, 100])
@pytest.mark.parametrize("M", [1, 3])
def test_fused_many_tied_candidates(M, n_tied):
    """Zero router weights and a bias of 1.0 on n_tied seeded experts: those tie above the rest and
    the K lowest indices among them are selected. Every lane group (experts with lane // 8 = g,
    lane = e % 64) holds one of them, so the candidates are exactly the tied experts: 40 fit in one
    wave (the in-wave sort), 100 do not (the ranking across waves)."""
    say("fused tied", n_tied, M)
    shape = synth.LayerShape()
    top = np.random.default_rng(11).choice(shape.n_routed, n_tied, replace=False)
    assert len(set(((top % 64) // 8).tolist())) == 8
    bias = np.zeros(shape.n_routed, dtype=np.float32)
    bias[top] = 1.0
    layer = _zero_router(Layer(0, 0, shape, M, bias=bias))
    L = _fused(layer)
    ridx, rw, _ = layer.oracle_route()
    want = np.sort(top)[:shape.topk]
    assert np.array_equal(ridx, np.tile(want, (M, 1)))
    assert L.topk_idx.cpu().numpy().tolist() == ridx.tolist()
    assert_close(L.y_f32.cpu().numpy(), layer.oracle_y(ridx, rw), what=f"{n_tied} tied M={M}")


def test_fused_matches_two_call_routing():
    say("fused vs two-call")
    layer = Layer(8, 0, synth.LayerShape(), 4)
    L = _fused(layer)
    idx, w = qws.moe_route_topk(layer.x_t, layer.wr_t, 8)
    assert torch.equal(idx.cpu(), L.topk_idx.cpu())
    assert torch.equal(w.cpu().view(torch.int32), L.topk_w.cpu().view(torch.int32))
    _, y32 = qws.moe_expert_gemv_mxfp4(_bank(layer), layer.x_t, idx, w)
    # the same products in another arithmetic: the fused layer's gate/up runs on the scaled FP4 x FP8
    # matrix op (x as two exact E4M3 parts), whose internal accumulation of 128 products is less
    # precise than float32 (measured on MI355X: up to ~8e-5 of one op's largest output), then the
    # down projection sums per block of 32 activations; 5e-5 of max|y| bounds the difference with
    # margin (measured 6e-6), far inside the 2e-3 both paths keep against the oracle
    assert_close(L.y_f32.cpu().numpy(), y32.cpu().numpy(), tol=5e-5, what="fused vs two-call")


def test_fused_deterministic_and_workspace_healthy():
    say("fused determinism")
    layer = Layer(9, 0, synth.LayerShape(), 2)
    ws = qws.moe_layer_workspace(2, 8, 512, 2560, 768, "cuda")
    a = _fused(layer, ws).y_f32.cpu().numpy()
    b = _fused(layer, ws).y_f32.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert qws.moe_workspace_errors(ws, 2, 8, 512, 768) == 0


def _multi(n, M, seed=30):
    shape = synth.LayerShape()
    layers = [Layer(seed, l, shape, M) for l in range(n)]
    Ls = [qws.MoeLayer(t.x_t, t.wr_t, _packed(t), 8) for t in layers]
    return layers, Ls, qws.MoeLayers(Ls)


@pytest.mark.parametrize("M", [1, 4])
def test_multi_layer_launch(M):
    say("multi-layer launch M", M)
    layers, Ls, seq = _multi(3, M)
    ws = qws.moe_layer_workspace(M, 8, 512, 2560, 768, "cuda")
    seq.run(ws)
    torch.cuda.synchronize()
    for t, L in zip(layers, Ls):
        ridx, rw, _ = t.oracle_route()
        assert np.array_equal(L.topk_idx.cpu().numpy(), ridx)
        assert_close(L.y_f32.cpu().numpy(), t.oracle_y(ridx, rw), what=f"layer {t.layer}")
        single = qws.moe_layer_mxfp4(qws.MoeLayer(t.x_t, t.wr_t, _packed(t), 8), workspace=ws)
        assert np.array_equal(single.y_f32.cpu().numpy().view(np.uint32), L.y_f32.cpu().numpy().view(np.uint32))
    assert qws.moe_workspace_errors(ws, M, 8, 512, 768) == 0


def test_multi_layer_graph_replay():
    say("multi-layer graph replay")
    layers, Ls, seq = _multi(4, 1, seed=31)
    ws = qws.moe_layer_workspace(1, 8, 512, 2560, 768, "cuda")
    seq.run(ws)
    torch.cuda.synchronize()
    ref = [L.y_f32.clone() for L in Ls]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq.run(ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq.run(ws)
    for i in range(5):
        for L in Ls:
            L.y_f32.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for L, r in zip(Ls, ref):
            assert torch.equal(L.y_f32.view(torch.int32), r.view(torch.int32)), f"replay {i}"
        seq.run(ws)                                                  # eager work between replays
        torch.cuda.synchronize()
    assert qws.moe_workspace_errors(ws, 1, 8, 512, 768) == 0


def test_decode_step_42_layers_sampled():
    """The full decode step's 42 layers (67.6 GB of seeded MXFP4 banks, packed task-major) in one launch; sampled
    layers against the oracle, all layers' routing against the oracle's."""
    say("decode step 42 layers")
    shape = synth.LayerShape()
    Ls, xs, wrs = [], [], []
    for l in range(synth.N_LAYERS):
        bank_t = synth.expert_bank_torch(0, l, shape, device="cuda")   # freed once packed
        wr = synth.router_weights(0, l, 512)
        x = synth.token_vectors(0, l, 1)
        wrs.append(wr)
        xs.append(x)
        from .helpers import bf16
        Ls.append(qws.MoeLayer(bf16(x), bf16(wr), qws.moe_pack_mxfp4(qws.ExpertBank.from_dict(bank_t, 512, True)), 8))
    seq = qws.MoeLayers(Ls)
    ws = qws.moe_layer_workspace(1, 8, 512, 2560, 768, "cuda")
    say("decode step: run")
    seq.run(ws)
    torch.cuda.synchronize()
    from oracle import moe as OM
    for l in range(synth.N_LAYERS):
        ridx, rw, _ = OM.route(xs[l], wrs[l], 8)
        assert np.array_equal(Ls[l].topk_idx.cpu().numpy(), ridx), f"layer {l} routing"
        if l in (0, 17, 41):
            experts = {e: synth.expert_np(0, l, e, shape) for e in set(ridx.reshape(-1).tolist()) | {512}}
            ref = OM.moe_layer(xs[l], ridx, rw, experts, 512)
            assert_close(Ls[l].y_f32.cpu().numpy(), ref, what=f"decode step layer {l}")
    assert qws.moe_workspace_errors(ws, 1, 8, 512, 768) == 0


# ------------------------------------------------------------------------------- chained sequences
def _chain(n, M, shape, seed):
    """Layers whose x is the previous layer's y_bf16 (layer 0 from the seeded token vectors)."""
    layers = [Layer(seed, l, shape, M) for l in range(n)]
    Ls = []
    for l, t in enumerate(layers):
        x = t.x_t if l == 0 else Ls[-1].y_bf16
        lg = torch.empty((M, shape.n_routed), dtype=torch.float32, device="cuda")
        Ls.append(qws.MoeLayer(x, t.wr_t, _packed(t), shape.topk, logits_out=lg))
    return layers, Ls, qws.MoeLayers(Ls)


def _oracle_chain_check(layers, Ls):
    """Each layer of the chain against the oracle, on the input the layer had: x_{l+1} is the
    kernel's bf16 y_l, whose rounding (RNE of the kernel's float32 y_l, checked bit for bit) is a
    decision taken in the kernel's precision; the oracle's float64 y_l would round some elements
    the other way, and with |y| growing ~40x per layer those flips compound along a chain.
    Routing must agree up to near-ties; after a layer whose routing needed the near-tie allowance,
    later layers are not compared. Returns layers compared."""
    compared = 0
    for l, (t, L) in enumerate(zip(layers, Ls)):
        if l > 0:
            t.x = Ls[l - 1].y_bf16.cpu().view(torch.int16).numpy().view(np.uint16)
        ridx, rw, rlg = t.oracle_route()
        near = check_topk(L.topk_idx.cpu().numpy(), L.logits_out.cpu().numpy(), rlg, t.shape.topk,
                          gpu_w=L.topk_w.cpu().numpy())
        if near:
            break
        y = t.oracle_y(ridx, rw)
        assert_close(L.y_f32.cpu().numpy(), y, what=f"chained layer {t.layer} M={t.M}")
        _assert_bf16_is_rne_of_f32(L.y_bf16, L.y_f32)
        compared += 1
    return compared


@pytest.mark.parametrize("M", [1, 4])
def test_chained_sequence_vs_oracle_chain(M):
    say("chained sequence M", M)
    layers, Ls, seq = _chain(4, M, synth.LayerShape(), seed=50 + M)
    ws = qws.moe_layer_workspace(M, 8, 512, 2560, 768, "cuda")
    seq.run(ws)
    torch.cuda.synchronize()
    assert qws.moe_workspace_errors(ws, M, 8, 512, 768) == 0
    assert _oracle_chain_check(layers, Ls) >= 1


@pytest.mark.parametrize("M,shape", [(1, synth.LayerShape()), (4, synth.LayerShape()), (2, TINY[1])])
def test_chained_sequence_matches_layer_by_layer(M, shape):
    """The barrier-free chained launch equals launching the layers one by one, bit for bit."""
    say("chained vs single M", M, shape)
    layers, Ls, seq = _chain(3, M, shape, seed=60 + M)
    ws = qws.moe_layer_workspace(M, shape.topk, shape.n_routed, shape.hidden, shape.inter, "cuda")
    seq.run(ws)
    torch.cuda.synchronize()
    chained = [(L.y_f32.clone(), L.topk_idx.clone()) for L in Ls]
    for L in Ls:                                           # x of layer l is y_bf16 of layer l-1
        qws.moe_layer_mxfp4(L, workspace=ws)
    torch.cuda.synchronize()
    for l, (L, (y, idx)) in enumerate(zip(Ls, chained)):
        assert torch.equal(idx, L.topk_idx), f"layer {l} routing"
        assert torch.equal(y.view(torch.int32), L.y_f32.view(torch.int32)), f"layer {l} output"
    assert qws.moe_workspace_errors(ws, M, shape.topk, shape.n_routed, shape.inter) == 0


def test_chained_graph_replay():
    say("chained graph replay")
    layers, Ls, seq = _chain(4, 1, synth.LayerShape(), seed=70)
    ws = qws.moe_layer_workspace(1, 8, 512, 2560, 768, "cuda")
    seq.run(ws)
    torch.cuda.synchronize()
    ref = [L.y_f32.clone() for L in Ls]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq.run(ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq.run(ws)
    for i in range(5):
        for L in Ls:
            L.y_f32.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for L, r in zip(Ls, ref):
            assert torch.equal(L.y_f32.view(torch.int32), r.view(torch.int32)), f"replay {i}"
        seq.run(ws)
        torch.cuda.synchronize()
    assert qws.moe_workspace_errors(ws, 1, 8, 512, 768) == 0


def _error_word_offset(ws: torch.Tensor) -> int:
    """Byte offset of the timeout count in a fused-layer workspace, found through the ABI: with
    every 32-bit word of the workspace holding its own index, moe_workspace_errors returns the index
    of the word it reads."""
    ws.view(torch.int32).copy_(torch.arange(ws.numel() // 4, dtype=torch.int32, device=ws.device))
    idx = qws.moe_workspace_errors(ws, 1, 8, 512, 768)
    ws.zero_()
    return 4 * idx


def test_earlier_timeouts_do_not_end_later_launches():
    """A timeout recorded by an earlier launch (the count and the give-up word, written here from the
    host) does not end the waits of a later launch: its outputs equal a healthy workspace's, bit for
    bit, and it adds nothing to the count. The give-up word is the 64-bit word 64 bytes after the
    32-bit count, holding the timed-out launch's number + 1; the launch counter (64-bit, 128 bytes
    before the count) holds the number of workgroups started in earlier launches."""
    say("stale timeout flag")
    layer = Layer(12, 0, synth.LayerShape(), 1)
    ref = _fused(layer).y_f32.clone()
    ws = qws.moe_layer_workspace(1, 8, 512, 2560, 768, "cuda")
    off = _error_word_offset(ws)
    _fused(layer, ws)                              # launch 0
    torch.cuda.synchronize()
    started = int(ws[off - 128:off - 120].view(torch.int64).item())
    G = torch.cuda.get_device_properties(0).multi_processor_count
    assert started == G                            # one workgroup per compute unit, one launch
    ws[off:off + 4].view(torch.int32).fill_(7)     # seven earlier timeouts
    ws[off + 64:off + 72].view(torch.int64).fill_(1)   # ... the last of them in launch 0
    for i in range(3):
        L = _fused(layer, ws)
        torch.cuda.synchronize()
        assert torch.equal(L.y_f32.view(torch.int32), ref.view(torch.int32)), f"launch {i + 1}"
        assert qws.moe_workspace_errors(ws, 1, 8, 512, 768) == 7
        ws[off + 64:off + 72].view(torch.int64).fill_(i + 2)   # as if this launch had timed out


@pytest.mark.parametrize("mode,M", [("single", 1), ("single", 4), ("independent", 1), ("chained", 1), ("chained", 4)])
def test_tag_wraparound_clears_stale_words(mode, M):
    """The 32-bit tags repeat after 2^20 launches on one workspace; the launch that starts the new
    cycle clears every tagged word (all copies of the polled words included) before any use. The
    launch counter is set from the host so that the next launch is number 2^20, whose tags equal
    launch 0's, after a launch 0 on other inputs whose words would otherwise pass for the new
    launch's: the outputs equal those of a fresh workspace, bit for bit, and nothing times out."""
    say("tag wrap-around", mode, M)
    shape = synth.LayerShape()
    G = torch.cuda.get_device_properties(0).multi_processor_count

    def make(seed):
        if mode == "single":
            t = Layer(seed, 0, shape, M)
            L = qws.MoeLayer(t.x_t, t.wr_t, _packed(t), shape.topk)
            return [L], (lambda ws: qws.moe_layer_mxfp4(L, workspace=ws))
        if mode == "independent":
            Ls = [qws.MoeLayer(t.x_t, t.wr_t, _packed(t), shape.topk) for t in (Layer(seed, l, shape, M) for l in range(3))]
        else:
            _, Ls, _ = _chain(3, M, shape, seed)
        seq = qws.MoeLayers(Ls)
        return Ls, (lambda ws: seq.run(ws))

    def outputs(Ls):
        return [L.y_f32.clone() for L in Ls]

    La, run_a = make(70)
    Lb, run_b = make(71)
    fresh = qws.moe_layer_workspace(M, shape.topk, shape.n_routed, shape.hidden, shape.inter, "cuda")
    run_b(fresh)
    torch.cuda.synchronize()
    ref = outputs(Lb)
    ws = qws.moe_layer_workspace(M, shape.topk, shape.n_routed, shape.hidden, shape.inter, "cuda")
    off = _error_word_offset(ws)
    run_a(ws)                                              # launch 0
    torch.cuda.synchronize()
    assert int(ws[off - 128:off - 120].view(torch.int64).item()) == G
    ws[off - 128:off - 120].view(torch.int64).fill_((1 << 20) * G)   # 2^20 launches started
    for i in range(2):                                     # launches 2^20 (clears) and 2^20 + 1
        run_b(ws)
        torch.cuda.synchronize()
        for l, (L, y) in enumerate(zip(Lb, ref)):
            assert torch.equal(L.y_f32.view(torch.int32), y.view(torch.int32)), f"launch {i}, layer {l}"
        assert qws.moe_workspace_errors(ws, M, shape.topk, shape.n_routed, shape.inter) == 0
