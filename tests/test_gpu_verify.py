"""GPU parity of the greedy verification epilogue (lmhead_verify_greedy_fp8): its logits equal the
FP8 head GEMV's bit for bit, each position's target is the argmax of those logits (ties to the
lower row) and agrees with the oracle's argmax wherever the top-2 gap allows, and the emitted
tokens follow the oracle's acceptance rule on windows built to accept 0 .. M-1 drafts; ragged
small heads, exact ties, the full 157,184-row head, and repeated calls on one workspace."""
import numpy as np
import pytest
import torch

import quantized_weight_streaming_amd as qws
import synth
from oracle import lmhead as OL
from oracle import verify as OV

from .helpers import ARGMAX_GAP, bf16, check_argmax, say

pytestmark = pytest.mark.gpu


def _run(h8, xt, draft, ws, logits=True):
    M = xt.shape[0]
    lg = torch.empty((M, h8.rows), dtype=torch.float32, device="cuda") if logits else None
    d = None if draft is None else torch.tensor(np.asarray(draft, dtype=np.int32), device="cuda")
    out = qws.lmhead_verify_greedy_fp8(h8, xt, d, ws, logits=lg)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, (None if lg is None else lg.cpu().numpy())


def _check_window(res, lg, draft):
    """The targets are the argmax of the kernel's own logits; the emitted prefix follows the oracle."""
    assert res["target"].tolist() == OV.argmax_first(lg).tolist()
    n, emitted = OV.greedy_accept(res["target"], np.asarray(draft, dtype=np.int64))
    assert int(res["n"][0]) == n
    assert res["emitted"][:n].tolist() == emitted.tolist()
    assert res["emitted"][n:].tolist() == [-1] * (len(res["emitted"]) - n)


def _drafts(target, rows):
    """For a = 0 .. M-1: drafts equal to the targets before position a and different at a."""
    M = len(target)
    out = []
    for a in range(M):
        d = [int(t) for t in target[:M - 1]]
        if a < M - 1:
            d[a] = (int(target[a]) + 1) % rows
        out.append(d)
    return out


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("rows,cols", [(1, 32), (999, 96), (4093, 256), (5000, 2560)])
def test_verify_small(M, rows, cols):
    say("verify small", M, rows, cols)
    w = synth.bf16_normal(4, 0, synth.HEAD, rows + cols, (rows, cols), 0.02)
    x = synth.token_vectors(4, 1, M, cols)
    xt = bf16(x)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    ws = qws.verify_workspace(M, "cuda")
    gemv = qws.lmhead_gemv_fp8(h8, xt).cpu().numpy()
    codes, scales = OL.fp8_rowquant(w)
    ref = OL.lmhead_fp8(codes, scales, x)
    res, lg = _run(h8, xt, [0] * (M - 1), ws)
    assert np.array_equal(lg.view(np.uint32), gemv.view(np.uint32))
    if rows > 1:   # the top-2 gap rule needs two rows
        check_argmax(lg, ref)
    else:
        assert res["target"].tolist() == [0] * M
    for draft in _drafts(res["target"], rows):
        res, lg = _run(h8, xt, draft, ws)
        _check_window(res, lg, draft)


def test_verify_exact_ties_go_to_the_lower_row():
    say("verify ties")
    rows, cols = 3000, 256
    w = synth.bf16_normal(5, 0, synth.HEAD, 0, (rows, cols), 0.02).copy()
    x = synth.token_vectors(5, 0, 2, cols)
    w[2500] = w[7] = w[1234] = np.where(x[0] & 0x8000, 0xC000, 0x4000)   # bf16 +-2 aligned with token 0
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    res, lg = _run(h8, bf16(x), [7], qws.verify_workspace(2, "cuda"))
    assert lg[0, 7] == lg[0, 1234] == lg[0, 2500] == lg[0].max()
    assert int(res["target"][0]) == 7
    _check_window(res, lg, [7])


def test_verify_workspace_is_reused():
    say("verify reuse")
    w = synth.bf16_normal(6, 0, synth.HEAD, 0, (4097, 544), 0.02)
    x = synth.token_vectors(6, 0, 4, 544)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    ws = qws.verify_workspace(4, "cuda")
    a, la = _run(h8, bf16(x), [1, 2, 3], ws)
    for _ in range(3):
        b, lb = _run(h8, bf16(x), [1, 2, 3], ws, logits=False)
        assert all(np.array_equal(a[k], b[k]) for k in a)
    _check_window(a, la, [1, 2, 3])


def test_verify_full_head_window():
    say("verify full head")
    w = synth.head_weights(0)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    x = synth.token_vectors(0, 8, 4)
    xt = bf16(x)
    ws = qws.verify_workspace(4, "cuda")
    res, lg = _run(h8, xt, [0, 0, 0], ws)
    assert np.array_equal(lg.view(np.uint32), qws.lmhead_gemv_fp8(h8, xt).cpu().numpy().view(np.uint32))
    codes, scales = OL.fp8_rowquant(w)
    ref = OL.lmhead_fp8(codes, scales, x)
    assert check_argmax(lg, ref, ARGMAX_GAP) >= 1
    for draft in _drafts(res["target"], h8.rows):
        res, lg = _run(h8, xt, draft, ws)
        _check_window(res, lg, draft)


def test_verify_in_a_hip_graph():
    """The head GEMV and both verification epilogues captured in one HIP graph: every replay (with
    eager work between the replays) equals the eager result."""
    say("verify graph replay")
    rows, cols = 6000, 512
    w = synth.bf16_normal(19, 0, synth.HEAD, 0, (rows, cols), 0.02)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    x = bf16(synth.token_vectors(19, 0, 4, cols))
    d = torch.tensor([1, 2, 3], dtype=torch.int32, device="cuda")
    u = torch.tensor([0.2, 0.4, 0.6, 0.8], dtype=torch.float32, device="cuda")
    ws_g, ws_s = qws.verify_workspace(4, "cuda"), qws.verify_workspace(4, "cuda")
    lg = torch.empty((4, rows), dtype=torch.float32, device="cuda")
    g_out = qws.lmhead_verify_greedy_fp8(h8, x, d, ws_g, logits=lg)
    s_out = qws.lmhead_verify_sample_fp8(h8, x, d, u, ws_s)
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in g_out.items()}
    want.update({"s_" + k: v.clone() for k, v in s_out.items()})
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qws.lmhead_verify_greedy_fp8(h8, x, d, ws_g, logits=lg, out=g_out)
        qws.lmhead_verify_sample_fp8(h8, x, d, u, ws_s, out=s_out)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in list(g_out.values()) + list(s_out.values()):
            v.zero_()                                  # eager work between the replays
        lg.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = dict(g_out)
        got.update({"s_" + k: v for k, v in s_out.items()})
        for k, v in want.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k}"
        assert torch.equal(lg, want["s_logits"])           # the greedy call's logits: the same values
