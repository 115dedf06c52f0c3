"""GPU parity of the sampled verification epilogue (lmhead_verify_sample_fp8) against the oracle
(oracle/verify.py): the ordered top-k rows equal the oracle's ranking of the kernel's own logits
(which equal the FP8 head GEMV's bit for bit), each position's token equals the oracle's sample
for the same uniform, and the emitted prefix follows the oracle's acceptance rule. Uniforms are
placed inside the oracle's probability intervals, away from their ends by more than float32
rounding of the cumulative sums can move them; positions whose top_p cut lies within 1e-5 of a
cumulative sum are left out of the token check (the cut is a float decision)."""
import numpy as np
import pytest
import torch

import quantized_weight_streaming_amd as qws
import synth
from oracle import lmhead as OL
from oracle import verify as OV

from .helpers import bf16, check_argmax, say

pytestmark = pytest.mark.gpu

PAGES = dict(temperature=0.6, top_k=29, top_p=0.95)   # the pages' sampled run


def _run(h8, xt, draft, u, ws, **kw):
    M = xt.shape[0]
    d = None if M == 1 else torch.tensor(np.asarray(draft, dtype=np.int32), device="cuda")
    ut = torch.tensor(np.asarray(u, dtype=np.float32), device="cuda")
    out = qws.lmhead_verify_sample_fp8(h8, xt, d, ut, ws, topk=True, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _cut_is_clear(row, temperature, top_k, top_p):
    """False when a cumulative probability of the ranked top_k lies within 1e-5 of top_p."""
    key = np.where(np.isnan(row), -np.inf, row.astype(np.float64))
    order = OV.ranked(key, min(top_k, key.size))
    p = np.exp((key[order] - key[order[0]]) / temperature)
    c = np.cumsum(p / p.sum())
    return bool(np.all(np.abs(c - top_p) > 1e-5)) or top_p == 1.0


def _interior_uniforms(row, temperature, top_k, top_p, rng, n):
    """n uniforms, each the midpoint of a kept token's interval of width >= 1e-3 (and u = 0)."""
    order, q = OV.sample_probs(row, temperature, top_k, top_p)
    c = np.concatenate([[0.0], np.cumsum(q)])
    wide = [j for j in range(len(q)) if q[j] >= 1e-3]
    pick = rng.choice(wide, size=n)
    return [0.0] + [float((c[j] + c[j + 1]) / 2 / c[-1]) for j in pick]


def _check(res, draft, u, kw, rows):
    lg = res["logits"]
    M = lg.shape[0]
    k = min(kw["top_k"], rows)
    for m in range(M):
        want = OV.ranked(lg[m], k).tolist() + [-1] * (kw["top_k"] - k)
        assert res["topk"][m].tolist() == want, f"top-k order, position {m}"
    clear = [m for m in range(M) if _cut_is_clear(lg[m], kw["temperature"], kw["top_k"], kw["top_p"])]
    want_tok = OV.sample_tokens(lg, kw["temperature"], kw["top_k"], kw["top_p"], u)
    for m in clear:
        assert int(res["token"][m]) == int(want_tok[m]), f"token of position {m} (u = {u[m]})"
    if len(clear) == M:
        n, emitted = OV.greedy_accept(res["token"], np.asarray(draft, dtype=np.int64))
        assert int(res["n"][0]) == n
        assert res["emitted"][:n].tolist() == emitted.tolist()
        assert res["emitted"][n:].tolist() == [-1] * (M - n)
    return len(clear)


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("rows,cols", [(1, 32), (40, 96), (999, 96), (4093, 256), (5000, 2560)])
@pytest.mark.parametrize("kw", [PAGES, dict(temperature=1.0, top_k=32, top_p=1.0),
                                dict(temperature=2.0, top_k=1, top_p=0.5), dict(temperature=0.6, top_k=5, top_p=0.3)])
def test_sample_small(M, rows, cols, kw):
    say("sample small", M, rows, cols, kw)
    w = synth.bf16_normal(9, 0, synth.HEAD, rows + cols, (rows, cols), 0.05)
    x = synth.token_vectors(9, 3, M, cols)
    xt = bf16(x)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    ws = qws.verify_workspace(M, "cuda")
    rng = np.random.default_rng(rows * 10 + M)
    res = _run(h8, xt, [0] * (M - 1), [0.5] * M, ws, **kw)
    gemv = qws.lmhead_gemv_fp8(h8, xt).cpu().numpy()
    assert np.array_equal(res["logits"].view(np.uint32), gemv.view(np.uint32))
    checked = 0
    for trial in range(3):
        u = [_interior_uniforms(res["logits"][m], kw["temperature"], kw["top_k"], kw["top_p"], rng, 3)[trial + 1]
             for m in range(M)]
        tok = OV.sample_tokens(res["logits"], kw["temperature"], kw["top_k"], kw["top_p"], u)
        for draft in ([int(t) for t in tok[:M - 1]], [(int(t) + 1) % rows for t in tok[:M - 1]]):
            res = _run(h8, xt, draft, u, ws, **kw)
            checked += _check(res, draft, u, kw, rows)
    assert checked >= 4 * M   # of the 6 M position checks, almost all have a clear top_p cut


def test_sample_ties_rank_the_lower_row_first():
    say("sample ties")
    rows, cols = 3000, 256
    w = synth.bf16_normal(10, 0, synth.HEAD, 0, (rows, cols), 0.02).copy()
    x = synth.token_vectors(10, 0, 2, cols)
    for r in (2500, 7, 1234, 2999, 64):
        w[r] = np.where(x[0] & 0x8000, 0xC000, 0x4000)    # bf16 +-2 aligned with token 0: equal top logits
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    ws = qws.verify_workspace(2, "cuda")
    kw = dict(temperature=1.0, top_k=8, top_p=1.0)
    res = _run(h8, bf16(x), [7], [0.0, 0.0], ws, **kw)
    lg = res["logits"]
    assert res["topk"][0].tolist()[:5] == [7, 64, 1234, 2500, 2999]
    assert int(res["token"][0]) == 7
    _check(res, [7], [0.0, 0.0], kw, rows)
    # u just past the first tied token's share picks the next tied row
    order, q = OV.sample_probs(lg[0], 1.0, 8, 1.0)
    u1 = float(q[0] + 1e-3)
    res = _run(h8, bf16(x), [7], [u1, 0.0], ws, **kw)
    assert int(res["token"][0]) == 64


@pytest.mark.parametrize("rows", [40000, 40001])
def test_sample_top_rows_clustered_in_one_workgroup(rows):
    """12 of the top 29 rows in one head workgroup (tiles 5 and 5 + 2048 of a 2,048-workgroup grid):
    its list of four keys is full, so its rows are read back from the logits (40,001 rows: the
    one-row-per-load path). Distinct top logits: each chosen row is +-v aligned with token 0's
    signs, v a different bf16 value per row (exact in E4M3 with its row scale)."""
    say(f"sample: clustered top rows, {rows} rows")
    cols = 256
    w = synth.bf16_normal(19, 0, synth.HEAD, 0, (rows, cols), 0.02).copy()
    x = synth.token_vectors(19, 0, 2, cols)
    rng = np.random.default_rng(19)
    cluster = sorted(rng.choice(np.r_[80:96, 16 * 2053:16 * 2054], 12, replace=False).tolist())
    others = rng.choice(np.setdiff1d(np.arange(rows), cluster), 20, replace=False).tolist()
    chosen = cluster + others
    order = rng.permutation(len(chosen))   # rank of each chosen row: a larger v for a lower rank
    for r, o in zip(chosen, order):
        v = 0x4100 - int(o)                 # bf16 codes 0x40E1 .. 0x4100 (7.0 .. 8.0)
        w[r] = np.where(x[0] & 0x8000, v | 0x8000, v)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    kw = dict(temperature=0.6, top_k=29, top_p=1.0)
    u = [0.37, 0.81]
    res = _run(h8, bf16(x), [0], u, qws.verify_workspace(2, "cuda"), **kw)
    want = [r for _, r in sorted(zip(order, chosen))][:29]
    assert res["topk"][0].tolist() == want
    assert set(cluster) <= set(want)
    _check(res, [0], u, kw, rows)


def test_sample_at_the_row_limit_reads_back_eight_tiles():
    """262,144 rows (2,048 head workgroups x 8 tiles, the most the sampled path takes): 20 of the
    top 29 rows in the eight tiles of one workgroup (its tiles t0 + 2048 i, t0 its first tile:
    tile 5 for workgroup 10, whose tiles pair with workgroup 2's on one XCD), so its 128 rows are
    read back."""
    say("sample: row limit, 8 tiles read back")
    rows, cols = 2048 * 16 * 8, 64
    w = synth.bf16_normal(20, 0, synth.HEAD, 0, (rows, cols), 0.02).copy()
    x = synth.token_vectors(20, 0, 1, cols)
    rng = np.random.default_rng(20)
    tiles = [5 + 2048 * i for i in range(8)]
    cluster = sorted(rng.choice(np.concatenate([np.arange(16 * t, 16 * t + 16) for t in tiles]), 20,
                                replace=False).tolist())
    others = rng.choice(np.setdiff1d(np.arange(rows), cluster), 12, replace=False).tolist()
    chosen = cluster + others
    order = rng.permutation(len(chosen))
    for r, o in zip(chosen, order):
        v = 0x4100 - int(o)
        w[r] = np.where(x[0] & 0x8000, v | 0x8000, v)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    kw = dict(temperature=0.6, top_k=29, top_p=1.0)
    res = _run(h8, bf16(x), [], [0.42], qws.verify_workspace(1, "cuda"), **kw)
    want = [r for _, r in sorted(zip(order, chosen))][:29]
    assert res["topk"][0].tolist() == want
    assert len(set(cluster) & set(want)) >= 17
    _check(res, [], [0.42], kw, rows)


def test_sample_more_candidates_than_rows():
    say("sample top_k > rows")
    rows, cols = 5, 64
    w = synth.bf16_normal(11, 0, synth.HEAD, 0, (rows, cols), 0.05)
    x = synth.token_vectors(11, 0, 1, cols)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    res = _run(h8, bf16(x), [], [0.999], qws.verify_workspace(1, "cuda"), **PAGES)
    assert res["topk"][0].tolist()[5:] == [-1] * 24
    _check(res, [], [0.999], PAGES, rows)


def test_sample_workspace_shared_with_greedy():
    say("sample + greedy on one workspace")
    w = synth.bf16_normal(12, 0, synth.HEAD, 0, (4097, 544), 0.05)
    x = synth.token_vectors(12, 0, 4, 544)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    ws = qws.verify_workspace(4, "cuda")
    u = [0.1, 0.5, 0.9, 0.3]
    a = _run(h8, bf16(x), [1, 2, 3], u, ws, **PAGES)
    d = torch.tensor([1, 2, 3], dtype=torch.int32, device="cuda")
    for _ in range(2):
        g = qws.lmhead_verify_greedy_fp8(h8, bf16(x), d, ws)
        b = _run(h8, bf16(x), [1, 2, 3], u, ws, **PAGES)
        assert all(np.array_equal(a[k], b[k]) for k in a)
    torch.cuda.synchronize()
    assert g["target"].cpu().tolist() == OV.argmax_first(a["logits"]).tolist()


def test_sample_full_head_window():
    say("sample full head")
    w = synth.head_weights(0)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    x = synth.token_vectors(0, 8, 4)
    xt = bf16(x)
    ws = qws.verify_workspace(4, "cuda")
    res = _run(h8, xt, [0, 0, 0], [0.5] * 4, ws, **PAGES)
    assert np.array_equal(res["logits"].view(np.uint32), qws.lmhead_gemv_fp8(h8, xt).cpu().numpy().view(np.uint32))
    codes, scales = OL.fp8_rowquant(w)
    assert check_argmax(res["logits"], OL.lmhead_fp8(codes, scales, x)) > 0
    rng = np.random.default_rng(13)
    checked = 0
    for trial in range(4):
        u = [_interior_uniforms(res["logits"][m], **PAGES, rng=rng, n=1)[1] for m in range(4)]
        tok = OV.sample_tokens(res["logits"], PAGES["temperature"], PAGES["top_k"], PAGES["top_p"], u)
        draft = [int(t) for t in tok[:3]]
        if trial % 2:
            draft[trial % 3] = (draft[trial % 3] + 1) % h8.rows
        res = _run(h8, xt, draft, u, ws, **PAGES)
        checked += _check(res, draft, u, PAGES, h8.rows)
    assert checked >= 12


def test_sample_many_ties_across_workgroups():
    """100 equal top logits on rows spread over many 16-row tiles (so over many head workgroups):
    the top 29 are the 29 lowest of those rows, and each tied token takes an equal share."""
    say("sample: 100 ties across workgroups")
    rows, cols = 40000, 256
    w = synth.bf16_normal(17, 0, synth.HEAD, 0, (rows, cols), 0.02).copy()
    x = synth.token_vectors(17, 0, 1, cols)
    tied = np.random.default_rng(17).choice(rows, 100, replace=False)
    w[tied] = np.where(x[0] & 0x8000, 0xC000, 0x4000)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    kw = dict(temperature=0.6, top_k=29, top_p=1.0)
    res = _run(h8, bf16(x), [], [0.5], qws.verify_workspace(1, "cuda"), **kw)
    assert res["topk"][0].tolist() == sorted(tied.tolist())[:29]
    assert int(res["token"][0]) == sorted(tied.tolist())[14]   # u = 0.5 of 29 equal shares
    _check(res, [], [0.5], kw, rows)


def test_sample_all_logits_equal():
    """x = 0: every logit is 0, the order is the row order, top_p 0.95 keeps 28 of 29 equal tokens."""
    say("sample: all logits equal")
    rows, cols = 9000, 128
    h8 = qws.lmhead_quantize_fp8(bf16(synth.bf16_normal(18, 0, synth.HEAD, 0, (rows, cols), 0.02)))
    x = np.zeros((2, cols), dtype=np.uint16)
    ws = qws.verify_workspace(2, "cuda")
    for u in (0.0, 0.5, 0.99):
        res = _run(h8, bf16(x), [3], [u, u], ws, **PAGES)
        assert res["topk"].tolist() == [list(range(29))] * 2
        assert res["token"].tolist() == [int(u * 28)] * 2
        assert int(res["n"][0]) == 1 + (int(u * 28) == 3)
