"""The allocation-free greedy verification (lmhead_verify_greedy_fp8_noalloc) through the C ABI:
its results equal lmhead_verify_greedy_fp8's (with a caller's workspace) bit for bit, on two
calls in a row, the second with a smaller window and a smaller head, and the outputs agree with
the oracle's argmax rule; a window past the scratch's size is refused."""
import ctypes as C

import numpy as np
import pytest
import torch

import quantized_weight_streaming_amd as qws
import synth
from oracle import lmhead as OL
from oracle import verify as OV
from quantized_weight_streaming_amd import _lib

from .helpers import bf16, say

pytestmark = pytest.mark.gpu


def _raw(head, x, draft, logits, out):
    """The entry point called through the C ABI directly (plain pointers, the current stream)."""
    lib = _lib.load()
    M = x.shape[0]
    st = lib.lmhead_verify_greedy_fp8_noalloc(C.byref(head.desc), x.data_ptr(), M,
                                              None if draft is None else draft.data_ptr(), logits.data_ptr(),
                                              out["target"].data_ptr(), out["emitted"].data_ptr(),
                                              out["n"].data_ptr(), torch.cuda.current_stream().cuda_stream)
    return st


def _case(rows, cols, M, seed):
    w = synth.bf16_normal(seed, 0, synth.HEAD, rows + cols, (rows, cols), 0.02)
    h8 = qws.lmhead_quantize_fp8(bf16(w))
    x = synth.token_vectors(seed, 1, M, cols)
    return w, h8, x


def test_noalloc_equals_workspace_path_twice_second_smaller():
    for i, (rows, cols, M) in enumerate(((157184, 2560, 4), (5000, 544, 2))):
        say("noalloc greedy", i, rows, cols, M)
        w, h8, x = _case(rows, cols, M, 40 + i)
        xt = bf16(x)
        # drafts equal to the window's own targets where possible, so a prefix is accepted
        ref_logits = torch.empty((M, rows), dtype=torch.float32, device="cuda")
        ws = qws.verify_workspace(M, "cuda")
        d0 = torch.zeros(max(M - 1, 0), dtype=torch.int32, device="cuda")
        ref = qws.lmhead_verify_greedy_fp8(h8, xt, d0 if M > 1 else None, ws, logits=ref_logits)
        draft = ref["target"][:M - 1].clone() if M > 1 else None
        ref = qws.lmhead_verify_greedy_fp8(h8, xt, draft, ws, logits=ref_logits)
        logits = torch.empty_like(ref_logits)
        out = {k: torch.full((n,), -7, dtype=torch.int32, device="cuda") for k, n in (("target", M), ("emitted", M), ("n", 1))}
        assert _raw(h8, xt, draft, logits, out) == _lib.QWS_OK
        torch.cuda.synchronize()
        assert torch.equal(logits.view(torch.int32), ref_logits.view(torch.int32))
        for k in ("target", "emitted", "n"):
            assert torch.equal(out[k], ref[k]), k
        # the oracle side: each target is the argmax of the logits (ties to the lower row)
        assert out["target"].cpu().numpy().tolist() == OV.argmax_first(logits.cpu().numpy()).tolist()
        assert int(out["n"].item()) == M                     # every draft equals its target
        if rows <= 5000:
            codes, scales = OL.fp8_rowquant(w)
            ref64 = OL.lmhead_fp8(codes, scales, x)
            err = float(np.max(np.abs(logits.cpu().numpy() - ref64)) / np.max(np.abs(ref64)))
            assert err <= 2e-3


def test_noalloc_refuses_a_window_past_the_scratch():
    say("noalloc refuses M = 5")
    _, h8, x = _case(64, 64, 4, 50)
    xt = bf16(x)
    z = torch.zeros(8, dtype=torch.int32, device="cuda")
    lg = torch.empty((5, 64), dtype=torch.float32, device="cuda")
    out = {"target": z, "emitted": z, "n": z}
    lib = _lib.load()
    st = lib.lmhead_verify_greedy_fp8_noalloc(C.byref(h8.desc), xt.data_ptr(), 5, z.data_ptr(), lg.data_ptr(),
                                              z.data_ptr(), z.data_ptr(), z.data_ptr(), None)
    assert st == _lib.QWS_ERR_SHAPE
