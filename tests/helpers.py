"""Shared pieces of the GPU parity tests: uploading seeded inputs, the oracle side of a layer, and
the comparison rules (tolerance, top-k with near-ties, argmax with a gap)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from oracle import formats as OF
from oracle import moe as OM

TOL = 2e-3          # max|err| / max|ref| for float outputs
ARGMAX_GAP = 1e-2   # LM-head argmax must agree where the oracle's top-2 gap exceeds this


def say(*a):
    """Name the case before each GPU step (flushed, so a dying box still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def bf16(bits: np.ndarray, device=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(device or dev())


def u8(a: np.ndarray, device=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device or dev())


def f32(a: np.ndarray, device=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device or dev())


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (scale if scale > 0 else 1.0))


def assert_close(got, ref, tol=TOL, what=""):
    e = rel_err(got, ref)
    assert np.all(np.isfinite(got)) or not np.all(np.isfinite(ref)), f"{what}: non-finite output"
    assert e <= tol, f"{what}: max|err|/max|ref| = {e:.3g} > {tol}"
    return e


def check_topk(gpu_idx: np.ndarray, gpu_logits: np.ndarray, ref_logits: np.ndarray, K: int,
               gpu_w: np.ndarray | None = None) -> int:
    """Top-k parity in two parts.

    (i) Always, bit for bit: the oracle's selection routine run on the GPU's own float32 logits
    gives the GPU's ordered indices (ties to the lower index), and, when gpu_w is given, the
    oracle's softmax over those logits gives the GPU's gate weights (2e-6 absolute: a float32 exp,
    sum of at most 8 terms and division, each within a few ulps of 1, against float64).
    (ii) Against the float64 oracle logits: where every adjacent gap among the oracle's top K+1
    logits exceeds tau = 4 * max|l_gpu - l_ref| (+ a float32 ulp floor), the ordered indices must
    be equal; otherwise the GPU's set must still be a valid top-K of the oracle logits within tau.
    Returns the number of tokens that needed that allowance."""
    near = 0
    for m in range(ref_logits.shape[0]):
        own = gpu_logits[m].astype(np.float64)[None]
        own_idx = OM.topk_select(own, K)[0]
        assert list(gpu_idx[m]) == list(own_idx), \
            f"token {m}: gpu {list(gpu_idx[m])} != oracle selection on the gpu logits {list(own_idx)}"
        if gpu_w is not None:
            own_w = OM.route_weights(own, own_idx[None])[0]
            err = float(np.max(np.abs(np.asarray(gpu_w[m], np.float64) - own_w)))
            assert err <= 2e-6, f"token {m}: gate weights differ from the oracle softmax of the gpu logits by {err:.3g}"
        ref = ref_logits[m]
        tau = 4 * float(np.max(np.abs(gpu_logits[m].astype(np.float64) - ref))) + 4e-7 * max(1.0, float(np.max(np.abs(ref))))
        order = OM.topk_select(ref[None], min(K + 1, ref.size))[0]
        gaps = -np.diff(ref[order])
        if np.all(gaps > tau):
            assert list(gpu_idx[m]) == list(order[:K]), f"token {m}: gpu {list(gpu_idx[m])} oracle {list(order[:K])}"
        else:
            near += 1
            sel = ref[np.asarray(gpu_idx[m])]
            rest = np.delete(ref, np.asarray(gpu_idx[m]))
            assert len(set(gpu_idx[m].tolist())) == K
            if rest.size:
                assert sel.min() >= rest.max() - tau, f"token {m}: invalid near-tie selection"
    return near


def check_argmax(gpu_logits: np.ndarray, ref_logits: np.ndarray, gap=ARGMAX_GAP) -> int:
    """argmax must agree wherever the oracle's top-2 gap exceeds `gap`; returns the rows checked
    (callers assert that it is above zero, so the rule cannot pass vacuously)."""
    checked = 0
    for m in range(ref_logits.shape[0]):
        top2 = np.sort(ref_logits[m])[-2:]
        if top2[1] - top2[0] > gap:
            checked += 1
            assert int(np.argmax(gpu_logits[m])) == int(np.argmax(ref_logits[m])), f"row {m}: argmax differs"
    return checked


# ------------------------------------------------------------------------------- layers
class Layer:
    """One MoE layer: a device bank (built on the GPU by the seeded generator), router weights and
    token vectors, plus the host-side oracle inputs regenerated per expert on demand."""

    def __init__(self, seed: int, layer: int, shape: synth.LayerShape, M: int, bias=None, device=None):
        self.seed, self.layer, self.shape, self.M = seed, layer, shape, M
        device = device or dev()
        self.bank_t = synth.expert_bank_torch(seed, layer, shape, device=device)
        self.wr = synth.router_weights(seed, layer, shape.n_routed, shape.hidden)
        self.x = synth.token_vectors(seed, layer, M, shape.hidden)
        self.bias = bias
        self.wr_t = bf16(self.wr, device)
        self.x_t = bf16(self.x, device)
        self.bias_t = None if bias is None else f32(bias, device)
        self._host = {}

    def expert(self, e):
        if e not in self._host:
            self._host[e] = synth.expert_np(self.seed, self.layer, e, self.shape)
        return self._host[e]

    def oracle_route(self):
        return OM.route(self.x, self.wr, self.shape.topk, self.bias)

    def oracle_y(self, idx, w):
        experts = {e: self.expert(e) for e in set(np.asarray(idx).reshape(-1).tolist()) | {self.shape.n_routed}
                   if 0 <= e <= self.shape.n_routed}
        return OM.moe_layer(self.x, idx, w, experts, self.shape.n_routed, self.shape.has_shared)


def fp8_tile_major(codes: np.ndarray) -> np.ndarray:
    """Row-major E4M3 codes [rows, cols] -> the library's tile-major bytes, from the header's
    definition: rows padded with zero codes to a multiple of 16; tile t at byte 16 t cols; chunk c
    (columns 16c .. 16c+15) of tile row i at byte 16 (16 c + i) of its tile."""
    rows, cols = codes.shape
    pad = (rows + 15) // 16 * 16
    full = np.zeros((pad, cols), dtype=np.uint8)
    full[:rows] = codes
    out = np.empty(pad * cols, dtype=np.uint8)
    for t in range(pad // 16):
        for c in range(cols // 16):
            for i in range(16):
                o = t * 16 * cols + (16 * c + i) * 16
                out[o:o + 16] = full[16 * t + i, 16 * c:16 * c + 16]
    return out
