"""Seeded synthetic inputs for the MoE decode step and the vocabulary LM head.

This module makes input bytes and nothing else: uniform MXFP4 nibble and scale bytes, bf16
Gaussian weights and activations, and the router biases that shape a routing regime. It holds
none of the method's arithmetic (no dequantisation, routing, SwiGLU, GEMV or quantisation).
The HIP path (through torch device tensors) and the CPU oracle both consume what it makes;
neither imports the other.

Two generators are used.

* Bulk MXFP4 bytes come from a counter hash: the 32-bit MurmurHash3 finaliser ("fmix32",
  Austin Appleby, MurmurHash3.cpp) applied to a Weyl sequence ``key + i * 0x9E3779B9 (mod 2^32)``.
  It is written twice, in numpy uint64 arithmetic and in torch int64 arithmetic with a split
  multiply that never overflows, so the device can build a 67 GB bank in seconds while the host
  regenerates the few experts the oracle needs, bit for bit.
* bf16 tensors come from numpy's PCG64 ``standard_normal`` (float32) keyed by
  ``SeedSequence([seed, layer, kind, index])``, scaled by sigma in float32, then rounded to bf16
  with round-to-nearest-even.

Workloads follow the pages' Ling-3.0-flash shapes: hidden 2560, moe_intermediate 768, 512 routed
experts with top-8 plus one shared expert, a 157,184 x 2,560 LM head, 42 layers.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# stream kinds, the third SeedSequence / hash-key component
ROUTER, GU_Q, GU_S, D_Q, D_S, X, HEAD, ZIPF, REGIME = range(9)

HIDDEN = 2560
INTER = 768
VOCAB = 157184
TOPK = 8
N_LAYERS = 42
# E8M0 bytes 119..123 are the exponents -8..-4: block scales uniform over 2^-8 .. 2^-4
SCALE_LO = 119
SCALE_N = 5
HEAD_CHUNK_ROWS = 4096

_M32 = 0xFFFFFFFF
_WEYL = 0x9E3779B9
_C1 = 0x85EBCA6B
_C2 = 0xC2B2AE35


@dataclass(frozen=True)
class LayerShape:
    hidden: int = HIDDEN
    inter: int = INTER
    n_routed: int = 512
    topk: int = TOPK
    has_shared: bool = True

    @property
    def n_experts(self) -> int:
        """Experts stored in a bank: the routed ones, then the shared one at index n_routed."""
        return self.n_routed + (1 if self.has_shared else 0)


# --------------------------------------------------------------------------- counter hash
def _fmix32_int(h: int) -> int:
    h ^= h >> 16
    h = (h * _C1) & _M32
    h ^= h >> 13
    h = (h * _C2) & _M32
    h ^= h >> 16
    return h


def hash_key(seed: int, layer: int, kind: int, index: int) -> int:
    """32-bit stream key from the four stream coordinates (each in [0, 2^32))."""
    k = 0x243F6A88
    for v in (seed, layer, kind, index):
        if not 0 <= v <= _M32:
            raise ValueError("hash coordinates must lie in [0, 2^32)")
        k = _fmix32_int(((k ^ v) + _WEYL) & _M32)
    return k


def _fmix32_np(h: np.ndarray) -> np.ndarray:
    m = np.uint64(_M32)
    h ^= h >> np.uint64(16)
    h *= np.uint64(_C1)
    h &= m
    h ^= h >> np.uint64(13)
    h *= np.uint64(_C2)
    h &= m
    h ^= h >> np.uint64(16)
    return h


def hash_words_np(key: int, n: int, start: int = 0) -> np.ndarray:
    """Words ``start .. start+n-1`` of stream ``key`` as uint64 values in [0, 2^32)."""
    i = np.arange(start, start + n, dtype=np.uint64)
    i *= np.uint64(_WEYL)
    i += np.uint64(key)
    i &= np.uint64(_M32)
    return _fmix32_np(i)


def uniform_bytes_np(key: int, nbytes: int) -> np.ndarray:
    """nbytes uniform bytes: word i supplies bytes 4i..4i+3, little-endian."""
    if nbytes % 4:
        raise ValueError("nbytes must be a multiple of 4")
    return hash_words_np(key, nbytes // 4).astype(np.uint32).view(np.uint8)


def scale_bytes_np(key: int, nbytes: int, lo: int = SCALE_LO, n: int = SCALE_N) -> np.ndarray:
    """nbytes E8M0 bytes uniform over lo .. lo+n-1; byte j = lo + floor(word(j) * n / 2^32)."""
    w = hash_words_np(key, nbytes)
    return (np.uint64(lo) + ((w * np.uint64(n)) >> np.uint64(32))).astype(np.uint8)


def _mul32_t(h, c: int):
    # (h * c) mod 2^32 for 0 <= h, c < 2^32 without leaving int64: split h in 16-bit halves
    return (((((h >> 16) * c) & 0xFFFF) << 16) + (h & 0xFFFF) * c) & _M32


def _fmix32_t(h):
    h = h ^ (h >> 16)
    h = _mul32_t(h, _C1)
    h = h ^ (h >> 13)
    h = _mul32_t(h, _C2)
    return h ^ (h >> 16)


def hash_words_torch(keys, n: int, device=None):
    """Words 0..n-1 for each key in ``keys`` (1-D int64 tensor) -> int64 tensor [len(keys), n]."""
    import torch

    keys = torch.as_tensor(keys, dtype=torch.int64, device=device).reshape(-1, 1)
    i = torch.arange(n, dtype=torch.int64, device=keys.device).reshape(1, -1)
    return _fmix32_t((i * _WEYL + keys) & _M32)


def uniform_bytes_torch(keys, nbytes: int, device=None):
    """Torch twin of :func:`uniform_bytes_np` for several keys -> uint8 tensor [len(keys), nbytes]."""
    import torch

    if nbytes % 4:
        raise ValueError("nbytes must be a multiple of 4")
    w = hash_words_torch(keys, nbytes // 4, device)
    out = torch.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255, w >> 24], dim=-1)
    return out.to(torch.uint8).reshape(w.shape[0], nbytes)


def scale_bytes_torch(keys, nbytes: int, lo: int = SCALE_LO, n: int = SCALE_N, device=None):
    """Torch twin of :func:`scale_bytes_np` -> uint8 tensor [len(keys), nbytes]."""
    import torch

    w = hash_words_torch(keys, nbytes, device)
    return (lo + ((w * n) >> 32)).to(torch.uint8)


# --------------------------------------------------------------------------- MXFP4 experts
def expert_byte_shapes(shape: LayerShape) -> dict:
    """Canonical (row-major) byte shapes of one expert's four MXFP4 tensors."""
    h, i = shape.hidden, shape.inter
    return {
        "gate_up_q": (2 * i, h // 2),
        "gate_up_s": (2 * i, h // 32),
        "down_q": (h, i // 2),
        "down_s": (h, i // 32),
    }


_KIND_OF = {"gate_up_q": GU_Q, "gate_up_s": GU_S, "down_q": D_Q, "down_s": D_S}


def expert_np(seed: int, layer: int, expert: int, shape: LayerShape) -> dict:
    """One expert's four canonical uint8 tensors (expert == n_routed is the shared expert)."""
    out = {}
    for name, shp in expert_byte_shapes(shape).items():
        key = hash_key(seed, layer, _KIND_OF[name], expert)
        n = shp[0] * shp[1]
        arr = scale_bytes_np(key, n) if name.endswith("_s") else uniform_bytes_np(key, n)
        out[name] = arr.reshape(shp)
    return out


def expert_bank_torch(seed: int, layer: int, shape: LayerShape, device=None, batch: int = 32,
                      out: dict | None = None) -> dict:
    """All experts of one layer as uint8 tensors [n_experts, rows, cols] built on ``device``.

    Bytes equal :func:`expert_np` for every expert. ``out`` may hold preallocated tensors to fill.
    """
    import torch

    n = shape.n_experts
    shapes = expert_byte_shapes(shape)
    if out is None:
        out = {k: torch.empty((n,) + s, dtype=torch.uint8, device=device) for k, s in shapes.items()}
    for name, shp in shapes.items():
        nbytes = shp[0] * shp[1]
        kind = _KIND_OF[name]
        for e0 in range(0, n, batch):
            e1 = min(n, e0 + batch)
            keys = torch.tensor([hash_key(seed, layer, kind, e) for e in range(e0, e1)],
                                dtype=torch.int64, device=device)
            if name.endswith("_s"):
                b = scale_bytes_torch(keys, nbytes, device=device)
            else:
                b = uniform_bytes_torch(keys, nbytes, device=device)
            out[name][e0:e1].copy_(b.reshape((e1 - e0,) + shp))
    return out


# --------------------------------------------------------------------------- bf16 tensors
def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u += np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_normal(seed: int, layer: int, kind: int, index: int, shape, sigma: float) -> np.ndarray:
    """bf16 bit patterns (uint16) of sigma * N(0, 1) draws, float32 scaled, RNE rounded."""
    n = int(np.prod(shape))
    rng = np.random.default_rng(np.random.SeedSequence([seed, layer, kind, index]))
    v = rng.standard_normal(n, dtype=np.float32)
    v *= np.float32(sigma)
    return f32_to_bf16_bits(v).reshape(shape)


def router_weights(seed: int, layer: int, n_routed: int, hidden: int = HIDDEN) -> np.ndarray:
    """Router matrix [n_routed, hidden], bf16 bits, entries N(0, 0.02^2)."""
    return bf16_normal(seed, layer, ROUTER, 0, (n_routed, hidden), 0.02)


def token_vectors(seed: int, layer: int, m: int, hidden: int = HIDDEN, first: int = 0) -> np.ndarray:
    """m activation vectors [m, hidden], bf16 bits, entries N(0, 1); vector j uses index first+j."""
    return np.stack([bf16_normal(seed, layer, X, first + j, (hidden,), 1.0) for j in range(m)])


def head_chunk(seed: int, chunk: int, rows: int, hidden: int = HIDDEN) -> np.ndarray:
    """Rows [chunk*4096, chunk*4096 + rows) of the LM-head weight, bf16 bits, N(0, 0.02^2)."""
    return bf16_normal(seed, 0, HEAD, chunk, (rows, hidden), 0.02)


def head_weights(seed: int, vocab: int = VOCAB, hidden: int = HIDDEN) -> np.ndarray:
    """The whole LM-head weight [vocab, hidden] as bf16 bits (built chunk by chunk)."""
    out = np.empty((vocab, hidden), dtype=np.uint16)
    for c in range(0, (vocab + HEAD_CHUNK_ROWS - 1) // HEAD_CHUNK_ROWS):
        r0 = c * HEAD_CHUNK_ROWS
        r1 = min(vocab, r0 + HEAD_CHUNK_ROWS)
        out[r0:r1] = head_chunk(seed, c, r1 - r0, hidden)
    return out


# --------------------------------------------------------------------------- routing regimes
def zipf_bias(seed: int, layer: int, n_routed: int, s: float = 1.1) -> np.ndarray:
    """Additive log-prior that concentrates routing: b_e = -s * ln(1 + pi(e)), pi a seeded
    permutation of the experts. float32 [n_routed]."""
    perm = np.random.default_rng(np.random.SeedSequence([seed, layer, ZIPF, 0])).permutation(n_routed)
    return (-s * np.log1p(perm.astype(np.float64))).astype(np.float32)


REGIMES = ("same", "half", "disjoint")


def regime_sets(seed: int, layer: int, regime: str, m: int, n_routed: int, k: int = TOPK) -> list:
    """Designated expert sets per token for a verification window of m tokens.

    same: every token gets one seeded set of k experts; disjoint: m*k distinct experts, k per
    token; half: k/2 experts shared by all tokens plus k/2 private ones per token.
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, layer, REGIME, REGIMES.index(regime)]))
    if regime == "same":
        s = rng.choice(n_routed, k, replace=False)
        return [sorted(int(e) for e in s) for _ in range(m)]
    if regime == "disjoint":
        p = rng.choice(n_routed, m * k, replace=False)
        return [sorted(int(e) for e in p[j * k:(j + 1) * k]) for j in range(m)]
    if regime == "half":
        h = k // 2
        p = rng.choice(n_routed, h + m * (k - h), replace=False)
        common = [int(e) for e in p[:h]]
        return [sorted(common + [int(e) for e in p[h + j * (k - h):h + (j + 1) * (k - h)]]) for j in range(m)]
    raise ValueError(f"unknown regime {regime!r}")


def regime_bias(sets: list, n_routed: int, boost: float = 30.0) -> np.ndarray:
    """float32 [m, n_routed]: +boost on each token's designated set, 0 elsewhere."""
    b = np.zeros((len(sets), n_routed), dtype=np.float32)
    for j, s in enumerate(sets):
        b[j, s] = np.float32(boost)
    return b
