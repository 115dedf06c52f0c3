"""The seeded input generator: numpy and torch twins agree byte for byte, draws are deterministic,
and the distributions are the stated ones."""
import hashlib

import numpy as np
import pytest
import torch

import synth


def test_numpy_and_torch_hash_agree():
    for key in (0, 1, synth.hash_key(3, 41, synth.GU_Q, 512), 0xFFFFFFFF):
        a = synth.uniform_bytes_np(key, 4096)
        b = synth.uniform_bytes_torch(torch.tensor([key]), 4096)[0].numpy()
        assert np.array_equal(a, b)
        assert np.array_equal(synth.scale_bytes_np(key, 777), synth.scale_bytes_torch(torch.tensor([key]), 777)[0].numpy())


def test_bank_torch_matches_per_expert_numpy():
    shape = synth.LayerShape(hidden=128, inter=64, n_routed=5, topk=2)
    bank = synth.expert_bank_torch(9, 2, shape, batch=2)
    for e in range(shape.n_experts):
        ref = synth.expert_np(9, 2, e, shape)
        for k, v in ref.items():
            assert np.array_equal(bank[k][e].numpy(), v), (e, k)


def test_deterministic_and_distinct():
    shape = synth.LayerShape()
    a = synth.expert_np(0, 0, 7, shape)
    b = synth.expert_np(0, 0, 7, shape)
    c = synth.expert_np(0, 0, 8, shape)
    h = lambda d: hashlib.sha256(b"".join(d[k].tobytes() for k in sorted(d))).hexdigest()
    assert h(a) == h(b) != h(c)
    assert a["gate_up_q"].shape == (1536, 1280) and a["down_s"].shape == (2560, 24)


def test_byte_distributions():
    key = synth.hash_key(0, 0, synth.GU_Q, 0)
    b = synth.uniform_bytes_np(key, 1 << 20)
    nib = np.concatenate([b & 15, b >> 4])
    cnt = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(cnt - 1 / 16) < 0.002)
    s = synth.scale_bytes_np(key, 100000)
    assert set(np.unique(s).tolist()) == {119, 120, 121, 122, 123}


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(v), want)


def test_normals_have_stated_scale():
    w = synth.router_weights(0, 0, 512).astype(np.uint32) << np.uint32(16)
    wf = w.view(np.float32)
    assert abs(wf.std() - 0.02) < 2e-4 and abs(wf.mean()) < 2e-4
    x = synth.token_vectors(0, 0, 4)
    assert x.shape == (4, 2560) and not np.array_equal(x[0], x[1])


def test_regimes_and_zipf():
    for regime, union in (("same", 8), ("half", 20), ("disjoint", 32)):
        sets = synth.regime_sets(0, 0, regime, 4, 512)
        assert all(len(s) == 8 and len(set(s)) == 8 for s in sets)
        assert len(set().union(*map(set, sets))) == union
    b = synth.zipf_bias(1, 0, 512)
    assert b.max() == 0.0 and abs(b.min() + 1.1 * np.log(512)) < 1e-5
    assert len(np.unique(b)) == 512


def test_head_chunks_are_independent():
    a = synth.head_chunk(0, 3, 16, 64)
    b = synth.head_chunk(0, 3, 16, 64)
    c = synth.head_chunk(0, 4, 16, 64)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
