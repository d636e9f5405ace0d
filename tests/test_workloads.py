"""The seeded input generators (CPU only): determinism, slicing and bf16 rounding."""
import numpy as np
import torch

import workloads as W


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    ours = W.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_tokens_slice_consistent_and_deterministic():
    w = W.workload("c3").with_(context=5000)
    a = W.tokens(w, "k", 0, 0, 0, 3000)
    b = W.tokens(w, "k", 0, 0, 1000, 2500)
    assert np.array_equal(a[1000:2500], b)
    assert np.array_equal(a, W.tokens(w, "k", 0, 0, 0, 3000))
    # values are bf16-representable
    assert np.array_equal(W.bf16_round(a), a)
    assert not np.array_equal(W.tokens(w, "k", 0, 0, 0, 100), W.tokens(w, "v", 0, 0, 0, 100))


def test_k_scale_applied_per_position():
    w = W.workload("c3").with_(dtype="f32")
    k = W.tokens(w, "k", 0, 0, 0, 1024)
    u = W.tokens(w.with_(k_scale=False), "k", 0, 0, 0, 1024)
    s = k / u
    # one factor per position, shared by heads and dims, in [1, inf)
    assert np.allclose(s, s[:, :1, :1], rtol=1e-6)
    assert s.min() >= 1.0 - 1e-6


def test_masks_and_lengths():
    m = W.retrieval_mask(W.workload("c4"))
    assert m.shape == (32, 8) and np.all(m.sum(axis=1) == 4)
    assert np.array_equal(W.retrieval_mask(W.workload("c1")), np.array([[1, 0]], dtype=np.uint8))
    assert W.retrieval_mask(W.workload("c2")).sum() == 8
    lens = W.initial_lengths(W.workload("c4"))
    assert lens.shape == (8,) and lens.min() >= 16384 and lens.max() <= 32768
    assert len(set(lens.tolist())) > 1
