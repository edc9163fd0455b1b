"""The seeded input generators: determinism, sub-range consistency, moments,
and the recipes of the five workloads."""
import math

import numpy as np
import pytest
import torch

import moe_inputs as mi


def test_ih4_deterministic_and_subrange():
    a = mi.ih4_normal(5000, 1.0, 3, mi.TAG_W1, 7, out_dtype=torch.float32)
    b = mi.ih4_normal(5000, 1.0, 3, mi.TAG_W1, 7, out_dtype=torch.float32)
    assert torch.equal(a, b)
    c = mi.ih4_normal(1000, 1.0, 3, mi.TAG_W1, 7, start=2000, out_dtype=torch.float32)
    assert torch.equal(a[2000:3000], c)
    d = mi.ih4_normal(5000, 1.0, 3, mi.TAG_W1, 8, out_dtype=torch.float32)
    assert not torch.equal(a, d)


def test_ih4_moments():
    sigma = 1 / math.sqrt(4096)
    z = mi.ih4_normal(1 << 20, sigma, 0, mi.TAG_X, 0, out_dtype=torch.float32).double()
    assert abs(z.mean().item()) < 3e-3 * sigma * 10
    assert z.std().item() == pytest.approx(sigma, rel=5e-3)
    k = ((z / sigma) ** 4).mean().item()
    assert k == pytest.approx(3.0 - 1.2 / 4, abs=0.03)       # Irwin-Hall(4) kurtosis 2.7
    assert (z.abs() / sigma).max().item() <= math.sqrt(12) + 1e-6


def test_bf16_rounding_is_rne():
    z = mi.ih4_normal(4096, 1.0, 0, mi.TAG_X, 0, out_dtype=torch.float32)
    bf = mi.ih4_normal(4096, 1.0, 0, mi.TAG_X, 0)
    assert torch.equal(z.to(torch.bfloat16), bf)


def test_routing_softmax_topk():
    cfg = mi.config(2).scaled(M=256)
    ids, w = mi.make_routing(cfg)
    assert ids.shape == (256, 8) and w.dtype == np.float32
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.all(np.diff(w, axis=1) <= 0)
    assert ids.min() >= 0 and ids.max() < 128


def test_batched_recipe():
    cfg = mi.config(4)
    counts, tok, w = mi.make_routing(cfg)
    assert counts.shape == (32,) and counts.max() <= 512
    assert counts[0] == 512 and counts[1] == 512           # the two hottest experts hit the cap
    assert 2800 < counts.sum() < 3600
    for e in range(32):
        assert np.all(tok[e, :counts[e]] >= 0) and np.all(tok[e, :counts[e]] < 512)
        assert np.all(tok[e, counts[e]:] == -1) and np.all(w[e, counts[e]:] == 0)
        assert np.all((w[e, :counts[e]] >= 0) & (w[e, :counts[e]] < 1))


def test_small_inputs_shapes():
    inp = mi.make_inputs(mi.config(0))
    assert inp.x.shape == (64, 256) and inp.x.dtype == torch.bfloat16
    assert inp.w1.shape == (8, 1024, 256) and inp.w2.shape == (8, 256, 512)
    assert torch.equal(inp.w1[3], mi.expert_w1(mi.config(0), 3))
    rows = np.array([5, 17])
    assert torch.equal(mi.activations(mi.config(0), rows=rows), inp.x[rows])
