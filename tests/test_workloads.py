"""The seeded input generator: determinism, shapes and planted structure."""
import math

import torch

import workloads as W


def test_prefill_tiny_is_deterministic_and_planted():
    cfg = W.CONFIGS[1]
    a = W.make_prefill(cfg)
    b = W.make_prefill(cfg)
    for key in ("q", "k", "v", "do"):
        assert torch.equal(a[key], b[key])
        assert a[key].dtype == torch.float32
    assert a["q"].shape == (1, 2, 256, 64) and a["k"].shape == (1, 2, 256, 64)
    assert abs(a["scale"] - 1 / 8) < 1e-15
    # logits have standard deviation about 3 (Q scaled by 3, scale 1/sqrt(d))
    s = (a["q"][0, 0] @ a["k"][0, 0].T) * a["scale"]
    assert 2.5 < s.std().item() < 3.5
    # every planted row has norm 4 and points along a later query row
    for h in range(2):
        ks, qs = W.planting_pairs(256, 8, "cpu", W.default_seed(1), h)
        assert (qs > ks).all() and (ks >= 0).all() and (qs <= 255).all()
    norms = a["k"][0].norm(dim=-1)
    assert ((norms - 4).abs() < 1e-4).sum() >= 8


def test_prefill_bf16_override_and_gqa():
    cfg = W.CONFIGS[3]
    x = W.make_prefill(cfg, n=300, hq=4, hkv=2, planted=5)
    assert x["q"].dtype == torch.bfloat16 and x["q"].shape == (1, 4, 300, 128)
    assert x["k"].shape == (1, 2, 300, 128)
    assert x["temps"].min() >= 1 and x["temps"].max() <= 4
    assert abs(x["scale"] - 1 / math.sqrt(128)) < 1e-15


def test_decode_inputs():
    cfg = W.CONFIGS[5]
    x = W.make_decode(cfg, cache=500, steps=3, batch=2, planted=4)
    assert x["k_cache"].shape == (2, 1, 503, 128)
    assert x["q_steps"].shape == (3, 2, 8, 128)
    y = W.make_decode(cfg, cache=500, steps=3, batch=2, planted=4)
    assert torch.equal(x["k_cache"], y["k_cache"]) and torch.equal(x["q_steps"], y["q_steps"])


def test_rademacher_probe():
    """The dO probe of the fidelity measurements: only -1 and +1, about half
    each, the same for the same seed and different for another seed."""
    a = W.rademacher((4, 1000), seed=7, dtype="f32")
    assert set(a.unique().tolist()) == {-1.0, 1.0}
    assert abs(float(a.mean())) < 0.05
    assert torch.equal(a, W.rademacher((4, 1000), seed=7, dtype="f32"))
    assert not torch.equal(a, W.rademacher((4, 1000), seed=8, dtype="f32"))
    assert W.rademacher((3, 5), seed=7).dtype == torch.bfloat16
