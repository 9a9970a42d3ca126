"""The seeded generators: deterministic bytes, shapes, mask counts, bf16 rounding."""

import hashlib

import numpy as np
import pytest
import torch

from workloads import CONFIGS, bf16_round, make_ce, make_fused, zipf_targets


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    a = make_fused(100, 64, 333, seed=7, bias_std=0.1, ignore_frac=0.1, targets="zipf")
    b = make_fused(100, 64, 333, seed=7, bias_std=0.1, ignore_frac=0.1, targets="zipf")
    assert _digest(a.hidden, a.weight, a.bias, a.targets) == \
        _digest(b.hidden, b.weight, b.bias, b.targets)
    c = make_fused(100, 64, 333, seed=8, bias_std=0.1, ignore_frac=0.1, targets="zipf")
    assert _digest(a.hidden) != _digest(c.hidden)


def test_bf16_round_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # ties to even
    ours = bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name,n_valid", [("tiny_f32", 230), ("ce_only", 7782),
                                          ("gemma_like", 8192), ("headline", 52428),
                                          ("qwen_like", 14746)])
def test_config_mask_counts(name, n_valid):
    c = CONFIGS[name]
    BT = getattr(c, "BT", None) or c.B
    frac = c.ignore_frac
    assert BT - int(round(frac * BT)) == n_valid
    if name == "tiny_f32":
        from workloads import make_config
        inp = make_config(name)
        assert int((inp.targets != -100).sum()) == n_valid
    if name == "ce_only":
        from workloads import ce_targets
        y = ce_targets(c.B, c.V, seed=c.seed, ignore_frac=c.ignore_frac)
        assert int((y != -100).sum()) == n_valid


def test_small_config_values():
    from workloads import make_config
    inp = make_config("tiny_f32")
    assert inp.hidden.shape == (256, 128) and inp.weight.shape == (4096, 128)
    assert inp.bias is None and inp.hidden.dtype == np.float32
    assert abs(inp.weight.std() - 128 ** -0.5) < 0.01
    ce = make_ce(64, 1000, seed=2, ignore_frac=0.05)
    assert np.array_equal(bf16_round(ce.logits), ce.logits)


def test_zipf_is_heavy_headed():
    rng = np.random.Generator(np.random.PCG64(0))
    y = zipf_targets(rng, 200000, 50000)
    assert y.min() >= 0 and y.max() < 50000
    p0 = (y == 0).mean()
    w = np.arange(1, 50001, dtype=np.float64) ** -1.1
    assert abs(p0 - 1 / w.sum()) < 0.01
