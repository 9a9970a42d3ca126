"""The no-allocation entry point (lce_ce_with_grad_inplace_noalloc) against the entry point it
varies (lce_ce_with_grad_inplace, with a workspace): the same kernels, so the same bits, on
two calls in a row of which the second is smaller (the scratch keeps the first call's
per-row values, which the second must not see), and at the largest size the scratch holds."""

import numpy as np
import pytest
import torch

import linear_cross_entropy_vocab_amd as lce
from workloads import make_ce
from gpu_util import dev

pytestmark = pytest.mark.gpu


def _pair(B, V, dt, mu, seed):
    inp = make_ce(B, V, dtype=dt, seed=seed, ignore_frac=0.1)
    x = dev(inp.logits, dt)
    y = dev(inp.targets)
    return x, y


def _outs():
    return dict(ce_sum=torch.empty((), dtype=torch.float32, device="cuda"),
                z_sum=torch.empty((), dtype=torch.float32, device="cuda"),
                n_valid=torch.empty((), dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point_on_two_calls(dt):
    print(f"no-allocation CE, {dt}", flush=True)
    for B, V, mu, seed in ((700, 5000, 1e-4, 81), (33, 1001, 0.0, 82)):  # the second call smaller
        x, y = _pair(B, V, dt, mu, seed)
        x_ref = x.clone()
        ref = lce.lce_ce_with_grad_inplace(x_ref, y, z_loss=mu)
        o = _outs()
        got = lce.lce_ce_with_grad_inplace_noalloc(x, y, z_loss=mu, out=o)
        torch.cuda.synchronize()
        assert torch.equal(x, x_ref), (B, V)                       # dlogits, bit for bit
        for a, b in zip(got, ref):
            assert torch.equal(a, b), (B, V)
        assert int(got[2].item()) == int((y != -100).sum().item())


def test_noalloc_largest_size_and_limit():
    B = lce.NOALLOC_MAX_ROWS
    print(f"no-allocation CE, B = {B}", flush=True)
    x, y = _pair(B, 64, "bf16", 0.0, 83)
    x_ref = x.clone()
    ref = lce.lce_ce_with_grad_inplace(x_ref, y)
    got = lce.lce_ce_with_grad_inplace_noalloc(x, y, out=_outs())
    torch.cuda.synchronize()
    assert torch.equal(x, x_ref)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    with pytest.raises(lce.LCEError) as e:
        lce.lce_ce_with_grad_inplace_noalloc(torch.empty(B + 1, 8, dtype=torch.bfloat16, device="cuda"),
                                             torch.zeros(B + 1, dtype=torch.int64, device="cuda"))
    assert e.value.status == 9
