"""Full-size GPU parity, in the launch configuration bench.py times, against the float64
oracle's values for the same seeded inputs (tests/expected/*.npz, written by
tests/expected/make_expected.py from oracle/ only).

Compared: n_valid (exact), the loss, every row's LSE, sampled rows of grad_input and
grad_W and sampled entries of grad_b (each computed by the oracle one row or one
vocabulary column at a time), plus properties that hold at any size: ignored rows of
grad_input are exactly zero, and without z-loss the vocabulary sum of grad_W vanishes.
The standalone kernel is checked on [8192, 128256] bf16 logits for both z-loss settings
(sums from the stored oracle values, sampled dlogit rows from the oracle at test time).
"""

import os

import numpy as np
import pytest
import torch

import oracle
import linear_cross_entropy_vocab_amd as lce
from workloads import CONFIGS, make_config
from gpu_util import TOL, CE_TOL, dev, host64, rel, rel_fro

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _expected(name):
    return np.load(os.path.join(HERE, "expected", f"{name}.npz"), allow_pickle=False)


@pytest.mark.parametrize("name", ["gemma_like", "headline", "qwen_like"])
def test_fused_full_size(name):
    c = CONFIGS[name]
    print(f"full-size fused parity: {name} BT={c.BT} H={c.H} V={c.V}", flush=True)
    exp = _expected(name)
    inp = make_config(name)
    tol = TOL[c.dtype]
    b = None if inp.bias is None else dev(inp.bias, c.dtype)
    r = lce.lce_fwd_bwd(dev(inp.hidden, c.dtype), dev(inp.weight, c.dtype), b, dev(inp.targets),
                        z_loss=c.z_loss, reduction=c.reduction, return_lse=True)
    torch.cuda.synchronize()
    assert int(r["n_valid"].item()) == int(exp["n_valid"])
    assert rel(r["loss"].item(), float(exp["loss"])) <= tol["loss"], (r["loss"].item(), float(exp["loss"]))
    lse = host64(r["lse"])
    assert np.max(np.abs(lse - exp["lse"]) / np.maximum(1.0, np.abs(exp["lse"]))) <= tol["lse"]
    rows = exp["rows"]
    gi = host64(r["grad_input"][torch.from_numpy(rows).cuda()])
    assert rel_fro(gi, exp["grad_input_rows"]) <= tol["grad"]
    vocab = exp["vocab"]
    gw = host64(r["grad_weight"][torch.from_numpy(vocab).cuda()])
    assert rel_fro(gw, exp["grad_weight_rows"]) <= tol["grad"]
    if "grad_bias" in exp.files:
        gb = host64(r["grad_bias"][torch.from_numpy(exp["bias_vocab"]).cuda()])
        assert rel_fro(gb, exp["grad_bias"]) <= tol["grad"]
    ign = torch.from_numpy(inp.targets == -100).cuda()
    if bool(ign.any()):
        assert int(torch.count_nonzero(r["grad_input"][ign])) == 0
    if c.z_loss == 0.0:
        gw_all = r["grad_weight"].float()
        col = gw_all.sum(dim=0)
        assert float(col.norm() / gw_all.norm()) <= tol["grad"]


@pytest.mark.parametrize("mu", [0.0, 1e-4])
def test_ce_full_size(mu):
    c = CONFIGS["ce_only"]
    print(f"full-size standalone CE parity: [{c.B}, {c.V}] mu={mu}", flush=True)
    exp = _expected("ce_only")
    tag = "mu0" if mu == 0.0 else "mu1e-4"
    inp = make_config("ce_only")
    sample = np.array([0, 1, 17, 4096, c.B - 1] + list(np.nonzero(inp.targets == -100)[0][:2]))
    ref_rows = oracle.ce_oracle(inp.logits[sample], inp.targets[sample], z_loss=mu)
    x = dev(inp.logits, "bf16")
    del inp.logits
    ce_sum, z_sum, nv = lce.lce_ce_with_grad_inplace(x, dev(inp.targets), z_loss=mu)
    torch.cuda.synchronize()
    tol = CE_TOL["bf16"]
    assert int(nv.item()) == int(exp["n_valid"])
    assert rel(ce_sum.item(), float(exp[f"ce_sum_{tag}"])) <= tol["sums"]
    if mu == 0.0:
        assert z_sum.item() == 0.0
    else:
        assert rel(z_sum.item(), float(exp[f"z_sum_{tag}"])) <= tol["sums"]
    d = host64(x[torch.from_numpy(sample).cuda()])
    assert rel_fro(d, ref_rows["dlogits"]) <= tol["dlogits"]
    ign = torch.from_numpy(inp.targets == -100).cuda()
    assert int(torch.count_nonzero(x[ign])) == 0
