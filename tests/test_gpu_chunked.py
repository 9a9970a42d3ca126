"""GPU parity of the token-chunked composition (lce_fwd_bwd_chunked: logits chunk written to
HBM, standalone cross-entropy in place, two GEMMs on the stored dlogits) against the float64
oracle, through the C ABI.  The composition computes the same loss and gradients as the fused
path ("Fused Linear Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It",
Strategy 1), so the oracle is the same one; the cases span several token chunks with a ragged
last chunk, several vocabulary ranges for grad_input, column chunks for H > 1024, bias,
z-loss, both reductions, the fp32 grad_W output, and the edge cases."""

import numpy as np
import pytest
import torch

import oracle
import linear_cross_entropy_vocab_amd as lce
from workloads import make_fused
from gpu_util import TOL, dev, host64, rel, rel_fro
from test_gpu_parity import check_fused

pytestmark = pytest.mark.gpu

# The composition stores the logits chunk in bf16 (the pages allow a bf16 or fp32 chunk; bf16
# holds twice the rows in the same bytes), so each row's LSE is that of logits rounded to
# bf16: off by at most the bf16 unit roundoff 2^-8 relative to the largest logit's size.
LSE_TOL = 2.0 ** -8


def run_chunked(inp, **kw):
    b = None if inp.bias is None else dev(inp.bias, inp.dtype)
    r = lce.lce_fwd_bwd(dev(inp.hidden, inp.dtype), dev(inp.weight, inp.dtype), b,
                        dev(inp.targets), z_loss=inp.z_loss, reduction=inp.reduction,
                        return_lse=True, method="chunked", **kw)
    torch.cuda.synchronize()
    return r


CASES = [
    # (BT, H, V, bias_std, z_loss, reduction, ignore_frac, seed): chunk rows, chunks, splits
    (200, 128, 1000, None, 0.0, "mean", 0.2, 41),     # 64-row chunks x 4, ragged
    (333, 256, 3001, 0.1, 1e-3, "sum", 0.1, 42),      # 64 x 6 (last 13 rows)
    (1500, 512, 20000, 0.1, 0.0, "mean", 0.1, 43),    # 128 x 12, 20 vocabulary ranges
    (700, 1280, 5000, None, 1e-4, "mean", 0.05, 44),  # 512 x 2, two column chunks of 768
    (65, 2304, 257, None, 0.0, "sum", 0.05, 45),      # one chunk, three column chunks
    (97, 200, 513, 0.2, 1e-2, "mean", 0.3, 46),       # H not a multiple of 128
    (1, 8, 5, None, 0.0, "mean", 0.0, 47),
    (64, 64, 1, 0.1, 0.0, "mean", 0.0, 48),           # V = 1
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in CASES])
def test_chunked_small_vs_oracle(case):
    BT, H, V, bstd, mu, red, ign, seed = case
    print(f"chunked case {case}", flush=True)
    inp = make_fused(BT, H, V, dtype="bf16", seed=seed, bias_std=bstd, ignore_frac=ign, z_loss=mu,
                     reduction=red)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=mu, reduction=red)
    r = run_chunked(inp)
    check_fused(inp, r, ref, lse_tol=LSE_TOL)


def test_chunked_grad_weight_fp32():
    inp = make_fused(333, 256, 3001, dtype="bf16", seed=42, bias_std=0.1, ignore_frac=0.1, z_loss=1e-3)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=1e-3)
    r32 = run_chunked(inp, grad_weight_fp32=True)
    assert r32["grad_weight"].dtype == torch.float32
    check_fused(inp, r32, ref, lse_tol=LSE_TOL)
    r16 = run_chunked(inp)
    # the bf16 output is the fp32 sum rounded once
    assert torch.equal(r32["grad_weight"].to(torch.bfloat16), r16["grad_weight"])
    assert torch.equal(r32["grad_input"], r16["grad_input"])


def test_chunked_matches_fused():
    inp = make_fused(1500, 512, 20000, dtype="bf16", seed=43, bias_std=0.1, ignore_frac=0.1)
    rc = run_chunked(inp)
    b = dev(inp.bias, "bf16")
    rf = lce.lce_fwd_bwd(dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), b, dev(inp.targets),
                         return_lse=True)
    torch.cuda.synchronize()
    assert int(rc["n_valid"].item()) == int(rf["n_valid"].item())
    assert rel(rc["loss"].item(), rf["loss"].item()) <= 1e-5
    assert float(((rc["lse"] - rf["lse"]).abs() / rf["lse"].abs().clamp(min=1.0)).max()) <= LSE_TOL
    for k in ("grad_input", "grad_weight", "grad_bias"):
        assert rel_fro(host64(rc[k]), host64(rf[k])) <= 1e-2, k


def test_chunked_edge_cases():
    inp = make_fused(150, 64, 300, dtype="bf16", seed=3, bias_std=0.1)
    inp.targets[:] = -100
    r = run_chunked(inp)
    assert r["loss"].item() == 0.0 and int(r["n_valid"].item()) == 0
    for k in ("grad_input", "grad_weight", "grad_bias"):
        assert torch.count_nonzero(r[k]) == 0, k
    empty = make_fused(0, 64, 300, dtype="bf16", seed=3)
    r = run_chunked(empty, out=dict(grad_weight=torch.full((300, 64), 7.0, dtype=torch.bfloat16,
                                                           device="cuda")))
    assert r["loss"].item() == 0.0 and int(r["n_valid"].item()) == 0
    assert torch.count_nonzero(r["grad_weight"]) == 0


def test_chunked_grad_subsets_and_determinism():
    inp = make_fused(333, 256, 3001, dtype="bf16", seed=49, bias_std=0.1, ignore_frac=0.1)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets)
    r = run_chunked(inp, grad_input=False, grad_weight=False, grad_bias=True)
    assert r["grad_input"] is None and r["grad_weight"] is None
    assert rel_fro(host64(r["grad_bias"]), ref["grad_bias"]) <= TOL["bf16"]["grad"]
    r = run_chunked(inp, grad_weight=False, grad_bias=False)
    assert rel_fro(host64(r["grad_input"]), ref["grad_input"]) <= TOL["bf16"]["grad"]
    a = run_chunked(inp)
    b = run_chunked(inp)
    for k in ("loss", "grad_input", "grad_weight", "grad_bias", "lse"):
        assert torch.equal(a[k], b[k]), k


def test_chunked_target_range_check():
    inp = make_fused(140, 64, 100, dtype="bf16", seed=5)
    inp.targets[77] = 100
    with pytest.raises(lce.LCEError) as e:
        run_chunked(inp, check_targets=True)
    assert e.value.status == 7
    r = run_chunked(inp)
    y = inp.targets.copy()
    y[77] = -100
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, y)
    check_fused(inp, r, ref, lse_tol=LSE_TOL)
