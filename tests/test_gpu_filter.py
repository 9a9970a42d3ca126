"""GPU parity of the gradient-filtering mode (lce_fwd_bwd_filtered, "Cut Cross Entropy
visualized", "Gradient Filtering") against the filtered float64 oracle.

Inputs make every tile decision unambiguous: a vocabulary range, aligned to the tiles and
holding no target, is pushed to probability ~e^-60 by its bias, and eps = 1e-6 sits far
from both e^-60 and the smallest probability any other tile can reach.  So the tile counts
must match the oracle exactly, and the gradients to the usual bf16 / fp32 tolerances.  The
oracle takes the call's tile shape (lce_filter_tile_shape: 256 x 64 on the stored-operand
GEMM's one-pass plan, 64 x 16 on the other kernels).
Covered: the pipelined kernel (bf16, H < 1024), the one-pass stored-operand backward (bf16,
from H = 1024: one and several vocabulary blocks, whole blocks without a kept tile, grad_W
over several token ranges) and the fp32 kernel; grad_b; both reductions; and eps below every
|dlogit|, where the filtered call must reproduce the exact call: bit for bit where both run
the same kernels (fp32, bf16 below H = 1024), within a quarter of the bf16 tolerance from
H = 1024 on (the plans of the two calls may cut the vocabulary into different blocks).
"""

import numpy as np
import pytest
import torch

import oracle
import linear_cross_entropy_vocab_amd as lce
from workloads import make_fused
from gpu_util import TOL, dev, host64, rel, rel_fro

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, BT, H, V, suppressed vocab range, reduction, z_loss, seed)
    ("bf16", 200, 256, 2048, (512, 1536), "mean", 0.0, 31),
    ("bf16", 333, 1024, 3001, (1024, 2048), "sum", 1e-3, 32),
    ("bf16", 150, 1152, 1500, (256, 1024), "mean", 0.0, 33),
    ("f32", 130, 128, 1200, (128, 896), "mean", 1e-3, 34),
    # 8 vocabulary blocks of 2560 entries: blocks 1-3 keep no tile at all
    ("bf16", 700, 1024, 20000, (2560, 10240), "mean", 1e-4, 36),
    # grad_W over two token ranges of 47 stages (flag pages not aligned to the ranges)
    ("bf16", 6000, 1024, 1500, (512, 1280), "mean", 0.0, 37),
]

_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _tiles(dtype, BT, H, V):
    return lce.filter_tile_shape(BT, H, V, _TORCH_DT[dtype])


def _inputs(dtype, BT, H, V, rng_v, seed, z_loss, reduction):
    inp = make_fused(BT, H, V, dtype=dtype, seed=seed, w_std=H ** -0.5, bias_std=0.1,
                     ignore_frac=0.1, z_loss=z_loss, reduction=reduction)
    lo, hi = rng_v
    inp.bias[lo:hi] = -60.0
    y = inp.targets.copy()
    sel = (y >= lo) & (y < hi)
    y[sel] = y[sel] % lo if lo > 0 else hi
    inp.targets = y
    return inp


def _run(inp, eps, counts=None):
    r = lce.lce_fwd_bwd(dev(inp.hidden, inp.dtype), dev(inp.weight, inp.dtype), dev(inp.bias, inp.dtype),
                        dev(inp.targets), z_loss=inp.z_loss, reduction=inp.reduction,
                        filter_eps=eps, filter_counts=counts)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}" for c in CASES])
def test_filtered_matches_filtered_oracle(case):
    dtype, BT, H, V, rv, reduction, mu, seed = case
    print(f"filtered parity {case}", flush=True)
    inp = _inputs(dtype, BT, H, V, rv, seed, mu, reduction)
    eps = 1e-6
    R, C = _tiles(dtype, BT, H, V)
    print(f"  tiles {R} x {C}", flush=True)
    ref = oracle.lce_oracle_filtered(inp.hidden, inp.weight, inp.bias, inp.targets, filter_eps=eps,
                                     z_loss=mu, reduction=reduction, stat_rows=R, stream_rows=C)
    counts = torch.zeros(4, dtype=torch.int64, device="cuda")
    r = _run(inp, eps, counts)
    c = counts.cpu().tolist()
    assert c == [ref["skipped_input"], ref["tiles_input"], ref["skipped_weight"], ref["tiles_weight"]]
    assert ref["skipped_input"] > 0 and ref["skipped_weight"] > 0
    tol = TOL[dtype]
    assert int(r["n_valid"].item()) == ref["n_valid"]
    assert rel(r["loss"].item(), ref["loss"]) <= tol["loss"]
    for k in ("grad_input", "grad_weight", "grad_bias"):
        assert rel_fro(host64(r[k]), ref[k]) <= tol["grad"], k
    # the vocabulary rows of skipped grad_W tiles get exactly zero grad_W and grad_b
    lo, hi = rv
    lo_r, hi_r = -(-lo // R) * R, (hi // R) * R
    if hi_r > lo_r:
        assert int(torch.count_nonzero(r["grad_weight"][lo_r:hi_r])) == 0
        assert int(torch.count_nonzero(r["grad_bias"][lo_r:hi_r])) == 0


@pytest.mark.parametrize("case", [("bf16", 700, 1024, 20000, (2560, 10240), "mean", 1e-4, 36),
                                  ("bf16", 6000, 1024, 1500, (512, 1280), "sum", 0.0, 37)],
                         ids=["8-blocks", "split-grad_W"])
def test_filtered_gradient_subsets(case):
    """A filtered call asked for one gradient only runs that product alone with the tile flags
    (grad_W and grad_b without the grad_input product, or grad_input by itself): each equals the
    filtered oracle's, and the counts of the tiles examined stay those of the full call."""
    dtype, BT, H, V, rv, reduction, mu, seed = case
    print(f"filtered gradient subsets {case}", flush=True)
    inp = _inputs(dtype, BT, H, V, rv, seed, mu, reduction)
    eps = 1e-6
    R, C = _tiles(dtype, BT, H, V)
    ref = oracle.lce_oracle_filtered(inp.hidden, inp.weight, inp.bias, inp.targets, filter_eps=eps,
                                     z_loss=mu, reduction=reduction, stat_rows=R, stream_rows=C)
    args = (dev(inp.hidden, dtype), dev(inp.weight, dtype), dev(inp.bias, dtype), dev(inp.targets))
    kw = dict(z_loss=mu, reduction=reduction, filter_eps=eps)
    tol = TOL[dtype]["grad"]
    counts = torch.zeros(4, dtype=torch.int64, device="cuda")
    w = lce.lce_fwd_bwd(*args, grad_input=False, filter_counts=counts, **kw)
    torch.cuda.synchronize()
    assert w["grad_input"] is None
    assert rel_fro(host64(w["grad_weight"]), ref["grad_weight"]) <= tol
    assert rel_fro(host64(w["grad_bias"]), ref["grad_bias"]) <= tol
    assert counts[2:].cpu().tolist() == [ref["skipped_weight"], ref["tiles_weight"]]
    del w
    i = lce.lce_fwd_bwd(*args, grad_weight=False, grad_bias=False, **kw)
    torch.cuda.synchronize()
    assert i["grad_weight"] is None and i["grad_bias"] is None
    assert rel_fro(host64(i["grad_input"]), ref["grad_input"]) <= tol


@pytest.mark.parametrize("dtype,H", [("bf16", 256), ("bf16", 1152), ("f32", 128)])
def test_tiny_eps_reproduces_exact_call(dtype, H):
    inp = make_fused(160, H, 1000, dtype=dtype, seed=35, w_std=H ** -0.5, bias_std=0.1,
                     ignore_frac=0.1)
    b = dev(inp.bias, dtype)
    args = (dev(inp.hidden, dtype), dev(inp.weight, dtype), b, dev(inp.targets))
    exact = lce.lce_fwd_bwd(*args)
    counts = torch.zeros(4, dtype=torch.int64, device="cuda")
    filt = lce.lce_fwd_bwd(*args, filter_eps=1e-38, filter_counts=counts)
    torch.cuda.synchronize()
    assert counts[0].item() == 0 and counts[2].item() == 0
    for k in ("loss", "grad_input", "grad_weight", "grad_bias"):
        if dtype == "f32" or H < 1024 or k == "loss":
            assert torch.equal(exact[k], filt[k]), k
        else:
            # bf16 from H = 1024: the exact call's backward runs on the stored-operand GEMM, the
            # filtered one on kernels that test each tile (the same values, summed in another
            # order)
            assert rel_fro(host64(filt[k]), host64(exact[k])) <= TOL[dtype]["grad"] / 4, k


# --------------------------------------------------------------------- vocabulary sorting

SORT_CASES = [
    # (dtype, BT, H, V, seed)
    ("bf16", 200, 256, 2048, 41),
    ("bf16", 150, 1152, 1500, 42),   # one-pass plan: grad_W rows through the order
    ("f32", 130, 128, 1200, 43),
    ("bf16", 6000, 1024, 1500, 44),  # ... from partial sums over two token ranges
]


def _sort_inputs(dtype, BT, H, V, seed):
    """Every 64th entry is "hot" (bias 20 + small distinct offsets) and holds all the targets;
    the others get distinct biases from -30 down in steps of 0.01, and W is tiny, so each
    entry's average logit is set by its bias alone (well separated: both orders agree) and
    every non-hot probability is ~e^-50, far below eps."""
    inp = make_fused(BT, H, V, dtype=dtype, seed=seed, w_std=1e-4, bias_std=None, ignore_frac=0.1)
    rng = np.random.default_rng(seed)
    hot = np.arange(0, V, 64)
    b = -30.0 - 0.01 * rng.permutation(V).astype(np.float64)
    b[hot] = 20.0 + 0.01 * np.arange(len(hot))
    inp.bias = b.astype(np.float32)
    if dtype == "bf16":
        inp.bias = torch.from_numpy(inp.bias).to(torch.bfloat16).float().numpy()
    y = inp.targets.copy()
    keep = y != -100
    y[keep] = hot[rng.integers(0, len(hot), size=int(keep.sum()))]
    inp.targets = y
    return inp


@pytest.mark.parametrize("case", SORT_CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}" for c in SORT_CASES])
def test_sorted_filtering_matches_oracle(case):
    dtype, BT, H, V, seed = case
    print(f"sorted filtering {case}", flush=True)
    inp = _sort_inputs(dtype, BT, H, V, seed)
    eps = 1e-6
    R, C = _tiles(dtype, BT, H, V)
    ref = oracle.lce_oracle_filtered(inp.hidden, inp.weight, inp.bias, inp.targets, filter_eps=eps, sort_vocab=True,
                                     stat_rows=R, stream_rows=C)
    plain = oracle.lce_oracle_filtered(inp.hidden, inp.weight, inp.bias, inp.targets, filter_eps=eps,
                                       stat_rows=R, stream_rows=C)
    assert ref["skipped_input"] > plain["skipped_input"] and ref["skipped_weight"] > plain["skipped_weight"]
    counts = torch.zeros(4, dtype=torch.int64, device="cuda")
    r = lce.lce_fwd_bwd(dev(inp.hidden, dtype), dev(inp.weight, dtype), dev(inp.bias, dtype), dev(inp.targets),
                        filter_eps=eps, filter_counts=counts, sort_vocab=True, return_lse=True)
    torch.cuda.synchronize()
    c = counts.cpu().tolist()
    assert c == [ref["skipped_input"], ref["tiles_input"], ref["skipped_weight"], ref["tiles_weight"]], c
    tol = TOL[dtype]
    assert int(r["n_valid"].item()) == ref["n_valid"]
    assert rel(r["loss"].item(), ref["loss"]) <= tol["loss"]
    for k in ("grad_input", "grad_weight", "grad_bias"):
        e = rel_fro(host64(r[k]), ref[k])
        assert e <= tol["grad"], (k, e)


SORT_GENERAL = [
    # (dtype, BT, H, V, bias, ignore_frac, targets, seed)
    ("bf16", 300, 256, 3001, True, 0.1, "zipf", 45),
    ("bf16", 150, 1152, 1500, False, 0.0, "uniform", 46),
    ("f32", 130, 128, 1200, True, 0.2, "zipf", 47),
    ("bf16", 64, 128, 700, True, 1.0, "uniform", 48),   # every row ignored: the order is the bias order
    ("bf16", 0, 128, 700, True, 0.0, "uniform", 49),    # empty batch
]


@pytest.mark.parametrize("case", SORT_GENERAL, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}" for c in SORT_GENERAL])
def test_sorted_tiny_eps_matches_exact_oracle(case):
    """With eps below every |dlogit| nothing is skipped, so the sorted call must give the exact
    loss and gradients in the original vocabulary order, whatever order the sort chose (near
    ties between averages may order differently in fp32 and fp64; the result does not depend
    on it)."""
    dtype, BT, H, V, with_bias, ign, tg, seed = case
    print(f"sorted tiny eps {case}", flush=True)
    inp = make_fused(BT, H, V, dtype=dtype, seed=seed, w_std=H ** -0.5, bias_std=0.5 if with_bias else None,
                     targets=tg, ignore_frac=ign)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets)
    counts = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    bias = dev(inp.bias, dtype) if with_bias else None
    r = lce.lce_fwd_bwd(dev(inp.hidden, dtype), dev(inp.weight, dtype), bias, dev(inp.targets),
                        filter_eps=1e-38, filter_counts=counts, sort_vocab=True, return_lse=True,
                        check_targets=True)
    torch.cuda.synchronize()
    c = counts.cpu().tolist()
    if ref["n_valid"] == 0:
        assert c[0] == c[1] and c[2] == c[3], c   # every dlogit is 0: every tile is skipped
    else:
        assert c[0] == 0 and c[2] == 0, c
    tol = TOL[dtype]
    assert int(r["n_valid"].item()) == ref["n_valid"]
    if ref["n_valid"] == 0:
        assert r["loss"].item() == 0.0
    else:
        assert rel(r["loss"].item(), ref["loss"]) <= tol["loss"]
    if BT > 0:
        lse = host64(r["lse"])
        assert np.max(np.abs(lse - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))) <= tol["lse"]
    keys = ("grad_input", "grad_weight", "grad_bias") if with_bias else ("grad_input", "grad_weight")
    for k in keys:
        want = ref[k]
        got = host64(r[k])
        if not np.any(want):
            assert not np.any(got), k
        else:
            assert rel_fro(got, want) <= tol["grad"], k


def test_sorted_call_checks_targets_before_sorting():
    inp = make_fused(100, 128, 500, dtype="bf16", seed=50, bias_std=0.1)
    y = inp.targets.copy()
    y[7] = 500
    with pytest.raises(lce.LCEError):
        lce.lce_fwd_bwd(dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.bias, "bf16"), dev(y),
                        filter_eps=1e-6, sort_vocab=True, check_targets=True)
    torch.cuda.synchronize()
