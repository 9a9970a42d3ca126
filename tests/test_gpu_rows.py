"""GPU parity of the per-row entry points (lce_rows_forward / lce_rows_backward: target
log-probability, softmax entropy, unreduced row loss, and the gradients of a per-row weighted
sum of them) against the float64 per-row oracle, through the C ABI, plus the autograd
wrapper.  The backward runs on the one-pass plan wherever it fits the one-chunk budget (every
case here but V = 1 and the 64 x 1088 x 70000 case, which take the token-chunked backward).  The forward takes every per-row statistic from the fp32 GEMM accumulator in one
pass over the vocabulary (no bf16 logits), so LSE, log-probability and entropy are held to the
fused path's LSE tolerance: |error| <= 2e-3 * max(1, |LSE|)."""

import numpy as np
import pytest
import torch

import oracle
import linear_cross_entropy_vocab_amd as lce
from workloads import make_fused
from gpu_util import TOL, dev, host64, rel_fro

pytestmark = pytest.mark.gpu

CASES = [
    # (BT, H, V, bias_std, z_loss, ignore_frac, seed)
    (200, 128, 1000, None, 0.0, 0.2, 61),
    (333, 256, 3001, 0.1, 1e-3, 0.1, 62),
    (700, 1280, 5000, 0.1, 1e-4, 0.05, 63),   # two token chunks, column chunks
    (97, 200, 513, None, 0.0, 0.3, 64),
    (64, 64, 1, 0.1, 0.0, 0.0, 65),           # V = 1: entropy 0, logprob 0
    (64, 1088, 70000, 0.1, 1e-4, 0.1, 75),    # no room for the one-pass plan: token-chunked backward
]


def _inputs(case):
    BT, H, V, bstd, mu, ign, seed = case
    inp = make_fused(BT, H, V, dtype="bf16", seed=seed, bias_std=bstd, ignore_frac=ign, z_loss=mu)
    b = None if inp.bias is None else dev(inp.bias, "bf16")
    return inp, dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), b, dev(inp.targets)


def _row_bound(ref):
    """The fused path's per-row LSE tolerance, relative to max(1, |LSE|)."""
    return TOL["bf16"]["lse"] * np.maximum(1.0, np.abs(ref["lse"]))


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in CASES])
def test_rows_forward_vs_oracle(case):
    print(f"rows forward case {case}", flush=True)
    inp, h, W, b, y = _inputs(case)
    ref = oracle.lce_rows_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=inp.z_loss)
    r = lce.lce_rows_forward(h, W, b, y, z_loss=inp.z_loss)
    torch.cuda.synchronize()
    assert int(r["n_valid"].item()) == ref["n_valid"]
    bound = _row_bound(ref)
    for k in ("lse", "logprobs", "entropy"):
        err = np.abs(host64(r[k]) - ref[k])
        assert np.all(err <= bound), (k, float((err / bound).max()))
    # row_loss adds mu LSE^2: its error also scales with 2 mu |LSE|
    err = np.abs(host64(r["row_loss"]) - ref["row_loss"])
    assert np.all(err <= bound * (1.0 + 2.0 * inp.z_loss * np.abs(ref["lse"]))), "row_loss"
    ign = inp.targets == -100
    assert np.all(host64(r["logprobs"])[ign] == 0.0) and np.all(host64(r["row_loss"])[ign] == 0.0)


@pytest.mark.parametrize("saved", [False, True], ids=["recomputed", "saved"])
@pytest.mark.parametrize("case", CASES + [(40, 2112, 9000, 0.1, 1e-4, 0.25, 66)],
                         ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in CASES] + ["40x2112x9000"])
def test_rows_backward_vs_oracle(case, saved):
    """Both forms of the backward: statistics recomputed from the stored bf16 logits chunk, and
    dlogits formed in the GEMM epilogue from the forward's saved LSE and entropy."""
    print(f"rows backward case {case} saved={saved}", flush=True)
    inp, h, W, b, y = _inputs(case)
    BT = inp.hidden.shape[0]
    rng = np.random.default_rng(case[-1])
    gl, gp, ge = (rng.normal(size=BT).astype(np.float32) for _ in range(3))
    ref = oracle.lce_rows_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=inp.z_loss,
                                 grad_row_loss=gl, grad_logprobs=gp, grad_entropy=ge)
    st = {}
    if saved:
        f = lce.lce_rows_forward(h, W, b, y, z_loss=inp.z_loss, outputs=("lse", "entropy"))
        st = dict(lse=f["lse"], entropy=f["entropy"], workspace=f["workspace"])
    r = lce.lce_rows_backward(h, W, b, y, grad_row_loss=dev(gl), grad_logprobs=dev(gp), grad_entropy=dev(ge),
                              z_loss=inp.z_loss, **st)
    torch.cuda.synchronize()
    for k in ("grad_input", "grad_weight", "grad_bias"):
        if ref[k] is None:
            continue
        e = rel_fro(host64(r[k]), ref[k])
        assert e <= TOL["bf16"]["grad"], (k, e)


ROWS_MASK = [
    # (BT, H, V, masked vocabulary ranges, z_loss, seed): whole 256-entry tiles of the forward
    # (the first, a middle one, the ragged last one) and a part of one tile, bias -inf
    (300, 256, 1500, ((0, 256), (512, 768), (1000, 1010)), 1e-3, 81),
    (130, 1152, 2000, ((0, 256), (1792, 2000)), 0.0, 82),
    (700, 1024, 5000, ((256, 512), (4864, 5000)), 1e-4, 83),
    (64, 1088, 70000, ((0, 256), (30000, 30256), (69888, 70000)), 1e-4, 84),   # token-chunked backward
]


@pytest.mark.parametrize("saved", [False, True], ids=["recomputed", "saved"])
@pytest.mark.parametrize("case", ROWS_MASK, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in ROWS_MASK])
def test_rows_minus_inf_bias_vs_oracle(case, saved):
    """Vocabulary entries masked with a -inf bias in the per-row forward and backward: a tile
    with no finite logit is skipped by the merge, and a masked entry (p = 0) adds nothing to
    the entropy or the dlogits, so its rows of grad_W and grad_b stay exactly 0."""
    BT, H, V, ranges, mu, seed = case
    print(f"rows masked-vocabulary case {case} saved={saved}", flush=True)
    inp = make_fused(BT, H, V, dtype="bf16", seed=seed, bias_std=0.1, ignore_frac=0.1, z_loss=mu)
    masked = np.zeros(V, dtype=bool)
    for a, b_ in ranges:
        masked[a:b_] = True
    keep = np.nonzero(~masked)[0]
    valid = inp.targets != -100
    inp.targets[:] = np.where(valid, keep[np.where(valid, inp.targets, 0) % keep.size], inp.targets)
    inp.bias[masked] = -np.inf
    h, W, b, y = dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.bias, "bf16"), dev(inp.targets)
    rng = np.random.default_rng(seed)
    gl, gp, ge = (rng.normal(size=BT).astype(np.float32) for _ in range(3))
    ref = oracle.lce_rows_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=mu,
                                 grad_row_loss=gl, grad_logprobs=gp, grad_entropy=ge)
    f = lce.lce_rows_forward(h, W, b, y, z_loss=mu)
    st = dict(lse=f["lse"], entropy=f["entropy"]) if saved else {}
    r = lce.lce_rows_backward(h, W, b, y, grad_row_loss=dev(gl), grad_logprobs=dev(gp), grad_entropy=dev(ge),
                              z_loss=mu, **st)
    torch.cuda.synchronize()
    bound = _row_bound(ref)
    for k in ("lse", "logprobs", "entropy"):
        err = np.abs(host64(f[k]) - ref[k])
        assert np.all(err <= bound), (k, float((err / bound).max()))
    for k in ("grad_input", "grad_weight", "grad_bias"):
        e = rel_fro(host64(r[k]), ref[k])
        assert e <= TOL["bf16"]["grad"], (k, e)
    mk = torch.from_numpy(masked).cuda()
    assert int(torch.count_nonzero(r["grad_weight"][mk])) == 0
    assert int(torch.count_nonzero(r["grad_bias"][mk])) == 0


def test_rows_backward_saved_matches_recomputed():
    """On the one-pass plan the recomputed form takes its statistics from the same per-row
    forward as the saved ones (on the token-chunked backward it recomputes them from the bf16
    logits chunk, so each dlogit is rounded after the logits' own rounding): close, and both
    deterministic."""
    inp, h, W, b, y = _inputs((700, 1280, 5000, 0.1, 1e-4, 0.05, 69))
    BT = inp.hidden.shape[0]
    rng = np.random.default_rng(69)
    g = [dev(rng.normal(size=BT).astype(np.float32)) for _ in range(3)]
    f = lce.lce_rows_forward(h, W, b, y, z_loss=inp.z_loss)
    kw = dict(grad_row_loss=g[0], grad_logprobs=g[1], grad_entropy=g[2], z_loss=inp.z_loss)
    r0 = lce.lce_rows_backward(h, W, b, y, **kw)
    r1 = lce.lce_rows_backward(h, W, b, y, lse=f["lse"], entropy=f["entropy"], **kw)
    r2 = lce.lce_rows_backward(h, W, b, y, lse=f["lse"], entropy=f["entropy"], **kw)
    torch.cuda.synchronize()
    for k in ("grad_input", "grad_weight", "grad_bias"):
        assert torch.equal(r1[k], r2[k]), k
        assert rel_fro(host64(r1[k]), host64(r0[k])) <= 5e-3, k
    with pytest.raises(ValueError):
        lce.lce_rows_backward(h, W, b, y, lse=f["lse"], **kw)


def test_rows_backward_single_upstreams_and_fp32_weight():
    inp, h, W, b, y = _inputs((333, 256, 3001, 0.1, 0.0, 0.1, 66))
    BT = inp.hidden.shape[0]
    ge = np.random.default_rng(66).normal(size=BT).astype(np.float32)
    ref = oracle.lce_rows_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, grad_entropy=ge)
    r = lce.lce_rows_backward(h, W, b, y, grad_entropy=dev(ge), grad_weight_fp32=True)
    torch.cuda.synchronize()
    assert r["grad_weight"].dtype == torch.float32
    for k in ("grad_input", "grad_weight", "grad_bias"):
        assert rel_fro(host64(r[k]), ref[k]) <= TOL["bf16"]["grad"], k
    # no upstream gradient at all: every gradient is zero
    z = lce.lce_rows_backward(h, W, b, y)
    torch.cuda.synchronize()
    for k in ("grad_input", "grad_weight", "grad_bias"):
        assert int(torch.count_nonzero(z[k])) == 0, k


def test_loss_weights_match_fused_gradients():
    inp, h, W, b, y = _inputs((333, 256, 3001, 0.1, 1e-3, 0.1, 67))
    valid = inp.targets != -100
    c = 1.0 / valid.sum()
    gl = np.where(valid, c, 0.0).astype(np.float32)
    r = lce.lce_rows_backward(h, W, b, y, grad_row_loss=dev(gl), z_loss=inp.z_loss)
    f = lce.lce_fwd_bwd(h, W, b, y, z_loss=inp.z_loss, method="chunked")
    torch.cuda.synchronize()
    for k in ("grad_input", "grad_weight", "grad_bias"):
        # (two separately rounded bf16 dlogits: about 2^-9 relative noise each)
        assert rel_fro(host64(r[k]), host64(f[k])) <= 5e-3, k


def test_autograd_wrapper():
    inp, h, W, b, y = _inputs((200, 128, 1000, 0.1, 0.0, 0.2, 68))
    BT = inp.hidden.shape[0]
    rng = np.random.default_rng(68)
    a1, a2, a3 = (rng.normal(size=BT).astype(np.float32) for _ in range(3))
    hh = h.clone().requires_grad_(True)
    WW = W.clone().requires_grad_(True)
    bb = b.clone().requires_grad_(True)
    lp, ent, rl = lce.linear_logprobs_entropy(hh, WW, y, bb)
    (lp * dev(a2)).sum().backward(retain_graph=True)
    g1 = hh.grad.clone()
    hh.grad = None
    WW.grad = None
    bb.grad = None
    total = (rl * dev(a1)).sum() + (lp * dev(a2)).sum() + (ent * dev(a3)).sum()
    total.backward()
    ref = oracle.lce_rows_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, grad_row_loss=a1,
                                 grad_logprobs=a2, grad_entropy=a3)
    assert rel_fro(host64(hh.grad), ref["grad_input"]) <= TOL["bf16"]["grad"]
    assert rel_fro(host64(WW.grad), ref["grad_weight"]) <= TOL["bf16"]["grad"]
    assert rel_fro(host64(bb.grad), ref["grad_bias"]) <= TOL["bf16"]["grad"]
    ref1 = oracle.lce_rows_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, grad_logprobs=a2)
    assert rel_fro(host64(g1), ref1["grad_input"]) <= TOL["bf16"]["grad"]


EDGE = [
    (130, 128, 257, 0.1, 0.0, 0.1, 71),       # last vocabulary tile holds one row
    (257, 64, 512, None, 1e-3, 0.0, 72),      # V a multiple of the tile; ragged token tile
    (40, 2112, 9000, 0.1, 1e-4, 0.25, 73),    # H > 1024, many vocabulary tiles
]


@pytest.mark.parametrize("case", EDGE, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in EDGE])
def test_rows_forward_edges_vs_oracle(case):
    print(f"rows forward edge case {case}", flush=True)
    inp, h, W, b, y = _inputs(case)
    ref = oracle.lce_rows_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=inp.z_loss)
    r = lce.lce_rows_forward(h, W, b, y, z_loss=inp.z_loss)
    # any subset of the outputs is the same values, bit for bit
    s = lce.lce_rows_forward(h, W, b, y, z_loss=inp.z_loss, outputs=("entropy",))
    torch.cuda.synchronize()
    assert s["lse"] is None and torch.equal(s["entropy"], r["entropy"])
    assert int(r["n_valid"].item()) == ref["n_valid"]
    bound = _row_bound(ref)
    for k in ("lse", "logprobs", "entropy"):
        err = np.abs(host64(r[k]) - ref[k])
        assert np.all(err <= bound), (k, float((err / bound).max()))
    err = np.abs(host64(r["row_loss"]) - ref["row_loss"])
    assert np.all(err <= bound * (1.0 + 2.0 * inp.z_loss * np.abs(ref["lse"]))), "row_loss"


def test_rows_forward_empty_batch_and_target_check():
    inp, h, W, b, y = _inputs((50, 128, 700, 0.1, 0.0, 0.1, 74))
    e = lce.lce_rows_forward(h[:0], W, b, y[:0], check_targets=True)
    torch.cuda.synchronize()
    assert int(e["n_valid"].item()) == 0 and e["lse"].numel() == 0
    bad = y.clone()
    bad[3] = 700
    with pytest.raises(lce.LCEError):
        lce.lce_rows_forward(h, W, b, bad, check_targets=True)
    torch.cuda.synchronize()
