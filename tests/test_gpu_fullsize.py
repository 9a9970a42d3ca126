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
from workloads import CONFIGS, make_config, make_fused
from gpu_util import TOL, CE_TOL, dev, host64, rel, rel_fro

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _expected(name):
    return np.load(os.path.join(HERE, "expected", f"{name}.npz"), allow_pickle=False)


# The token-chunked composition keeps its logits chunk in bf16, so its LSE is that of
# bf16-rounded logits (within 2^-8 relative); loss and gradients keep the bf16 tolerances.
CHUNKED_LSE_TOL = 2.0 ** -8


@pytest.mark.parametrize("method", ["fused", "chunked"])
@pytest.mark.parametrize("name", ["gemma_like", "headline", "qwen_like"])
def test_fused_full_size(name, method):
    c = CONFIGS[name]
    print(f"full-size {method} parity: {name} BT={c.BT} H={c.H} V={c.V}", flush=True)
    exp = _expected(name)
    inp = make_config(name)
    tol = TOL[c.dtype]
    b = None if inp.bias is None else dev(inp.bias, c.dtype)
    r = lce.lce_fwd_bwd(dev(inp.hidden, c.dtype), dev(inp.weight, c.dtype), b, dev(inp.targets),
                        z_loss=c.z_loss, reduction=c.reduction, return_lse=True, method=method)
    torch.cuda.synchronize()
    assert int(r["n_valid"].item()) == int(exp["n_valid"])
    assert rel(r["loss"].item(), float(exp["loss"])) <= tol["loss"], (r["loss"].item(), float(exp["loss"]))
    lse = host64(r["lse"])
    lse_tol = tol["lse"] if method == "fused" else CHUNKED_LSE_TOL
    assert np.max(np.abs(lse - exp["lse"]) / np.maximum(1.0, np.abs(exp["lse"]))) <= lse_tol
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


@pytest.mark.parametrize("saved", [False, True], ids=["recomputed", "saved"])
def test_rows_full_size_headline(saved):
    """Per-row outputs and their backward at the headline size (statistics recomputed, or the
    forward's LSE and entropy passed in): sampled rows against the per-row oracle (each row's
    values and grad_input row depend on that row only), and the vocabulary sum of grad_W,
    which vanishes for logprob and entropy upstreams alone."""
    c = CONFIGS["headline"]
    print(f"full-size per-row parity: headline BT={c.BT} H={c.H} V={c.V}", flush=True)
    inp = make_config("headline")
    h, W, y = dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.targets)
    f = lce.lce_rows_forward(h, W, None, y)
    rng = np.random.default_rng(4)
    gp = rng.normal(size=c.BT).astype(np.float32)
    ge = rng.normal(size=c.BT).astype(np.float32)
    st = dict(lse=f["lse"], entropy=f["entropy"]) if saved else {}
    g = lce.lce_rows_backward(h, W, None, y, grad_logprobs=dev(gp), grad_entropy=dev(ge), workspace=f["workspace"],
                              **st)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 777, 30000, c.BT - 1] + list(np.nonzero(inp.targets == -100)[0][:2]))
    ref = oracle.lce_rows_oracle(inp.hidden[rows], inp.weight, None, inp.targets[rows],
                                 grad_logprobs=gp[rows], grad_entropy=ge[rows])
    # (one pass from the fp32 accumulator: the fused path's LSE tolerance)
    bound = TOL["bf16"]["lse"] * np.maximum(1.0, np.abs(ref["lse"]))
    sel = torch.from_numpy(rows).cuda()
    for k in ("lse", "logprobs", "entropy", "row_loss"):
        err = np.abs(host64(f[k][sel]) - ref[k])
        assert np.all(err <= bound), (k, float((err / bound).max()))
    gi = host64(g["grad_input"][sel])
    assert rel_fro(gi, ref["grad_input"]) <= TOL["bf16"]["grad"]
    gw = g["grad_weight"].float()
    assert float(gw.sum(dim=0).norm() / gw.norm()) <= TOL["bf16"]["grad"]


@pytest.mark.parametrize("name", ["headline", "gemma_like"])
def test_filtered_tiny_eps_full_size(name):
    """Gradient filtering at full size (the one-pass stored-operand backward with tile flags,
    grad_W over token ranges at the headline, in one range at gemma_like): with eps below every
    |dlogit| no tile is skipped, the loss is the exact call's bit for bit (the forward is shared)
    and the gradients stay within a quarter of the bf16 tolerance of it; with vocabulary
    sorting on top (grad_W rows through the order), the loss and gradients (returned in the
    original vocabulary order) stay within the bf16 tolerances of the exact call."""
    c = CONFIGS[name]
    print(f"full-size filtering, tiny eps: {name} BT={c.BT} H={c.H} V={c.V}", flush=True)
    inp = make_config(name)
    b = None if inp.bias is None else dev(inp.bias, c.dtype)
    args = (dev(inp.hidden, c.dtype), dev(inp.weight, c.dtype), b, dev(inp.targets))
    kw = dict(z_loss=c.z_loss, reduction=c.reduction)
    exact = lce.lce_fwd_bwd(*args, **kw)
    counts = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    filt = lce.lce_fwd_bwd(*args, filter_eps=1e-38, filter_counts=counts, **kw)
    torch.cuda.synchronize()
    cnt = counts.cpu().tolist()
    # every tile of both gradient products tested once, none skipped
    R, C = lce.filter_tile_shape(c.BT, c.H, c.V, torch.bfloat16)
    assert cnt == [0, -(-c.BT // R) * -(-c.V // C), 0, -(-c.V // R) * -(-c.BT // C)], (cnt, R, C)
    keys = ["loss", "grad_input", "grad_weight"] + (["grad_bias"] if b is not None else [])
    tol = TOL[c.dtype]
    for k in keys:
        if k == "loss":
            assert torch.equal(exact[k], filt[k]), k  # (the forward is shared)
        else:
            e = float((filt[k].float() - exact[k].float()).norm() / exact[k].float().norm())
            assert e <= tol["grad"] / 4, (k, e)
    del filt
    srt = lce.lce_fwd_bwd(*args, filter_eps=1e-38, sort_vocab=True, **kw)
    torch.cuda.synchronize()
    assert int(srt["n_valid"].item()) == int(exact["n_valid"].item())
    assert rel(srt["loss"].item(), exact["loss"].item()) <= tol["loss"]
    for k in keys[1:]:
        e = float((srt[k].float() - exact[k].float()).norm() / exact[k].float().norm())
        assert e <= tol["grad"], (k, e)


@pytest.mark.parametrize("name", ["headline", "gemma_like", "qwen_like"])
def test_filtered_full_size_sampled_tiles(name):
    """Gradient filtering at full size with the bench's threshold (eps = 2^-12, "Cut Cross
    Entropy visualized", "Gradient Filtering"), against the filtered oracle on sampled tiles
    in the call's own tile shape: grad_input of the first and last token tiles, grad_W (and
    grad_b) of the first, a middle and the last vocabulary tile, each computed by the oracle
    from the definitions (every token's LSE from the stored oracle values).  Where the
    filtered values differ from the exact ones by more than twice the bf16 tolerance, the GPU
    must be within a quarter of that difference of the filtered oracle, so that the tiles it
    skipped are the oracle's; a tile with every block skipped must come out exactly zero."""
    c = CONFIGS[name]
    print(f"full-size filtering, sampled tiles: {name} BT={c.BT} H={c.H} V={c.V}", flush=True)
    exp = _expected(name)
    inp = make_config(name)
    eps = 2.0 ** -12
    R, C = lce.filter_tile_shape(c.BT, c.H, c.V, torch.bfloat16)
    b = None if inp.bias is None else dev(inp.bias, c.dtype)
    counts = torch.zeros(4, dtype=torch.int64, device="cuda")
    r = lce.lce_fwd_bwd(dev(inp.hidden, c.dtype), dev(inp.weight, c.dtype), b, dev(inp.targets),
                        z_loss=c.z_loss, reduction=c.reduction, filter_eps=eps, filter_counts=counts)
    torch.cuda.synchronize()
    cnt = counts.cpu().tolist()
    assert cnt[1] == -(-c.BT // R) * -(-c.V // C) and cnt[3] == -(-c.V // R) * -(-c.BT // C), cnt
    assert 0 < cnt[0] < cnt[1] and 0 <= cnt[2] < cnt[3], cnt
    tol = TOL[c.dtype]["grad"]
    kw = dict(stat_rows=R, stream_rows=C, filter_eps=eps, z_loss=c.z_loss, reduction=c.reduction)

    def check(got, filt, exact, what):
        if not np.any(filt):
            assert not np.any(got), what  # every block skipped
            return
        d = rel_fro(filt, exact)
        e = rel_fro(got, filt)
        print(f"  {what}: filtered vs exact {d:.4f}, GPU vs filtered {e:.4f}", flush=True)
        assert e <= tol, (what, e)
        if d > 2 * tol:
            assert e <= d / 4, (what, e, d)

    for t0 in (0, (c.BT - 1) // R * R):
        o = oracle.filtered_grad_input_tile(inp.hidden, inp.weight, inp.bias, inp.targets, t0, **kw)
        got = host64(r["grad_input"][t0:t0 + R])
        check(got, o["grad_input"], o["grad_input_exact"], f"grad_input tokens {t0}..")
    for v0 in (0, (c.V // 2) // R * R, (c.V - 1) // R * R):
        o = oracle.filtered_grad_weight_tile(inp.hidden, inp.weight, inp.bias, inp.targets, v0, exp["lse"], **kw)
        got = host64(r["grad_weight"][v0:v0 + R])
        check(got, o["grad_weight"], o["grad_weight_exact"], f"grad_W entries {v0}..")
        if b is not None:
            check(host64(r["grad_bias"][v0:v0 + R]), o["grad_bias"], o["grad_bias_exact"], f"grad_b entries {v0}..")


def test_long_sequence_dlogits_blocks_under_2gib():
    """400000 tokens, H = 2048, V = 32000: the one-chunk budget (3.9 GiB) would hold a 3 GiB
    block of stored transposed dlogits, but every block is kept under 2^31 bytes (one buffer
    descriptor with 32-bit offsets per block), so the call runs the one-pass backward.
    Sampled tokens' LSE and grad_input rows against the oracle; grad_W by its vanishing
    vocabulary sum (no z-loss); ignored rows of grad_input exactly zero."""
    BT, H, V = 400000, 2048, 32000
    print(f"long-sequence fused call: BT={BT} H={H} V={V}", flush=True)
    inp = make_fused(BT, H, V, seed=11, ignore_frac=0.05)
    tol = TOL["bf16"]
    r = lce.lce_fwd_bwd(dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), None, dev(inp.targets),
                        reduction="mean", return_lse=True, method="fused")
    torch.cuda.synchronize()
    assert int(r["n_valid"].item()) == int((inp.targets != -100).sum())
    rows = np.random.default_rng(5).choice(BT, 24, replace=False)
    rows[:2] = [0, BT - 1]
    lse = host64(r["lse"][torch.from_numpy(rows).cuda()])
    want = oracle.lse_rows(inp.hidden, inp.weight, None, rows)
    assert np.max(np.abs(lse - want) / np.maximum(1.0, np.abs(want))) <= tol["lse"]
    gi = host64(r["grad_input"][torch.from_numpy(rows).cuda()])
    assert rel_fro(gi, oracle.grad_input_rows(inp.hidden, inp.weight, None, inp.targets, rows)) <= tol["grad"]
    ign = torch.from_numpy(inp.targets == -100).cuda()
    assert bool(ign.any()) and int(torch.count_nonzero(r["grad_input"][ign])) == 0
    gw = r["grad_weight"].float()
    assert torch.isfinite(gw).all()
    assert float(gw.sum(dim=0).norm() / gw.norm()) <= tol["grad"]
