"""Pins of the float64 oracle against things other than itself.

Each test ties the oracle to a closed form, an invariant, a textbook routine
(torch.nn.functional.cross_entropy / logsumexp with autograd, float64, CPU),
central finite differences, a pure-Python brute force, or numbers printed on
the pages.  Mutation tests at the end plant plausible mistakes into the oracle
(on the CPU) and check that at least one pin catches each.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import lce as olce
from workloads import make_fused, make_ce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _small(BT=37, H=16, V=53, seed=0, bias=True, ignore_frac=0.2, w_std=0.5):
    inp = make_fused(BT, H, V, dtype="f32", seed=seed, w_std=w_std,
                     bias_std=0.3 if bias else None, ignore_frac=ignore_frac)
    return inp.hidden.astype(np.float64), inp.weight.astype(np.float64), \
        None if inp.bias is None else inp.bias.astype(np.float64), inp.targets


def _torch_ref(h, W, b, y, reduction, mu):
    """Loss and grads from torch's own cross_entropy/logsumexp + autograd, float64."""
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = None if b is None else torch.tensor(b, requires_grad=True)
    yt = torch.tensor(y)
    z = ht @ Wt.T
    if bt is not None:
        z = z + bt
    valid = yt != -100
    n_valid = int(valid.sum())
    ce = F.cross_entropy(z, yt, ignore_index=-100, reduction="sum")
    zl = (torch.logsumexp(z, dim=1)[valid] ** 2).sum()
    c = 1.0 / max(n_valid, 1) if reduction == "mean" else 1.0
    L = c * (ce + mu * zl)
    L.backward()
    return (L.item(), ht.grad.numpy(), Wt.grad.numpy(),
            None if bt is None else bt.grad.numpy())


# --------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("mu", [0.0, 1e-2])
def test_zero_weight_gives_log_V(reduction, mu):
    h, W, _, y = _small(BT=29, H=8, V=1000, bias=False)
    W[:] = 0.0
    out = oracle.lce_oracle(h, W, None, y, reduction=reduction, z_loss=mu)
    n = int((y != -100).sum())
    logV = math.log(1000)
    assert np.all(out["lse"] == logV)  # sum of V exact ones, then log: bit-exact
    per = logV + mu * logV * logV
    expect = per if reduction == "mean" else n * per
    assert out["loss"] == pytest.approx(expect, rel=1e-15)
    # gradient of each valid row: c * (1/V * (1 + 2 mu log V) - onehot)
    c = 1.0 / n if reduction == "mean" else 1.0
    assert np.all(out["grad_input"] == 0.0)  # grad_input = G . W = 0 because W = 0
    gw = out["grad_weight"]
    # grad_W[v] = sum_t G[t, v] h[t]; check one column by hand
    valid = y != -100
    G = np.where(valid[:, None], c * (1.0 + 2 * mu * logV) / 1000.0, 0.0) * np.ones((29, 1000))
    G[np.nonzero(valid)[0], y[valid]] -= c
    np.testing.assert_allclose(gw, G.T @ h, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_zero_weight_grad_bias_closed_form(reduction):
    """W = 0 with a bias: every row's logits are b, so LSE = log sum e^b for every row and
    grad_b[v] = c (n_valid softmax(b)_v (1 + 2 mu LSE) - #{t valid: y_t = v})."""
    h, W, b, y = _small(BT=41, H=8, V=300)
    W[:] = 0.0
    mu = 2e-2
    out = oracle.lce_oracle(h, W, b, y, reduction=reduction, z_loss=mu)
    bb = b.astype(np.float64)
    L = math.log(float(np.sum(np.exp(bb))))
    p = np.exp(bb) / np.sum(np.exp(bb))
    valid = y != -100
    n = int(valid.sum())
    c = 1.0 / n if reduction == "mean" else 1.0
    count = np.bincount(y[valid], minlength=300)
    np.testing.assert_allclose(out["lse"], L, rtol=1e-14)
    np.testing.assert_allclose(out["grad_bias"], c * (n * p * (1.0 + 2.0 * mu * L) - count), rtol=1e-11, atol=1e-14)


def test_all_ignored_gives_zero():
    h, W, b, y = _small()
    y[:] = -100
    out = oracle.lce_oracle(h, W, b, y, z_loss=1e-3)
    assert out["n_valid"] == 0 and out["loss"] == 0.0
    assert np.all(out["grad_input"] == 0) and np.all(out["grad_weight"] == 0)
    assert np.all(out["grad_bias"] == 0)


def test_single_class_vocab():
    h, W, b, y = _small(V=1, ignore_frac=0.0)
    y[:] = 0
    out = oracle.lce_oracle(h, W, b, y)
    assert abs(out["loss"]) < 1e-15
    assert np.abs(out["grad_input"]).max() < 1e-15
    assert np.abs(out["grad_weight"]).max() < 1e-15


# --------------------------------------------------------------------- invariants

def test_bias_shift_invariance():
    h, W, b, y = _small()
    kappa = 3.75
    a = oracle.lce_oracle(h, W, b, y)
    s = oracle.lce_oracle(h, W, b + kappa, y)
    assert s["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(s["lse"], a["lse"] + kappa, rtol=1e-14)
    for k in ("grad_input", "grad_weight", "grad_bias"):
        np.testing.assert_allclose(s[k], a[k], rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("mu", [0.0, 0.05])
def test_dlogit_row_invariants(mu):
    h, W, b, y = _small()
    X = h @ W.T + b
    out = oracle.ce_oracle(X, y, z_loss=mu)
    d = out["dlogits"]
    valid = y != -100
    lse = out["lse"]
    # ignored rows are exactly zero ([P3] "Kernel design")
    assert np.all(d[~valid] == 0.0)
    # rows sum to 2 mu LSE (0 without z-loss): sum p = 1, one -1 at the target
    np.testing.assert_allclose(d[valid].sum(axis=1), 2 * mu * lse[valid], atol=1e-13)
    # target entry is p_y (1 + 2 mu LSE) - 1, all others positive
    rows = np.nonzero(valid)[0]
    p = np.exp(X - lse[:, None])
    np.testing.assert_allclose(d[rows, y[rows]], p[rows, y[rows]] * (1 + 2 * mu * lse[rows]) - 1,
                               rtol=1e-13)
    mask = np.ones_like(d, dtype=bool)
    mask[rows, y[rows]] = False
    mask[~valid] = False
    assert np.all(d[mask] > 0)


def test_grad_weight_and_bias_sum_to_zero_without_zloss():
    h, W, b, y = _small()
    out = oracle.lce_oracle(h, W, b, y)
    np.testing.assert_allclose(out["grad_weight"].sum(axis=0), 0.0, atol=1e-14)
    assert abs(out["grad_bias"].sum()) < 1e-14
    valid = y != -100
    assert np.all(out["grad_input"][~valid] == 0.0)


# --------------------------------------------------------------------- textbook routine

@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("mu", [0.0, 1e-2])
def test_matches_torch_autograd(reduction, bias, mu):
    h, W, b, y = _small(bias=bias)
    out = oracle.lce_oracle(h, W, b, y, reduction=reduction, z_loss=mu)
    L, gi, gw, gb = _torch_ref(h, W, b, y, reduction, mu)
    assert out["loss"] == pytest.approx(L, rel=1e-12)
    np.testing.assert_allclose(out["grad_input"], gi, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["grad_weight"], gw, rtol=1e-10, atol=1e-14)
    if bias:
        np.testing.assert_allclose(out["grad_bias"], gb, rtol=1e-10, atol=1e-14)
    else:
        assert out["grad_bias"] is None


def test_matches_torch_at_workload_like_scale():
    """A larger, chunked case: exercise row chunking against torch in one shot."""
    h, W, b, y = _small(BT=300, H=64, V=5000, bias=True, w_std=0.125)
    out = oracle.lce_oracle(h, W, b, y, rows_per_chunk=17)
    L, gi, gw, gb = _torch_ref(h, W, b, y, "mean", 0.0)
    assert out["loss"] == pytest.approx(L, rel=1e-12)
    np.testing.assert_allclose(out["grad_input"], gi, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(out["grad_weight"], gw, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(out["grad_bias"], gb, rtol=1e-9, atol=1e-15)


def test_ce_oracle_matches_torch():
    ce = make_ce(19, 301, dtype="f32", seed=3, ignore_frac=0.2)
    X = ce.logits.astype(np.float64)
    y = ce.targets
    for mu in (0.0, 1e-3):
        out = oracle.ce_oracle(X, y, z_loss=mu)
        Xt = torch.tensor(X, requires_grad=True)
        yt = torch.tensor(y)
        v = yt != -100
        L = F.cross_entropy(Xt, yt, ignore_index=-100, reduction="sum") + \
            mu * (torch.logsumexp(Xt, 1)[v] ** 2).sum()
        L.backward()
        assert out["ce_sum"] + mu * out["z_sum"] == pytest.approx(L.item(), rel=1e-13)
        np.testing.assert_allclose(out["dlogits"], Xt.grad.numpy(), rtol=1e-11, atol=1e-15)
        if mu == 0.0:
            assert out["z_sum"] == 0.0


# --------------------------------------------------------------------- finite differences

@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("mu", [0.0, 0.03])
def test_central_finite_differences(reduction, mu):
    h, W, b, y = _small(BT=7, H=4, V=6, seed=11, bias=True, ignore_frac=0.3, w_std=0.8)
    assert (y == -100).any() and (y != -100).any()
    out = oracle.lce_oracle(h, W, b, y, reduction=reduction, z_loss=mu)
    eps = 1e-6

    def L(hh, WW, bb):
        return oracle.lce_oracle(hh, WW, bb, y, reduction=reduction, z_loss=mu,
                                 grads=False)["loss"]

    for name, arr, grad in (("h", h, out["grad_input"]), ("W", W, out["grad_weight"]),
                            ("b", b, out["grad_bias"])):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            ap = arr.copy()
            am = arr.copy()
            ap[i] += eps
            am[i] -= eps
            args_p = {"h": (ap, W, b), "W": (h, ap, b), "b": (h, W, ap)}[name]
            args_m = {"h": (am, W, b), "W": (h, am, b), "b": (h, W, am)}[name]
            fd[i] = (L(*args_p) - L(*args_m)) / (2 * eps)
        err = np.abs(fd - grad).max() / max(np.abs(grad).max(), 1e-12)
        assert err < 1e-7, (name, err)


# --------------------------------------------------------------------- brute force

def _brute(h, W, b, y, reduction, mu):
    BT, H = len(h), len(h[0])
    V = len(W)
    valid = [int(t) != -100 for t in y]
    n = sum(valid)
    c = (1.0 / max(n, 1)) if reduction == "mean" else 1.0
    terms = []
    gi = [[0.0] * H for _ in range(BT)]
    gw = [[0.0] * H for _ in range(V)]
    gb = [0.0] * V
    for t in range(BT):
        z = [math.fsum(h[t][k] * W[v][k] for k in range(H)) + (b[v] if b is not None else 0.0)
             for v in range(V)]
        m = max(z)
        lse = m + math.log(math.fsum(math.exp(zz - m) for zz in z))
        if not valid[t]:
            continue
        terms.append(lse - z[int(y[t])] + mu * lse * lse)
        g = [c * (math.exp(z[v] - lse) * (1 + 2 * mu * lse) - (1.0 if v == int(y[t]) else 0.0))
             for v in range(V)]
        for k in range(H):
            gi[t][k] = math.fsum(g[v] * W[v][k] for v in range(V))
        for v in range(V):
            for k in range(H):
                gw[v][k] += g[v] * h[t][k]
            gb[v] += g[v]
    return c * math.fsum(terms), gi, gw, gb


@pytest.mark.parametrize("reduction,mu", [("mean", 0.0), ("sum", 0.02)])
def test_brute_force_python_loops(reduction, mu):
    h, W, b, y = _small(BT=9, H=5, V=11, seed=5, bias=True, ignore_frac=0.25)
    out = oracle.lce_oracle(h, W, b, y, reduction=reduction, z_loss=mu)
    L, gi, gw, gb = _brute(h.tolist(), W.tolist(), b.tolist(), y.tolist(), reduction, mu)
    assert out["loss"] == pytest.approx(L, rel=1e-14)
    np.testing.assert_allclose(out["grad_input"], np.array(gi), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out["grad_weight"], np.array(gw), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out["grad_bias"], np.array(gb), rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------- consistency

def test_fused_equals_ce_on_materialised_logits():
    h, W, b, y = _small()
    for reduction, mu in (("mean", 0.0), ("sum", 1e-2), ("mean", 1e-2)):
        f = oracle.lce_oracle(h, W, b, y, reduction=reduction, z_loss=mu)
        ce = oracle.ce_oracle(h @ W.T + b, y, z_loss=mu)
        c = f["scale"]
        assert f["loss"] == pytest.approx(c * (ce["ce_sum"] + mu * ce["z_sum"]), rel=1e-13)
        G = c * ce["dlogits"]
        np.testing.assert_allclose(f["grad_input"], G @ W, rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(f["grad_weight"], G.T @ h, rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(f["grad_bias"], G.sum(0), rtol=1e-11, atol=1e-15)


def test_row_pieces_equal_full_oracle():
    h, W, b, y = _small(BT=50, V=97)
    mu = 1e-2
    full = oracle.lce_oracle(h, W, b, y, z_loss=mu)
    rows = np.array([0, 3, 17, 49])
    vocab = np.array([0, 5, 50, 96])
    lse = oracle.lse_all(h, W, b, rows_per_chunk=7)
    np.testing.assert_allclose(lse, full["lse"], rtol=1e-14)
    np.testing.assert_allclose(oracle.lse_rows(h, W, b, rows), full["lse"][rows], rtol=1e-14)
    np.testing.assert_allclose(oracle.grad_input_rows(h, W, b, y, rows, z_loss=mu),
                               full["grad_input"][rows], rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(oracle.grad_weight_rows(h, W, b, y, vocab, lse, z_loss=mu),
                               full["grad_weight"][vocab], rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(oracle.grad_bias_entries(h, W, b, y, vocab, lse, z_loss=mu),
                               full["grad_bias"][vocab], rtol=1e-11, atol=1e-15)


def test_minus_inf_bias_equals_smaller_vocabulary():
    """Entries whose bias is -inf contribute e^-inf = 0 to every LSE ("Cut Cross Entropy
    visualized", "Forward Kernel": the accumulation starts from -inf): the problem reduces
    exactly to the vocabulary without them, and their grad_W rows and grad_b entries are 0."""
    h, W, b, y = _small(BT=41, V=70, ignore_frac=0.1)
    masked = np.zeros(70, dtype=bool)
    masked[[0, 1, 2, 33, 34, 69]] = True
    keep = np.nonzero(~masked)[0]
    # targets only on kept entries (a target on a masked entry has an infinite loss)
    valid = y != -100
    y = np.where(valid, keep[y % keep.size], y)
    bm = b.copy()
    bm[masked] = -np.inf
    new_id = np.full(70, -1)
    new_id[keep] = np.arange(keep.size)
    yr = np.where(valid, new_id[np.where(valid, y, 0)], y)
    for reduction, mu in (("mean", 0.0), ("sum", 1e-2)):
        full = oracle.lce_oracle(h, W, bm, y, reduction=reduction, z_loss=mu)
        red = oracle.lce_oracle(h, W[keep], b[keep], yr, reduction=reduction, z_loss=mu)
        assert np.isfinite(full["loss"])
        assert full["loss"] == pytest.approx(red["loss"], rel=1e-13)
        np.testing.assert_allclose(full["lse"], red["lse"], rtol=1e-14)
        np.testing.assert_allclose(full["grad_input"], red["grad_input"], rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(full["grad_weight"][keep], red["grad_weight"], rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(full["grad_bias"][keep], red["grad_bias"], rtol=1e-11, atol=1e-15)
        assert np.all(full["grad_weight"][masked] == 0.0) and np.all(full["grad_bias"][masked] == 0.0)


def test_ce_oracle_selected_rows_equal_full_call():
    """ce_oracle's dlogit_rows branch (only the listed rows of dlogits, in that order) returns
    exactly the full call's rows and the same sums."""
    inp = make_ce(29, 301, dtype="f32", seed=5, ignore_frac=0.2)
    rows = np.array([28, 0, 3, 3, 17])
    for mu in (0.0, 1e-2):
        full = oracle.ce_oracle(inp.logits, inp.targets, z_loss=mu, rows_per_chunk=4)
        part = oracle.ce_oracle(inp.logits, inp.targets, z_loss=mu, dlogit_rows=rows)
        assert part["dlogits"].shape == (rows.size, 301)
        np.testing.assert_array_equal(part["dlogits"], full["dlogits"][rows])
        assert part["ce_sum"] == full["ce_sum"] and part["z_sum"] == full["z_sum"]
        assert part["n_valid"] == full["n_valid"]
        np.testing.assert_array_equal(part["lse"], full["lse"])


def test_target_out_of_range_raises():
    h, W, b, y = _small()
    y = y.copy()
    y[3] = W.shape[0]
    with pytest.raises(oracle.TargetRangeError):
        oracle.lce_oracle(h, W, b, y)
    y[3] = -1
    with pytest.raises(oracle.TargetRangeError):
        oracle.ce_oracle(h @ W.T, y)


# --------------------------------------------------------------------- page-printed numbers

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split("=")
                vals[k] = int(v)
    return vals


def test_liger_chunk_table_from_first_page():
    g = _read_golden("liger_chunk_table.txt")
    plan = oracle.liger_chunk_plan(g["BT"], g["V"], g["H"])
    for k in ("inc_factor", "chunk_size", "num_chunks", "chunk_bytes"):
        assert plan[k] == g[k], k


# --------------------------------------------------------------------- planted mistakes

def _pins_fail(monkeypatch, target, replacement):
    monkeypatch.setattr(olce, target, replacement)
    failures = 0
    for fn in (lambda: test_matches_torch_autograd("mean", True, 1e-2),
               lambda: test_matches_torch_autograd("sum", False, 0.0),
               lambda: test_bias_shift_invariance(),
               lambda: test_dlogit_row_invariants(0.0),
               lambda: test_zero_weight_gives_log_V("mean", 1e-2)):
        try:
            fn()
        except AssertionError:
            failures += 1
    return failures


def test_planted_mistakes_are_caught(monkeypatch):
    orig_dl = olce._dlogits
    orig_lse = olce._lse
    orig_logits = olce._logits
    orig_scale = olce._scale
    mutants = {
        "_dlogits": [
            lambda z, lse, y, v, c, mu: -orig_dl(z, lse, y, v, c, mu),            # wrong sign
            lambda z, lse, y, v, c, mu: orig_dl(z, lse, y, v, c, 0.0),            # dropped z-loss term
            lambda z, lse, y, v, c, mu: orig_dl(z, lse, np.where(v, y, 0),        # mask dropped
                                                np.ones_like(v), c, mu),
            lambda z, lse, y, v, c, mu: orig_dl(z, lse, np.where(v, (y + 1) % z.shape[1], y),
                                                v, c, mu),                        # wrong target index
        ],
        "_lse": [
            lambda z: z.max(axis=1),                                              # dropped log-sum term
            lambda z: np.log(np.exp(z - z.max(1, keepdims=True)).sum(axis=1)),   # dropped max
        ],
        "_logits": [
            lambda h, W, b: h @ W.T,                                              # bias dropped
        ],
        "_scale": [
            lambda n, r: 1.0 / max(n + 1, 1) if r == "mean" else 1.0,             # off-by-one count
        ],
    }
    for target, fns in mutants.items():
        for fn in fns:
            assert _pins_fail(monkeypatch, target, fn) > 0, target
            monkeypatch.setattr(olce, target, {"_dlogits": orig_dl, "_lse": orig_lse,
                                               "_logits": orig_logits,
                                               "_scale": orig_scale}[target])
