"""Pins of the per-row oracle (row loss, log-probabilities, entropy and the gradients of a
per-row weighted sum of them) against things other than itself: closed forms (uniform
softmax, two classes), invariants (bias shift), torch's log_softmax / softmax with autograd
in float64, central finite differences, a pure-Python brute force, and the fused oracle.
Planted mistakes in the oracle's pieces are each caught by at least one pin."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import lce as olce
from workloads import make_fused


def _small(BT=23, H=8, V=29, seed=0, bias=True, ignore_frac=0.25, w_std=0.7):
    inp = make_fused(BT, H, V, dtype="f32", seed=seed, w_std=w_std,
                     bias_std=0.3 if bias else None, ignore_frac=ignore_frac)
    return inp.hidden.astype(np.float64), inp.weight.astype(np.float64), \
        None if inp.bias is None else inp.bias.astype(np.float64), inp.targets


def _upstream(BT, seed):
    r = np.random.default_rng(seed)
    return r.normal(size=BT), r.normal(size=BT), r.normal(size=BT)


def _torch_rows(h, W, b, y, mu, gl, gp, ge):
    """Per-row outputs from torch's own log_softmax/softmax, and autograd of
    sum(gl * row_loss + gp * logprobs + ge * entropy), float64."""
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = None if b is None else torch.tensor(b, requires_grad=True)
    yt = torch.tensor(y)
    z = ht @ Wt.T
    if bt is not None:
        z = z + bt
    valid = yt != -100
    ls = F.log_softmax(z, dim=1)
    lse = torch.logsumexp(z, dim=1)
    ysafe = torch.where(valid, yt, torch.zeros_like(yt))
    lp = torch.where(valid, ls.gather(1, ysafe[:, None])[:, 0], torch.zeros_like(lse))
    ent = -(F.softmax(z, dim=1) * ls).sum(dim=1)
    rl = torch.where(valid, -lp + mu * lse * lse, torch.zeros_like(lse))
    total = (torch.tensor(gl) * rl).sum() + (torch.tensor(gp) * lp).sum() + (torch.tensor(ge) * ent).sum()
    total.backward()
    return dict(row_loss=rl.detach().numpy(), logprobs=lp.detach().numpy(), entropy=ent.detach().numpy(),
                lse=lse.detach().numpy(), grad_input=ht.grad.numpy(), grad_weight=Wt.grad.numpy(),
                grad_bias=None if bt is None else bt.grad.numpy())


# --------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("mu", [0.0, 0.05])
def test_uniform_softmax(mu):
    h, W, b, y = _small(seed=1, bias=False)
    W = np.zeros_like(W)
    out = oracle.lce_rows_oracle(h, W, None, y, z_loss=mu)
    V = W.shape[0]
    logV = math.log(V)
    valid = y != -100
    assert np.all(out["lse"] == logV)
    np.testing.assert_allclose(out["entropy"], logV, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(out["logprobs"], np.where(valid, -logV, 0.0))
    np.testing.assert_allclose(out["row_loss"], np.where(valid, logV + mu * logV * logV, 0.0),
                               rtol=1e-15)


def test_two_classes_entropy():
    h, W, b, y = _small(BT=31, H=6, V=2, seed=2)
    out = oracle.lce_rows_oracle(h, W, b, y)
    z = h @ W.T + b
    q = 1.0 / (1.0 + np.exp(-(z[:, 0] - z[:, 1])))     # P(class 0), logistic form
    ent = -(q * np.log(q) + (1 - q) * np.log(1 - q))
    np.testing.assert_allclose(out["entropy"], ent, rtol=1e-12)


def test_bias_shift_invariance():
    h, W, b, y = _small(seed=3)
    gl, gp, ge = _upstream(len(y), 3)
    a = oracle.lce_rows_oracle(h, W, b, y, grad_row_loss=gl, grad_logprobs=gp, grad_entropy=ge)
    c = oracle.lce_rows_oracle(h, W, b + 2.5, y, grad_row_loss=gl, grad_logprobs=gp, grad_entropy=ge)
    np.testing.assert_allclose(c["lse"], a["lse"] + 2.5, rtol=1e-13)
    for k in ("logprobs", "entropy", "row_loss", "grad_input", "grad_weight", "grad_bias"):
        np.testing.assert_allclose(c[k], a[k], rtol=1e-9, atol=1e-12, err_msg=k)


def test_masked_entries_equal_removed_entries():
    """Entries masked with a -inf bias (p = 0) are the same as entries that do not exist: every
    per-row output and every gradient of the kept entries equals that of the problem over the
    kept entries alone (targets renumbered), and the masked rows of grad_W and grad_b are 0."""
    h, W, b, y = _small(seed=5)
    V = W.shape[0]
    masked = np.zeros(V, dtype=bool)
    masked[[0, 3, 4, V - 1]] = True
    keep = np.nonzero(~masked)[0]
    y = y.copy()
    valid = y != -100
    y[valid] = keep[y[valid] % keep.size]
    bm = b.copy()
    bm[masked] = -np.inf
    gl, gp, ge = _upstream(len(y), 5)
    a = oracle.lce_rows_oracle(h, W, bm, y, z_loss=0.03, grad_row_loss=gl, grad_logprobs=gp, grad_entropy=ge)
    pos = np.full(V, -1)
    pos[keep] = np.arange(keep.size)
    yk = np.where(valid, pos[np.where(valid, y, 0)], y)
    c = oracle.lce_rows_oracle(h, W[keep], b[keep], yk, z_loss=0.03, grad_row_loss=gl, grad_logprobs=gp,
                               grad_entropy=ge)
    for k in ("lse", "logprobs", "entropy", "row_loss", "grad_input"):
        assert np.all(np.isfinite(a[k])), k
        np.testing.assert_allclose(a[k], c[k], rtol=1e-12, atol=1e-13, err_msg=k)
    np.testing.assert_allclose(a["grad_weight"][keep], c["grad_weight"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a["grad_bias"][keep], c["grad_bias"], rtol=1e-12, atol=1e-13)
    assert np.all(a["grad_weight"][masked] == 0.0) and np.all(a["grad_bias"][masked] == 0.0)


# --------------------------------------------------------------------- textbook routine

@pytest.mark.parametrize("mu,bias", [(0.0, True), (0.02, True), (0.0, False)])
def test_matches_torch_autograd(mu, bias):
    h, W, b, y = _small(seed=4, bias=bias)
    gl, gp, ge = _upstream(len(y), 4)
    out = oracle.lce_rows_oracle(h, W, b, y, z_loss=mu, grad_row_loss=gl, grad_logprobs=gp, grad_entropy=ge)
    ref = _torch_rows(h, W, b, y, mu, gl, gp, ge)
    for k in ("row_loss", "logprobs", "entropy", "lse", "grad_input", "grad_weight", "grad_bias"):
        if ref[k] is None:
            assert out[k] is None
            continue
        np.testing.assert_allclose(out[k], ref[k], rtol=1e-10, atol=1e-12, err_msg=k)


@pytest.mark.parametrize("which", ["row_loss", "logprobs", "entropy"])
def test_each_upstream_alone(which):
    h, W, b, y = _small(seed=5)
    gl, gp, ge = _upstream(len(y), 5)
    z = np.zeros(len(y))
    args = dict(row_loss=(gl, z, z), logprobs=(z, gp, z), entropy=(z, z, ge))[which]
    out = oracle.lce_rows_oracle(h, W, b, y, z_loss=0.01, grad_row_loss=args[0], grad_logprobs=args[1],
                                 grad_entropy=args[2])
    ref = _torch_rows(h, W, b, y, 0.01, *args)
    for k in ("grad_input", "grad_weight", "grad_bias"):
        np.testing.assert_allclose(out[k], ref[k], rtol=1e-10, atol=1e-12, err_msg=k)


# --------------------------------------------------------------------- finite differences

def test_central_finite_differences():
    h, W, b, y = _small(BT=6, H=3, V=5, seed=6, ignore_frac=0.3, w_std=0.9)
    assert (y == -100).any() and (y != -100).any()
    gl, gp, ge = _upstream(len(y), 6)
    mu = 0.04
    out = oracle.lce_rows_oracle(h, W, b, y, z_loss=mu, grad_row_loss=gl, grad_logprobs=gp, grad_entropy=ge)
    eps = 1e-6

    def F_(hh, WW, bb):
        r = oracle.lce_rows_oracle(hh, WW, bb, y, z_loss=mu)
        return float(np.dot(gl, r["row_loss"]) + np.dot(gp, r["logprobs"]) + np.dot(ge, r["entropy"]))

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
            fd[i] = (F_(*args_p) - F_(*args_m)) / (2 * eps)
        err = np.abs(fd - grad).max() / max(np.abs(grad).max(), 1e-12)
        assert err < 1e-7, (name, err)


# --------------------------------------------------------------------- brute force

def test_brute_force_python_loops():
    h, W, b, y = _small(BT=7, H=4, V=9, seed=7)
    out = oracle.lce_rows_oracle(h, W, b, y)
    for t in range(len(y)):
        z = [math.fsum(h[t][k] * W[v][k] for k in range(h.shape[1])) + b[v] for v in range(W.shape[0])]
        m = max(z)
        s = math.fsum(math.exp(zz - m) for zz in z)
        p = [math.exp(zz - m) / s for zz in z]
        ent = -math.fsum(pp * math.log(pp) for pp in p)
        assert out["entropy"][t] == pytest.approx(ent, rel=1e-13)
        if y[t] != -100:
            assert out["logprobs"][t] == pytest.approx(math.log(p[int(y[t])]), rel=1e-13)
        else:
            assert out["logprobs"][t] == 0.0


# --------------------------------------------------------------------- consistency

@pytest.mark.parametrize("reduction,mu", [("mean", 0.0), ("sum", 0.01)])
def test_loss_weights_give_fused_gradients(reduction, mu):
    h, W, b, y = _small(seed=8)
    fused = oracle.lce_oracle(h, W, b, y, z_loss=mu, reduction=reduction)
    gl = np.full(len(y), fused["scale"])
    out = oracle.lce_rows_oracle(h, W, b, y, z_loss=mu, grad_row_loss=gl)
    assert math.fsum(out["row_loss"].tolist()) * fused["scale"] == pytest.approx(fused["loss"], rel=1e-13)
    for k in ("grad_input", "grad_weight", "grad_bias"):
        np.testing.assert_allclose(out[k], fused[k], rtol=1e-11, atol=1e-14, err_msg=k)


# --------------------------------------------------------------------- planted mistakes

def _pins_fail(monkeypatch, target, replacement):
    monkeypatch.setattr(olce, target, replacement)
    failures = 0
    for fn in (lambda: test_matches_torch_autograd(0.02, True),
               lambda: test_two_classes_entropy(),
               lambda: test_uniform_softmax(0.05),
               lambda: test_each_upstream_alone("entropy")):
        try:
            fn()
        except AssertionError:
            failures += 1
    return failures


def test_planted_mistakes_are_caught(monkeypatch):
    orig_ml = olce._mean_logit
    orig_rc = olce._row_coefficients
    mutants = {
        "_mean_logit": [
            lambda z, lse: (np.exp(z - lse[:, None])).sum(axis=1),               # dropped z factor
            lambda z, lse: z.mean(axis=1),                                        # unweighted mean
        ],
        "_row_coefficients": [
            lambda L, ez, v, gl, gp, ge, mu: (lambda a, b, c: (a, -b, c))(*orig_rc(L, ez, v, gl, gp, ge, mu)),
            lambda L, ez, v, gl, gp, ge, mu: (lambda a, b, c: (a - ge * ez, b, c))(*orig_rc(L, ez, v, gl, gp, ge, mu)),
            lambda L, ez, v, gl, gp, ge, mu: orig_rc(L, ez, v, gl, -gp, ge, mu),   # logprob sign
            lambda L, ez, v, gl, gp, ge, mu: orig_rc(L, ez, np.ones_like(v), gl, gp, ge, mu),  # mask dropped
        ],
    }
    for target, fns in mutants.items():
        for fn in fns:
            assert _pins_fail(monkeypatch, target, fn) > 0, target
            monkeypatch.setattr(olce, target, {"_mean_logit": orig_ml, "_row_coefficients": orig_rc}[target])
