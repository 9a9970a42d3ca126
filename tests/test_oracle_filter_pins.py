"""Pins of the gradient-filtering oracle (``oracle.lce_oracle_filtered``).

It follows "Cut Cross Entropy visualized", "Gradient Filtering": a dlogits block whose
entries are all below filter_eps contributes nothing to the gradient GEMMs.  Pinned by:
  * eps = 0 skips nothing and gives exactly the unfiltered oracle;
  * an eps above every |dlogit| skips every tile and gives zero gradients, loss unchanged;
  * a vocabulary range pushed to probability ~e^-60 by its bias, aligned to the tiles and
    holding no target, is skipped exactly where the tile geometry says (counts checked
    tile by tile), and the gradients move by less than what was dropped;
  * a pure-Python brute force with its own block loop (2 x 3 tiles, so that skipped and
    kept blocks mix in both GEMMs) agrees to rounding.
"""

import math

import numpy as np
import pytest

import oracle
from workloads import make_fused


def _case(BT, H, V, seed=0, bias=True, ignore_frac=0.2, w_std=0.5):
    inp = make_fused(BT, H, V, dtype="f32", seed=seed, w_std=w_std,
                     bias_std=0.3 if bias else None, ignore_frac=ignore_frac)
    b = None if inp.bias is None else inp.bias.astype(np.float64)
    return inp.hidden.astype(np.float64), inp.weight.astype(np.float64), b, inp.targets


@pytest.mark.parametrize("mu", [0.0, 1e-2])
def test_zero_eps_is_unfiltered(mu):
    h, W, b, y = _case(150, 8, 300, seed=1)
    ref = oracle.lce_oracle(h, W, b, y, z_loss=mu)
    f = oracle.lce_oracle_filtered(h, W, b, y, filter_eps=0.0, z_loss=mu)
    assert f["skipped_input"] == 0 and f["skipped_weight"] == 0
    assert f["loss"] == ref["loss"]
    np.testing.assert_allclose(f["grad_input"], ref["grad_input"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f["grad_weight"], ref["grad_weight"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f["grad_bias"], ref["grad_bias"], rtol=1e-12, atol=1e-15)


def test_huge_eps_skips_everything():
    h, W, b, y = _case(70, 8, 90, seed=2)
    ref = oracle.lce_oracle(h, W, b, y)
    f = oracle.lce_oracle_filtered(h, W, b, y, filter_eps=1e9)
    assert f["tiles_input"] == 2 * 6 and f["tiles_weight"] == 2 * 5  # ceil(70/64)*ceil(90/16), ...
    assert f["skipped_input"] == f["tiles_input"] and f["skipped_weight"] == f["tiles_weight"]
    assert f["loss"] == ref["loss"]
    assert not f["grad_input"].any() and not f["grad_weight"].any() and not f["grad_bias"].any()


def test_suppressed_vocabulary_block_is_skipped_where_the_tiles_say():
    BT, H, V = 150, 8, 192
    h, W, b, y = _case(BT, H, V, seed=3, ignore_frac=0.1)
    b = b.copy()
    b[64:128] = -60.0                       # p ~ e^-60 there
    y = np.where((y >= 64) & (y < 128), y - 64, y)  # no target in the suppressed range
    eps = 1e-12
    ref = oracle.lce_oracle(h, W, b, y)
    f = oracle.lce_oracle_filtered(h, W, b, y, filter_eps=eps)
    n_tok64, n_tok16 = -(-BT // 64), -(-BT // 16)
    # grad_input tiles are 64 tokens x 16 vocab: vocab tiles 4..7 of every token tile
    assert f["skipped_input"] == 4 * n_tok64
    # grad_W tiles are 64 vocab x 16 tokens: vocab tile 1 of every token tile
    assert f["skipped_weight"] == n_tok16
    # what was dropped is below eps per entry; the gradients move by at most that much
    c = ref["scale"]
    bound_in = c * eps * np.abs(W).sum(axis=0).max() * 1.01
    assert np.abs(f["grad_input"] - ref["grad_input"]).max() <= bound_in
    assert np.abs(f["grad_weight"][64:128]).max() == 0.0
    np.testing.assert_allclose(f["grad_weight"][:64], ref["grad_weight"][:64], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f["grad_weight"][128:], ref["grad_weight"][128:], rtol=1e-12, atol=1e-15)
    assert np.abs(f["grad_bias"][64:128]).max() == 0.0


def _brute_filtered(h, W, b, y, eps, sr, tr, mu=0.0):
    """Pure-Python filtered gradients (mean reduction) with its own block loop."""
    BT, H, V = len(h), len(h[0]), len(W)
    valid = [yy != -100 for yy in y]
    n = sum(valid)
    c = 1.0 / max(n, 1)
    G = [[0.0] * V for _ in range(BT)]
    for t in range(BT):
        z = [math.fsum(h[t][k] * W[v][k] for k in range(H)) + b[v] for v in range(V)]
        m = max(z)
        lse = m + math.log(math.fsum(math.exp(zz - m) for zz in z))
        if valid[t]:
            for v in range(V):
                G[t][v] = math.exp(z[v] - lse) * (1 + 2 * mu * lse) - (1.0 if v == y[t] else 0.0)

    def keep(rows_of, cols_of, r, col):  # block of (r, col) in a [rows_of x cols_of] grid
        r0, c0 = (r // sr) * sr, (col // tr) * tr
        return not all(abs(rows_of(rr, cc)) < eps
                       for rr in range(r0, min(r0 + sr, len_rows(rows_of)))
                       for cc in range(c0, min(c0 + tr, len_cols(rows_of))))

    def len_rows(f):
        return BT if f is gin else V

    def len_cols(f):
        return V if f is gin else BT

    def gin(r, col):  # tokens x vocab
        return G[r][col]

    def gwt(r, col):  # vocab x tokens
        return G[col][r]

    gi = [[c * math.fsum(G[t][v] * W[v][k] for v in range(V) if keep(gin, gin, t, v))
           for k in range(H)] for t in range(BT)]
    kw = [[keep(gwt, gwt, v, t) for t in range(BT)] for v in range(V)]
    gw = [[c * math.fsum(G[t][v] * h[t][k] for t in range(BT) if kw[v][t]) for k in range(H)]
          for v in range(V)]
    gb = [c * math.fsum(G[t][v] for t in range(BT) if kw[v][t]) for v in range(V)]
    return gi, gw, gb


def test_brute_force_with_mixed_blocks():
    h, W, b, y = _case(11, 3, 13, seed=4, w_std=3.0)
    eps = 0.05
    f = oracle.lce_oracle_filtered(h, W, b, y, filter_eps=eps, stat_rows=2, stream_rows=3)
    assert 0 < f["skipped_input"] < f["tiles_input"]   # some blocks skipped, some kept
    assert 0 < f["skipped_weight"] < f["tiles_weight"]
    gi, gw, gb = _brute_filtered(h.tolist(), W.tolist(), b.tolist(), y.tolist(), eps, 2, 3)
    np.testing.assert_allclose(f["grad_input"], np.array(gi), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f["grad_weight"], np.array(gw), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f["grad_bias"], np.array(gb), rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------- vocabulary sorting

def test_logit_average_is_the_logit_of_the_mean_hidden_row():
    # linearity: the batch mean of z_t = W h_t + b over the rows that count is W hbar + b
    inp = make_fused(90, 12, 70, dtype="f32", seed=31, bias_std=0.4, ignore_frac=0.2)
    avg, perm = oracle.vocab_sort_order(inp.hidden, inp.weight, inp.bias, inp.targets)
    valid = inp.targets != -100
    hbar = inp.hidden.astype(np.float64)[valid].mean(axis=0)
    np.testing.assert_allclose(avg, inp.weight.astype(np.float64) @ hbar + inp.bias, rtol=1e-12, atol=1e-14)
    assert sorted(perm.tolist()) == list(range(70))
    assert np.all(np.diff(avg[perm]) <= 0.0)


def test_sort_ties_keep_vocabulary_order():
    inp = make_fused(20, 8, 12, dtype="f32", seed=32, bias_std=None)
    W = inp.weight.copy()
    W[[3, 7, 10]] = W[5]                     # four entries with the same average logit
    avg, perm = oracle.vocab_sort_order(inp.hidden, W, None, inp.targets)
    tied = [v for v in perm if v in (3, 5, 7, 10)]
    assert tied == [3, 5, 7, 10]


def test_sorting_changes_nothing_without_filtering():
    inp = make_fused(100, 16, 300, dtype="f32", seed=33, bias_std=0.3, ignore_frac=0.1, z_loss=1e-3)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=1e-3)
    r = oracle.lce_oracle_filtered(inp.hidden, inp.weight, inp.bias, inp.targets, filter_eps=0.0,
                                   z_loss=1e-3, sort_vocab=True)
    for k in ("grad_input", "grad_weight", "grad_bias"):
        np.testing.assert_allclose(r[k], ref[k], rtol=1e-10, atol=1e-15, err_msg=k)
    assert r["skipped_input"] == 0 and r["skipped_weight"] == 0


def test_sorting_clusters_the_likely_entries():
    # 16 "hot" ids, every 16th one, take nearly all the probability and are the targets:
    # unsorted, every 16-entry tile and every 64-entry block holds one, so nothing is
    # skipped; sorted, they fill the first tile, and of the 16 grad_input tiles (64 tokens x
    # 16 entries) 15 are negligible, of the 16 grad_W tiles (64 entries x 16 tokens) 12.
    BT, H, V = 64, 8, 256
    inp = make_fused(BT, H, V, dtype="f32", seed=34, w_std=0.01, bias_std=None)
    hot = np.arange(0, V, 16)
    b = np.full(V, -20.0)
    b[hot] = 20.0
    y = hot[np.arange(BT) % 16]
    kw = dict(filter_eps=1e-6)
    plain = oracle.lce_oracle_filtered(inp.hidden, inp.weight, b, y, **kw)
    srt = oracle.lce_oracle_filtered(inp.hidden, inp.weight, b, y, sort_vocab=True, **kw)
    assert (plain["skipped_input"], plain["tiles_input"]) == (0, 16)
    assert (plain["skipped_weight"], plain["tiles_weight"]) == (0, 16)
    assert (srt["skipped_input"], srt["tiles_input"]) == (15, 16)
    assert (srt["skipped_weight"], srt["tiles_weight"]) == (12, 16)
    assert set(srt["vocab_perm"][:16].tolist()) == set(hot.tolist())
    ref = oracle.lce_oracle(inp.hidden, inp.weight, b, y)
    for k in ("grad_input", "grad_weight", "grad_bias"):
        np.testing.assert_allclose(srt[k], ref[k], rtol=0, atol=1e-9, err_msg=k)


@pytest.mark.parametrize("R,C", [(64, 16), (256, 64)])
@pytest.mark.parametrize("mu,reduction", [(0.0, "mean"), (1e-2, "sum")])
def test_tile_pieces_reassemble_the_filtered_oracle(R, C, mu, reduction):
    """The one-tile pieces used by full-size checks (filtered_grad_input_tile over R tokens,
    filtered_grad_weight_tile over R vocabulary entries given every row's LSE) put back
    together give lce_oracle_filtered's gradients and skip counts, with ragged last tiles in
    both directions and an eps at which both kept and skipped blocks occur."""
    BT, V = 3 * R - 7, 5 * R + 3
    h, W, b, y = _case(BT, 8, V, seed=5, w_std=1.5)
    eps = 0.1
    full = oracle.lce_oracle_filtered(h, W, b, y, filter_eps=eps, z_loss=mu, reduction=reduction,
                                      stat_rows=R, stream_rows=C)
    assert 0 < full["skipped_input"] < full["tiles_input"]
    assert 0 < full["skipped_weight"] < full["tiles_weight"]
    ref = oracle.lce_oracle(h, W, b, y, z_loss=mu, reduction=reduction)
    kw = dict(stat_rows=R, stream_rows=C, filter_eps=eps, z_loss=mu, reduction=reduction)
    gi, gie, ski, nbi = [], [], 0, 0
    for t0 in range(0, BT, R):
        t = oracle.filtered_grad_input_tile(h, W, b, y, t0, **kw)
        gi.append(t["grad_input"])
        gie.append(t["grad_input_exact"])
        ski += t["skipped"]
        nbi += t["blocks"]
    np.testing.assert_allclose(np.concatenate(gi), full["grad_input"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(np.concatenate(gie), ref["grad_input"], rtol=1e-12, atol=1e-15)
    assert (ski, nbi) == (full["skipped_input"], full["tiles_input"])
    gw, gb, gwe, gbe, skw, nbw = [], [], [], [], 0, 0
    for v0 in range(0, V, R):
        t = oracle.filtered_grad_weight_tile(h, W, b, y, v0, ref["lse"], **kw)
        gw.append(t["grad_weight"])
        gb.append(t["grad_bias"])
        gwe.append(t["grad_weight_exact"])
        gbe.append(t["grad_bias_exact"])
        skw += t["skipped"]
        nbw += t["blocks"]
    np.testing.assert_allclose(np.concatenate(gw), full["grad_weight"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(np.concatenate(gb), full["grad_bias"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(np.concatenate(gwe), ref["grad_weight"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(np.concatenate(gbe), ref["grad_bias"], rtol=1e-12, atol=1e-15)
    assert (skw, nbw) == (full["skipped_weight"], full["tiles_weight"])
