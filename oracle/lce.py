"""Plain float64 definitions of fused linear cross-entropy and its gradients.

Sources (page title, then section / equation):
  [P1] "Fused Linear Cross-Entropy: The Math, the Memory Wall, and Two Ways
       Around It" -- "The setting" (per-token forward, mean reduction with
       ignore_index -100), "The identity that makes fused fwbw possible" (boxed
       dl/dz = softmax(z) - onehot(y); consequence 3, the max-shifted LSE),
       "From dlogits to grad_input and grad_W" (scaled dlogits; boxed
       grad_input and grad_W GEMMs; grad_b column sum), "The chunk-size trick"
       (inc_factor / chunk_size / num_chunks table).
  [P2] "Cut Cross Entropy visualized" -- "Breakdown: Forward Pass" (inputs E,
       C, bias, targets; mean and sum reductions), "Breakdown: Backward Pass"
       (S = exp(z - LSE), S - Y).
  [P3] "Greyhound -- Cross-Entropy" -- opening formulas (loss_i and the z-loss
       term z_i = LSE_i**2), "Kernel design" (softmax term scaled by the z-loss
       derivative before the target column is adjusted; ignored rows get a zero
       gradient and are not counted), "Raw kernel helper" (loss = ce_sum /
       max(n_valid, 1)).

Readings where the pages leave a step open:
  * z-loss in the fused loss: L = c * sum_valid [LSE - z_y + mu * LSE**2]; its
    logit gradient is p * (1 + 2 mu LSE) - onehot(y).
  * c = 1 / max(n_valid, 1) for "mean" (so an all-ignored batch gives 0, as the
    clamp in [P3] does), c = 1 for "sum".
  * A target outside [0, V) that is not ignore_index is an error.
  * The standalone helper's dlogits are the unscaled gradient of
    ce_sum + mu * z_sum.

Memory is bounded by processing rows in chunks; each row is still computed on
its own from the definition, so chunking changes nothing numerically beyond
BLAS summation order.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

IGNORE_INDEX = -100
_CHUNK_BYTES = 1 << 28  # rows per chunk chosen so a float64 [rows, V] block is <= 256 MiB


class TargetRangeError(ValueError):
    """A target is neither ignore_index nor a vocabulary id."""


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _valid_mask(targets: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    """Rows that count: y != ignore_index ([P1] "The setting"); others must be in [0, V)."""
    y = np.asarray(targets, dtype=np.int64)
    valid = y != ignore_index
    bad = valid & ((y < 0) | (y >= V))
    if np.any(bad):
        raise TargetRangeError(f"{int(bad.sum())} targets outside [0, {V}) and != {ignore_index}")
    return valid


def _scale(n_valid: int, reduction: str) -> float:
    """c = 1/max(n_valid, 1) for mean ([P1] mean reduction; [P3] clamp), 1 for sum ([P2])."""
    if reduction == "mean":
        return 1.0 / max(n_valid, 1)
    if reduction == "sum":
        return 1.0
    raise ValueError(f"reduction must be 'mean' or 'sum', got {reduction!r}")


def _rows_per_chunk(V: int) -> int:
    return max(1, _CHUNK_BYTES // (8 * max(V, 1)))


def _logits(h: np.ndarray, W: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """z = W . hidden[t] (+ b) for a block of rows ([P1] "The setting"; bias per [P2] inputs)."""
    z = h @ W.T
    if b is not None:
        z = z + b[None, :]
    return z


def _lse(z: np.ndarray) -> np.ndarray:
    """LSE(z) = max z + log sum exp(z - max z), per row ([P1] consequence 3)."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def _dlogits(z: np.ndarray, lse: np.ndarray, y: np.ndarray, valid: np.ndarray,
             c: float, mu: float) -> np.ndarray:
    """c * valid * (softmax(z) * (1 + 2 mu LSE) - onehot(y)) ([P1] boxed identity and
    scaled dlogits; [P3] z-loss derivative applied before the target column)."""
    p = np.exp(z - lse[:, None])
    g = p * (1.0 + 2.0 * mu * lse)[:, None]
    rows = np.nonzero(valid)[0]
    g[rows, y[rows]] -= 1.0
    g[~valid, :] = 0.0
    return c * g


def lce_oracle(hidden, weight, bias, targets, *, ignore_index: int = IGNORE_INDEX,
               z_loss: float = 0.0, reduction: str = "mean", grads: bool = True,
               rows_per_chunk: Optional[int] = None) -> dict:
    """Fused linear cross-entropy: loss and (optionally) grad_input, grad_W, grad_b.

    hidden [BT, H], weight [V, H] (nn.Linear layout), bias [V] or None, targets
    [BT] int.  Returns a dict with loss, n_valid, lse [BT], ce_sum, z_sum and,
    with grads=True, grad_input [BT, H], grad_weight [V, H], grad_bias [V] or None.
    All float results are float64.
    """
    h = _f64(hidden)
    W = _f64(weight)
    b = _f64(bias)
    y = np.asarray(targets, dtype=np.int64)
    BT, H = h.shape
    V = W.shape[0]
    valid = _valid_mask(y, V, ignore_index)
    n_valid = int(valid.sum())
    c = _scale(n_valid, reduction)
    mu = float(z_loss)

    lse = np.empty(BT)
    zy = np.zeros(BT)
    gi = np.zeros((BT, H)) if grads else None
    gw = np.zeros((V, H)) if grads else None
    gb = np.zeros(V) if (grads and b is not None) else None
    R = rows_per_chunk or _rows_per_chunk(V)
    for r0 in range(0, BT, R):
        r1 = min(BT, r0 + R)
        z = _logits(h[r0:r1], W, b)
        lse[r0:r1] = _lse(z)
        vr = valid[r0:r1]
        idx = np.nonzero(vr)[0]
        zy[r0 + idx] = z[idx, y[r0:r1][idx]]
        if grads:
            g = _dlogits(z, lse[r0:r1], y[r0:r1], vr, c, mu)
            gi[r0:r1] = g @ W                      # grad_input = dlogits . W
            gw += g.T @ h[r0:r1]                   # grad_W = dlogits^T . hidden
            if gb is not None:
                gb += g.sum(axis=0)                # grad_b = sum_t dlogits[t, :]
    ce_terms = np.where(valid, lse - zy, 0.0)
    z_terms = np.where(valid, lse * lse, 0.0)
    ce_sum = math.fsum(ce_terms.tolist())
    z_sum = math.fsum(z_terms.tolist()) if mu != 0.0 else 0.0
    loss = c * (ce_sum + mu * z_sum)
    out = dict(loss=loss, n_valid=n_valid, lse=lse, z_target=zy, ce_sum=ce_sum, z_sum=z_sum,
               scale=c)
    if grads:
        out.update(grad_input=gi, grad_weight=gw, grad_bias=gb)
    return out


def _mean_logit(z: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """E_p[z] = sum_v p_v z_v per row, p = exp(z - LSE); an entry with p_v = 0 (a logit of
    -inf: a vocabulary entry masked by a -inf bias) adds nothing, the limit of p log p -> 0
    in the entropy -sum_v p_v log p_v."""
    p = np.exp(z - lse[:, None])
    return (p * np.where(p > 0.0, z, 0.0)).sum(axis=1)


def _row_coefficients(lse, ez, valid, gl, gp, ge, mu):
    """(alpha, beta, gamma) of dlogits = p * (alpha + beta * z) - gamma * onehot(y) for the
    upstream gradients gl (row loss), gp (logprobs), ge (entropy); see lce_rows_oracle."""
    vf = valid.astype(np.float64)
    alpha = vf * (gl * (1.0 + 2.0 * mu * lse) - gp) + ge * ez
    beta = -ge
    gamma = vf * (gl - gp)
    return alpha, beta, gamma


def lce_rows_oracle(hidden, weight, bias, targets, *, ignore_index: int = IGNORE_INDEX,
                    z_loss: float = 0.0, grad_row_loss=None, grad_logprobs=None,
                    grad_entropy=None, rows_per_chunk: Optional[int] = None) -> dict:
    """Per-row outputs of the LM head for RL-style use, and their gradients.

    [P1] "Strategy 2" names the per-row quantities an RL trainer keeps (each row's
    log-probability of its target and the entropy of its softmax, beside the LSE); the
    pages give no formulas for them, so the textbook definitions are used:
      row_loss[t] = valid_t * (LSE_t - z_t[y_t] + mu * LSE_t**2)   (the fused loss per row)
      logprobs[t] = valid_t * (z_t[y_t] - LSE_t)                    (log softmax at the target)
      entropy[t]  = -sum_v p_tv log p_tv = LSE_t - sum_v p_tv z_tv   (every row)
    With per-row upstream gradients (gl, gp, ge; any may be None = 0) the gradients are
    those of  sum_t gl_t row_loss_t + gp_t logprobs_t + ge_t entropy_t.  By the chain rule
    through p = softmax(z) (d LSE / dz_v = p_v; d (sum_u p_u z_u) / dz_v = p_v (1 + z_v - E[z])):
      dlogits[t, v] = p_tv * (alpha_t + beta_t * z_tv) - gamma_t * [v == y_t]
      alpha_t = valid_t * (gl_t * (1 + 2 mu LSE_t) - gp_t) + ge_t * E_t[z]
      beta_t  = -ge_t
      gamma_t = valid_t * (gl_t - gp_t)
    and grad_input = dlogits . W, grad_W = dlogits^T . hidden, grad_b = sum_t dlogits
    ([P1] "From dlogits to grad_input and grad_W").
    """
    h = _f64(hidden)
    W = _f64(weight)
    b = _f64(bias)
    y = np.asarray(targets, dtype=np.int64)
    BT, H = h.shape
    V = W.shape[0]
    valid = _valid_mask(y, V, ignore_index)
    mu = float(z_loss)
    gl = None if grad_row_loss is None else _f64(grad_row_loss)
    gp = None if grad_logprobs is None else _f64(grad_logprobs)
    ge = None if grad_entropy is None else _f64(grad_entropy)
    want_grads = gl is not None or gp is not None or ge is not None

    lse = np.empty(BT)
    zy = np.zeros(BT)
    ez = np.empty(BT)
    gi = np.zeros((BT, H)) if want_grads else None
    gw = np.zeros((V, H)) if want_grads else None
    gb = np.zeros(V) if (want_grads and b is not None) else None
    R = rows_per_chunk or _rows_per_chunk(V)
    for r0 in range(0, BT, R):
        r1 = min(BT, r0 + R)
        z = _logits(h[r0:r1], W, b)
        L = _lse(z)
        lse[r0:r1] = L
        ez[r0:r1] = _mean_logit(z, L)
        vr = valid[r0:r1]
        idx = np.nonzero(vr)[0]
        zy[r0 + idx] = z[idx, y[r0:r1][idx]]
        if want_grads:
            n = r1 - r0
            glc = gl[r0:r1] if gl is not None else np.zeros(n)
            gpc = gp[r0:r1] if gp is not None else np.zeros(n)
            gec = ge[r0:r1] if ge is not None else np.zeros(n)
            alpha, beta, gamma = _row_coefficients(L, ez[r0:r1], vr, glc, gpc, gec, mu)
            p = np.exp(z - L[:, None])
            # (p = 0 entries, masked by a -inf bias, have zero gradient: p (alpha + beta z) -> 0)
            g = p * (alpha[:, None] + beta[:, None] * np.where(p > 0.0, z, 0.0))
            g[idx, y[r0:r1][idx]] -= gamma[idx]
            gi[r0:r1] = g @ W
            gw += g.T @ h[r0:r1]
            if gb is not None:
                gb += g.sum(axis=0)
    row_loss = np.where(valid, lse - zy + mu * lse * lse, 0.0)
    logprobs = np.where(valid, zy - lse, 0.0)
    entropy = lse - ez
    out = dict(lse=lse, row_loss=row_loss, logprobs=logprobs, entropy=entropy, mean_z=ez,
               n_valid=int(valid.sum()))
    if want_grads:
        out.update(grad_input=gi, grad_weight=gw, grad_bias=gb)
    return out


def _block_keep(g: np.ndarray, rows: int, cols: int, eps: float):
    """Mask of g [R, C] that is False inside every (rows x cols) block, aligned at 0, whose
    entries all have |g| < eps ([P2] "Gradient Filtering": a block is skipped only if
    every value in it is below the threshold), and the number of such blocks."""
    R, C = g.shape
    keep = np.ones_like(g, dtype=bool)
    skipped = 0
    for r0 in range(0, R, rows):
        for c0 in range(0, C, cols):
            if np.all(np.abs(g[r0:r0 + rows, c0:c0 + cols]) < eps):
                keep[r0:r0 + rows, c0:c0 + cols] = False
                skipped += 1
    return keep, skipped


def vocab_sort_order(hidden, weight, bias, targets, *, ignore_index: int = IGNORE_INDEX,
                     rows_per_chunk: Optional[int] = None):
    """Vocabulary sorting of [P2] "Vocabulary Sorting": each vocabulary entry's average logit
    over the batch (here over the rows that count, divided by max(n_valid, 1)), and the order
    of the entries by decreasing average logit (ties by increasing id).  Returns
    (logit_avg [V], perm [V]) with perm[i] = the id at sorted position i."""
    h = _f64(hidden)
    W = _f64(weight)
    b = _f64(bias)
    y = np.asarray(targets, dtype=np.int64)
    BT = h.shape[0]
    V = W.shape[0]
    valid = _valid_mask(y, V, ignore_index)
    total = np.zeros(V)
    R = rows_per_chunk or _rows_per_chunk(V)
    for r0 in range(0, BT, R):
        r1 = min(BT, r0 + R)
        z = _logits(h[r0:r1], W, b)
        total += z[valid[r0:r1]].sum(axis=0)
    avg = total / max(int(valid.sum()), 1)
    perm = np.argsort(-avg, kind="stable")
    return avg, perm


def lce_oracle_filtered(hidden, weight, bias, targets, *, filter_eps: float,
                        ignore_index: int = IGNORE_INDEX, z_loss: float = 0.0,
                        reduction: str = "mean", stat_rows: int = 64,
                        stream_rows: int = 16, sort_vocab: bool = False) -> dict:
    """The gradients with CCE-style gradient filtering ([P2] "Gradient Filtering").

    Each gradient GEMM sees the dlogits in tiles; a tile whose entries are all below
    filter_eps in magnitude contributes nothing (its contribution is zeroed, not
    deferred).  The tiles are those of the GEMM that produces the gradient:
      grad_input: stat_rows tokens x stream_rows vocabulary entries (aligned at 0);
      grad_W and grad_b: stat_rows vocabulary entries x stream_rows tokens.
    Reading: the threshold applies to the dlogits of the summed loss, valid * (softmax *
    (1 + 2 mu LSE) - onehot), i.e. before the 1/n_valid of the mean, so that the test
    depends on the size of an entry relative to the others in its row and not on the
    batch size.  The loss is not affected.  Returns the lce_oracle dict with the filtered
    gradients and the tile counts skipped_input / tiles_input, skipped_weight /
    tiles_weight.
    With sort_vocab, the vocabulary is first put in the order of vocab_sort_order
    ([P2] "Vocabulary Sorting": W rows, bias entries and target ids permuted), the filtered
    gradients are computed in that order (so the tiles group entries of similar average
    logit), and grad_W / grad_b are returned in the original order (plus vocab_perm and
    logit_avg).
    """
    if sort_vocab:
        avg, perm = vocab_sort_order(hidden, weight, bias, targets, ignore_index=ignore_index)
        pos = np.empty_like(perm)
        pos[perm] = np.arange(len(perm))
        y0 = np.asarray(targets, dtype=np.int64)
        ys = np.where(y0 == ignore_index, y0, pos[np.clip(y0, 0, len(perm) - 1)])
        Ws = _f64(weight)[perm]
        bs = None if bias is None else _f64(bias)[perm]
        out = lce_oracle_filtered(hidden, Ws, bs, ys, filter_eps=filter_eps, ignore_index=ignore_index,
                                  z_loss=z_loss, reduction=reduction, stat_rows=stat_rows,
                                  stream_rows=stream_rows)
        gw = np.empty_like(out["grad_weight"])
        gw[perm] = out["grad_weight"]
        out["grad_weight"] = gw
        if out["grad_bias"] is not None:
            gb = np.empty_like(out["grad_bias"])
            gb[perm] = out["grad_bias"]
            out["grad_bias"] = gb
        out.update(vocab_perm=perm, logit_avg=avg)
        return out
    h = _f64(hidden)
    W = _f64(weight)
    b = _f64(bias)
    y = np.asarray(targets, dtype=np.int64)
    BT, H = h.shape
    V = W.shape[0]
    out = lce_oracle(hidden, weight, bias, targets, ignore_index=ignore_index, z_loss=z_loss,
                     reduction=reduction, grads=False)
    valid = _valid_mask(y, V, ignore_index)
    c = out["scale"]
    mu = float(z_loss)
    lse = out["lse"]
    gi = np.zeros((BT, H))
    gw = np.zeros((V, H))
    gb = np.zeros(V) if b is not None else None
    a = max(stat_rows, stream_rows)
    R = max(a, (_rows_per_chunk(V) // a) * a)  # chunks start on tile boundaries of both GEMMs
    skipped_in = skipped_w = 0
    for r0 in range(0, BT, R):
        r1 = min(BT, r0 + R)
        g = _dlogits(_logits(h[r0:r1], W, b), lse[r0:r1], y[r0:r1], valid[r0:r1], 1.0, mu)
        k_in, n_in = _block_keep(g, stat_rows, stream_rows, filter_eps)
        k_wt, n_w = _block_keep(g.T, stat_rows, stream_rows, filter_eps)
        skipped_in += n_in
        skipped_w += n_w
        gi[r0:r1] = c * (np.where(k_in, g, 0.0) @ W)       # grad_input = dlogits . W
        g_w = np.where(k_wt.T, g, 0.0)
        gw += c * (g_w.T @ h[r0:r1])                       # grad_W = dlogits^T . hidden
        if gb is not None:
            gb += c * g_w.sum(axis=0)                      # grad_b = sum_t dlogits[t, :]
    out.update(grad_input=gi, grad_weight=gw, grad_bias=gb,
               skipped_input=skipped_in, tiles_input=-(-BT // stat_rows) * -(-V // stream_rows),
               skipped_weight=skipped_w, tiles_weight=-(-V // stat_rows) * -(-BT // stream_rows))
    return out


def ce_oracle(logits, targets, *, ignore_index: int = IGNORE_INDEX, z_loss: float = 0.0,
              rows_per_chunk: Optional[int] = None, dlogit_rows=None) -> dict:
    """Standalone cross-entropy on existing logits ([P3] opening formulas, "Kernel design").

    Returns ce_sum = sum_valid (LSE - x_y), z_sum = sum_valid LSE**2 (0 when z-loss is
    off), n_valid, lse [B] and dlogits [B, V] = valid * (softmax * (1 + 2 mu LSE) - onehot),
    the unscaled gradient of ce_sum + mu * z_sum.  With dlogit_rows (an index array) only
    those rows of dlogits are returned, in that order (bounds memory for large inputs).
    """
    y = np.asarray(targets, dtype=np.int64)
    B, V = np.shape(logits)
    valid = _valid_mask(y, V, ignore_index)
    mu = float(z_loss)
    lse = np.empty(B)
    xy = np.zeros(B)
    full = dlogit_rows is None
    d = np.empty((B, V)) if full else None
    R = rows_per_chunk or _rows_per_chunk(V)
    for r0 in range(0, B, R):
        r1 = min(B, r0 + R)
        z = _f64(logits[r0:r1])
        lse[r0:r1] = _lse(z)
        vr = valid[r0:r1]
        idx = np.nonzero(vr)[0]
        xy[r0 + idx] = z[idx, y[r0:r1][idx]]
        if full:
            d[r0:r1] = _dlogits(z, lse[r0:r1], y[r0:r1], vr, 1.0, mu)
    if not full:
        rows = np.asarray(dlogit_rows)
        z = _f64(np.asarray(logits)[rows])
        d = _dlogits(z, lse[rows], y[rows], valid[rows], 1.0, mu)
    ce_sum = math.fsum(np.where(valid, lse - xy, 0.0).tolist())
    z_sum = math.fsum(np.where(valid, lse * lse, 0.0).tolist()) if mu != 0.0 else 0.0
    return dict(ce_sum=ce_sum, z_sum=z_sum, n_valid=int(valid.sum()), lse=lse, dlogits=d)


# ---------------------------------------------------------------------------
# Row-at-a-time pieces for full-size checks: each output entry is computed from
# the same definitions as above, one row (or one vocabulary column) at a time.
# ---------------------------------------------------------------------------

def lse_rows(hidden, weight, bias, rows) -> np.ndarray:
    """LSE of z_t = W . hidden[t] + b for the listed token rows."""
    W = _f64(weight)
    b = _f64(bias)
    h = _f64(np.asarray(hidden)[np.asarray(rows)])
    return _lse(_logits(h, W, b))


def lse_all(hidden, weight, bias, rows_per_chunk: Optional[int] = None) -> np.ndarray:
    """LSE of every token row (the forward statistic the backward reuses, [P2] backward)."""
    hidden = np.asarray(hidden)
    BT = hidden.shape[0]
    V = np.asarray(weight).shape[0]
    W = _f64(weight)
    b = _f64(bias)
    out = np.empty(BT)
    R = rows_per_chunk or _rows_per_chunk(V)
    for r0 in range(0, BT, R):
        r1 = min(BT, r0 + R)
        out[r0:r1] = _lse(_logits(_f64(hidden[r0:r1]), W, b))
    return out


def grad_input_rows(hidden, weight, bias, targets, rows, *, ignore_index: int = IGNORE_INDEX,
                    z_loss: float = 0.0, reduction: str = "mean") -> np.ndarray:
    """Rows of grad_input = dlogits . W for the listed tokens ([P1] boxed grad_input)."""
    W = _f64(weight)
    b = _f64(bias)
    y_all = np.asarray(targets, dtype=np.int64)
    V = W.shape[0]
    valid_all = _valid_mask(y_all, V, ignore_index)
    c = _scale(int(valid_all.sum()), reduction)
    rows = np.asarray(rows)
    z = _logits(_f64(np.asarray(hidden)[rows]), W, b)
    lse = _lse(z)
    g = _dlogits(z, lse, y_all[rows], valid_all[rows], c, float(z_loss))
    return g @ W


def _dlogit_columns(hidden, weight, bias, targets, vocab, lse, ignore_index, z_loss, reduction,
                    rows_per_chunk=None):
    """dlogits[:, v] for the listed vocabulary ids, given every row's LSE."""
    hidden = np.asarray(hidden)
    W = _f64(weight)
    b = _f64(bias)
    y = np.asarray(targets, dtype=np.int64)
    V = W.shape[0]
    valid = _valid_mask(y, V, ignore_index)
    c = _scale(int(valid.sum()), reduction)
    mu = float(z_loss)
    vocab = np.asarray(vocab)
    Wv = W[vocab]
    bv = None if b is None else b[vocab]
    BT = hidden.shape[0]
    G = np.empty((BT, vocab.shape[0]))
    R = rows_per_chunk or max(1, (1 << 26) // max(vocab.shape[0], 1))
    for r0 in range(0, BT, R):
        r1 = min(BT, r0 + R)
        z = _f64(hidden[r0:r1]) @ Wv.T
        if bv is not None:
            z = z + bv[None, :]
        p = np.exp(z - lse[r0:r1, None]) * (1.0 + 2.0 * mu * lse[r0:r1])[:, None]
        p -= (y[r0:r1, None] == vocab[None, :])
        p[~valid[r0:r1], :] = 0.0
        G[r0:r1] = c * p
    return G


def grad_weight_rows(hidden, weight, bias, targets, vocab, lse, *,
                     ignore_index: int = IGNORE_INDEX, z_loss: float = 0.0,
                     reduction: str = "mean") -> np.ndarray:
    """Rows grad_W[v, :] = sum_t dlogits[t, v] hidden[t, :] ([P1] boxed grad_W), given LSE."""
    G = _dlogit_columns(hidden, weight, bias, targets, vocab, np.asarray(lse, np.float64),
                        ignore_index, z_loss, reduction)
    return G.T @ _f64(hidden)


def grad_bias_entries(hidden, weight, bias, targets, vocab, lse, *,
                      ignore_index: int = IGNORE_INDEX, z_loss: float = 0.0,
                      reduction: str = "mean") -> np.ndarray:
    """Entries grad_b[v] = sum_t dlogits[t, v] ([P1] grad_b column sum), given LSE."""
    G = _dlogit_columns(hidden, weight, bias, targets, vocab, np.asarray(lse, np.float64),
                        ignore_index, z_loss, reduction)
    return G.sum(axis=0)


def filtered_grad_input_tile(hidden, weight, bias, targets, t0, *, stat_rows: int, stream_rows: int,
                             filter_eps: float, ignore_index: int = IGNORE_INDEX, z_loss: float = 0.0,
                             reduction: str = "mean") -> dict:
    """grad_input of one token tile under gradient filtering ([P2] "Gradient Filtering"), as
    lce_oracle_filtered computes it: the tokens t0 .. t0 + stat_rows - 1 (t0 a multiple of
    stat_rows; fewer at the end of the batch) against the whole vocabulary, in blocks of
    stream_rows entries aligned at 0; a block whose unscaled dlogits are all below filter_eps in
    magnitude adds nothing.  Each of these rows depends only on its own token, so the tile is
    computed exactly as the full call would, from the rows' own logits.  Returns grad_input
    (the filtered rows), grad_input_exact (the same rows unfiltered), skipped and blocks."""
    W = _f64(weight)
    b = _f64(bias)
    y_all = np.asarray(targets, dtype=np.int64)
    V = W.shape[0]
    valid_all = _valid_mask(y_all, V, ignore_index)
    c = _scale(int(valid_all.sum()), reduction)
    rows = np.arange(t0, min(int(t0) + stat_rows, y_all.shape[0]))
    z = _logits(_f64(np.asarray(hidden)[rows]), W, b)
    g = _dlogits(z, _lse(z), y_all[rows], valid_all[rows], 1.0, float(z_loss))
    keep, skipped = _block_keep(g, stat_rows, stream_rows, filter_eps)
    return dict(grad_input=c * (np.where(keep, g, 0.0) @ W), grad_input_exact=c * (g @ W),
                skipped=skipped, blocks=-(-V // stream_rows))


def filtered_grad_weight_tile(hidden, weight, bias, targets, v0, lse, *, stat_rows: int, stream_rows: int,
                              filter_eps: float, ignore_index: int = IGNORE_INDEX, z_loss: float = 0.0,
                              reduction: str = "mean") -> dict:
    """grad_W and grad_b of one vocabulary tile under gradient filtering ([P2] "Gradient
    Filtering"), as lce_oracle_filtered computes them: the entries v0 .. v0 + stat_rows - 1
    (v0 a multiple of stat_rows; fewer at the end of the vocabulary) against every token, in
    blocks of stream_rows tokens aligned at 0, given every token's LSE; a block whose
    unscaled dlogits are all below filter_eps in magnitude adds nothing.  Returns grad_weight,
    grad_bias (the filtered rows and entries), their unfiltered values, skipped and blocks."""
    V = np.asarray(weight).shape[0]
    BT = np.asarray(hidden).shape[0]
    vocab = np.arange(v0, min(int(v0) + stat_rows, V))
    y = np.asarray(targets, dtype=np.int64)
    c = _scale(int(_valid_mask(y, V, ignore_index).sum()), reduction)
    G = _dlogit_columns(hidden, weight, bias, targets, vocab, np.asarray(lse, np.float64), ignore_index, z_loss,
                        "sum")  # (unscaled: the threshold applies before c)
    keep_t, skipped = _block_keep(G.T, stat_rows, stream_rows, filter_eps)
    Gk = np.where(keep_t.T, G, 0.0)
    h = _f64(hidden)
    return dict(grad_weight=c * (Gk.T @ h), grad_weight_exact=c * (G.T @ h), grad_bias=c * Gk.sum(axis=0),
                grad_bias_exact=c * G.sum(axis=0), skipped=skipped, blocks=-(-BT // stream_rows))


def liger_chunk_plan(BT: int, V: int, H: int) -> dict:
    """Token-chunk sizing of [P1] "The chunk-size trick": inc_factor = ceil(V/H),
    chunk_size = next power of two >= ceil(BT/inc_factor), num_chunks = ceil(BT/chunk_size),
    and the bytes of one fp32 logits chunk (chunk_size x V x 4), the extra-memory budget."""
    inc = -(-V // H)
    need = -(-BT // inc)
    cs = 1
    while cs < need:
        cs *= 2
    return dict(inc_factor=inc, chunk_size=cs, num_chunks=-(-BT // cs), chunk_bytes=cs * V * 4)
