"""Write the oracle's expected values for the full-size workloads (tests/expected/*.npz).

Calls only the float64 oracle (oracle/) on the seeded inputs of workloads/; nothing here
comes from the HIP path.  Full-size parity tests compare the GPU against these files:
loss, n_valid and every row's LSE exactly as the oracle computes them, plus sampled rows
of grad_input, grad_W and entries of grad_b (each computed from the definitions one row
or one vocabulary column at a time).

    python tests/expected/make_expected.py [name ...]      # a few minutes per workload
"""

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import CONFIGS, make_config  # noqa: E402


def sample_rows(y, n, seed):
    rng = np.random.default_rng(seed)
    BT = y.shape[0]
    ign = np.nonzero(y == -100)[0]
    rows = {0, BT - 1, BT // 2}
    rows.update(ign[:2].tolist())
    rows.update(rng.choice(BT, size=n, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def sample_vocab(y, V, n, seed):
    rng = np.random.default_rng(seed + 1)
    vals = {0, 1, 2, V - 1, V // 2}
    valid_y = y[y != -100]
    vals.update(valid_y[:4].tolist())
    vals.update(rng.choice(V, size=n, replace=False).tolist())
    return np.array(sorted(vals), dtype=np.int64)


def fused(name):
    c = CONFIGS[name]
    inp = make_config(name)
    t = time.time()
    out = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=c.z_loss,
                            reduction=c.reduction, grads=False)
    print(f"{name}: forward {time.time() - t:.1f}s loss={out['loss']!r}", flush=True)
    rows = sample_rows(inp.targets, 24, c.seed)
    vocab = sample_vocab(inp.targets, c.V, 24, c.seed)
    gi = oracle.grad_input_rows(inp.hidden, inp.weight, inp.bias, inp.targets, rows,
                                z_loss=c.z_loss, reduction=c.reduction)
    gw = oracle.grad_weight_rows(inp.hidden, inp.weight, inp.bias, inp.targets, vocab, out["lse"],
                                 z_loss=c.z_loss, reduction=c.reduction)
    extra = {}
    if inp.bias is not None:
        bvocab = sample_vocab(inp.targets, c.V, 250, c.seed + 7)
        extra["bias_vocab"] = bvocab
        extra["grad_bias"] = oracle.grad_bias_entries(inp.hidden, inp.weight, inp.bias, inp.targets,
                                                      bvocab, out["lse"], z_loss=c.z_loss,
                                                      reduction=c.reduction)
    np.savez_compressed(os.path.join(HERE, f"{name}.npz"), loss=out["loss"], ce_sum=out["ce_sum"],
                        z_sum=out["z_sum"], n_valid=out["n_valid"], lse=out["lse"], rows=rows,
                        grad_input_rows=gi.astype(np.float32), vocab=vocab,
                        grad_weight_rows=gw.astype(np.float32), **extra)
    print(f"{name}: done {time.time() - t:.1f}s", flush=True)


def ce_only():
    c = CONFIGS["ce_only"]
    inp = make_config("ce_only")
    res = {}
    for tag, mu in (("mu0", 0.0), ("mu1e-4", 1e-4)):
        t = time.time()
        out = oracle.ce_oracle(inp.logits, inp.targets, z_loss=mu, dlogit_rows=np.array([0]))
        res[f"ce_sum_{tag}"] = out["ce_sum"]
        res[f"z_sum_{tag}"] = out["z_sum"]
        print(f"ce_only {tag}: {time.time() - t:.1f}s ce_sum={out['ce_sum']!r}", flush=True)
    np.savez_compressed(os.path.join(HERE, "ce_only.npz"), lse=out["lse"], n_valid=out["n_valid"], **res)


if __name__ == "__main__":
    names = sys.argv[1:] or ["ce_only", "gemma_like", "qwen_like", "headline"]
    for n in names:
        if n == "ce_only":
            ce_only()
        else:
            fused(n)
