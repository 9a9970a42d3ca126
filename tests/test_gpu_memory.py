"""Extra device memory of the default training paths at full size: the autograd wrappers
(linear_cross_entropy, and the per-row linear_logprobs_entropy; forward and backward) must stay
within one logits chunk beyond their inputs, outputs and gradients, the budget of "Fused Linear Cross-Entropy: The Math, the Memory
Wall, and Two Ways Around It", "The chunk-size trick" / "Memory profile" (Liger's fp32 chunk
of next_pow2(ceil(BT / ceil(V / H))) rows: 360,949,760 bytes at BT = 65535, V = 176245).
Measured with the torch allocator's peak around the call; the loss is checked against the
oracle's stored value so that the measured call is the real one."""

import os

import numpy as np
import pytest
import torch

import linear_cross_entropy_vocab_amd as lce
from oracle import liger_chunk_plan
from workloads import CONFIGS, make_config
from gpu_util import TOL, dev, rel

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("name", ["headline", "gemma_like", "qwen_like"])
def test_autograd_extra_memory_within_one_logits_chunk(name):
    c = CONFIGS[name]
    print(f"extra device memory, autograd path: {name} BT={c.BT} H={c.H} V={c.V}", flush=True)
    exp = np.load(os.path.join(HERE, "expected", f"{name}.npz"), allow_pickle=False)
    inp = make_config(name)
    h = dev(inp.hidden, c.dtype).requires_grad_(True)
    W = dev(inp.weight, c.dtype).requires_grad_(True)
    b = None if inp.bias is None else dev(inp.bias, c.dtype).requires_grad_(True)
    y = dev(inp.targets)
    del inp
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    loss = lce.linear_cross_entropy(h, W, y, b, z_loss=c.z_loss, reduction=c.reduction)
    loss.backward()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    # what is left after the backward is the gradients (and the loss): the rest of the peak
    # was transient, the extra memory of the op, as the allocator holds it (large blocks
    # rounded up to 2 MiB)
    extra = peak - torch.cuda.memory_allocated()
    budget = liger_chunk_plan(c.BT, c.V, c.H)["chunk_bytes"]
    ws = lce.fwd_bwd_workspace_bytes(c.BT, c.H, c.V, torch.bfloat16)
    print(f"  peak delta {peak - base} B, extra {extra} B, workspace {ws} B, budget {budget} B", flush=True)
    assert extra <= budget, (extra, budget)
    assert extra <= ws + (2 << 20), (extra, ws)
    assert rel(loss.item(), float(exp["loss"])) <= TOL[c.dtype]["loss"]
    assert torch.isfinite(W.grad.float().norm())


@pytest.mark.parametrize("name", ["headline", "gemma_like", "qwen_like"])
def test_rows_autograd_extra_memory_within_one_logits_chunk(name):
    """The per-row autograd path (linear_logprobs_entropy, forward and backward of a weighted
    sum of its three outputs) within the same one-chunk budget."""
    c = CONFIGS[name]
    print(f"extra device memory, per-row autograd path: {name} BT={c.BT} H={c.H} V={c.V}", flush=True)
    inp = make_config(name)
    h = dev(inp.hidden, c.dtype).requires_grad_(True)
    W = dev(inp.weight, c.dtype).requires_grad_(True)
    b = None if inp.bias is None else dev(inp.bias, c.dtype).requires_grad_(True)
    y = dev(inp.targets)
    rng = np.random.default_rng(9)
    wl, we = (dev(rng.normal(size=c.BT).astype(np.float32)) for _ in range(2))
    del inp
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    lp, ent, rl = lce.linear_logprobs_entropy(h, W, y, b, z_loss=c.z_loss)
    ((lp * wl).sum() + (ent * we).sum() + rl.sum()).backward()
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - torch.cuda.memory_allocated()
    budget = liger_chunk_plan(c.BT, c.V, c.H)["chunk_bytes"]
    print(f"  extra {extra} B, budget {budget} B", flush=True)
    assert extra <= budget, (extra, budget)
    assert torch.isfinite(W.grad.float().norm()) and torch.isfinite(h.grad.float().norm())
