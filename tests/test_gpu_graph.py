"""The fused call (pipelined backward; one-pass plan, exact and filtered), the token-chunked
composition and the per-row backward captured in a HIP graph (through torch's
graph capture on the caller's stream) and replayed several times, with eager work and
synchronisations between the replays: every replay must reproduce the eager outputs bit for
bit (the library enqueues kernels only, so a caller can capture it; no memset nodes)."""

import pytest
import torch

import linear_cross_entropy_vocab_amd as lce
from workloads import make_fused
from gpu_util import dev

pytestmark = pytest.mark.gpu


CASES = [
    # (BT, H, V, method, filter_eps)
    (333, 256, 3001, "fused", 0.0),       # pipelined backward
    (333, 256, 3001, "chunked", 0.0),
    (700, 1024, 20000, "fused", 0.0),     # one-pass plan: 8 vocabulary blocks, running sum
    (700, 1024, 20000, "fused", 1e-4),    # the same with tile flags
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[3]}-{c[0]}x{c[1]}x{c[2]}" + ("-filtered" if c[4] else "")
                                             for c in CASES])
def test_graph_replays_match_eager(case):
    BT, H, V, method, eps = case
    inp = make_fused(BT, H, V, dtype="bf16", seed=71, bias_std=0.1, ignore_frac=0.1, z_loss=1e-3)
    h, W, b, y = dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.bias, "bf16"), dev(inp.targets)
    kw = dict(z_loss=inp.z_loss, reduction="mean", return_lse=True, method=method)
    counts = None
    if eps > 0:
        counts = torch.zeros(4, dtype=torch.int64, device="cuda")
        kw.update(filter_eps=eps, filter_counts=counts)
    eager = lce.lce_fwd_bwd(h, W, b, y, **kw)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items() if isinstance(v, torch.Tensor) and k != "workspace"}
    ref_counts = None if counts is None else counts.clone()
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    ws = torch.empty_like(eager["workspace"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        lce.lce_fwd_bwd(h, W, b, y, out=out, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    for t in out.values():
        t.zero_()
    with torch.cuda.graph(g):
        lce.lce_fwd_bwd(h, W, b, y, out=out, workspace=ws, **kw)
    for rep in range(3):
        for t in out.values():
            t.fill_(7)             # eager work between replays
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), (case, rep, k)
        if counts is not None:
            assert torch.equal(counts, ref_counts), (case, rep, counts.tolist())


def test_rows_backward_graph_replays_match_eager():
    """The per-row backward on the one-pass plan, captured and replayed the same way."""
    inp = make_fused(700, 1024, 20000, dtype="bf16", seed=72, bias_std=0.1, ignore_frac=0.1)
    h, W, b, y = dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.bias, "bf16"), dev(inp.targets)
    g = torch.randn(700, device="cuda")
    f = lce.lce_rows_forward(h, W, b, y)
    kw = dict(grad_logprobs=g, grad_entropy=0.5 * g, lse=f["lse"], entropy=f["entropy"], workspace=f["workspace"])
    eager = lce.lce_rows_backward(h, W, b, y, **kw)
    torch.cuda.synchronize()
    ref = {k: eager[k].clone() for k in ("grad_input", "grad_weight", "grad_bias")}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lce.lce_rows_backward(h, W, b, y, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):  # (the gradients come from the graph's memory pool)
        r = lce.lce_rows_backward(h, W, b, y, **kw)
    out = {k: r[k] for k in ref}
    for rep in range(3):
        for t in out.values():
            t.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), (rep, k)
