"""The fused call and the token-chunked composition captured in a HIP graph (through torch's
graph capture on the caller's stream) and replayed several times, with eager work and
synchronisations between the replays: every replay must reproduce the eager outputs bit for
bit (the library enqueues kernels only, so a caller can capture it; no memset nodes)."""

import pytest
import torch

import linear_cross_entropy_vocab_amd as lce
from workloads import make_fused
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("method", ["fused", "chunked"])
def test_graph_replays_match_eager(method):
    inp = make_fused(333, 256, 3001, dtype="bf16", seed=71, bias_std=0.1, ignore_frac=0.1, z_loss=1e-3)
    h, W, b, y = dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.bias, "bf16"), dev(inp.targets)
    kw = dict(z_loss=inp.z_loss, reduction="mean", return_lse=True, method=method)
    eager = lce.lce_fwd_bwd(h, W, b, y, **kw)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items() if isinstance(v, torch.Tensor) and k != "workspace"}
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
            assert torch.equal(out[k], v), (method, rep, k)
