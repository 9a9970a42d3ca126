"""GPU parity of the HIP path (through the C ABI) against the float64 oracle on the same
seeded inputs, at sizes the oracle finishes in seconds: several tiles, ragged tails,
each kernel variant (single-chunk and column-chunked backward, bf16 and fp32 MFMA),
bias, z-loss, both reductions, and the edge cases (V = 1, all rows ignored, empty batch,
H not a multiple of the per-wave K quarter)."""

import numpy as np
import pytest
import torch

import oracle
import linear_cross_entropy_vocab_amd as lce
from workloads import make_config, make_fused, make_ce
from gpu_util import TOL, CE_TOL, dev, host64, rel, rel_fro

pytestmark = pytest.mark.gpu


def run_fused(inp, **kw):
    b = None if inp.bias is None else dev(inp.bias, inp.dtype)
    r = lce.lce_fwd_bwd(dev(inp.hidden, inp.dtype), dev(inp.weight, inp.dtype), b,
                        dev(inp.targets), z_loss=inp.z_loss, reduction=inp.reduction,
                        return_lse=True, **kw)
    torch.cuda.synchronize()
    return r


def check_fused(inp, r, ref, lse_tol=None):
    tol = TOL[inp.dtype]
    assert int(r["n_valid"].item()) == ref["n_valid"]
    assert rel(r["loss"].item(), ref["loss"]) <= tol["loss"] or abs(ref["loss"]) < 1e-12 and \
        abs(r["loss"].item()) < 1e-6, (r["loss"].item(), ref["loss"])
    lse = host64(r["lse"])
    lse_tol = tol["lse"] if lse_tol is None else lse_tol
    assert np.max(np.abs(lse - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))) <= lse_tol
    for k in ("grad_input", "grad_weight", "grad_bias"):
        if ref.get(k) is None or r.get(k) is None:
            continue
        e = rel_fro(host64(r[k]), ref[k])
        assert e <= tol["grad"], (k, e)
    # rows of ignored tokens get an exactly zero grad_input
    if r["grad_input"] is not None:
        ign = inp.targets == -100
        if ign.any():
            assert np.all(host64(r["grad_input"])[ign] == 0.0)


CASES = [
    # (dtype, BT, H, V, bias_std, z_loss, reduction, ignore_frac, seed)
    ("bf16", 200, 128, 1000, None, 0.0, "mean", 0.2, 11),
    ("bf16", 333, 256, 3001, 0.1, 1e-3, "sum", 0.1, 12),
    ("bf16", 130, 1024, 700, None, 0.0, "mean", 0.0, 13),   # one-pass backward, one vocabulary block
    ("bf16", 97, 200, 513, 0.2, 1e-2, "mean", 0.3, 14),
    ("bf16", 100, 1152, 600, 0.1, 1e-4, "mean", 0.1, 15),
    ("bf16", 65, 2304, 257, None, 0.0, "sum", 0.05, 16),
    ("f32", 77, 520, 300, 0.1, 1e-3, "mean", 0.1, 17),
    ("f32", 150, 64, 2000, None, 0.0, "sum", 0.2, 18),
    ("bf16", 1, 8, 5, None, 0.0, "mean", 0.0, 19),
    ("bf16", 64, 64, 1, 0.1, 0.0, "mean", 0.0, 20),
    # H >= 1024 with room in the budget: the backward on stored dlogits blocks.  One pass
    # (grad_input summed over the vocabulary blocks as hi + lo): 9, 4 and 3 blocks, the last
    # ragged; two passes: one vocabulary block, two token blocks
    ("bf16", 700, 1024, 20000, 0.1, 1e-4, "mean", 0.1, 25),
    ("bf16", 600, 1152, 9000, 0.1, 1e-4, "mean", 0.1, 21),
    ("bf16", 300, 2112, 5000, None, 0.0, "sum", 0.2, 22),
    ("bf16", 2000, 1280, 300, 0.2, 1e-3, "mean", 0.3, 23),
    ("bf16", 64, 1088, 70000, None, 0.0, "mean", 0.1, 24),   # budget too small for a block: column-chunked kernel
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}" for c in CASES])
def test_fused_small_vs_oracle(case):
    dt, BT, H, V, bstd, mu, red, ign, seed = case
    print(f"case {case}", flush=True)
    inp = make_fused(BT, H, V, dtype=dt, seed=seed, bias_std=bstd, ignore_frac=ign, z_loss=mu,
                     reduction=red)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=mu, reduction=red)
    r = run_fused(inp)
    check_fused(inp, r, ref)


def test_tiny_f32_config():
    inp = make_config("tiny_f32")
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=inp.z_loss,
                            reduction=inp.reduction)
    r = run_fused(inp)
    assert int(r["n_valid"].item()) == 230
    check_fused(inp, r, ref)


def test_all_ignored_and_empty():
    inp = make_fused(50, 64, 300, dtype="bf16", seed=3, bias_std=0.1)
    inp.targets[:] = -100
    r = run_fused(inp)
    assert r["loss"].item() == 0.0 and int(r["n_valid"].item()) == 0
    assert torch.count_nonzero(r["grad_input"]) == 0
    assert torch.count_nonzero(r["grad_weight"]) == 0
    assert torch.count_nonzero(r["grad_bias"]) == 0
    empty = make_fused(0, 64, 300, dtype="bf16", seed=3)
    r = run_fused(empty, out=dict(grad_weight=torch.full((300, 64), 7.0, dtype=torch.bfloat16,
                                                          device="cuda")))
    assert r["loss"].item() == 0.0 and int(r["n_valid"].item()) == 0
    assert torch.count_nonzero(r["grad_weight"]) == 0  # fully overwritten with zeros


MASK_CASES = [
    # (dtype, BT, H, V, masked vocabulary ranges, z_loss, method): whole 256-entry vocabulary
    # tiles of the forward (the first one, a middle one, the ragged last one) with bias -inf
    ("bf16", 300, 256, 1500, ((0, 256), (512, 768)), 1e-3, "fused"),
    ("f32", 150, 128, 1300, ((0, 256), (768, 1024), (1280, 1300)), 0.0, "fused"),
    ("bf16", 600, 1152, 9000, ((0, 256), (4096, 4352)), 1e-4, "fused"),   # one-pass backward (stored dlogits)
    ("bf16", 300, 256, 1500, ((0, 256), (1280, 1500)), 0.0, "chunked"),
    ("bf16", 2000, 1280, 300, ((0, 256),), 1e-3, "fused"),                  # two-pass backward
    ("bf16", 700, 1024, 20000, ((0, 256), (9984, 10240)), 1e-4, "filtered"),  # flagged tiles, eps 2^-20
    ("bf16", 700, 1024, 20000, ((0, 256), (9984, 10240)), 1e-4, "sorted"),    # and the vocabulary sorted
    ("bf16", 300, 256, 1500, ((0, 256), (512, 768)), 1e-3, "sorted"),          # sorted, pipelined backward
]


@pytest.mark.parametrize("case", MASK_CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[6]}" for c in MASK_CASES])
def test_minus_inf_bias_tiles_vs_oracle(case):
    """Vocabulary entries masked with a -inf bias contribute e^-inf = 0 ("Cut Cross Entropy
    visualized", "Forward Kernel": the LSE accumulation starts from -inf), also when a whole
    vocabulary tile of the forward is masked (its partial LSE is -inf and the merge skips it)."""
    dt, BT, H, V, ranges, mu, method = case
    print(f"masked-vocabulary case {case}", flush=True)
    inp = make_fused(BT, H, V, dtype=dt, seed=BT + V, bias_std=0.1, ignore_frac=0.1, z_loss=mu)
    masked = np.zeros(V, dtype=bool)
    for a, b in ranges:
        masked[a:b] = True
    keep = np.nonzero(~masked)[0]
    valid = inp.targets != -100
    inp.targets[:] = np.where(valid, keep[np.where(valid, inp.targets, 0) % keep.size], inp.targets)
    inp.bias[masked] = -np.inf
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=mu)
    assert np.isfinite(ref["loss"])
    kw = (dict(filter_eps=2.0 ** -20) if method == "filtered" else
          dict(filter_eps=2.0 ** -20, sort_vocab=True) if method == "sorted" else dict(method=method))
    r = run_fused(inp, **kw)
    lse_tol = 2.0 ** -8 if method == "chunked" else None  # (bf16 logits chunk)
    check_fused(inp, r, ref, lse_tol=lse_tol)
    for k in ("grad_weight", "grad_bias"):
        g = r[k][torch.from_numpy(masked).cuda()]
        assert int(torch.count_nonzero(g)) == 0, k


def _offset_copy(x: torch.Tensor, k: int) -> torch.Tensor:
    """x copied into a fresh buffer k elements past its (256-byte aligned) start."""
    big = torch.zeros(x.numel() + 16, dtype=x.dtype, device=x.device)
    v = big[k:k + x.numel()]
    v.copy_(x)
    return v


@pytest.mark.parametrize("shape", [(333, 256, 3001), (700, 1024, 20000), (130, 1152, 600)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bias_at_any_element_offset(shape):
    """A bf16 bias that starts 1, 3 or 7 elements past a 16-byte boundary (a view into a larger
    buffer) gives bit for bit the results of the same bias at an aligned address: the fused
    call, the per-row forward and backward, and the token-chunked composition (the forward
    kernels take the bias entries of a tile from the 16-byte boundary below the tile)."""
    BT, H, V = shape
    print(f"offset-bias case {shape}", flush=True)
    inp = make_fused(BT, H, V, dtype="bf16", seed=BT + H, bias_std=0.3, ignore_frac=0.1, z_loss=1e-4)
    h, w, y = dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.targets)
    b0 = dev(inp.bias, "bf16")
    assert b0.data_ptr() % 16 == 0
    ref = lce.lce_fwd_bwd(h, w, b0, y, z_loss=1e-4, return_lse=True)
    rf0 = lce.lce_rows_forward(h, w, b0, y, z_loss=1e-4)
    gl = torch.linspace(-1.0, 1.0, BT, device="cuda", dtype=torch.float32)
    rb0 = lce.lce_rows_backward(h, w, b0, y, grad_row_loss=gl, grad_entropy=0.5 * gl, z_loss=1e-4)
    ch0 = lce.lce_fwd_bwd(h, w, b0, y, z_loss=1e-4, method="chunked")
    torch.cuda.synchronize()
    oref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=1e-4)
    check_fused(inp, ref, oref)
    for k in (1, 3, 7):
        b = _offset_copy(b0, k)
        assert b.data_ptr() % 16 == 2 * k
        r = lce.lce_fwd_bwd(h, w, b, y, z_loss=1e-4, return_lse=True)
        rf = lce.lce_rows_forward(h, w, b, y, z_loss=1e-4)
        rb = lce.lce_rows_backward(h, w, b, y, grad_row_loss=gl, grad_entropy=0.5 * gl, z_loss=1e-4)
        ch = lce.lce_fwd_bwd(h, w, b, y, z_loss=1e-4, method="chunked")
        torch.cuda.synchronize()
        for name, x, x0 in (("fused", r, ref), ("rows forward", rf, rf0), ("rows backward", rb, rb0),
                            ("chunked", ch, ch0)):
            for key, t0 in x0.items():
                if isinstance(t0, torch.Tensor) and key != "workspace":  # (scratch contents)
                    assert torch.equal(x[key], t0), (name, key, k)


@pytest.mark.parametrize("shape", [(120, 256, 900), (600, 1152, 9000), (700, 1024, 20000)],
                         ids=["pipelined", "one-pass", "one-pass-1024"])
def test_grad_subsets(shape):
    BT, H, V = shape
    inp = make_fused(BT, H, V, dtype="bf16", seed=21, bias_std=0.1, ignore_frac=0.1)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets)
    r = run_fused(inp, grad_input=False, grad_weight=False, grad_bias=True)
    assert r["grad_input"] is None and r["grad_weight"] is None
    assert rel_fro(host64(r["grad_bias"]), ref["grad_bias"]) <= TOL["bf16"]["grad"]
    r = run_fused(inp, grad_weight=False, grad_bias=False)
    assert rel_fro(host64(r["grad_input"]), ref["grad_input"]) <= TOL["bf16"]["grad"]


def test_fused_grad_weight_fp32():
    inp = make_fused(333, 256, 3001, dtype="bf16", seed=12, bias_std=0.1, ignore_frac=0.1, z_loss=1e-3)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=1e-3)
    r32 = run_fused(inp, grad_weight_fp32=True)
    assert r32["grad_weight"].dtype == torch.float32
    check_fused(inp, r32, ref)
    r16 = run_fused(inp)
    # the bf16 output is the same fp32 accumulator rounded once more
    assert torch.equal(r32["grad_weight"].to(torch.bfloat16), r16["grad_weight"])
    for shape, seed in (((65, 2304, 257), 16),      # column-chunked kernel
                        ((300, 2112, 5000), 22)):   # two-pass backward
        big = make_fused(*shape, dtype="bf16", seed=seed, ignore_frac=0.05)
        a32 = run_fused(big, grad_weight_fp32=True)
        a16 = run_fused(big)
        assert torch.equal(a32["grad_weight"].to(torch.bfloat16), a16["grad_weight"]), shape


@pytest.mark.parametrize("shape", [(333, 256, 3001), (6000, 1024, 1500), (4096, 2304, 3000), (2000, 1280, 300)],
                         ids=["pipelined", "one-pass-1024-split", "one-pass", "two-pass"])
def test_grad_bias_closed_form_identical_rows(shape):
    """grad_b when every token has the same softmax (W = 0, so z_t = b for every t): by the
    dlogits formula ("Fused Linear Cross-Entropy: ...", "The identity that makes fused fwbw
    possible"; z-loss factor of "Greyhound — Cross-Entropy", "Kernel design") the sum over
    tokens is n_valid p (1 + 2 mu LSE(b)) - count_v, with p = softmax(b) and count_v the
    targets equal to v: grad_b = that / n_valid.  24 entries hold most of the mass and the
    targets are drawn from p, so count_v nearly cancels n_valid p_v: a sum of per-token
    bf16-rounded dlogits (each rounded the same way) is off by 1.5-3% here, the fp32 sums stay
    within bf16 output rounding.  grad_input = G . 0 is exactly zero."""
    BT, H, V = shape
    mu = 1e-3
    inp = make_fused(BT, H, V, dtype="bf16", seed=27, w_std=0.0, bias_std=0.5, ignore_frac=0.1, z_loss=mu)
    rng = np.random.default_rng(27)
    hot = rng.choice(V, size=24, replace=False)
    b = inp.bias.astype(np.float64) - 2.0
    b[hot] = 3.0 + 0.05 * np.arange(24)
    inp.bias = torch.from_numpy(b.astype(np.float32)).to(torch.bfloat16).float().numpy()
    b = inp.bias.astype(np.float64)
    L = float(np.log(np.sum(np.exp(b - b.max()))) + b.max())
    p = np.exp(b - L)
    y = inp.targets.copy()
    keep = y != -100
    y[keep] = rng.choice(V, size=int(keep.sum()), p=p / p.sum())
    inp.targets = y
    r = run_fused(inp)
    n = int(keep.sum())
    count = np.bincount(y[keep], minlength=V).astype(np.float64)
    want = (n * p * (1.0 + 2.0 * mu * L) - count) / n
    e = rel_fro(host64(r["grad_bias"]), want)
    assert e <= 2.0 ** -8, e
    assert int(torch.count_nonzero(r["grad_input"])) == 0


@pytest.mark.parametrize("shape", [(333, 256, 3001), (600, 1152, 9000), (700, 1024, 20000), (2000, 1280, 300)],
                         ids=["pipelined", "one-pass", "one-pass-1024", "two-pass"])
def test_deterministic_bits(shape):
    inp = make_fused(*shape, dtype="bf16", seed=12, bias_std=0.1, ignore_frac=0.1, z_loss=1e-3)
    a = run_fused(inp)
    b = run_fused(inp)
    for k in ("loss", "grad_input", "grad_weight", "grad_bias", "lse"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("ignore_index", [0, -1, 7])
@pytest.mark.parametrize("shape", [(200, 128, 1000), (700, 1024, 20000)], ids=lambda s: "x".join(map(str, s)))
def test_custom_ignore_index_vs_oracle(shape, ignore_index):
    """ignore_index other than -100, including a vocabulary id (its rows count for nothing, in
    the fused call, the token-chunked composition, the per-row outputs and the standalone CE)."""
    BT, H, V = shape
    print(f"ignore_index case {shape} {ignore_index}", flush=True)
    inp = make_fused(BT, H, V, dtype="bf16", seed=BT + ignore_index, bias_std=0.1, ignore_frac=0.0, z_loss=1e-4)
    rng = np.random.default_rng(BT)
    inp.targets[rng.random(BT) < 0.2] = ignore_index
    inp.targets[:3] = ignore_index
    h, W, b, y = dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.bias, "bf16"), dev(inp.targets)
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=1e-4, ignore_index=ignore_index)
    for method in ("fused", "chunked"):
        r = lce.lce_fwd_bwd(h, W, b, y, z_loss=1e-4, ignore_index=ignore_index, return_lse=True, method=method)
        torch.cuda.synchronize()
        lse_tol = 2.0 ** -8 if method == "chunked" else TOL["bf16"]["lse"]  # (chunked: bf16 logits chunk)
        lse = host64(r["lse"])
        assert np.max(np.abs(lse - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))) <= lse_tol, method
        assert int(r["n_valid"].item()) == ref["n_valid"], method
        assert rel(r["loss"].item(), ref["loss"]) <= TOL["bf16"]["loss"], method
        for k in ("grad_input", "grad_weight", "grad_bias"):
            assert rel_fro(host64(r[k]), ref[k]) <= TOL["bf16"]["grad"], (method, k)
        ign = inp.targets == ignore_index
        assert np.all(host64(r["grad_input"])[ign] == 0.0), method
    rr = oracle.lce_rows_oracle(inp.hidden, inp.weight, inp.bias, inp.targets, z_loss=1e-4,
                                ignore_index=ignore_index)
    f = lce.lce_rows_forward(h, W, b, y, z_loss=1e-4, ignore_index=ignore_index)
    torch.cuda.synchronize()
    assert int(f["n_valid"].item()) == rr["n_valid"]
    bound = TOL["bf16"]["lse"] * np.maximum(1.0, np.abs(rr["lse"]))
    for k in ("logprobs", "entropy"):
        assert np.all(np.abs(host64(f[k]) - rr[k]) <= bound), k
    ce = make_ce(64, 1000, dtype="bf16", seed=5, ignore_frac=0.0)
    ce.targets[::3] = ignore_index
    cref = oracle.ce_oracle(ce.logits, ce.targets, z_loss=1e-4, ignore_index=ignore_index)
    x = dev(ce.logits, "bf16")
    ce_sum, z_sum, nv = lce.lce_ce_with_grad_inplace(x, dev(ce.targets), z_loss=1e-4, ignore_index=ignore_index)
    torch.cuda.synchronize()
    assert int(nv.item()) == cref["n_valid"]
    assert rel(ce_sum.item(), cref["ce_sum"]) <= CE_TOL["bf16"]["sums"]
    assert rel_fro(host64(x), cref["dlogits"]) <= CE_TOL["bf16"]["dlogits"]


@pytest.mark.parametrize("shape", [(200, 128, 1000), (700, 1024, 20000), (300, 2112, 5000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_large_logits_vs_oracle(shape):
    """Logits in the hundreds (hidden scaled by 40, a bias of +-50): the exponentials stay
    relative to the running maximum everywhere, so the loss, LSE and gradients stay finite and
    match the oracle (fused call, per-row outputs)."""
    BT, H, V = shape
    print(f"large-logits case {shape}", flush=True)
    inp = make_fused(BT, H, V, dtype="bf16", seed=BT + 3, bias_std=0.1, ignore_frac=0.1, z_loss=1e-4)
    inp.hidden[:] = (inp.hidden * 40.0).astype(inp.hidden.dtype)
    inp.bias[:] = np.where(np.arange(V) % 2 == 0, 50.0, -50.0).astype(inp.bias.dtype)
    h, W, b, y = dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), dev(inp.bias, "bf16"), dev(inp.targets)
    hb, Wb, bb = host64(h), host64(W), host64(b)   # the bf16 values the kernels see
    ref = oracle.lce_oracle(hb, Wb, bb, inp.targets, z_loss=1e-4)
    assert np.all(np.isfinite(ref["lse"])) and np.max(np.abs(ref["lse"])) > 100.0
    r = lce.lce_fwd_bwd(h, W, b, y, z_loss=1e-4, return_lse=True)
    torch.cuda.synchronize()
    assert rel(r["loss"].item(), ref["loss"]) <= TOL["bf16"]["loss"]
    lse = host64(r["lse"])
    assert np.max(np.abs(lse - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))) <= TOL["bf16"]["lse"]
    for k in ("grad_input", "grad_weight", "grad_bias"):
        g = host64(r[k])
        assert np.all(np.isfinite(g)), k
        assert rel_fro(g, ref[k]) <= TOL["bf16"]["grad"], k
    rr = oracle.lce_rows_oracle(hb, Wb, bb, inp.targets, z_loss=1e-4)
    f = lce.lce_rows_forward(h, W, b, y, z_loss=1e-4)
    torch.cuda.synchronize()
    bound = TOL["bf16"]["lse"] * np.maximum(1.0, np.abs(rr["lse"]))
    for k in ("lse", "logprobs", "entropy"):
        assert np.all(np.abs(host64(f[k]) - rr[k]) <= bound), k


def test_concurrent_calls_on_two_streams():
    """Two calls in flight at once on two streams (separate workspaces; the library keeps no
    state between calls) give bit for bit the results of the same calls made one at a time:
    fused calls with the one-pass and the pipelined backward, and per-row outputs."""
    cases = [(700, 1024, 20000, 0.1), (600, 1152, 9000, None), (333, 256, 3001, 0.1)]
    inputs = []
    for BT, H, V, bstd in cases:
        inp = make_fused(BT, H, V, dtype="bf16", seed=BT + 11, bias_std=bstd, ignore_frac=0.1, z_loss=1e-4)
        b = None if inp.bias is None else dev(inp.bias, "bf16")
        inputs.append((dev(inp.hidden, "bf16"), dev(inp.weight, "bf16"), b, dev(inp.targets)))

    def run(i):
        h, W, b, y = inputs[i]
        r = lce.lce_fwd_bwd(h, W, b, y, z_loss=1e-4, return_lse=True)
        f = lce.lce_rows_forward(h, W, b, y, z_loss=1e-4)
        return {**{k: v for k, v in r.items() if isinstance(v, torch.Tensor) and k != "workspace"},
                **{"rows_" + k: v for k, v in f.items() if isinstance(v, torch.Tensor) and k != "workspace"}}

    alone = [run(i) for i in range(len(cases))]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    together = [None] * len(cases)
    for rep in range(3):
        for i, st in enumerate(streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                together[i] = run(i)
        torch.cuda.synchronize()
        for i in range(len(cases)):
            for k, v in alone[i].items():
                assert torch.equal(together[i][k], v), (rep, i, k)


def test_target_range_check():
    inp = make_fused(40, 64, 100, dtype="bf16", seed=5)
    inp.targets[7] = 100  # == V: out of range
    with pytest.raises(lce.LCEError) as e:
        run_fused(inp, check_targets=True)
    assert e.value.status == 7
    # without the check the row counts as ignored
    r = run_fused(inp)
    y = inp.targets.copy()
    y[7] = -100
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, y)
    check_fused(inp, r, ref)


def test_autograd_wrapper_scales_by_upstream_grad():
    inp = make_fused(64, 128, 500, dtype="f32", seed=8, bias_std=0.1, ignore_frac=0.1)
    h = dev(inp.hidden).requires_grad_(True)
    W = dev(inp.weight).requires_grad_(True)
    b = dev(inp.bias).requires_grad_(True)
    y = dev(inp.targets)
    loss = lce.linear_cross_entropy(h, W, y, b)
    (2.5 * loss).backward()
    ref = oracle.lce_oracle(inp.hidden, inp.weight, inp.bias, inp.targets)
    assert rel(loss.item(), ref["loss"]) < 1e-5
    assert rel_fro(host64(h.grad), 2.5 * ref["grad_input"]) < 1e-4
    assert rel_fro(host64(W.grad), 2.5 * ref["grad_weight"]) < 1e-4
    assert rel_fro(host64(b.grad), 2.5 * ref["grad_bias"]) < 1e-4


# ------------------------------------------------------------------ standalone CE

CE_CASES = [
    ("bf16", 64, 1000, 0.0, 0.1, 31),
    ("bf16", 64, 1000, 1e-3, 0.1, 32),
    ("bf16", 33, 1001, 1e-4, 0.2, 33),     # row bytes not a multiple of 16: streaming path
    ("f32", 16, 5000, 1e-3, 0.1, 34),
    ("f32", 6, 70000, 0.0, 0.0, 35),       # too long for the register cache: streaming path
    ("bf16", 8, 131072, 1e-4, 0.25, 36),   # largest register-cached bf16 row
    ("bf16", 5, 1, 0.0, 0.2, 37),
    ("bf16", 6, 20000, 1e-4, 0.2, 38),     # 3 vectors per thread, cached as 4: partial upper half
    ("f32", 5, 13000, 0.0, 0.0, 39),       # 4 per thread, the last one partial
    ("bf16", 4, 150000, 0.0, 0.25, 40),    # past the register cache, 16-byte rows: vector stream
    ("f16", 64, 1000, 1e-3, 0.1, 41),      # IEEE half logits
    ("f16", 6, 20000, 0.0, 0.2, 42),
    ("f16", 8, 131072, 1e-4, 0.25, 43),    # largest register-cached half row
    ("f16", 4, 150000, 1e-4, 0.0, 44),     # vector stream
    ("f16", 7, 1001, 0.0, 0.1, 45),        # scalar stream (row bytes not a multiple of 16)
]


@pytest.mark.parametrize("case", CE_CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}-mu{c[3]}" for c in CE_CASES])
def test_ce_small_vs_oracle(case):
    dt, B, V, mu, ign, seed = case
    print(f"ce case {case}", flush=True)
    inp = make_ce(B, V, dtype=dt, seed=seed, ignore_frac=ign)
    ref = oracle.ce_oracle(inp.logits, inp.targets, z_loss=mu)
    x = dev(inp.logits, dt)
    ptr = x.data_ptr()
    ce_sum, z_sum, nv = lce.lce_ce_with_grad_inplace(x, dev(inp.targets), z_loss=mu)
    torch.cuda.synchronize()
    assert x.data_ptr() == ptr
    tol = CE_TOL[dt]
    assert int(nv.item()) == ref["n_valid"]
    assert rel(ce_sum.item(), ref["ce_sum"]) <= tol["sums"]
    if mu == 0.0:
        assert z_sum.item() == 0.0
    else:
        assert rel(z_sum.item(), ref["z_sum"]) <= tol["sums"]
    d = host64(x)
    assert rel_fro(d, ref["dlogits"]) <= tol["dlogits"]
    ign_rows = inp.targets == -100
    assert np.all(d[ign_rows] == 0.0)


@pytest.mark.parametrize("case", [c for c in CE_CASES if c[2] > 1][:6] + [CE_CASES[9], CE_CASES[10]],
                         ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_ce_masked_entries_vs_oracle(case):
    """Logits of -inf (vocabulary entries masked out; never a counted target) add e^-inf = 0 to
    the LSE and get a dlogit of exactly 0, on each row-length path of the kernel."""
    dt, B, V, mu, ign, seed = case
    print(f"ce masked case {case}", flush=True)
    inp = make_ce(B, V, dtype=dt, seed=seed, ignore_frac=ign)
    rng = np.random.default_rng(seed)
    masked = rng.random(V) < 0.3
    masked[0] = True
    masked[V - 1] = True
    keep = np.nonzero(~masked)[0]
    valid = inp.targets != -100
    inp.targets[:] = np.where(valid, keep[np.where(valid, inp.targets, 0) % keep.size], inp.targets)
    logits = np.array(inp.logits, dtype=np.float32)
    logits[:, masked] = -np.inf
    ref = oracle.ce_oracle(logits, inp.targets, z_loss=mu)
    assert np.isfinite(ref["ce_sum"])
    x = dev(logits, dt)
    ce_sum, z_sum, nv = lce.lce_ce_with_grad_inplace(x, dev(inp.targets), z_loss=mu)
    torch.cuda.synchronize()
    tol = CE_TOL[dt]
    assert int(nv.item()) == ref["n_valid"]
    assert rel(ce_sum.item(), ref["ce_sum"]) <= tol["sums"]
    d = host64(x)
    assert np.all(np.isfinite(d))
    assert np.all(d[:, masked] == 0.0)
    assert rel_fro(d, ref["dlogits"]) <= tol["dlogits"]


def test_ce_empty_batch():
    x = torch.empty(0, 100, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(0, dtype=torch.int64, device="cuda")
    ce_sum, z_sum, nv = lce.lce_ce_with_grad_inplace(x, y, z_loss=1e-4)
    assert ce_sum.item() == 0.0 and z_sum.item() == 0.0 and int(nv.item()) == 0


def test_stream_bandwidth_helper_moves_the_bytes():
    """The bandwidth-measurement helper (read, write, copy) does what it says on a small buffer."""
    import ctypes
    lib = lce.load()
    src = torch.arange(4096, dtype=torch.int32, device="cuda")
    dst = torch.full_like(src, 7)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nb = src.numel() * 4
    assert lib.lce_stream_bandwidth(2, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nb, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert lib.lce_stream_bandwidth(1, None, ctypes.c_void_p(dst.data_ptr()), nb, st) == 0
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dst)) == 0
    assert lib.lce_stream_bandwidth(0, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(sink.data_ptr()), nb, st) == 0
    assert lib.lce_stream_bandwidth(3, None, ctypes.c_void_p(dst.data_ptr()), nb, st) == 6
    torch.cuda.synchronize()
