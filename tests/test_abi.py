"""The C ABI on the CPU: the library loads, exports every declared symbol, sizes its
workspace within the one-logits-chunk budget, and rejects bad arguments on the host
before any HIP call (fake but well-formed device pointers are passed, so reaching a
launch would be a bug these tests would expose)."""

import ctypes
import math
import os
import re

import pytest

from linear_cross_entropy_vocab_amd import _lib
from oracle import liger_chunk_plan
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lce.h")

BF16, F32 = _lib.DTYPE_BF16, _lib.DTYPE_F32
MEAN, SUM = _lib.REDUCTION_MEAN, _lib.REDUCTION_SUM


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_symbols_are_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:lce_status|size_t|const char\*)\s+(lce_\w+)\s*\(", text, re.M))
    assert declared == set(_lib.EXPORTS), declared ^ set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert b"gfx950" in lib.lce_version()
    for code in range(10):
        assert lib.lce_status_string(code)
    names = [lib.lce_stage_name(k).decode() for k in range(_lib.NUM_STAGES)]
    assert names == ["targets", "fwd_lse", "target_logit", "merge", "loss", "bwd_dinput", "bwd_dweight"]
    assert lib.lce_stage_name(_lib.NUM_STAGES) is None and lib.lce_stage_name(-1) is None


@pytest.mark.parametrize("name", ["tiny_f32", "gemma_like", "headline", "qwen_like"])
def test_workspace_within_one_logits_chunk(lib, name):
    c = CONFIGS[name]
    dt = BF16 if c.dtype == "bf16" else F32
    ws = lib.lce_fwd_bwd_workspace_bytes(c.BT, c.H, c.V, dt, 0)
    budget = liger_chunk_plan(c.BT, c.V, c.H)["chunk_bytes"]
    assert 0 < ws <= budget, (ws, budget)


@pytest.mark.parametrize("H", [1024, 1152, 2048, 2304, 4096])
def test_workspace_within_budget_over_shapes(lib, H):
    """The backward's block plans (one pass from H = 1024, two passes above; the filtered calls'
    one-pass plan with its tile flags) size their region
    to what the forward leaves of the one-chunk budget: over a grid of token and vocabulary
    counts the workspace never exceeds it (budget of "Fused Linear Cross-Entropy: The Math,
    the Memory Wall, and Two Ways Around It", "The chunk-size trick")."""
    for BT in (1, 64, 130, 700, 4096, 16384, 65535):
        for V in (1, 300, 3001, 20000, 151936, 256128):
            ws = lib.lce_fwd_bwd_workspace_bytes(BT, H, V, BF16, 0)
            budget = liger_chunk_plan(BT, V, H)["chunk_bytes"]
            base = 16 + 8 * BT + 16 * ((BT + 255) // 256) + 8 * BT + 4 * V + 4 * BT * ((V + 255) // 256)
            # (the forward's own pieces come first; the plans only add within the budget)
            assert ws <= max(budget, base + 64 * 256), (BT, H, V, ws, budget)


ERR_ARG = 6  # LCE_ERR_ARG


def test_filter_tile_shape(lib):
    """Filter tiles (host query): 256 x 64 where the bf16 backward takes the one-pass
    stored-operand plan (from H = 1024, the plan fitting the one-chunk workspace), 64 x 16 on
    the other kernels; invalid sizes, dtypes and NULL outputs are refused."""
    def shape(BT, H, V, dt):
        r, c = ctypes.c_int64(-1), ctypes.c_int64(-1)
        st = lib.lce_filter_tile_shape(BT, H, V, dt, ctypes.byref(r), ctypes.byref(c))
        return st, r.value, c.value
    for name in ("headline", "gemma_like", "qwen_like"):
        cf = CONFIGS[name]
        assert shape(cf.BT, cf.H, cf.V, BF16) == (_lib.LCE_OK, 256, 64), name
        assert shape(cf.BT, cf.H, cf.V, F32) == (_lib.LCE_OK, 64, 16), name
    assert shape(200, 256, 2048, BF16) == (_lib.LCE_OK, 64, 16)       # pipelined kernel
    assert shape(2000, 1280, 300, BF16) == (_lib.LCE_OK, 64, 16)      # no room for the one-pass plan
    assert shape(700, 1024, 20000, BF16) == (_lib.LCE_OK, 256, 64)
    assert shape(10, 12, 10, BF16)[0] == ERR_ARG
    assert shape(10, 64, 0, BF16)[0] == ERR_ARG
    assert shape(10, 64, 10, 7)[0] == ERR_ARG
    assert lib.lce_filter_tile_shape(10, 64, 10, BF16, None, None) == ERR_ARG


@pytest.mark.parametrize("name", ["gemma_like", "headline", "qwen_like"])
def test_rows_workspace_within_one_logits_chunk(lib, name):
    """The per-row entry points (forward, and the backward on the one-pass plan) keep their
    workspace within the same one-chunk budget as the fused call."""
    c = CONFIGS[name]
    lib.lce_rows_workspace_bytes.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_uint32]
    lib.lce_rows_workspace_bytes.restype = ctypes.c_size_t
    ws = lib.lce_rows_workspace_bytes(c.BT, c.H, c.V, BF16, 0)
    budget = liger_chunk_plan(c.BT, c.V, c.H)["chunk_bytes"]
    assert 0 < ws <= budget, (ws, budget)


def test_workspace_sizes(lib):
    assert lib.lce_fwd_bwd_workspace_bytes(-1, 64, 10, BF16, 0) == 0
    assert lib.lce_fwd_bwd_workspace_bytes(10, 12, 10, BF16, 0) == 0   # H % 8 != 0
    assert lib.lce_fwd_bwd_workspace_bytes(10, 64, 0, BF16, 0) == 0
    assert lib.lce_fwd_bwd_workspace_bytes(10, 64, 10, 7, 0) == 0
    assert lib.lce_fwd_bwd_workspace_bytes(0, 64, 10, BF16, 0) > 0
    B, V = 8192, 128256
    ws = lib.lce_ce_workspace_bytes(B, V, BF16)
    assert 0 < ws <= 16 * B
    assert lib.lce_ce_workspace_bytes(-1, V, BF16) == 0


# Fake device addresses: 16-byte aligned, never dereferenced on the host.
P = 0x7f0000000000
OK_WS = 1 << 40


def fused(lib, **kw):
    a = dict(hidden=P, W=P + 0x100000, bias=None, targets=P + 0x200000, BT=100, H=64, V=1000,
             dtype=BF16, ignore=-100, mu=0.0, red=MEAN, flags=0, loss=P + 0x300000,
             gi=P + 0x400000, gw=P + 0x500000, gb=None, nv=P + 0x600000, lse=None,
             ws=P + 0x700000, wsb=OK_WS, stream=None)
    a.update(kw)
    return lib.lce_fwd_bwd(a["hidden"], a["W"], a["bias"], a["targets"], a["BT"], a["H"], a["V"],
                           a["dtype"], a["ignore"], a["mu"], a["red"], a["flags"], a["loss"], a["gi"],
                           a["gw"], a["gb"], a["nv"], a["lse"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), 1), (dict(loss=None), 1), (dict(ws=None), 1), (dict(hidden=None), 1),
    (dict(targets=None), 1),
    (dict(BT=-1), 2), (dict(V=0), 2), (dict(H=0), 2), (dict(H=12), 2), (dict(H=4), 2),
    (dict(V=1 << 31), 2),
    (dict(dtype=2), 3), (dict(dtype=-1), 3),
    (dict(hidden=P + 8), 4), (dict(W=P + 4), 4), (dict(gi=P + 2), 4), (dict(ws=P + 8), 4),
    (dict(targets=P + 4), 4), (dict(loss=P + 2), 4),
    (dict(wsb=16), 5),
    (dict(red=2), 6), (dict(mu=-1.0), 6), (dict(mu=float("nan")), 6), (dict(mu=float("inf")), 6),
    (dict(gb=P + 0x800000), 6), (dict(flags=4), 6),
])
def test_fused_host_errors(lib, kw, status):
    assert fused(lib, **kw) == status


def fused_filtered(lib, eps, counts=None, **kw):
    a = dict(hidden=P, W=P + 0x100000, bias=None, targets=P + 0x200000, BT=100, H=64, V=1000,
             dtype=BF16, ignore=-100, mu=0.0, red=MEAN, flags=0, loss=P + 0x300000,
             gi=P + 0x400000, gw=P + 0x500000, gb=None, nv=P + 0x600000, lse=None,
             ws=P + 0x700000, wsb=OK_WS, stream=None)
    a.update(kw)
    return lib.lce_fwd_bwd_filtered(a["hidden"], a["W"], a["bias"], a["targets"], a["BT"], a["H"],
                                    a["V"], a["dtype"], a["ignore"], a["mu"], a["red"], a["flags"],
                                    a["loss"], a["gi"], a["gw"], a["gb"], a["nv"], a["lse"], a["ws"],
                                    a["wsb"], a["stream"], eps, counts)


@pytest.mark.parametrize("eps,counts,kw,status", [
    (-1e-3, None, {}, 6), (math.nan, None, {}, 6), (math.inf, None, {}, 6),
    (1e-3, P + 4, {}, 4),                 # misaligned count buffer
    (1e-3, None, dict(W=None), 1),        # the usual checks still apply
    (1e-3, None, dict(H=12), 2),
])
def test_filtered_host_errors(lib, eps, counts, kw, status):
    assert fused_filtered(lib, eps, counts, **kw) == status


def test_sort_vocab_flag(lib):
    # only the filtered entry takes it; its workspace adds the sorted copies of W, the bias and
    # the targets, the order and the sort keys; BT and V are capped at 2^24
    S = _lib.FLAG_SORT_VOCAB
    BT, H, V = 100, 64, 1000
    ws0 = lib.lce_fwd_bwd_workspace_bytes(BT, H, V, BF16, 0)
    ws1 = lib.lce_fwd_bwd_workspace_bytes(BT, H, V, BF16, S)
    assert ws1 >= ws0 + V * H * 2 + BT * 4 + V * 8
    assert lib.lce_fwd_bwd_workspace_bytes(BT, H, V, F32, S) >= ws1 + V * H * 2
    assert fused(lib, flags=S) == 6
    assert fused_filtered(lib, 1e-3, flags=S, wsb=ws0) == 5
    assert fused_filtered(lib, 1e-3, flags=S, BT=(1 << 24) + 1) == 2
    assert fused_filtered(lib, 1e-3, flags=S, V=(1 << 24) + 1) == 2
    assert fused_filtered(lib, 1e-3, flags=S | 8) == 6


def chunked(lib, **kw):
    a = dict(hidden=P, W=P + 0x100000, bias=None, targets=P + 0x200000, BT=100, H=64, V=1000,
             dtype=BF16, ignore=-100, mu=0.0, red=MEAN, flags=0, loss=P + 0x300000,
             gi=P + 0x400000, gw=P + 0x500000, gb=None, nv=P + 0x600000, lse=None,
             ws=P + 0x700000, wsb=OK_WS, stream=None)
    a.update(kw)
    return lib.lce_fwd_bwd_chunked(a["hidden"], a["W"], a["bias"], a["targets"], a["BT"], a["H"], a["V"],
                                   a["dtype"], a["ignore"], a["mu"], a["red"], a["flags"], a["loss"], a["gi"],
                                   a["gw"], a["gb"], a["nv"], a["lse"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), 1), (dict(loss=None), 1), (dict(ws=None), 1), (dict(targets=None), 1),
    (dict(BT=-1), 2), (dict(V=0), 2), (dict(H=12), 2), (dict(V=(1 << 22) + 1), 2),
    (dict(dtype=F32), 3), (dict(dtype=7), 3),
    (dict(hidden=P + 8), 4), (dict(gw=P + 4), 4), (dict(targets=P + 4), 4),
    (dict(wsb=16), 5),
    (dict(red=2), 6), (dict(mu=-1.0), 6), (dict(gb=P + 0x800000), 6), (dict(flags=4), 6),
])
def test_chunked_host_errors(lib, kw, status):
    assert chunked(lib, **kw) == status


def rows_fwd(lib, **kw):
    a = dict(hidden=P, W=P + 0x100000, bias=None, targets=P + 0x200000, BT=100, H=64, V=1000,
             dtype=BF16, ignore=-100, mu=0.0, flags=0, lse=P + 0x300000, lp=None, ent=None, rl=None,
             nv=None, ws=P + 0x700000, wsb=OK_WS, stream=None)
    a.update(kw)
    return lib.lce_rows_forward(a["hidden"], a["W"], a["bias"], a["targets"], a["BT"], a["H"], a["V"], a["dtype"],
                                a["ignore"], a["mu"], a["flags"], a["lse"], a["lp"], a["ent"], a["rl"], a["nv"],
                                a["ws"], a["wsb"], a["stream"])


def rows_bwd(lib, **kw):
    a = dict(hidden=P, W=P + 0x100000, bias=None, targets=P + 0x200000, BT=100, H=64, V=1000,
             dtype=BF16, ignore=-100, mu=0.0, flags=0, gl=P + 0x300000, gp=None, ge=None,
             lse=None, ent=None, gi=P + 0x400000, gw=P + 0x500000, gb=None, ws=P + 0x700000, wsb=OK_WS,
             stream=None)
    a.update(kw)
    return lib.lce_rows_backward(a["hidden"], a["W"], a["bias"], a["targets"], a["BT"], a["H"], a["V"],
                                 a["dtype"], a["ignore"], a["mu"], a["flags"], a["gl"], a["gp"], a["ge"], a["lse"],
                                 a["ent"], a["gi"], a["gw"], a["gb"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), 1), (dict(ws=None), 1), (dict(targets=None), 1), (dict(BT=-1), 2), (dict(H=12), 2),
    (dict(dtype=F32), 3), (dict(lse=P + 2), 4), (dict(ent=P + 0x800002), 4), (dict(wsb=16), 5),
    (dict(mu=float("nan")), 6), (dict(flags=2), 6),
])
def test_rows_forward_host_errors(lib, kw, status):
    assert rows_fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), 1), (dict(hidden=None), 1), (dict(V=0), 2), (dict(dtype=F32), 3), (dict(gl=P + 2), 4),
    (dict(gi=P + 8), 4), (dict(wsb=16), 5), (dict(gb=P + 0x800000), 6), (dict(flags=8), 6),
    (dict(lse=P + 0x600000), 6), (dict(ent=P + 0x600000), 6), (dict(lse=P + 0x600002, ent=P + 0x610000), 4),
])
def test_rows_backward_host_errors(lib, kw, status):
    assert rows_bwd(lib, **kw) == status


def test_chunked_workspace(lib):
    # one bf16 logits chunk (twice the rows of the pages' fp32 chunk), the grad_input partial
    # sums and the fp32 grad_W sum (left out when grad_W itself is fp32)
    BT, H, V = 65535, 1024, 176245
    ws = lib.lce_fwd_bwd_chunked_workspace_bytes(BT, H, V, BF16, 0)
    ws32 = lib.lce_fwd_bwd_chunked_workspace_bytes(BT, H, V, BF16, _lib.FLAG_GRAD_W_FP32)
    chunk = 1024 * ((V + 63) // 64 * 64) * 2
    assert ws - ws32 >= V * H * 4
    assert chunk < ws32 < chunk + 256 * 1024 * 1024
    assert lib.lce_fwd_bwd_chunked_workspace_bytes(BT, H, V, F32, 0) == 0
    assert lib.lce_fwd_bwd_chunked_workspace_bytes(0, H, V, BF16, 0) > 0


def test_fused_errors_before_device_work_with_empty_batch(lib):
    # BT = 0 may pass NULL hidden/targets; a too-small workspace is still rejected on the host
    assert fused(lib, BT=0, hidden=None, targets=None, wsb=0) == 5


def ce(lib, **kw):
    a = dict(logits=P, targets=P + 0x100000, B=10, V=1000, dtype=BF16, ignore=-100, mu=0.0,
             ce=P + 0x200000, z=P + 0x300000, nv=P + 0x400000, ws=P + 0x500000, wsb=OK_WS, stream=None)
    a.update(kw)
    return lib.lce_ce_with_grad_inplace(a["logits"], a["targets"], a["B"], a["V"], a["dtype"],
                                        a["ignore"], a["mu"], a["ce"], a["z"], a["nv"], a["ws"],
                                        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), 1), (dict(ce=None), 1), (dict(z=None), 1), (dict(ws=None), 1),
    (dict(B=-1), 2), (dict(V=0), 2), (dict(V=1 << 31), 2), (dict(dtype=5), 3),
    (dict(logits=P + 2), 4), (dict(ws=P + 4), 4), (dict(targets=P + 4), 4),
    (dict(wsb=8), 5), (dict(mu=-0.5), 6), (dict(mu=math.nan), 6),
])
def test_ce_host_errors(lib, kw, status):
    assert ce(lib, **kw) == status


def test_status_strings_are_distinct(lib):
    s = {lib.lce_status_string(k) for k in range(10)}
    assert len(s) == 10


def test_python_binding_refuses_cpu_tensors():
    import torch
    import linear_cross_entropy_vocab_amd as lce
    h = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        lce.lce_fwd_bwd(h, torch.zeros(5, 8), None, torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError):
        lce.lce_ce_with_grad_inplace(torch.zeros(4, 5), torch.zeros(4, dtype=torch.int64))


def test_oracle_not_imported_by_product_package():
    pkg = os.path.join(ROOT, "linear_cross_entropy_vocab_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


def test_noalloc_ce_host_errors(lib):
    """The no-allocation cross-entropy checks its arguments on the host, before it looks up
    its scratch or touches the device: rows beyond the scratch, bad shapes, dtypes, pointers."""
    p = ctypes.c_void_p(1 << 20)  # well-formed fake device pointers: never dereferenced here
    f = lib.lce_ce_with_grad_inplace_noalloc
    nmax = _lib.NOALLOC_MAX_ROWS
    assert f(p, p, nmax + 1, 10, BF16, -100, 0.0, p, p, p, None) == 9      # LCE_ERR_SCRATCH_LIMIT
    assert f(p, p, -1, 10, BF16, -100, 0.0, p, p, p, None) == 2            # shape
    assert f(p, p, 4, 0, BF16, -100, 0.0, p, p, p, None) == 2
    assert f(p, p, 4, 10, 7, -100, 0.0, p, p, p, None) == 3                # dtype
    assert f(p, p, 4, 10, BF16, -100, 0.0, None, p, p, None) == 1          # NULL output
    assert f(p, p, 4, 10, BF16, -100, -1.0, p, p, p, None) == 6            # z-loss < 0
    assert f(ctypes.c_void_p((1 << 20) + 2), p, 4, 10, BF16, -100, 0.0, p, p, p, None) == 4  # alignment
    assert b"scratch" in lib.lce_status_string(9)
