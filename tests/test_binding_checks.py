"""The Python binding checks every tensor it passes to the C ABI (shape, dtype, device,
contiguity) and raises before loading or calling the library: the C side receives raw
pointers and sizes only, so a mismatched tensor would otherwise be read or written out of
bounds on the device.  CPU only: the library is replaced by a stub that fails if reached."""

import pytest
import torch

import linear_cross_entropy_vocab_amd as lce

bf = torch.bfloat16
i64 = torch.int64


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def _fail():
        raise AssertionError("the library was reached before the argument check")
    monkeypatch.setattr(lce, "load", _fail)


def _ok(BT=6, H=8, V=5, dtype=bf, bias=True):
    return (torch.zeros(BT, H, dtype=dtype), torch.zeros(V, H, dtype=dtype),
            torch.zeros(V, dtype=dtype) if bias else None, torch.zeros(BT, dtype=i64))


FUSED_BAD = [
    ("weight H", lambda h, W, b, y: (h, torch.zeros(5, 9, dtype=bf), b, y), {}, ValueError, "weight must be"),
    ("hidden 1-D", lambda h, W, b, y: (h.reshape(-1), W, b, y), {}, ValueError, "hidden must be 2-D"),
    ("bias length", lambda h, W, b, y: (h, W, torch.zeros(6, dtype=bf), y), {}, ValueError, "bias must be"),
    ("bias 2-D", lambda h, W, b, y: (h, W, torch.zeros(5, 1, dtype=bf), y), {}, ValueError, "bias must be"),
    ("targets length", lambda h, W, b, y: (h, W, b, torch.zeros(7, dtype=i64)), {}, ValueError, "targets must be"),
    ("targets 2-D", lambda h, W, b, y: (h, W, b, y.reshape(2, 3)), {}, ValueError, "targets must be"),
    ("targets dtype", lambda h, W, b, y: (h, W, b, y.to(torch.int32)), {}, TypeError, "int64"),
    ("mixed dtype", lambda h, W, b, y: (h, W.float(), b, y), {}, TypeError, "share a dtype"),
    ("out grad_input", None, dict(out=dict(grad_input=torch.zeros(6, 9, dtype=bf))), ValueError, "grad_input"),
    ("out grad_input dtype", None, dict(out=dict(grad_input=torch.zeros(6, 8))), TypeError, "grad_input"),
    ("out grad_weight", None, dict(out=dict(grad_weight=torch.zeros(4, 8, dtype=bf))), ValueError, "grad_weight"),
    ("out grad_weight fp32", None, dict(out=dict(grad_weight=torch.zeros(5, 8, dtype=bf)), grad_weight_fp32=True),
     TypeError, "grad_weight"),
    ("out grad_bias", None, dict(out=dict(grad_bias=torch.zeros(4, dtype=bf))), ValueError, "grad_bias"),
    ("out lse", None, dict(out=dict(lse=torch.zeros(5)), return_lse=True), ValueError, "lse"),
    ("out loss", None, dict(out=dict(loss=torch.zeros(2))), ValueError, "loss"),
    ("out n_valid", None, dict(out=dict(n_valid=torch.zeros(1))), TypeError, "n_valid"),
    ("workspace", None, dict(workspace=torch.zeros(16)), TypeError, "workspace"),
    ("filter counts", None, dict(filter_eps=1e-3, filter_counts=torch.zeros(3, dtype=i64)), TypeError, "filter_counts"),
    ("reduction", None, dict(reduction="none"), ValueError, "reduction"),
    ("grad_bias without bias", "nobias", dict(grad_bias=True), ValueError, "grad_bias needs a bias"),
]


@pytest.mark.parametrize("case", FUSED_BAD, ids=[c[0] for c in FUSED_BAD])
@pytest.mark.parametrize("method", ["fused", "chunked"])
def test_fused_arguments_checked_before_the_library(case, method):
    _, edit, kw, exc, msg = case
    args = _ok(bias=edit != "nobias")
    if callable(edit):
        args = edit(*args)
    if method == "chunked" and "filter_eps" in kw:
        pytest.skip("filtering is a fused-only option")
    with pytest.raises(exc, match=msg):
        lce.lce_fwd_bwd(*args, method=method, **kw)


def test_cpu_tensors_refused_after_shape_checks():
    with pytest.raises(ValueError, match="GPU"):
        lce.lce_fwd_bwd(*_ok())


ROWS_BAD = [
    ("fp32 inputs", lambda: _ok(dtype=torch.float32), {}, TypeError, "bf16"),
    ("targets length", lambda: _ok()[:3] + (torch.zeros(2, dtype=i64),), {}, ValueError, "targets must be"),
    ("weight H", lambda: (_ok()[0], torch.zeros(5, 7, dtype=bf)) + _ok()[2:], {}, ValueError, "weight must be"),
]


@pytest.mark.parametrize("case", ROWS_BAD, ids=[c[0] for c in ROWS_BAD])
def test_rows_arguments_checked_before_the_library(case):
    _, mk, kw, exc, msg = case
    with pytest.raises(exc, match=msg):
        lce.lce_rows_forward(*mk(), **kw)
    with pytest.raises(exc, match=msg):
        lce.lce_rows_backward(*mk(), **kw)


def test_rows_backward_upstream_length_checked():
    h, W, b, y = _ok()
    with pytest.raises(TypeError, match="BT elements"):
        lce.lce_rows_backward(h, W, b, y, grad_logprobs=torch.zeros(5))
    with pytest.raises(ValueError, match="grad_bias needs a bias"):
        lce.lce_rows_backward(h, W, None, y, grad_bias=True)


CE_BAD = [
    ("targets length", (torch.zeros(4, 5, dtype=bf), torch.zeros(3, dtype=i64)), {}, ValueError, "targets must be"),
    ("logits 1-D", (torch.zeros(20, dtype=bf), torch.zeros(4, dtype=i64)), {}, ValueError, "logits must be 2-D"),
    ("targets dtype", (torch.zeros(4, 5, dtype=bf), torch.zeros(4, dtype=torch.int32)), {}, TypeError, "int64"),
    ("logits dtype", (torch.zeros(4, 5, dtype=torch.float64), torch.zeros(4, dtype=i64)), {}, TypeError, "dtype"),
    ("out ce_sum", (torch.zeros(4, 5, dtype=bf), torch.zeros(4, dtype=i64)),
     dict(out=dict(ce_sum=torch.zeros(2))), ValueError, "ce_sum"),
    ("out n_valid", (torch.zeros(4, 5, dtype=bf), torch.zeros(4, dtype=i64)),
     dict(out=dict(n_valid=torch.zeros(1, dtype=torch.int32))), TypeError, "n_valid"),
]


@pytest.mark.parametrize("case", CE_BAD, ids=[c[0] for c in CE_BAD])
def test_ce_arguments_checked_before_the_library(case):
    _, args, kw, exc, msg = case
    with pytest.raises(exc, match=msg):
        lce.lce_ce_with_grad_inplace(*args, **kw)


def test_autograd_method_is_fused_unless_asked():
    import inspect
    assert inspect.signature(lce.linear_cross_entropy).parameters["method"].default == "fused"
    with pytest.raises(ValueError, match="method"):
        lce.linear_cross_entropy(*_ok()[:2], _ok()[3], method="auto")
