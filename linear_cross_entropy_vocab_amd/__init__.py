"""Fused linear cross-entropy for MI355X (gfx950): Python binding of liblce.so.

Every step of the computation runs in the HIP kernels behind the C ABI
(include/lce.h); this module only marshals torch tensors (device memory and the
current stream) into that ABI.  There is no CPU or PyTorch fallback: if the
library is missing or the tensors are not on a GPU, the calls raise.

  lce_fwd_bwd(hidden, weight, bias, targets, ...)   -> dict(loss, grad_input, grad_weight, grad_bias, n_valid, lse)
  lce_ce_with_grad_inplace(logits, targets, ...)    -> (ce_sum, z_sum, n_valid); logits become dlogits
  linear_cross_entropy(hidden, weight, targets, bias=None, ...)  -> loss with autograd
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import LCEError, load  # noqa: F401

__all__ = ["lce_fwd_bwd", "lce_ce_with_grad_inplace", "linear_cross_entropy", "fwd_bwd_workspace_bytes",
           "ce_workspace_bytes", "stage_names", "version", "LCEError", "load"]

_DTYPES = {torch.bfloat16: _lib.DTYPE_BF16, torch.float32: _lib.DTYPE_F32, torch.float16: _lib.DTYPE_F16}
_REDUCTIONS = {"mean": _lib.REDUCTION_MEAN, "sum": _lib.REDUCTION_SUM}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")
    return _DTYPES[t.dtype]


def _need_gpu(*ts):
    """Every tensor on one GPU and contiguous (the C ABI takes raw device pointers)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU (no CPU path exists)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"all tensors must be on one device ({dev} and {t.device} given)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _tensor(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, not {type(t).__name__}")
    return t


def _expect(t, name, shape, dtype):
    """A caller-supplied tensor (input or out=) must have exactly this shape and dtype: the
    library writes and reads through raw pointers, so a mismatch would reach out of bounds."""
    if t is None:
        return
    _tensor(t, name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _expect_scalar(t, name, dtype):
    if t is None:
        return
    _tensor(t, name)
    if t.numel() != 1:
        raise ValueError(f"{name} must hold exactly one element, not {t.numel()}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _expect_workspace(ws):
    if ws is None:
        return
    _tensor(ws, "workspace")
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")


def _check_problem(hidden, weight, bias, targets):
    """[BT, H] hidden, [V, H] weight, [V] bias (or None) of one dtype, [BT] int64 targets."""
    _tensor(hidden, "hidden")
    _tensor(weight, "weight")
    _tensor(targets, "targets")
    if hidden.dim() != 2:
        raise ValueError(f"hidden must be 2-D [BT, H], not of shape {tuple(hidden.shape)}")
    BT, H = hidden.shape
    if weight.dim() != 2 or weight.shape[1] != H:
        raise ValueError(f"weight must be [V, {H}], not of shape {tuple(weight.shape)}")
    V = weight.shape[0]
    if bias is not None:
        _tensor(bias, "bias")
        if tuple(bias.shape) != (V,):
            raise ValueError(f"bias must be [{V}], not of shape {tuple(bias.shape)}")
    if tuple(targets.shape) != (BT,):
        raise ValueError(f"targets must be [{BT}], not of shape {tuple(targets.shape)}")
    if targets.dtype != torch.int64:
        raise TypeError("targets must be int64")
    if weight.dtype != hidden.dtype or (bias is not None and bias.dtype != hidden.dtype):
        raise TypeError("hidden, weight and bias must share a dtype")
    return BT, H, V


def version() -> str:
    return load().lce_version().decode()


def stage_names():
    lib = load()
    return [lib.lce_stage_name(k).decode() for k in range(_lib.NUM_STAGES)]


def fwd_bwd_workspace_bytes(BT: int, H: int, V: int, dtype: torch.dtype) -> int:
    return int(load().lce_fwd_bwd_workspace_bytes(BT, H, V, _DTYPES[dtype], 0))


def filter_tile_shape(BT: int, H: int, V: int, dtype: torch.dtype):
    """(R, C): the gradient-filtering tiles of lce_fwd_bwd_filtered for these sizes, R tokens x C
    vocabulary entries for grad_input and R entries x C tokens for grad_W and grad_b."""
    r, c = ctypes.c_int64(0), ctypes.c_int64(0)
    _lib.check(load().lce_filter_tile_shape(BT, H, V, _DTYPES[dtype], ctypes.byref(r), ctypes.byref(c)),
               "lce_filter_tile_shape")
    return int(r.value), int(c.value)


def chunked_workspace_bytes(BT: int, H: int, V: int, dtype: torch.dtype, grad_weight_fp32: bool = False) -> int:
    flags = _lib.FLAG_GRAD_W_FP32 if grad_weight_fp32 else 0
    return int(load().lce_fwd_bwd_chunked_workspace_bytes(BT, H, V, _DTYPES[dtype], flags))


def ce_workspace_bytes(B: int, V: int, dtype: torch.dtype) -> int:
    return int(load().lce_ce_workspace_bytes(B, V, _DTYPES[dtype]))


def lce_fwd_bwd(hidden: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                targets: torch.Tensor, *, ignore_index: int = -100, z_loss: float = 0.0,
                reduction: str = "mean", grad_input: bool = True, grad_weight: bool = True,
                grad_bias: Optional[bool] = None, return_lse: bool = False,
                check_targets: bool = False, workspace: Optional[torch.Tensor] = None,
                out: Optional[dict] = None, events=None, filter_eps: float = 0.0,
                filter_counts: Optional[torch.Tensor] = None, method: str = "fused",
                grad_weight_fp32: bool = False, sort_vocab: bool = False) -> dict:
    """One call of lce_fwd_bwd: loss and the requested gradients (fully overwritten).

    `out` may hold preallocated tensors under the keys loss, grad_input, grad_weight,
    grad_bias, n_valid, lse; `events` = (start_list, stop_list) of hipEvent_t handles
    selects lce_fwd_bwd_profiled.  filter_eps > 0 selects lce_fwd_bwd_filtered (lossy
    gradient filtering); filter_counts (int64 [4] on the device) then receives the skipped
    and examined tile counts of the grad_input and grad_W passes.  method="chunked" selects
    lce_fwd_bwd_chunked (the token-chunked composition; bf16 only).  grad_weight_fp32 (bf16
    inputs) makes grad_weight a float32 tensor (in the chunked composition it then holds the
    sum over the chunks directly);
    method="auto" takes the fused path (the one within one logits chunk of extra memory; measured
    as fast as the composition at H = 4096 and faster at 2304).
    sort_vocab (with filter_eps > 0) orders the vocabulary by average logit before filtering.
    """
    if sort_vocab and not filter_eps > 0.0:
        raise ValueError("sort_vocab needs filter_eps > 0 (it only changes which tiles are skipped)")
    if method not in ("fused", "chunked", "auto"):
        raise ValueError(f"method must be 'fused', 'chunked' or 'auto', not {method!r}")
    if method == "auto":
        # the fused path's one-pass backward above H = 1024 measured 73.8 vs 74.1 ms (H = 4096)
        # and 35.5 vs 62.0 ms (H = 2304) against the composition, with a tenth of its memory;
        # at H = 1024 the composition is faster but needs 6.7x the memory
        method = "fused"
    chunked = method == "chunked"
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'sum', not {reduction!r}")
    BT, H, V = _check_problem(hidden, weight, bias, targets)
    if grad_weight_fp32 and hidden.dtype != torch.bfloat16:
        raise ValueError("grad_weight_fp32 applies to bf16 inputs")
    if chunked and (filter_eps > 0.0 or events is not None):
        raise ValueError("filter_eps and events are not supported with method='chunked'")
    dt = _dtype_code(hidden)
    if grad_bias is None:
        grad_bias = bias is not None
    if grad_bias and bias is None:
        raise ValueError("grad_bias needs a bias")
    o = dict(out or {})
    _expect_scalar(o.get("loss"), "out['loss']", torch.float32)
    _expect(o.get("grad_input") if grad_input else None, "out['grad_input']", (BT, H), hidden.dtype)
    _expect(o.get("grad_weight") if grad_weight else None, "out['grad_weight']", (V, H),
            torch.float32 if grad_weight_fp32 else weight.dtype)
    _expect(o.get("grad_bias") if grad_bias else None, "out['grad_bias']", (V,), None if bias is None else bias.dtype)
    _expect_scalar(o.get("n_valid"), "out['n_valid']", torch.int64)
    _expect(o.get("lse") if return_lse else None, "out['lse']", (BT,), torch.float32)
    _expect_workspace(workspace)
    if filter_counts is not None:
        _tensor(filter_counts, "filter_counts")
        if filter_counts.dtype != torch.int64 or filter_counts.numel() < 4:
            raise TypeError("filter_counts must be an int64 tensor of 4 elements")
    _need_gpu(hidden, weight, bias, targets, *(o.get(k) for k in ("loss", "grad_input", "grad_weight",
                                                                 "grad_bias", "n_valid", "lse")),
              workspace, filter_counts)
    lib = load()
    dev = hidden.device
    loss = o.get("loss")
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    gi = o.get("grad_input") if grad_input else None
    if grad_input and gi is None:
        gi = torch.empty_like(hidden)
    gw = o.get("grad_weight") if grad_weight else None
    if grad_weight and gw is None:
        gw = torch.empty_like(weight, dtype=torch.float32 if grad_weight_fp32 else weight.dtype)
    gb = o.get("grad_bias") if grad_bias else None
    if grad_bias and gb is None:
        gb = torch.empty_like(bias)
    nv = o.get("n_valid")
    if nv is None:
        nv = torch.empty((), dtype=torch.int64, device=dev)
    lse = o.get("lse") if return_lse else None
    if return_lse and lse is None:
        lse = torch.empty(BT, dtype=torch.float32, device=dev)
    flags = _lib.FLAG_CHECK_TARGETS if check_targets else 0
    if sort_vocab:
        flags |= _lib.FLAG_SORT_VOCAB
    if grad_weight_fp32:
        flags |= _lib.FLAG_GRAD_W_FP32
    ws_fn = lib.lce_fwd_bwd_chunked_workspace_bytes if chunked else lib.lce_fwd_bwd_workspace_bytes
    need = int(ws_fn(BT, H, V, dt, flags))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (_ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets), BT, H, V, dt, ignore_index,
            float(z_loss), _REDUCTIONS[reduction], flags, _ptr(loss), _ptr(gi), _ptr(gw), _ptr(gb),
            _ptr(nv), _ptr(lse), _ptr(workspace), workspace.numel(), stream)
    if chunked:
        st = lib.lce_fwd_bwd_chunked(*args)
    elif filter_eps > 0.0:
        if events is not None:
            raise ValueError("events are not supported with filter_eps")
        st = lib.lce_fwd_bwd_filtered(*args, float(filter_eps), _ptr(filter_counts))
    elif events is None:
        st = lib.lce_fwd_bwd(*args)
    else:
        arr_t = ctypes.c_void_p * _lib.NUM_STAGES
        ev0 = arr_t(*[ctypes.c_void_p(e) for e in events[0]])
        ev1 = arr_t(*[ctypes.c_void_p(e) for e in events[1]])
        st = lib.lce_fwd_bwd_profiled(*args, ev0, ev1)
    _lib.check(st, "lce_fwd_bwd_chunked" if chunked else "lce_fwd_bwd")
    return dict(loss=loss, grad_input=gi, grad_weight=gw, grad_bias=gb, n_valid=nv, lse=lse,
                workspace=workspace)


def rows_workspace_bytes(BT: int, H: int, V: int, dtype: torch.dtype, grad_weight_fp32: bool = False) -> int:
    flags = _lib.FLAG_GRAD_W_FP32 if grad_weight_fp32 else 0
    return int(load().lce_rows_workspace_bytes(BT, H, V, _DTYPES[dtype], flags))


def _rows_common(hidden, weight, bias, targets):
    BT, H, V = _check_problem(hidden, weight, bias, targets)
    if hidden.dtype != torch.bfloat16:
        raise TypeError("the per-row entry points take bf16 hidden, weight and bias")
    return BT, H, V


def lce_rows_forward(hidden: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                     targets: torch.Tensor, *, ignore_index: int = -100, z_loss: float = 0.0,
                     outputs=("lse", "logprobs", "entropy", "row_loss"), check_targets: bool = False,
                     workspace: Optional[torch.Tensor] = None) -> dict:
    """lce_rows_forward: per-row LSE, target log-probability, softmax entropy and row loss
    (reduction 'none'), each only if named in `outputs`; also n_valid."""
    BT, H, V = _rows_common(hidden, weight, bias, targets)
    _expect_workspace(workspace)
    _need_gpu(hidden, weight, bias, targets, workspace)
    lib = load()
    dev = hidden.device
    res = {k: (torch.empty(BT, dtype=torch.float32, device=dev) if k in outputs else None)
           for k in ("lse", "logprobs", "entropy", "row_loss")}
    nv = torch.empty((), dtype=torch.int64, device=dev)
    flags = _lib.FLAG_CHECK_TARGETS if check_targets else 0
    need = int(lib.lce_rows_workspace_bytes(BT, H, V, _lib.DTYPE_BF16, flags))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = lib.lce_rows_forward(_ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets), BT, H, V, _lib.DTYPE_BF16,
                              ignore_index, float(z_loss), flags, _ptr(res["lse"]), _ptr(res["logprobs"]),
                              _ptr(res["entropy"]), _ptr(res["row_loss"]), _ptr(nv), _ptr(workspace),
                              workspace.numel(), stream)
    _lib.check(st, "lce_rows_forward")
    res.update(n_valid=nv, workspace=workspace)
    return res


def lce_rows_backward(hidden: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                      targets: torch.Tensor, *, grad_row_loss: Optional[torch.Tensor] = None,
                      grad_logprobs: Optional[torch.Tensor] = None, grad_entropy: Optional[torch.Tensor] = None,
                      ignore_index: int = -100, z_loss: float = 0.0, grad_input: bool = True,
                      grad_weight: bool = True, grad_bias: Optional[bool] = None,
                      grad_weight_fp32: bool = False, check_targets: bool = False,
                      lse: Optional[torch.Tensor] = None, entropy: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> dict:
    """lce_rows_backward: gradients of sum_t gl_t row_loss_t + gp_t logprobs_t + ge_t entropy_t
    (upstream gradients float32 [BT] on the device, or None for zeros).  `lse` and `entropy`,
    both or neither, are lce_rows_forward's outputs for the same inputs: with them the backward
    does not recompute them (the dlogits come straight from the GEMM accumulator)."""
    BT, H, V = _rows_common(hidden, weight, bias, targets)
    if (lse is None) != (entropy is None):
        raise ValueError("pass both lse and entropy, or neither")
    ups = []
    for g in (grad_row_loss, grad_logprobs, grad_entropy, lse, entropy):
        if g is not None:
            _tensor(g, "per-row gradient")
            if g.dtype != torch.float32 or g.numel() != BT:
                raise TypeError("per-row gradients and saved outputs must be float32 with BT elements")
            g = g.contiguous()
        ups.append(g)
    if grad_bias is None:
        grad_bias = bias is not None
    if grad_bias and bias is None:
        raise ValueError("grad_bias needs a bias")
    _expect_workspace(workspace)
    _need_gpu(hidden, weight, bias, targets, *ups, workspace)
    lib = load()
    gi = torch.empty_like(hidden) if grad_input else None
    gw = torch.empty_like(weight, dtype=torch.float32 if grad_weight_fp32 else weight.dtype) if grad_weight else None
    gb = torch.empty_like(bias) if grad_bias else None
    flags = (_lib.FLAG_CHECK_TARGETS if check_targets else 0) | (_lib.FLAG_GRAD_W_FP32 if grad_weight_fp32 else 0)
    dev = hidden.device
    need = int(lib.lce_rows_workspace_bytes(BT, H, V, _lib.DTYPE_BF16, flags))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = lib.lce_rows_backward(_ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets), BT, H, V, _lib.DTYPE_BF16,
                               ignore_index, float(z_loss), flags, _ptr(ups[0]), _ptr(ups[1]), _ptr(ups[2]),
                               _ptr(ups[3]), _ptr(ups[4]), _ptr(gi), _ptr(gw), _ptr(gb), _ptr(workspace), workspace.numel(), stream)
    _lib.check(st, "lce_rows_backward")
    return dict(grad_input=gi, grad_weight=gw, grad_bias=gb, workspace=workspace)


class _LinearRows(torch.autograd.Function):
    """(logprobs, entropy, row_loss) per row; the backward recomputes the logits block by
    block, forming the dlogits from the saved LSE and entropy (within the same one-chunk
    workspace as the forward)."""

    @staticmethod
    def forward(ctx, hidden, weight, bias, targets, ignore_index, z_loss):
        h, W = hidden.contiguous(), weight.contiguous()
        b = None if bias is None else bias.contiguous()
        y = targets.contiguous()
        r = lce_rows_forward(h, W, b, y, ignore_index=ignore_index, z_loss=z_loss,
                             outputs=("lse", "logprobs", "entropy", "row_loss"))
        ent = r["entropy"]
        ctx.save_for_backward(h, W, b, y, r["lse"], ent.clone())
        ctx.opts = (ignore_index, z_loss)
        return r["logprobs"], r["entropy"], r["row_loss"]

    @staticmethod
    def backward(ctx, g_lp, g_ent, g_rl):
        h, W, b, y, lse, ent = ctx.saved_tensors
        ignore_index, z_loss = ctx.opts

        def f32(g):
            return None if g is None else g.to(torch.float32).contiguous()

        r = lce_rows_backward(h, W, b, y, grad_row_loss=f32(g_rl), grad_logprobs=f32(g_lp),
                              grad_entropy=f32(g_ent), ignore_index=ignore_index, z_loss=z_loss,
                              lse=lse, entropy=ent,
                              grad_input=ctx.needs_input_grad[0], grad_weight=ctx.needs_input_grad[1],
                              grad_bias=b is not None and ctx.needs_input_grad[2])
        return r["grad_input"], r["grad_weight"], r["grad_bias"], None, None, None


def linear_logprobs_entropy(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                            bias: Optional[torch.Tensor] = None, *, ignore_index: int = -100,
                            z_loss: float = 0.0):
    """Differentiable per-row (logprobs, entropy, row_loss) of hidden @ weight.T + bias (bf16):
    the target log-probability, the softmax entropy, and the unreduced loss (reduction 'none')."""
    return _LinearRows.apply(hidden, weight, bias, targets, ignore_index, z_loss)


def lce_ce_with_grad_inplace(logits: torch.Tensor, targets: torch.Tensor, *, ignore_index: int = -100,
                             z_loss: float = 0.0, workspace: Optional[torch.Tensor] = None,
                             out: Optional[dict] = None):
    """Cross-entropy on existing logits; logits are overwritten with dlogits.

    Returns device tensors (ce_sum, z_sum, n_valid); the mean loss is
    ce_sum / n_valid.clamp(min=1).
    """
    _tensor(logits, "logits")
    _tensor(targets, "targets")
    if logits.dim() != 2:
        raise ValueError(f"logits must be 2-D [B, V], not of shape {tuple(logits.shape)}")
    B, V = logits.shape
    if tuple(targets.shape) != (B,):
        raise ValueError(f"targets must be [{B}], not of shape {tuple(targets.shape)}")
    dt = _dtype_code(logits)
    if targets.dtype != torch.int64:
        raise TypeError("targets must be int64")
    o = dict(out or {})
    _expect_scalar(o.get("ce_sum"), "out['ce_sum']", torch.float32)
    _expect_scalar(o.get("z_sum"), "out['z_sum']", torch.float32)
    _expect_scalar(o.get("n_valid"), "out['n_valid']", torch.int64)
    _expect_workspace(workspace)
    _need_gpu(logits, targets, o.get("ce_sum"), o.get("z_sum"), o.get("n_valid"), workspace)
    lib = load()
    dev = logits.device
    ce = o.get("ce_sum")
    if ce is None:
        ce = torch.empty((), dtype=torch.float32, device=dev)
    zs = o.get("z_sum")
    if zs is None:
        zs = torch.empty((), dtype=torch.float32, device=dev)
    nv = o.get("n_valid")
    if nv is None:
        nv = torch.empty((), dtype=torch.int64, device=dev)
    need = int(lib.lce_ce_workspace_bytes(B, V, dt))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = lib.lce_ce_with_grad_inplace(_ptr(logits), _ptr(targets), B, V, dt, ignore_index, float(z_loss),
                                      _ptr(ce), _ptr(zs), _ptr(nv), _ptr(workspace), workspace.numel(),
                                      stream)
    _lib.check(st, "lce_ce_with_grad_inplace")
    return ce, zs, nv


def lce_ce_with_grad_inplace_noalloc(logits: torch.Tensor, targets: torch.Tensor, *, ignore_index: int = -100,
                                     z_loss: float = 0.0, out: Optional[dict] = None):
    """lce_ce_with_grad_inplace_noalloc: the standalone cross-entropy without a workspace (the
    library's fixed per-GPU scratch, at most NOALLOC_MAX_ROWS rows).  The C call allocates
    nothing; with `out` holding ce_sum, z_sum and n_valid, neither does this binding."""
    _tensor(logits, "logits")
    _tensor(targets, "targets")
    if logits.dim() != 2:
        raise ValueError(f"logits must be 2-D [B, V], not of shape {tuple(logits.shape)}")
    B, V = logits.shape
    if tuple(targets.shape) != (B,):
        raise ValueError(f"targets must be [{B}], not of shape {tuple(targets.shape)}")
    dt = _dtype_code(logits)
    if targets.dtype != torch.int64:
        raise TypeError("targets must be int64")
    o = dict(out or {})
    _expect_scalar(o.get("ce_sum"), "out['ce_sum']", torch.float32)
    _expect_scalar(o.get("z_sum"), "out['z_sum']", torch.float32)
    _expect_scalar(o.get("n_valid"), "out['n_valid']", torch.int64)
    _need_gpu(logits, targets, o.get("ce_sum"), o.get("z_sum"), o.get("n_valid"))
    lib = load()
    dev = logits.device
    ce = o.get("ce_sum")
    if ce is None:
        ce = torch.empty((), dtype=torch.float32, device=dev)
    zs = o.get("z_sum")
    if zs is None:
        zs = torch.empty((), dtype=torch.float32, device=dev)
    nv = o.get("n_valid")
    if nv is None:
        nv = torch.empty((), dtype=torch.int64, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = lib.lce_ce_with_grad_inplace_noalloc(_ptr(logits), _ptr(targets), B, V, dt, ignore_index, float(z_loss),
                                              _ptr(ce), _ptr(zs), _ptr(nv), stream)
    _lib.check(st, "lce_ce_with_grad_inplace_noalloc")
    return ce, zs, nv


NOALLOC_MAX_ROWS = _lib.NOALLOC_MAX_ROWS


class _LinearCrossEntropy(torch.autograd.Function):
    """Loss with gradients computed in the same fused call (the backward only rescales).

    The gradients are those of the loss itself (upstream gradient 1), rounded once to the
    input dtype by the library.  The backward multiplies them in place by the upstream
    gradient g (each product formed in fp32, then rounded to the input dtype): exact for g = 1
    (the usual case of a loss) and for powers of two; otherwise bf16 outputs carry a second
    rounding (relative error up to 2^-8 more per element).  In place, so that the backward
    allocates nothing beyond the gradients themselves; a second backward through the same
    graph therefore raises (the saved gradients have been modified)."""

    @staticmethod
    def forward(ctx, hidden, weight, bias, targets, ignore_index, z_loss, reduction, method):
        r = lce_fwd_bwd(hidden.contiguous(), weight.contiguous(),
                        None if bias is None else bias.contiguous(), targets.contiguous(),
                        ignore_index=ignore_index, z_loss=z_loss, reduction=reduction, method=method,
                        grad_input=ctx.needs_input_grad[0], grad_weight=ctx.needs_input_grad[1],
                        grad_bias=bias is not None and ctx.needs_input_grad[2])
        ctx.save_for_backward(r["grad_input"], r["grad_weight"], r["grad_bias"])
        return r["loss"]

    @staticmethod
    def backward(ctx, g):
        gi, gw, gb = ctx.saved_tensors
        scale = None if g is None else g.to(torch.float32)

        def mul(t):
            if t is None or scale is None:
                return t
            return t.mul_(scale)

        return mul(gi), mul(gw), mul(gb), None, None, None, None, None


def linear_cross_entropy(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, *, ignore_index: int = -100,
                         z_loss: float = 0.0, reduction: str = "mean", method: str = "fused") -> torch.Tensor:
    """loss = reduction over rows of CE(hidden @ weight.T + bias, targets) (+ z-loss), differentiable.

    method="fused" (default) keeps the extra device memory within one logits chunk (the
    workspace of lce_fwd_bwd_workspace_bytes); method="chunked" opts into the token-chunked
    composition, which is faster at H = 4096 but needs several times that memory."""
    if method not in ("fused", "chunked"):
        raise ValueError(f"method must be 'fused' or 'chunked', not {method!r}")
    return _LinearCrossEntropy.apply(hidden, weight, bias, targets, ignore_index, z_loss, reduction, method)
