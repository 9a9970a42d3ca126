"""Benchmark: fused linear cross-entropy forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-ce]
                    [--no-filter] [--filter-eps E] [--copy-calibration]

One step = one lce_fwd_bwd call (loss, grad_input, grad_W) on the headline LM-head
workload BT=65535, H=1024, V=176245, bf16, mean reduction, no bias, 20% of the targets
ignored; inputs are seeded synthetic data already resident in HBM.  Prints ONE JSON line:
whole-job tokens/s, the dominant kernel's roofline position (per-kernel HIP events
recorded by the library on the launch stream during the timed steps; algorithmic flops
2 BT V H per GEMM of the method, and beside them the executed flops with the logits
recomputed in each gradient kernel), the same fused step on the Gemma-like and Qwen-like
workloads (under "configs"), the float64 CPU
oracle timed on a bounded sample of the same workload, and the standalone
cross-entropy kernel's HBM throughput on [8192, 128256] bf16 logits, and (under
"filtered") the lossy gradient-filtering mode on the same workload: its step time, skipped
tile fractions and distance from the exact gradients.  Under "vendor_gemm_reference" (per
workload) the vendor GEMM library's rate on the step's three contractions with the logits
materialised: a measured reference for these shapes on this device, not a path of the
library.

The `traffic` fields are HBM bytes per launch from FETCH_SIZE / WRITE_SIZE counter runs of
this script (profiles/hbm_traffic.json, scaled by the same counters' reading for a plain
copy of known size, which --copy-calibration adds); they are null when the kernel's
sources have changed since those counters were taken.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused LCE fwd+bwd tokens/s & MFMA util (BT=65535,H=1024,V=176245 bf16)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
COPY_CAL_BYTES = 1 << 30    # size of the calibration copy (--copy-calibration)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_busy.json")
FILTER_EPS = 2.0 ** -12     # gradient-filtering threshold of the lossy leg (a bf16-scale floor)


def _hip():
    lib = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def _event(hip):
    e = ctypes.c_void_p()
    if hip.hipEventCreate(ctypes.byref(e)) != 0:
        raise RuntimeError("hipEventCreate failed")
    return e.value


def _elapsed(hip, a, b):
    ms = ctypes.c_float()
    if hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
        return float("nan")
    return ms.value


def measure_extra_hbm(lce, torch, h, W, y, kw, ws_bytes) -> dict:
    """Peak device memory one fused call adds beyond its inputs and preallocated outputs: the
    torch allocator's peak delta around a call whose workspace the binding allocates (so it
    is counted), and the device's free memory before and after a call with every buffer
    preallocated (the library itself must not allocate)."""
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    lce.lce_fwd_bwd(h, W, None, y, **kw)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=h.device)
    kw2 = dict(kw, workspace=ws)
    lce.lce_fwd_bwd(h, W, None, y, **kw2)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    lce.lce_fwd_bwd(h, W, None, y, **kw2)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    del ws
    return {"torch_peak_delta_bytes": int(peak), "device_free_delta_bytes": int(free0 - free1),
            "workspace_bytes": int(ws_bytes)}


def _sha(path: str) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _profile_value(path: str, kernel: str, key: str):
    """A per-kernel figure from a committed counter summary, or None when the summary is
    missing or the kernel's sources changed since the counters were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    for rel, sha in rec["sources"].items():
        fp = os.path.join(ROOT, rel)
        if not os.path.exists(fp) or _sha(fp) != sha:
            return None
    return rec[key]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the
    summary is missing or the kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    for rel, sha in rec["sources"].items():
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path) or _sha(path) != sha:
            return None
    return rec["hbm_bytes_per_launch"]


def bench_filtered(lce, torch, h, W, y, kw, exact, eps, steps, BT, sort_vocab=False) -> dict:
    """The lossy gradient-filtering mode on the same workload: time per step, the fraction
    of skipped tiles in each gradient pass, and how far its gradients are from the exact
    ones (relative Frobenius norm of the difference)."""
    counts = torch.zeros(4, dtype=torch.int64, device="cuda")
    out = dict(loss=torch.empty_like(exact["loss"]), grad_input=torch.empty_like(exact["grad_input"]),
               grad_weight=torch.empty_like(exact["grad_weight"]), n_valid=torch.empty_like(exact["n_valid"]))
    fkw = dict(kw, out=out)
    bias = fkw.pop("bias", None)
    if bias is not None:
        out["grad_bias"] = torch.empty_like(bias)
    r = lce.lce_fwd_bwd(h, W, bias, y, filter_eps=eps, filter_counts=counts, sort_vocab=sort_vocab, **fkw)
    fkw["workspace"] = r["workspace"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        lce.lce_fwd_bwd(h, W, bias, y, filter_eps=eps, filter_counts=counts, sort_vocab=sort_vocab, **fkw)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    c = counts.cpu().tolist()

    def rdiff(a, b):
        a = a.float()
        b = b.float()
        return float((a - b).norm() / b.norm())

    return {"filter_eps": eps, "sort_vocab": sort_vocab, "ms_per_step": ms, "tokens_per_s": BT / (ms * 1e-3),
            "skip_fraction_grad_input": c[0] / max(c[1], 1), "skip_fraction_grad_weight": c[2] / max(c[3], 1),
            "grad_rel_diff_vs_exact": {"grad_input": rdiff(out["grad_input"], exact["grad_input"]),
                                        "grad_weight": rdiff(out["grad_weight"], exact["grad_weight"])},
            "loss_equal": bool(torch.equal(out["loss"], exact["loss"]))}


def bench_chunked(lce, torch, h, W, b, y, kw, exact, steps, BT) -> dict:
    """The token-chunked composition on the same workload: time per step, its extra device
    memory, and how far its results are from the fused path's (relative differences)."""
    ckw = {k: v for k, v in kw.items() if k not in ("workspace", "out")}
    r = lce.lce_fwd_bwd(h, W, b, y, method="chunked", **ckw)
    torch.cuda.synchronize()
    out = {k: r[k] for k in ("loss", "grad_input", "grad_weight", "grad_bias", "n_valid") if r[k] is not None}
    ws = r["workspace"]
    ws_bytes = ws.numel()
    t0 = time.perf_counter()
    for _ in range(steps):
        lce.lce_fwd_bwd(h, W, b, y, method="chunked", workspace=ws, out=out, **ckw)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps

    def rdiff(a, c):
        a = a.float()
        c = c.float()
        return float((a - c).norm() / c.norm())

    diffs = {k: rdiff(out[k], exact[k]) for k in ("grad_input", "grad_weight", "grad_bias")
             if out.get(k) is not None and exact.get(k) is not None}
    diffs["loss"] = abs(out["loss"].item() - exact["loss"].item()) / abs(exact["loss"].item())
    del out, ws, r
    # fp32 grad_W output (the chunked composition then sums into it directly), both methods
    fp32 = {}
    for method in ("fused", "chunked"):
        r = lce.lce_fwd_bwd(h, W, b, y, method=method, grad_weight_fp32=True, **ckw)
        torch.cuda.synchronize()
        o = {k: r[k] for k in ("loss", "grad_input", "grad_weight", "grad_bias", "n_valid") if r[k] is not None}
        t0 = time.perf_counter()
        for _ in range(steps):
            lce.lce_fwd_bwd(h, W, b, y, method=method, grad_weight_fp32=True, workspace=r["workspace"], out=o, **ckw)
        torch.cuda.synchronize()
        msf = (time.perf_counter() - t0) * 1e3 / steps
        fp32[method] = {"ms_per_step": msf, "workspace_bytes": int(r["workspace"].numel()),
                        "grad_weight_rel_diff_vs_bf16_fused": rdiff(o["grad_weight"], exact["grad_weight"])}
        del r, o
    return {"ms_per_step": ms, "tokens_per_s": BT / (ms * 1e-3), "workspace_bytes": int(ws_bytes),
            "rel_diff_vs_fused": diffs, "grad_weight_fp32": fp32}


def bench_rows(lce, torch, h, W, b, y, steps, BT) -> dict:
    """Per-row outputs for RL-style use on the same workload: the forward (LSE, target
    log-probability, entropy, row loss) and the backward of a per-row weighted sum of them,
    given the forward's LSE and entropy (and, for comparison, recomputing them)."""
    r = lce.lce_rows_forward(h, W, b, y)
    ws = r["workspace"]
    g = [torch.randn(BT, device="cuda", dtype=torch.float32) for _ in range(3)]
    lce.lce_rows_backward(h, W, b, y, grad_row_loss=g[0], grad_logprobs=g[1], grad_entropy=g[2],
                          lse=r["lse"], entropy=r["entropy"], workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        lce.lce_rows_forward(h, W, b, y, workspace=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        lce.lce_rows_backward(h, W, b, y, grad_row_loss=g[0], grad_logprobs=g[1], grad_entropy=g[2],
                              lse=r["lse"], entropy=r["entropy"], workspace=ws)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(steps):
        lce.lce_rows_backward(h, W, b, y, grad_row_loss=g[0], grad_logprobs=g[1], grad_entropy=g[2],
                              workspace=ws)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    fwd = (t1 - t0) * 1e3 / steps
    bwd = (t2 - t1) * 1e3 / steps
    return {"forward_ms": fwd, "backward_ms": bwd, "backward_recompute_stats_ms": (t3 - t2) * 1e3 / steps,
            "tokens_per_s": BT / ((fwd + bwd) * 1e-3),
            "workspace_bytes": int(ws.numel()),
            "mean_entropy": float(r["entropy"].mean().item())}


def one_pass_backward(stage_ms) -> bool:
    """The library's one-pass backward (bf16, H > 1024, when its planner prefers it) computes
    grad_input, grad_W and grad_b in the grad_input stage from one recompute of the dlogits,
    leaving the grad_W stage empty."""
    return stage_ms["bwd_dweight"] < 0.02 * stage_ms["bwd_dinput"]


def executed_flops(stage_ms, btvh) -> float:
    """Executed flops of a step: the forward GEMM and, per gradient stage, the recompute of the
    logits and the gradient GEMM (10 BT V H); one recompute in the one-pass backward (8)."""
    return (8 if one_pass_backward(stage_ms) else 10) * btvh


def _stage_roofline(stage_ms, btvh, dom=None):
    """Roofline position of the slowest stage: algorithmic flops (the method's 2 BT V H per
    GEMM: logits, grad_input, grad_W) and executed flops (with the logits recomputed inside
    each gradient stage) per launch over its mean event time, against dense bf16 peak.  In
    the one-pass backward the grad_input stage holds both gradient GEMMs and one recompute."""
    algo = {"fwd_lse": 2 * btvh, "bwd_dinput": 2 * btvh, "bwd_dweight": 2 * btvh}
    execd = {"fwd_lse": 2 * btvh, "bwd_dinput": 4 * btvh, "bwd_dweight": 4 * btvh}
    if one_pass_backward(stage_ms):
        algo["bwd_dinput"], execd["bwd_dinput"] = 4 * btvh, 6 * btvh
    if dom is None:
        dom = max(algo, key=lambda n: stage_ms[n])
    a = algo[dom] / (stage_ms[dom] * 1e-3) / 1e12
    e = execd[dom] / (stage_ms[dom] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": a, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": a / PEAK_BF16_TFLOPS, "kernel": dom, "algorithmic_flops_per_launch": algo[dom],
            "achieved_executed": e, "frac_executed": e / PEAK_BF16_TFLOPS,
            "executed_flops_per_launch": execd[dom]}
    if dom == "bwd_dinput" and one_pass_backward(stage_ms):
        # the stage is the whole backward: per vocabulary block one transposed-dlogits forward
        # launch and one grouped grad_W + grad_input GEMM launch (plus a partial-sum reduce)
        dom = "bwd_onepass"
        roof["kernel"] = dom
        roof["launch"] = "one backward stage (per vocabulary block: transposed dlogits, grouped grad_W + grad_input GEMM)"
    return dom, roof


def vendor_gemm_reference(torch, h, W, reps: int = 3) -> dict:
    """The vendor GEMM library (hipBLASLt, through torch.matmul) on the three contractions of
    one step with the logits materialised: z = h W^T [BT, V], grad_input = G W and
    grad_W = G^T h for a bf16 [BT, V] matrix G.  Plain GEMMs, no LSE epilogue, no recompute,
    BT*V*2 bytes of logits in HBM: a measured reference for what this device's MFMAs deliver
    on these shapes (the clock throttles under dense MFMA load), not a path of the library."""
    BT, H = h.shape
    V = W.shape[0]
    z = torch.empty((BT, V), dtype=h.dtype, device=h.device)
    gi = torch.empty_like(h)
    gw = torch.empty_like(W)
    flop = 2.0 * BT * V * H
    res = {"library": "hipBLASLt via torch.matmul", "logits_bytes": int(z.numel() * z.element_size())}
    for key, f in (("logits", lambda: torch.matmul(h, W.t(), out=z)),
                   ("grad_input", lambda: torch.matmul(z, W, out=gi)),
                   ("grad_weight", lambda: torch.matmul(z.t(), h, out=gw))):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[key] = {"ms": ms, "tflops": flop / (ms * 1e-3) / 1e12}
    res["three_gemms_ms"] = sum(res[k]["ms"] for k in ("logits", "grad_input", "grad_weight"))
    del z, gi, gw
    torch.cuda.empty_cache()
    return res


def bench_config(lce, torch, name, steps, warmup, log, vendor=True) -> dict:
    """The fused step (lce_fwd_bwd: loss and every gradient) on another named LM-head workload:
    wall time per step, per-stage event times, the slowest stage's roofline position, and the
    extra device memory of one call against the one-logits-chunk budget."""
    from oracle import liger_chunk_plan
    from workloads import CONFIGS, make_config
    c = CONFIGS[name]
    log(f"generating {name}")
    inp = make_config(name)
    dt = torch.bfloat16
    h = torch.from_numpy(inp.hidden).to(dt).cuda()
    W = torch.from_numpy(inp.weight).to(dt).cuda()
    b = None if inp.bias is None else torch.from_numpy(inp.bias).to(dt).cuda()
    y = torch.from_numpy(inp.targets).cuda()
    del inp
    kw = dict(reduction=c.reduction, z_loss=c.z_loss)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    r = lce.lce_fwd_bwd(h, W, b, y, **kw)
    torch.cuda.synchronize()
    out_bytes = sum(r[k].numel() * r[k].element_size() for k in ("loss", "grad_input", "grad_weight",
                                                                  "grad_bias", "n_valid") if r[k] is not None)
    peak_extra = torch.cuda.max_memory_allocated() - base - out_bytes
    ws = r["workspace"]
    out = {k: r[k] for k in ("loss", "grad_input", "grad_weight", "grad_bias", "n_valid") if r[k] is not None}
    for _ in range(warmup):
        lce.lce_fwd_bwd(h, W, b, y, out=out, workspace=ws, **kw)
    hip = _hip()
    n_st = len(lce.stage_names())
    evs = [([_event(hip) for _ in range(n_st)], [_event(hip) for _ in range(n_st)]) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        lce.lce_fwd_bwd(h, W, b, y, out=out, workspace=ws, events=evs[k], **kw)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    names = lce.stage_names()
    st = {n: float(np.mean([_elapsed(hip, e[0][i], e[1][i]) for e in evs])) for i, n in enumerate(names)}
    for e in evs:
        for x in e[0] + e[1]:
            hip.hipEventDestroy(ctypes.c_void_p(x))
    btvh = float(c.BT) * c.V * c.H
    _, roof = _stage_roofline(st, btvh)
    budget = liger_chunk_plan(c.BT, c.V, c.H)["chunk_bytes"]
    res = {"workload": f"{name}: BT={c.BT}, H={c.H}, V={c.V}, bf16, {c.reduction}"
                       + (", bias" if b is not None else "") + (f", z-loss {c.z_loss:g}" if c.z_loss else ""),
           "ms_per_step": ms, "tokens_per_s": c.BT / (ms * 1e-3),
           "tflops_useful": 6 * btvh / (ms * 1e-3) / 1e12,
           "tflops_executed": executed_flops(st, btvh) / (ms * 1e-3) / 1e12,
           "backward": "one pass" if one_pass_backward(st) else "two gradient stages",
           "useful_frac": 6 * btvh / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "stage_ms": st, "roofline": roof, "n_valid": int(out["n_valid"].item()),
           "loss": float(out["loss"].item()),
           "extra_hbm_bytes": int(ws.numel()), "extra_hbm_torch_peak_bytes": int(peak_extra),
           "extra_hbm_budget_bytes": int(budget)}
    del r, out, ws
    torch.cuda.empty_cache()
    if vendor:
        res["vendor_gemm_reference"] = vendor_gemm_reference(torch, h, W)
    del h, W, b, y
    torch.cuda.empty_cache()
    return res


def cpu_baseline(inp, n_tokens: int) -> dict:
    """The float64 oracle (as it stands) on the first n_tokens rows of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    h = inp.hidden[:n_tokens]
    y = inp.targets[:n_tokens]
    t = time.perf_counter()
    oracle.lce_oracle(h, inp.weight, inp.bias, y, z_loss=inp.z_loss, reduction=inp.reduction)
    dt = time.perf_counter() - t
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n_tokens} tokens of the workload, full V and H, loss + grad_input + "
                      f"grad_W in float64 ({dt:.1f} s)"}


def bench_ce(lce, torch, steps: int) -> dict:
    from workloads import CONFIGS, make_ce
    c = CONFIGS["ce_only"]
    inp = make_ce(c.B, c.V, dtype=c.dtype, seed=c.seed, logit_std=c.logit_std, ignore_frac=c.ignore_frac)
    x = torch.from_numpy(inp.logits).to(torch.bfloat16).cuda()
    y = torch.from_numpy(inp.targets).cuda()
    del inp
    out = dict(ce_sum=torch.empty((), dtype=torch.float32, device="cuda"),
               z_sum=torch.empty((), dtype=torch.float32, device="cuda"),
               n_valid=torch.empty((), dtype=torch.int64, device="cuda"))
    ws = torch.empty(lce.ce_workspace_bytes(c.B, c.V, torch.bfloat16), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        lce.lce_ce_with_grad_inplace(x, y, workspace=ws, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        lce.lce_ce_with_grad_inplace(x, y, workspace=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    algo_bytes = 2 * c.B * c.V * 2 + 8 * c.B
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    # references: plain device streams of the same bytes show what rate this device sustains
    # (the library's own read-only, write-only and copy kernels, 16-byte accesses, and torch's
    # copy); the copy moves what the cross-entropy moves, one read and one write per element
    dst = torch.empty_like(x)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    nbytes = x.numel() * x.element_size()
    lib = lce.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def stream_ms(mode, src, dstp):
        for _ in range(2):
            assert lib.lce_stream_bandwidth(mode, src, dstp, nbytes, stream) == 0
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            lib.lce_stream_bandwidth(mode, src, dstp, nbytes, stream)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_read = stream_ms(0, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(sink.data_ptr()))
    ms_write = stream_ms(1, None, ctypes.c_void_p(dst.data_ptr()))
    ms_lcopy = stream_ms(2, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(dst.data_ptr()))
    dst.copy_(x)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        dst.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms_copy = e0.elapsed_time(e1) / steps
    copy_gbs = 2 * nbytes / (ms_copy * 1e-3) / 1e9
    lcopy_gbs = 2 * nbytes / (ms_lcopy * 1e-3) / 1e9
    stream_rates = {"bytes": nbytes, "read_GBs": nbytes / (ms_read * 1e-3) / 1e9,
                    "write_GBs": nbytes / (ms_write * 1e-3) / 1e9, "copy_GBs": lcopy_gbs,
                    "torch_copy_GBs": copy_gbs}
    del dst, sink
    # the other variants of the same workload: z-loss on, and fp16 / fp32 logits
    variants = []
    for dt, mu in (("bf16", 1e-4), ("f16", 0.0), ("f32", 0.0)):
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
        xv = x.to(tdt)
        wsv = torch.empty(lce.ce_workspace_bytes(c.B, c.V, tdt), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            lce.lce_ce_with_grad_inplace(xv, y, z_loss=mu, workspace=wsv, out=out)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            lce.lce_ce_with_grad_inplace(xv, y, z_loss=mu, workspace=wsv, out=out)
        e1.record()
        torch.cuda.synchronize()
        msv = e0.elapsed_time(e1) / steps
        bv = 2 * c.B * c.V * xv.element_size() + 8 * c.B
        variants.append({"dtype": dt, "z_loss": mu, "ms": msv, "GB/s": bv / (msv * 1e-3) / 1e9,
                         "frac": bv / (msv * 1e-3) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": bv})
        del xv, wsv
    return {"workload": f"standalone CE+dlogits in place, [{c.B}, {c.V}] bf16, z-loss 0",
            "ms": ms, "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic("ce_rows")},
            "algorithmic_bytes": algo_bytes,
            "device_stream": stream_rates,
            "frac_of_best_copy": gbs / max(lcopy_gbs, copy_gbs),
            "variants": variants}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ce", action="store_true")
    ap.add_argument("--no-filter", action="store_true", help="skip the gradient-filtering leg")
    ap.add_argument("--filter-zipf", action="store_true",
                    help="only measure gradient filtering on the Zipf-target workloads (Gemma-like, "
                         "Qwen-like) and print one JSON line per workload")
    ap.add_argument("--filter-eps", type=float, default=FILTER_EPS)
    ap.add_argument("--no-chunked", action="store_true", help="skip the token-chunked composition leg")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip the vendor GEMM reference (hipBLASLt on the step's three contractions)")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row outputs leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the fused step on the Gemma-like and Qwen-like workloads")
    ap.add_argument("--compare-methods", action="store_true",
                    help="only time the fused path and the token-chunked composition on the three "
                         "LM-head workloads and print one JSON line per workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference dispatch for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (asked for --gpus {args.gpus}); the fused op "
              f"has no multi-GPU path here", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_cross_entropy_vocab_amd as lce
    from workloads import CONFIGS, make_config

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.compare_methods:
        for name in ("gemma_like", "headline", "qwen_like"):
            c = CONFIGS[name]
            log(f"generating {name}")
            inp = make_config(name)
            dt = torch.bfloat16
            hh = torch.from_numpy(inp.hidden).to(dt).cuda()
            WW = torch.from_numpy(inp.weight).to(dt).cuda()
            bb = None if inp.bias is None else torch.from_numpy(inp.bias).to(dt).cuda()
            yy = torch.from_numpy(inp.targets).cuda()
            del inp
            kw2 = dict(reduction=c.reduction, z_loss=c.z_loss)
            ex = lce.lce_fwd_bwd(hh, WW, bb, yy, **kw2)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                ex = lce.lce_fwd_bwd(hh, WW, bb, yy, out=ex, workspace=ex["workspace"], **kw2)
            torch.cuda.synchronize()
            ms_f = (time.perf_counter() - t0) * 1e3 / args.steps
            log(f"{name}: fused {ms_f:.1f} ms")
            res_c = bench_chunked(lce, torch, hh, WW, bb, yy, kw2, ex, args.steps, c.BT)
            log(f"{name}: chunked {res_c['ms_per_step']:.1f} ms")
            print(json.dumps({"workload": f"{name}: BT={c.BT}, H={c.H}, V={c.V}",
                              "fused_ms_per_step": ms_f, "fused_workspace_bytes": int(ex["workspace"].numel()),
                              "chunked": res_c}), flush=True)
            del hh, WW, bb, yy, ex
            torch.cuda.empty_cache()
        return

    if args.filter_zipf:
        for name in ("gemma_like", "qwen_like"):
            c = CONFIGS[name]
            log(f"generating {name}")
            inp = make_config(name)
            dt = torch.bfloat16
            hh = torch.from_numpy(inp.hidden).to(dt).cuda()
            WW = torch.from_numpy(inp.weight).to(dt).cuda()
            bb = None if inp.bias is None else torch.from_numpy(inp.bias).to(dt).cuda()
            yy = torch.from_numpy(inp.targets).cuda()
            del inp
            kw2 = dict(reduction=c.reduction, z_loss=c.z_loss)
            ex = lce.lce_fwd_bwd(hh, WW, bb, yy, **kw2)
            torch.cuda.synchronize()
            hip = _hip()
            n_st = len(lce.stage_names())
            evs = [([_event(hip) for _ in range(n_st)], [_event(hip) for _ in range(n_st)])
                   for _ in range(args.steps)]
            t0 = time.perf_counter()
            for k in range(args.steps):
                ex = lce.lce_fwd_bwd(hh, WW, bb, yy, out=ex, events=evs[k], **kw2)
            torch.cuda.synchronize()
            ms_exact = (time.perf_counter() - t0) * 1e3 / args.steps
            st_ms = {n: float(np.mean([_elapsed(hip, e[0][i], e[1][i]) for e in evs]))
                     for i, n in enumerate(lce.stage_names())}
            for e in evs:
                for x in e[0] + e[1]:
                    hip.hipEventDestroy(ctypes.c_void_p(x))
            log(f"{name}: exact {ms_exact:.1f} ms, stages {st_ms}")
            for srt in (False, True):
                res_f = bench_filtered(lce, torch, hh, WW, yy, dict(kw2, bias=bb), ex, args.filter_eps,
                                       args.steps, c.BT, sort_vocab=srt)
                res_f.update(workload=f"{name}: BT={c.BT}, H={c.H}, V={c.V}, Zipf(1.1) targets",
                             exact_ms_per_step=ms_exact, exact_stage_ms=st_ms)
                print(json.dumps(res_f), flush=True)
            del hh, WW, bb, yy, ex
            torch.cuda.empty_cache()
        return

    c = CONFIGS["headline"]
    log("generating the headline workload")
    inp = make_config("headline")
    dev = torch.device("cuda:0")
    h = torch.from_numpy(inp.hidden).to(torch.bfloat16).to(dev)
    W = torch.from_numpy(inp.weight).to(torch.bfloat16).to(dev)
    y = torch.from_numpy(inp.targets).to(dev)
    BT, H, V = c.BT, c.H, c.V
    out = dict(loss=torch.empty((), dtype=torch.float32, device=dev), grad_input=torch.empty_like(h),
               grad_weight=torch.empty_like(W), n_valid=torch.empty((), dtype=torch.int64, device=dev))
    ws_bytes = lce.fwd_bwd_workspace_bytes(BT, H, V, torch.bfloat16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kw = dict(reduction=c.reduction, z_loss=c.z_loss, workspace=ws, out=out)

    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter readings give the
        # factor that turns those counters into bytes for the kernels measured beside it.
        src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: {COPY_CAL_BYTES} bytes copied")

    log(f"warmup x{args.warmup}")
    for _ in range(args.warmup):
        lce.lce_fwd_bwd(h, W, None, y, **kw)
    torch.cuda.synchronize()
    hbm = measure_extra_hbm(lce, torch, h, W, y, dict(kw, workspace=None), ws_bytes)
    log(f"timing x{args.steps}")

    hip = _hip()
    n_st = len(lce.stage_names())
    evs = [([_event(hip) for _ in range(n_st)], [_event(hip) for _ in range(n_st)]) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        lce.lce_fwd_bwd(h, W, None, y, events=evs[k], **kw)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = t1 - t0
    ms_step = sec * 1e3 / args.steps
    names = lce.stage_names()
    stage_ms = {n: float(np.mean([_elapsed(hip, e[0][i], e[1][i]) for e in evs])) for i, n in enumerate(names)}
    for e in evs:
        for x in e[0] + e[1]:
            hip.hipEventDestroy(ctypes.c_void_p(x))

    btvh = float(BT) * V * H
    dom, roof = _stage_roofline(stage_ms, btvh)
    roof["traffic"] = measured_traffic(dom)
    roof["mfma_busy_counter"] = _profile_value(MFMA_FILE, dom, "mfma_busy")
    executed = executed_flops(stage_ms, btvh) / (ms_step * 1e-3) / 1e12
    useful = 6 * btvh / (ms_step * 1e-3) / 1e12
    n_valid = int(out["n_valid"].item())
    loss = float(out["loss"].item())

    res = {
        "metric": METRIC,
        "value": BT * args.steps / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; hidden ~ N(0,1), W ~ N(0, 1/H), uniform targets, 20% ignored)",
        "config": {"workload": "headline LM head: BT=65535, H=1024, V=176245, bf16, mean, no bias",
                   "BT": BT, "H": H, "V": V, "reduction": c.reduction, "n_valid": n_valid,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "tflops_executed": executed,
        "tflops_useful": useful,
        "mfma_util_executed": executed / PEAK_BF16_TFLOPS,
        "useful_frac": useful / PEAK_BF16_TFLOPS,
        "stage_ms": stage_ms,
        "extra_hbm_bytes": ws_bytes,
        "extra_hbm_budget_bytes": 512 * V * 4,
        "extra_hbm_measured": hbm,
        "loss": loss,
    }
    log(f"fused step {ms_step:.2f} ms")
    if not args.no_configs:
        res["configs"] = {}
        for name in ("gemma_like", "qwen_like"):
            res["configs"][name] = bench_config(lce, torch, name, min(args.steps, 10), min(args.warmup, 2), log,
                                                vendor=not args.no_vendor_gemm)
            log(f"{name}: fused step {res['configs'][name]['ms_per_step']:.2f} ms")
    if not args.no_vendor_gemm:
        log("vendor GEMM reference (materialised logits)")
        res["vendor_gemm_reference"] = vendor_gemm_reference(torch, h, W)
    if not args.no_chunked:
        log("token-chunked composition leg")
        res["chunked"] = bench_chunked(lce, torch, h, W, None, y, kw, out, args.steps, BT)
    if not args.no_rows:
        log("per-row outputs leg")
        res["rows"] = bench_rows(lce, torch, h, W, None, y, args.steps, BT)
    if not args.no_filter:
        log(f"gradient filtering, eps {args.filter_eps:g}")
        res["filtered"] = bench_filtered(lce, torch, h, W, y, kw, out, args.filter_eps, args.steps, BT)
    if not args.no_ce:
        log("standalone cross-entropy")
        res["standalone_ce"] = bench_ce(lce, torch, max(args.steps, 10))
    if not args.no_cpu_baseline:
        log(f"cpu baseline on {args.cpu_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
