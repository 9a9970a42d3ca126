"""Helpers shared by the GPU parity tests (inputs to device, error metrics, tolerances)."""

import numpy as np
import torch

# Tolerances for fused linear cross-entropy against the float64 oracle: bf16 inputs with fp32
# accumulation, and fp32 inputs (fp32 MFMA, no reduced-precision operands).
TOL = {
    "bf16": dict(loss=1e-3, grad=1e-2, lse=2e-3),
    "f32": dict(loss=1e-5, grad=1e-4, lse=1e-5),
}
# Standalone cross-entropy: dlogits rounded to the logits' dtype.
CE_TOL = {
    "bf16": dict(sums=1e-3, dlogits=1e-2),
    # fp16 logits: sums in fp32 from exact inputs; dlogits rounded once to half (2^-11)
    "f16": dict(sums=1e-5, dlogits=1e-3),
    "f32": dict(sums=1e-5, dlogits=1e-5),
}

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}


def dev(a, dtype="f32"):
    """numpy float32 array (bf16-representable for bf16) -> contiguous device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.int64:
        return t.cuda()
    return t.to(TORCH_DT[dtype]).cuda().contiguous()


def host64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return num
    return num / den


def rel(got, ref):
    return abs(float(got) - float(ref)) / max(abs(float(ref)), 1e-30)
