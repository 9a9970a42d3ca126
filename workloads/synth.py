"""Seeded generators for the five workloads of fused linear cross-entropy.

Every array is drawn from numpy's PCG64 with one child stream per tensor
(``SeedSequence(seed).spawn(4)``: hidden, weight, bias, targets), so the same
seed gives the same bytes on any machine.  Values for bf16 workloads are drawn
in float32 and rounded to the nearest bf16 (ties to even) here, once; the GPU
receives exactly those values and the float64 oracle upcasts them exactly.

Shapes follow the pages' workloads:
  * the headline LM-head shape BT=65535, H=1024, V=176245 ("Fused Linear
    Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It", section
    "The engineering wall" and "Putting numbers on it");
  * a Gemma-2-2B-like head, 8192 tokens x 256128 vocab ("Cut Cross Entropy
    visualized", section "Naively computing Cross Entropy is Expensive");
  * standalone logits of shape [8192, 128256] ("Greyhound - Cross-Entropy",
    section "Usage");
  * a Qwen3-4B-like head with H=4096, V=151936 (first page, "The setting").

Distribution readings: N(0, s) is read as standard deviation s, except the
weight init written N(0, 1/H), read as variance 1/H (std H**-0.5).  Zipf(1.1)
targets put P(y=k) proportional to (k+1)**-1.1 on [0, V), sampled by inverse
CDF.  "x% ignored" masks exactly round(x*BT) positions chosen by a seeded
permutation.  None of this is the method's arithmetic.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

IGNORE_INDEX = -100


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    # finite inputs only: u + 0x8000 stays below 2**32 for every finite float32
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return x


def zipf_targets(rng: np.random.Generator, n: int, V: int, s: float = 1.1) -> np.ndarray:
    """Draw n ids in [0, V) with P(k) proportional to (k+1)**-s (truncated, normalised)."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    y = np.searchsorted(cdf, u, side="right")
    return np.minimum(y, V - 1).astype(np.int64)


def _mask_ignored(rng: np.random.Generator, y: np.ndarray, frac: float) -> np.ndarray:
    n_ign = int(round(frac * y.shape[0]))
    if n_ign:
        pos = rng.permutation(y.shape[0])[:n_ign]
        y = y.copy()
        y[pos] = IGNORE_INDEX
    return y


@dataclasses.dataclass(frozen=True)
class FusedConfig:
    name: str
    BT: int
    H: int
    V: int
    dtype: str  # "f32" or "bf16"
    w_std: float
    bias_std: Optional[float]
    targets: str  # "uniform" or "zipf"
    ignore_frac: float
    z_loss: float
    reduction: str
    seed: int


@dataclasses.dataclass(frozen=True)
class CEConfig:
    name: str
    B: int
    V: int
    dtype: str
    logit_std: float
    ignore_frac: float
    reduction: str
    seed: int


CONFIGS = {
    "tiny_f32": FusedConfig("tiny_f32", 256, 128, 4096, "f32", 128 ** -0.5, None,
                            "uniform", 0.10, 0.0, "mean", 1),
    "ce_only": CEConfig("ce_only", 8192, 128256, "bf16", 2.0, 0.05, "sum", 2),
    "gemma_like": FusedConfig("gemma_like", 8192, 2304, 256128, "bf16", 0.02, None,
                              "zipf", 0.0, 0.0, "mean", 3),
    "headline": FusedConfig("headline", 65535, 1024, 176245, "bf16", 1024 ** -0.5, None,
                            "uniform", 0.20, 0.0, "mean", 4),
    "qwen_like": FusedConfig("qwen_like", 16384, 4096, 151936, "bf16", 0.02, 0.1,
                             "zipf", 0.10, 1e-4, "mean", 5),
}


@dataclasses.dataclass
class FusedInputs:
    hidden: np.ndarray          # [BT, H] float32 (bf16-representable for bf16 workloads)
    weight: np.ndarray          # [V, H]
    bias: Optional[np.ndarray]  # [V] or None
    targets: np.ndarray         # [BT] int64
    dtype: str
    z_loss: float
    reduction: str


@dataclasses.dataclass
class CEInputs:
    logits: np.ndarray   # [B, V] float32 (bf16-representable for bf16)
    targets: np.ndarray  # [B] int64
    dtype: str


def make_fused(BT: int, H: int, V: int, *, dtype: str = "bf16", seed: int = 0,
               h_std: float = 1.0, w_std: Optional[float] = None,
               bias_std: Optional[float] = None, targets: str = "uniform",
               ignore_frac: float = 0.0, z_loss: float = 0.0,
               reduction: str = "mean") -> FusedInputs:
    """Seeded fused-LCE inputs of any shape (used for the named configs and small cases)."""
    if w_std is None:
        w_std = H ** -0.5 if H > 0 else 1.0
    ss = np.random.SeedSequence(seed).spawn(4)
    g_h, g_w, g_b, g_y = (np.random.Generator(np.random.PCG64(s)) for s in ss)
    h = g_h.standard_normal((BT, H), dtype=np.float32)
    if h_std != 1.0:
        h *= np.float32(h_std)
    w = g_w.standard_normal((V, H), dtype=np.float32)
    w *= np.float32(w_std)
    b = None
    if bias_std is not None:
        b = g_b.standard_normal((V,), dtype=np.float32) * np.float32(bias_std)
    if targets == "uniform":
        y = g_y.integers(0, V, size=BT, dtype=np.int64)
    elif targets == "zipf":
        y = zipf_targets(g_y, BT, V)
    else:
        raise ValueError(targets)
    y = _mask_ignored(g_y, y, ignore_frac)
    if dtype == "bf16":
        h = bf16_round(h)
        w = bf16_round(w)
        if b is not None:
            b = bf16_round(b)
    elif dtype != "f32":
        raise ValueError(dtype)
    return FusedInputs(h, w, b, y, dtype, float(z_loss), reduction)


def make_ce(B: int, V: int, *, dtype: str = "bf16", seed: int = 0, logit_std: float = 2.0,
            ignore_frac: float = 0.0) -> CEInputs:
    """Seeded logits/labels for the standalone cross-entropy kernel."""
    ss = np.random.SeedSequence(seed).spawn(2)
    g_x = np.random.Generator(np.random.PCG64(ss[0]))
    x = g_x.standard_normal((B, V), dtype=np.float32)
    x *= np.float32(logit_std)
    y = ce_targets(B, V, seed=seed, ignore_frac=ignore_frac)
    if dtype == "bf16":
        x = bf16_round(x)
    elif dtype == "f16":
        x = x.astype(np.float16).astype(np.float32)  # nearest even in IEEE half
    elif dtype != "f32":
        raise ValueError(dtype)
    return CEInputs(x, y, dtype)


def ce_targets(B: int, V: int, *, seed: int = 0, ignore_frac: float = 0.0) -> np.ndarray:
    """Labels of the standalone workload (uniform ids, then the ignore mask)."""
    g_y = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(2)[1]))
    y = g_y.integers(0, V, size=B, dtype=np.int64)
    return _mask_ignored(g_y, y, ignore_frac)


def make_config(name: str):
    """Inputs of one named workload (seed = its number in the list of five)."""
    c = CONFIGS[name]
    if isinstance(c, CEConfig):
        return make_ce(c.B, c.V, dtype=c.dtype, seed=c.seed, logit_std=c.logit_std,
                       ignore_frac=c.ignore_frac)
    return make_fused(c.BT, c.H, c.V, dtype=c.dtype, seed=c.seed, w_std=c.w_std,
                      bias_std=c.bias_std, targets=c.targets, ignore_frac=c.ignore_frac,
                      z_loss=c.z_loss, reduction=c.reduction)
