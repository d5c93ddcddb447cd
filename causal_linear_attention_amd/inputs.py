"""Seeded synthetic inputs for the causal linear attention workloads.

This module only draws numbers: it holds none of the attention arithmetic, and
both the HIP path and the CPU oracle are fed from it.  Everything is drawn on
the CPU with a ``torch.Generator`` seeded per workload, in this order: q, k, v
(fp32 standard normal, each scaled by 1/sqrt(d) of its own width), then dO
(standard normal) when the workload has a backward pass, then one Bernoulli
row mask per q, k, v for the outlier rows.  Values are rounded once to the
workload dtype; the oracle later widens the same stored values exactly.

The shapes are the ones the pages report training and benchmarking at: the
TransNormerLLM-15B attention layer (40 heads x 128 = embedding 5120, sequence
6144; research.elamur.ai summary of Lightning Attention-2, key points), tile
sizes 64/128/256 (page "Lightning Attention", section 2 and section 4), and a
fixed-token length sweep from 1K to 128K tokens (same summary: tokens per GPU
per second against sequence length).
"""
from dataclasses import dataclass, replace
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    d: int
    dv: int
    block: int
    dtype: str              # "f32" or "bf16"
    decay: bool             # per-head decay lam_h, else lam = 1
    seed: int
    backward: bool
    outlier_frac: float = 0.0
    outlier_scale: float = 8.0

    @property
    def tokens(self):
        return self.B * self.T

    @property
    def chains(self):
        return self.B * self.H


def head_decays(H):
    """lam_h = exp(-2^(-8 (h+1) / H)) for h = 0..H-1, computed in fp64, rounded once to fp32."""
    vals = [math.exp(-(2.0 ** (-8.0 * (h + 1) / H))) for h in range(H)]
    return torch.tensor(vals, dtype=torch.float64).to(torch.float32)


_SWEEP = [(128, 1024), (32, 4096), (8, 16384), (2, 65536), (1, 131072)]

WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_fwd", 1, 1, 256, 64, 64, 64, "f32", False, 0, False),
        Workload("bf16_fwd_t2k", 4, 16, 2048, 64, 64, 64, "bf16", True, 1, False),
        Workload("tnl15b_layer", 2, 40, 6144, 128, 128, 128, "bf16", True, 2, True),
        *[Workload(f"sweep131k_t{T // 1024}k", B, 16, T, 128, 128, 128, "bf16", False, 3, True)
          for B, T in _SWEEP],
        Workload("long128k_outliers", 1, 40, 131072, 128, 128, 256, "bf16", True, 4, True,
                 outlier_frac=0.01),
    ]
}

SWEEP_NAMES = [f"sweep131k_t{T // 1024}k" for _, T in _SWEEP]


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make(w, with_grad_out=None):
    """Draw the inputs of workload ``w`` (a Workload or its name) on the CPU.

    Returns a dict with q, k, v ([B, H, T, d] / [B, H, T, dv] in the workload
    dtype), do (or None), decay (fp32 [H] or None) and the workload itself.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    want_do = w.backward if with_grad_out is None else with_grad_out
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    dt = torch_dtype(w.dtype)
    q = torch.randn(w.B, w.H, w.T, w.d, generator=g) / math.sqrt(w.d)
    k = torch.randn(w.B, w.H, w.T, w.d, generator=g) / math.sqrt(w.d)
    v = torch.randn(w.B, w.H, w.T, w.dv, generator=g) / math.sqrt(w.dv)
    do = torch.randn(w.B, w.H, w.T, w.dv, generator=g) if want_do else None
    if w.outlier_frac > 0:
        for x in (q, k, v):
            rows = torch.rand(w.B, w.H, w.T, generator=g) < w.outlier_frac
            x[rows] *= w.outlier_scale
    out = {
        "q": q.to(dt), "k": k.to(dt), "v": v.to(dt),
        "do": None if do is None else do.to(dt),
        "decay": head_decays(w.H) if w.decay else None,
        "workload": w,
    }
    return out


def make_random(B, H, T, d, dv, dtype="bf16", seed=0, decay="heads", block=64, backward=True):
    """Inputs of an arbitrary small shape (parity cases), drawn like the named workloads.

    ``decay`` is "heads" (lam_h as above), "none" (lam = 1) or a float in (0, 1]
    applied to every head.
    """
    w = Workload(f"random_{B}x{H}x{T}x{d}x{dv}", B, H, T, d, dv, block, dtype,
                 decay != "none", seed, backward)
    x = make(w)
    if isinstance(decay, float):
        x["decay"] = torch.full((H,), decay, dtype=torch.float32)
    return x


def with_overrides(w, **kw):
    """A copy of workload ``w`` with some fields replaced."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return replace(w, **kw)
