"""The seeded input generator: determinism, shapes, dtypes, decays, outlier rows."""
import math

import torch

from causal_linear_attention_amd import inputs


def test_named_workloads_shapes():
    w = inputs.WORKLOADS
    assert (w["tnl15b_layer"].H * w["tnl15b_layer"].d) == 5120
    assert {inputs.WORKLOADS[n].tokens for n in inputs.SWEEP_NAMES} == {131072}
    assert [inputs.WORKLOADS[n].T for n in inputs.SWEEP_NAMES] == [1024, 4096, 16384, 65536, 131072]


def test_deterministic_and_dtypes():
    a = inputs.make("tiny_fp32_fwd")
    b = inputs.make("tiny_fp32_fwd")
    assert a["q"].dtype == torch.float32 and a["do"] is None and a["decay"] is None
    for n in ("q", "k", "v"):
        assert torch.equal(a[n], b[n])
    c = inputs.make("bf16_fwd_t2k")
    assert c["q"].dtype == torch.bfloat16 and c["q"].shape == (4, 16, 2048, 64)
    # N(0,1)/sqrt(d): per-element std close to 1/8
    assert abs(c["q"].float().std().item() - 1 / 8) < 2e-3


def test_head_decays():
    lam = inputs.head_decays(16)
    assert lam.dtype == torch.float32
    ref = [math.exp(-(2.0 ** (-8.0 * (h + 1) / 16))) for h in range(16)]
    assert torch.allclose(lam.double(), torch.tensor(ref, dtype=torch.float64), rtol=1e-7, atol=0)
    assert abs(lam[0].item() - 0.4931) < 1e-4 and abs(lam[-1].item() - 0.99610) < 1e-4
    lam40 = inputs.head_decays(40)
    assert abs(lam40[0].item() - 0.4187) < 1e-4
    assert bool(((lam40 > 0) & (lam40 <= 1)).all())


def test_outlier_rows():
    w = inputs.with_overrides("long128k_outliers", T=8192, H=8)
    x = inputs.make(w)
    g = torch.Generator().manual_seed(w.seed)
    norms = x["q"].float().norm(dim=-1)                 # rows x8 have norm ~8
    frac = (norms > 3.0).float().mean().item()
    assert 0.007 < frac < 0.013, frac
    assert x["do"].float().norm(dim=-1).max().item() < 3 * math.sqrt(w.dv)
