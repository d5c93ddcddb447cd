"""Seeded random shapes through every entry point, against the oracle.

Each case draws B, H, T, d, d_v, dtype, tile length and decay from a fixed generator (the draw is the
same on every run), so together the cases cover ragged last tiles, split and unsplit chains, both
bf16 staging paths and the fp32 path in combinations the hand-picked cases do not.  Bars as
elsewhere: max|gpu - ref| / max|ref| <= 1e-5 (fp32 inputs), <= 2e-2 (bf16 inputs).
"""
import numpy as np
import pytest
import torch

import causal_linear_attention_amd as la2
from causal_linear_attention_amd import inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
DEV = "cuda:0"


def f64(t):
    return t.detach().double().cpu().numpy()


def rel_err(got, ref):
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(np.asarray(got) - ref))) / (scale if scale > 0 else 1.0)


def draw(i):
    rng = np.random.default_rng(1000 + i)
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    d, dv = (int(x) for x in rng.choice([64, 128], size=2))
    if dtype == "f32":
        dv = 64 * int(rng.integers(1, 3))
    block = int(rng.choice([64, 128, 256] if dtype == "bf16" else [16, 32, 64]))
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 6))
    T = int(rng.integers(1, 1500))
    decay = ["heads", "none", float(rng.uniform(0.3, 1.0))][int(rng.integers(0, 3))]
    return B, H, T, d, dv, dtype, block, decay


CASES = [draw(i) for i in range(24)]


def lam_of(x):
    return None if x["decay"] is None else x["decay"].double().numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}T{}d{}dv{}{}tb{}-{}".format(*c))
def test_random_shape(case):
    B, H, T, d, dv, dtype, block, decay = case
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=T + 7 * d, decay=decay, backward=True)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    lam = lam_of(x)
    host = [f64(x[n]) for n in ("q", "k", "v", "do")]
    g = torch.Generator().manual_seed(T)
    s_in = (torch.randn((B, H, d, dv), generator=g) * 0.3).float()
    gs = (torch.randn((B, H, d, dv), generator=g) * 0.3).float()

    o = la2.forward(q, k, v, dec, block)
    grads = la2.backward(q, k, v, do, dec, block)
    o_s, s_out = la2.forward_state(q, k, v, dec, block, s_in.to(DEV))
    grads_s = la2.backward_state(q, k, v, do, dec, block, s_in.to(DEV), gs.to(DEV))
    torch.cuda.synchronize()

    ref_o = oracle.forward(*host[:3], lam)
    ref_g = oracle.backward(*host, lam)
    ref_os, ref_s = oracle.forward_state(*host[:3], lam, f64(s_in))
    ref_gs = oracle.backward_state(*host, lam, f64(s_in), f64(gs))
    checks = [("o", o, ref_o), ("dq", grads[0], ref_g[0]), ("dk", grads[1], ref_g[1]), ("dv", grads[2], ref_g[2]),
              ("o_state", o_s, ref_os), ("state_out", s_out, ref_s)]
    checks += [(n, a, r) for n, a, r in zip(("dq_s", "dk_s", "dv_s", "dstate_in"), grads_s, ref_gs)]
    errs = {n: rel_err(f64(a), r) for n, a, r in checks}
    print(case, " ".join(f"{n} {e:.1e}" for n, e in errs.items()), flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, bad
