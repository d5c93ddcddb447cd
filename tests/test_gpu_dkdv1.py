"""The dK/dV pass of the two-pass backward on the producer/consumer walk of the one-pass backward
(la2_bwd1_bf16.hip without its dQ and S: bf16, d = d_v = 128, no carried state), with and without a
decay, against the oracle and against the eight-wave fused dK/dV kernel it replaces there (forced
through the test build): unsplit and split chains, forced segment lengths and state pieces, ragged
and one-position sequences, per-head, strong and underflowing decays.  dq comes from the dQ pass in
both runs, so it is compared too."""
import numpy as np
import pytest
import torch

import causal_linear_attention_amd as la2
from causal_linear_attention_amd import binding, inputs
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


def f64(t):
    return t.detach().double().cpu().numpy()


def rel_err(got, ref):
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (scale if scale > 0 else 1.0)


def two_pass(x, block, **plan):
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    with binding.plan_override(two_pass_backward=True, **plan):
        g = la2.backward(q, k, v, do, dec, block)
        torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("B,H,T,block,decay,plan", [
    (2, 3, 1000, 128, "heads", {}),             # 6 chains: split by the plan
    (16, 16, 300, 128, "heads", {}),            # 256 chains: one segment each
    (16, 16, 300, 128, "none", {}),
    (1, 2, 1, 128, "heads", {}), (1, 2, 65, 64, 0.5, {}), (1, 2, 129, 256, "none", {}),
    (1, 3, 1111, 128, "heads", {"seg_tiles": 1}), (1, 3, 1111, 128, 0.9, {"seg_tiles": 3, "state_sub": 3}),
    (1, 2, 700, 128, 1e-3, {"seg_tiles": 2}),   # lam^j underflows from j = 13 on
    (1, 1, 5000, 16, "heads", {}),
])
def test_dkdv_walk_against_oracle_and_fused_kernel(B, H, T, block, decay, plan):
    x = inputs.make_random(B, H, T, 128, 128, dtype="bf16", seed=1200 + T, decay=decay)
    g = two_pass(x, block, **plan)
    g_old = two_pass(x, block, legacy_dkdv=True, **plan)
    lam = None if x["decay"] is None else x["decay"].double().numpy()
    ref = oracle.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), lam)
    errs = [rel_err(f64(a), r) for a, r in zip(g, ref)]
    diffs = [rel_err(f64(a), f64(b)) for a, b in zip(g, g_old)]
    print((B, H, T, block, decay, plan), "dq dk dv vs oracle", " ".join(f"{e:.2e}" for e in errs),
          "vs the fused kernel", " ".join(f"{e:.2e}" for e in diffs), flush=True)
    for t in g:
        assert np.isfinite(f64(t)).all()
    for n, e in zip(("dq", "dk", "dv"), errs):
        assert e <= TOL, (n, e)
    for n, e in zip(("dq", "dk", "dv"), diffs):
        assert e <= TOL, (n, e)


def test_dkdv_walk_tnl15b_layer_shape():
    """The TNL-15B layer shape (2 x 40 chains of 6144 positions, per-head decay): every chain split,
    every output element against the oracle."""
    x = inputs.make("tnl15b_layer")
    w = x["workload"]
    g = two_pass(x, w.block)
    ref = oracle.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), x["decay"].double().numpy())
    errs = [rel_err(f64(a), r) for a, r in zip(g, ref)]
    print(w.name, "dq dk dv vs oracle", " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= TOL
