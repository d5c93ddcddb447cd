"""The producer/consumer forward scan (la2_fwd1_bf16.hip: bf16, d = d_v = 128) against the oracle
and against the eight-wave scan kernel it replaces there (forced through the test build), on
unsplit and split chains, forced segment lengths and state pieces, every tile length, ragged and tiny
sequences, without and with a decay (per-head, strong, and so small that most weights underflow);
with the final state of the training step's forward; as the dQ pass of the two-pass backward (state
read transposed)."""
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


def lam_of(x):
    return None if x["decay"] is None else x["decay"].double().numpy()


def forward(x, block, **plan):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    with binding.plan_override(**plan):
        ws = la2.workspace_for(q, v, block, True)
        o = torch.empty_like(v)
        la2.la2_forward(q, k, v, dec, o, block, ws)
        torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("B,H,T,block,plan", [
    (2, 3, 1000, 128, {}),                      # 6 chains, split by the plan
    (16, 16, 300, 128, {}),                     # 256 chains, one segment each
    (1, 2, 1, 128, {}), (1, 2, 63, 64, {}), (1, 2, 64, 128, {}), (1, 2, 65, 32, {}), (1, 2, 129, 256, {}),
    (1, 3, 1111, 128, {"seg_tiles": 1}), (1, 3, 1111, 128, {"seg_tiles": 3}),
    (1, 3, 1111, 64, {"seg_tiles": 5, "state_sub": 5}),
    (1, 1, 5000, 16, {}),
])
def test_forward_against_oracle_and_legacy(B, H, T, block, plan):
    x = inputs.make_random(B, H, T, 128, 128, dtype="bf16", seed=900 + T, decay="none")
    o = forward(x, block, **plan)
    o_old = forward(x, block, legacy_forward=True, **plan)
    ref = oracle.forward(*(f64(x[n]) for n in ("q", "k", "v")), None)
    e, e_old = rel_err(f64(o), ref), rel_err(f64(o_old), ref)
    d = rel_err(f64(o), f64(o_old))
    print((B, H, T, block, plan), f"vs oracle {e:.2e} (eight-wave kernel {e_old:.2e}), vs each other {d:.2e}",
          flush=True)
    assert e <= TOL and d <= TOL


@pytest.mark.parametrize("B,H,T,block,plan,decay", [
    (2, 3, 1000, 128, {}, "heads"),             # 6 chains, split by the plan
    (16, 16, 300, 128, {}, "heads"),            # 256 chains, one segment each
    (1, 2, 1, 128, {}, "heads"), (1, 2, 65, 32, {}, 0.5), (1, 2, 129, 256, {}, 0.5),
    (1, 3, 1111, 128, {"seg_tiles": 3}, "heads"), (1, 3, 1111, 64, {"seg_tiles": 5, "state_sub": 5}, 0.9),
    (1, 1, 5000, 16, {}, "heads"),
    (1, 2, 700, 128, {"seg_tiles": 2}, 1e-3),   # lam^j underflows from j = 13 on
])
def test_decay_forward_against_oracle_and_legacy(B, H, T, block, plan, decay):
    x = inputs.make_random(B, H, T, 128, 128, dtype="bf16", seed=950 + T, decay=decay)
    o = forward(x, block, **plan)
    o_old = forward(x, block, legacy_forward=True, **plan)
    ref = oracle.forward(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x))
    e, e_old = rel_err(f64(o), ref), rel_err(f64(o_old), ref)
    d = rel_err(f64(o), f64(o_old))
    print((B, H, T, block, plan, decay), f"vs oracle {e:.2e} (eight-wave kernel {e_old:.2e}), vs each other {d:.2e}",
          flush=True)
    assert np.isfinite(f64(o)).all()
    assert e <= TOL and d <= TOL


def test_decay_dq_pass():
    """With a decay the backward keeps the two passes; its dQ pass runs this scan on the forward's
    states read transposed."""
    x = inputs.make_random(1, 3, 1111, 128, 128, dtype="bf16", seed=88, decay="heads")
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    dec = x["decay"].to(DEV)
    for plan in ({}, {"seg_tiles": 2}):
        with binding.plan_override(**plan):
            dq, dk, dv = la2.backward(q, k, v, do, dec, 128)
            torch.cuda.synchronize()
        ref = oracle.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), lam_of(x))
        for a, r in zip((dq, dk, dv), ref):
            assert rel_err(f64(a), r) <= TOL


def test_final_state_for_the_one_pass_backward():
    """The training step's forward writes each chain's final state: with it the one-pass backward
    matches the oracle (split chains: the state of the last segment)."""
    x = inputs.make_random(2, 3, 1500, 128, 128, dtype="bf16", seed=77, decay="none")
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    for plan in ({}, {"seg_tiles": 2}):
        with binding.plan_override(**plan):
            ws = la2.workspace_for(q, v, 128, True)
            o = torch.empty_like(v)
            la2.la2_forward(q, k, v, None, o, 128, ws)
            g = tuple(torch.empty_like(t) for t in (q, k, v))
            la2.la2_backward_saved(q, k, v, None, do, *g, 128, ws)
            torch.cuda.synchronize()
        ref = oracle.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), None)
        errs = [rel_err(f64(a), r) for a, r in zip(g, ref)]
        print(plan, "dq dk dv", " ".join(f"{e:.2e}" for e in errs), flush=True)
        assert max(errs) <= TOL


def test_dq_pass_reads_states_transposed():
    """The two-pass backward's dQ pass runs this scan with the forward's states read transposed."""
    x = inputs.make_random(1, 3, 1111, 128, 128, dtype="bf16", seed=78, decay="none")
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    with binding.plan_override(seg_tiles=2, two_pass_backward=True):
        dq, dk, dv = la2.backward(q, k, v, do, None, 128)
        torch.cuda.synchronize()
    ref = oracle.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), None)
    for a, r in zip((dq, dk, dv), ref):
        assert rel_err(f64(a), r) <= TOL


@pytest.mark.parametrize("decay", ["none", "heads", 0.5])
def test_forward_state_out_without_state_in(decay):
    """la2_forward_state with no carried-in state runs this kernel and writes the exact final state
    (a ragged last tile: with a decay its weights count only the tile's real rows), with the same o as
    la2_forward."""
    x = inputs.make_random(1, 2, 777, 128, 128, dtype="bf16", seed=79, decay=decay)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    for plan in ({}, {"seg_tiles": 2}):
        with binding.plan_override(**plan):
            o, s_out = la2.forward_state(q, k, v, dec, 128, None)
            o_plain = la2.forward(q, k, v, dec, 128)
            torch.cuda.synchronize()
        o_ref, s_ref = oracle.forward_state(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x), None)
        assert rel_err(f64(o), o_ref) <= TOL
        assert rel_err(f64(s_out), s_ref) <= 1e-2
        assert torch.equal(o, o_plain)
