"""The one-pass backward of the training step without decay (la2_forward then la2_backward_saved on
one backward-sized workspace, bf16, d = d_v = 128): dq, dk and dv from a single reverse walk, checked
element by element against the oracle and against the two-pass backward (dQ pass + dK/dV pass, forced
through the test build) on unsplit and split chains, forced segment lengths and state pieces, every
tile length and ragged or tiny sequences."""
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


def train_step(q, k, v, do, block):
    ws = la2.workspace_for(q, v, block, True)
    o = torch.empty_like(v)
    la2.la2_forward(q, k, v, None, o, block, ws)
    g = tuple(torch.empty_like(t) for t in (q, k, v))
    la2.la2_backward_saved(q, k, v, None, do, *g, block, ws)
    torch.cuda.synchronize()
    return o, g


def check(B, H, T, block, seed, **plan):
    x = inputs.make_random(B, H, T, 128, 128, dtype="bf16", seed=seed, decay="none")
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    with binding.plan_override(**plan):
        o, g = train_step(q, k, v, do, block)
    with binding.plan_override(two_pass_backward=True, **plan):
        _, g2 = train_step(q, k, v, do, block)
    ref = oracle.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), None)
    errs = [rel_err(f64(a), r) for a, r in zip(g, ref)]
    diffs = [rel_err(f64(a), f64(b)) for a, b in zip(g, g2)]
    print((B, H, T, block, plan), "dq dk dv vs oracle", " ".join(f"{e:.2e}" for e in errs),
          "vs two-pass", " ".join(f"{e:.2e}" for e in diffs), flush=True)
    for n, e in zip(("dq", "dk", "dv"), errs):
        assert e <= TOL, (n, e)
    for n, e in zip(("dq", "dk", "dv"), diffs):
        assert e <= TOL, (n, e)
    return g


@pytest.mark.parametrize("B,H,T,block", [
    (2, 3, 1000, 128),     # 6 chains: split into segments by the plan
    (16, 16, 300, 128),    # 256 chains: one segment each
    (1, 2, 1, 128), (1, 2, 63, 128), (1, 2, 64, 128), (1, 2, 65, 128), (1, 2, 129, 128),
    (1, 4, 2000, 64),      # 64-position forward tiles
    (1, 2, 1500, 256),
    (1, 1, 5000, 16),
])
def test_one_pass_backward(B, H, T, block):
    check(B, H, T, block, seed=700 + T)


@pytest.mark.parametrize("seg_tiles,state_sub", [(1, 0), (2, 0), (3, 0), (4, 2), (6, 3)])
def test_one_pass_backward_forced_segments(seg_tiles, state_sub):
    """Segments of forced lengths (every hand-over of the forward state and of the reverse state),
    and reverse state passes over finer pieces than the segments."""
    check(1, 3, 1111, 128, seed=71 + seg_tiles, seg_tiles=seg_tiles, state_sub=state_sub)


def test_one_pass_backward_narrow_forward_slices():
    """The forward run as two 64-wide value slices (its final states written per slice)."""
    check(1, 2, 900, 128, seed=5, slice_width=64, seg_tiles=2)


def test_one_pass_backward_twice_on_one_workspace():
    """The saved backward leaves the forward's states in place: a second call gives the same bits."""
    x = inputs.make_random(1, 4, 3000, 128, 128, dtype="bf16", seed=9, decay="none")
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    ws = la2.workspace_for(q, v, 128, True)
    o = torch.empty_like(v)
    la2.la2_forward(q, k, v, None, o, 128, ws)
    runs = []
    for _ in range(2):
        g = tuple(torch.empty_like(t) for t in (q, k, v))
        la2.la2_backward_saved(q, k, v, None, do, *g, 128, ws)
        runs.append(g)
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_autograd_uses_one_pass_backward():
    """lightning_attention's backward (no decay) is the one-pass backward and matches the oracle."""
    x = inputs.make_random(2, 2, 700, 128, 128, dtype="bf16", seed=12, decay="none")
    q, k, v = (x[n].to(DEV).requires_grad_(True) for n in ("q", "k", "v"))
    do = x["do"].to(DEV)
    la2.lightning_attention(q, k, v, None, 128).backward(do)
    ref = oracle.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), None)
    for t, r in zip((q.grad, k.grad, v.grad), ref):
        assert rel_err(f64(t), r) <= TOL
