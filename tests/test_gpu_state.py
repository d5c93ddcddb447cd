"""Carried states and one-token decode steps on the GPU, through the C ABI, against the oracle.

The oracle's ``forward_state`` (pinned by the closed forms of the outputs and the final state and
by split-and-carry invariance) is the reference.  Bars as for the plain passes: max|gpu - ref| /
max|ref| <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs, on every output and on the final state.
"""
import numpy as np
import pytest
import torch

import causal_linear_attention_amd as la2
from causal_linear_attention_amd import binding, inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
DEV = "cuda:0"


def f64(t):
    return t.detach().double().cpu().numpy()


def rel_err(got, ref):
    ref = np.asarray(ref)
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(np.asarray(got) - ref))) / (scale if scale > 0 else 1.0)


def lam_of(x):
    return None if x["decay"] is None else x["decay"].double().numpy()


def seeded_state(B, H, d, dv, seed):
    """A carried-in state: fp32 values both sides read exactly."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((B, H, d, dv), generator=g) * 0.5).to(torch.float32)


def to_dev(x):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    decay = None if x["decay"] is None else x["decay"].to(DEV)
    return q, k, v, decay


CASES = [
    # (B, H, T, d, dv, dtype, block, decay)
    (1, 2, 777, 128, 128, "bf16", 128, "heads"),      # split chains, ragged last tile
    (1, 2, 50, 128, 128, "bf16", 128, "heads"),       # one short tile
    (2, 3, 700, 64, 128, "bf16", 64, "heads"),        # direct-to-LDS path
    (1, 3, 333, 128, 64, "bf16", 256, "none"),
    (16, 16, 200, 128, 128, "bf16", 128, "heads"),    # 256 chains: unsplit, state read at the start
    (1, 2, 300, 64, 64, "f32", 32, "heads"),
    (16, 16, 70, 64, 64, "f32", 64, "none"),          # fp32, unsplit
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}T{c[2]}d{c[3]}dv{c[4]}{c[5]}tb{c[6]}{c[7]}")
def test_forward_state_matches_oracle(case):
    B, H, T, d, dv, dtype, block, decay = case
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=61 + T, decay=decay, backward=False)
    s_in = seeded_state(B, H, d, dv, 7 + T)
    q, k, v, dec = to_dev(x)
    o, s_out = la2.forward_state(q, k, v, dec, block, state_in=s_in.to(DEV))
    ref_o, ref_s = oracle.forward_state(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x), f64(s_in))
    torch.cuda.synchronize()
    eo, es = rel_err(f64(o), ref_o), rel_err(f64(s_out), ref_s)
    print(case, f"o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    # without a carried-in state: the plain forward's o, and the final state from zero
    o0, s0 = la2.forward_state(q, k, v, dec, block)
    ref_o0, ref_s0 = oracle.forward_state(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x), None)
    torch.cuda.synchronize()
    assert rel_err(f64(o0), ref_o0) <= TOL[dtype] and rel_err(f64(s0), ref_s0) <= TOL[dtype]
    assert torch.equal(o0, la2.forward(q, k, v, dec, block))


@pytest.mark.parametrize("seg_tiles,slice_width,sub", [(1, 0, 0), (3, 0, 0), (0, 64, 0), (2, 64, 0), (4, 0, 2)])
def test_forward_state_plans(seg_tiles, slice_width, sub):
    """Forced segment splits (prefix with a carried-in state), state pieces finer than the segments
    and 64-wide value slices."""
    x = inputs.make_random(2, 2, 600, 128, 128, dtype="bf16", seed=71, decay="heads", backward=False)
    s_in = seeded_state(2, 2, 128, 128, 73)
    q, k, v, dec = to_dev(x)
    with binding.plan_override(seg_tiles=seg_tiles, state_sub=sub, slice_width=slice_width):
        o, s_out = la2.forward_state(q, k, v, dec, 128, state_in=s_in.to(DEV))
    ref_o, ref_s = oracle.forward_state(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x), f64(s_in))
    torch.cuda.synchronize()
    assert rel_err(f64(o), ref_o) <= 2e-2 and rel_err(f64(s_out), ref_s) <= 2e-2


@pytest.mark.parametrize("dtype,d,dv,block", [("bf16", 128, 128, 128), ("bf16", 64, 128, 64), ("f32", 64, 64, 64)])
def test_chunked_prefill_in_place(dtype, d, dv, block):
    """A sequence run in uneven chunks, one state buffer updated in place, equals the whole run."""
    B, H, T = 1, 4, 1000
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=83, decay="heads", backward=False)
    q, k, v, dec = to_dev(x)
    state = torch.zeros((B, H, d, dv), dtype=torch.float32, device=DEV)
    outs, t = [], 0
    for n in (300, 1, 450, 249):
        sl = slice(t, t + n)
        qc, kc, vc = (a[:, :, sl].contiguous() for a in (q, k, v))
        oc = torch.empty_like(vc)
        ws = la2.workspace_for(qc, vc, block, False)
        la2.la2_forward_state(qc, kc, vc, dec, state, oc, state, block, ws)
        outs.append(oc)
        t += n
    ref_o, ref_s = oracle.forward_state(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x), None)
    torch.cuda.synchronize()
    assert rel_err(f64(torch.cat(outs, dim=2)), ref_o) <= TOL[dtype]
    assert rel_err(f64(state), ref_s) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,dv,decay", [("bf16", 128, 128, "heads"), ("bf16", 64, 128, "none"),
                                              ("bf16", 128, 64, "heads"), ("f32", 64, 64, "heads"),
                                              ("f32", 128, 128, "none")])
def test_decode_steps_continue_a_prefill(dtype, d, dv, decay):
    """Prefill T0 positions with la2_forward_state, then generate 6 positions with la2_decode_step;
    outputs and final state against the oracle's whole-sequence run."""
    B, H, T0, N = 2, 3, 257, 6
    x = inputs.make_random(B, H, T0 + N, d, dv, dtype=dtype, seed=97 + d + dv, decay=decay, backward=False)
    q, k, v, dec = to_dev(x)
    block = 128 if dtype == "bf16" else 64
    _, state = la2.forward_state(q[:, :, :T0].contiguous(), k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(),
                                 dec, block)
    outs = []
    for t in range(T0, T0 + N):
        outs.append(la2.decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                    state, dec))
    ref_o, ref_s = oracle.forward_state(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x), None)
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=2)
    eo, es = rel_err(f64(got), ref_o[:, :, T0:]), rel_err(f64(state), ref_s)
    print(dtype, d, dv, decay, f"o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("B,d,dv", [(260, 128, 128), (513, 128, 64)])
def test_decode_streamed_state(B, d, dv):
    """Over 256 MiB of states (B x 16 heads) the decode step streams them with the nontemporal
    policy: two steps from a random fp32 state, outputs and states of sampled sequences against the
    oracle's state-carrying forward from the same state."""
    H = 16
    assert B * H * d * dv * 4 > (256 << 20)
    x = inputs.make_random(B, H, 2, d, dv, dtype="bf16", seed=131 + dv, decay="heads", backward=False)
    q, k, v, dec = to_dev(x)
    s0 = seeded_state(B, H, d, dv, 7)
    state = s0.to(DEV)
    outs = [la2.decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(), state, dec)
            for t in range(2)]
    torch.cuda.synchronize()
    rows = [0, B // 2, B - 1]
    ref_o, ref_s = oracle.forward_state(*(f64(x[n])[rows] for n in ("q", "k", "v")), lam_of(x),
                                        s0[rows].double().numpy())
    got = torch.stack(outs, dim=2)[rows]
    eo, es = rel_err(f64(got), ref_o), rel_err(f64(state[rows]), ref_s)
    print(B, d, dv, f"o {eo:.2e} state {es:.2e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_decode_step_from_zero_is_one_position():
    """From a zero state a decode step is the one-position forward: o = (k . q) v."""
    x = inputs.make_random(3, 5, 1, 128, 64, dtype="bf16", seed=5, decay="heads", backward=False)
    q, k, v, dec = to_dev(x)
    state = torch.zeros((3, 5, 128, 64), dtype=torch.float32, device=DEV)
    o = la2.decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(), state, dec)
    ref = oracle.forward(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x))[:, :, 0]
    torch.cuda.synchronize()
    assert rel_err(f64(o), ref) <= 2e-2
    assert rel_err(f64(state), np.einsum("bhi,bhj->bhij", f64(x["k"])[:, :, 0], f64(x["v"])[:, :, 0])) <= 1e-6


# ---- backward from carried states ----------------------------------------------------------------

BCASES = [
    # (B, H, T, d, dv, dtype, block, decay)
    (1, 2, 777, 128, 128, "bf16", 128, "heads"),      # fused dk/dv, split chains, ragged last tile
    (2, 3, 700, 64, 128, "bf16", 64, "heads"),        # separate reverse scans (d != d_v), split
    (16, 16, 200, 128, 128, "bf16", 128, "heads"),    # 256 chains: unsplit, states read directly
    (1, 3, 333, 128, 64, "bf16", 128, "none"),
    (2, 2, 64, 128, 128, "bf16", 64, "heads"),        # one fused tile: the only tile carries the gradient
    (1, 1, 50, 64, 64, "bf16", 64, "heads"),          # one ragged tile
    (1, 2, 300, 64, 64, "f32", 32, "heads"),
    (16, 16, 70, 64, 64, "f32", 64, "heads"),         # fp32, unsplit
]


def check_backward_state(B, H, T, d, dv, dtype, block, decay, seed, with_in=True, with_out=True):
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=seed, decay=decay, backward=True)
    q, k, v, dec = to_dev(x)
    do = x["do"].to(DEV)
    s_in = seeded_state(B, H, d, dv, seed + 1) if with_in else None
    g_out = seeded_state(B, H, d, dv, seed + 2) if with_out else None
    dq, dk, dv_, ds_in = la2.backward_state(q, k, v, do, dec, block,
                                            None if s_in is None else s_in.to(DEV),
                                            None if g_out is None else g_out.to(DEV))
    ref = oracle.backward_state(*(f64(x[n]) for n in ("q", "k", "v", "do")), lam_of(x),
                                None if s_in is None else f64(s_in), None if g_out is None else f64(g_out))
    torch.cuda.synchronize()
    errs = [rel_err(f64(g), r) for g, r in zip((dq, dk, dv_, ds_in), ref)]
    print((B, H, T, d, dv, dtype, block, decay, with_in, with_out), " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= TOL[dtype], errs


@pytest.mark.parametrize("case", BCASES, ids=lambda c: f"B{c[0]}H{c[1]}T{c[2]}d{c[3]}dv{c[4]}{c[5]}tb{c[6]}{c[7]}")
def test_backward_state_matches_oracle(case):
    check_backward_state(*case, seed=301 + case[2])


@pytest.mark.parametrize("with_in,with_out", [(True, False), (False, True), (False, False)])
def test_backward_state_partial(with_in, with_out):
    check_backward_state(1, 3, 500, 128, 128, "bf16", 128, "heads", 17, with_in, with_out)
    check_backward_state(1, 3, 500, 64, 128, "bf16", 64, "heads", 19, with_in, with_out)


@pytest.mark.parametrize("plan", [{"seg_tiles": 2}, {"seg_tiles": 4, "state_sub": 2},
                                  {"separate_dkdv": True, "seg_tiles": 3}, {"slice_width": 64, "seg_tiles": 2}],
                         ids=lambda e: ",".join(f"{k}={v}" for k, v in e.items()))
def test_backward_state_plans(plan):
    with binding.plan_override(**plan):
        check_backward_state(1, 2, 777, 128, 128, "bf16", 128, "heads", 23)
        check_backward_state(1, 2, 601, 64, 64, "f32", 32, "heads", 29)


@pytest.mark.parametrize("dtype,d,block", [("bf16", 128, 128), ("bf16", 64, 64), ("f32", 64, 32)])
def test_chunked_training(dtype, d, block):
    """One sequence trained in uneven chunks: forwards carried through the states, backwards in
    reverse order with each chunk's d(state_in) passed to the previous chunk as d(state_out); the
    chunk gradients together equal the oracle's whole-sequence ones."""
    B, H, T = 1, 4, 1000
    x = inputs.make_random(B, H, T, d, d, dtype=dtype, seed=83, decay="heads", backward=True)
    q, k, v, dec = to_dev(x)
    do = x["do"].to(DEV)
    G = seeded_state(B, H, d, d, 89)
    cuts = [0, 300, 301, 751, 1000]
    states = [None]
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = slice(a, b)
        _, s_next = la2.forward_state(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(),
                                      dec, block, state_in=states[-1])
        states.append(s_next)
    grads, g_out = [], G.to(DEV)
    for c in range(len(cuts) - 2, -1, -1):
        sl = slice(cuts[c], cuts[c + 1])
        dq, dk, dv_, g_out = la2.backward_state(*(t[:, :, sl].contiguous() for t in (q, k, v, do)), dec, block,
                                                states[c], g_out)
        grads.append((dq, dk, dv_))
    grads.reverse()
    ref = oracle.backward_state(*(f64(x[n]) for n in ("q", "k", "v", "do")), lam_of(x), None, f64(G))
    torch.cuda.synchronize()
    for i in range(3):
        got = torch.cat([g[i] for g in grads], dim=2)
        assert rel_err(f64(got), ref[i]) <= TOL[dtype], i
    assert rel_err(f64(g_out), ref[3]) <= TOL[dtype]


def test_autograd_chunked_training_matches_whole():
    """lightning_attention_state in PyTorch autograd: a loss over a sequence run in two chunks (the
    second from the first's state, through which gradients flow) gives the whole run's gradients."""
    x = inputs.make_random(1, 3, 600, 128, 128, dtype="bf16", seed=97, decay="heads", backward=True)
    dec = x["decay"].to(DEV)
    do = x["do"].to(DEV)
    G = seeded_state(1, 3, 128, 128, 98).to(DEV)

    def grads(cut):
        q, k, v = (x[n].to(DEV).requires_grad_(True) for n in ("q", "k", "v"))
        if cut is None:
            o, s = la2.lightning_attention_state(q, k, v, None, dec, 128)
        else:
            sl1, sl2 = slice(0, cut), slice(cut, 600)
            o1, s1 = la2.lightning_attention_state(q[:, :, sl1], k[:, :, sl1], v[:, :, sl1], None, dec, 128)
            o2, s = la2.lightning_attention_state(q[:, :, sl2], k[:, :, sl2], v[:, :, sl2], s1, dec, 128)
            o = torch.cat([o1, o2], dim=2)
        loss = (o.float() * do.float()).sum() + (s * G).sum()
        loss.backward()
        return q.grad, k.grad, v.grad

    whole = grads(None)
    chunked = grads(257)
    torch.cuda.synchronize()
    ref = oracle.backward_state(*(f64(x[n]) for n in ("q", "k", "v", "do")), lam_of(x), None, f64(G))
    for a, b, r in zip(whole, chunked, ref):
        assert rel_err(f64(a), r) <= 2e-2 and rel_err(f64(b), r) <= 2e-2
