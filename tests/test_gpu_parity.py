"""HIP path vs the CPU oracle, through the C ABI.

Bars (max|gpu - ref| / max|ref| over each output tensor): 1e-5 for fp32 inputs,
2e-2 for bf16 inputs.  Every case compares every output element with the
whole-sequence oracle: small shapes that span several tiles with ragged tails,
and the named workloads at full size in the benchmark's launch configuration
(the oracle run chain by chain).
"""
import os

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


def run_gpu(x, block, backward=True):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    decay = None if x["decay"] is None else x["decay"].to(DEV)
    o = la2.forward(q, k, v, decay, block=block)
    out = {"o": o}
    if backward:
        out["dq"], out["dk"], out["dv"] = la2.backward(q, k, v, x["do"].to(DEV), decay, block=block)
    torch.cuda.synchronize()
    return out


def check_full(x, block, backward=True, tol=None):
    w = x["workload"]
    tol = tol or TOL[w.dtype]
    got = run_gpu(x, block, backward)
    lam = lam_of(x)
    args = [f64(x[n]) for n in ("q", "k", "v")]
    errs = {"o": rel_err(f64(got["o"]), oracle.forward(*args, lam))}
    if backward:
        ref = oracle.backward(*args, f64(x["do"]), lam)
        for n, r in zip(("dq", "dk", "dv"), ref):
            errs[n] = rel_err(f64(got[n]), r)
    print(w.name, block, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{w.name} T_B={block} {n}: {e:.3e} > {tol}"
    return got


SMALL = [
    # (B, H, T, d, dv, dtype, block, decay)
    (2, 3, 1000, 64, 64, "bf16", 64, "heads"),
    (2, 3, 1000, 128, 128, "bf16", 128, "heads"),
    (1, 2, 777, 128, 64, "bf16", 256, "heads"),
    (1, 2, 500, 64, 128, "bf16", 128, "none"),
    (1, 1, 4096, 128, 128, "bf16", 128, 0.999),
    (2, 2, 300, 128, 128, "f32", 64, "heads"),
    (1, 3, 257, 64, 64, "f32", 16, "heads"),
    (1, 2, 200, 128, 64, "f32", 32, 0.5),
    (1, 2, 333, 64, 128, "f32", 64, "none"),
]


@pytest.mark.parametrize("B,H,T,d,dv,dtype,block,decay", SMALL, ids=lambda v: str(v))
def test_small_shapes(B, H, T, d, dv, dtype, block, decay):
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=B * 1000 + T, decay=decay)
    check_full(x, block)


def test_many_chains_no_split():
    # 272 chains fill the GPU, so every chain runs as one segment (no workspace)
    x = inputs.make_random(16, 17, 200, 64, 64, dtype="bf16", seed=5, decay="heads")
    assert la2.la2_workspace_bytes(16, 17, 200, 64, 64, 64, torch.bfloat16, True) == 0
    check_full(x, 64)


@pytest.mark.parametrize("seg_tiles", [1, 2, 3])
def test_forced_segments(seg_tiles):
    x = inputs.make_random(1, 2, 700, 128, 128, dtype="bf16", seed=9, decay="heads")
    with binding.plan_override(seg_tiles=seg_tiles):
        check_full(x, 64)


@pytest.mark.parametrize("T,d,dtype,block,seg_tiles,sub", [
    (700, 128, "bf16", 64, 4, 2),     # 11 tiles: 3 segments of 2 state pieces, last piece 1 tile
    (700, 128, "bf16", 64, 4, 4),     # pieces of one tile
    (1000, 128, "bf16", 128, 4, 4),   # 128-position tiles (the fused dk/dv pass keeps 64)
    (520, 64, "bf16", 64, 4, 2),      # last segment one piece of one tile
    (300, 64, "f32", 32, 4, 2),
])
def test_state_sub_segments(T, d, dtype, block, seg_tiles, sub):
    """State-only passes over finer pieces than the output segments (start states read from the
    first piece forward, the last piece reverse), forward + backward against the oracle, and the
    saved-state backward bitwise equal to the recomputing one."""
    x = inputs.make_random(1, 3, T, d, d, dtype=dtype, seed=61 + T, decay="heads")
    with binding.plan_override(seg_tiles=seg_tiles, state_sub=sub):
        check_full(x, block)
        q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
        decay = x["decay"].to(DEV)
        ws = la2.workspace_for(q, v, block, True)
        o = torch.empty_like(v)
        la2.la2_forward(q, k, v, decay, o, block, ws)
        g = tuple(torch.empty_like(t) for t in (q, k, v))
        la2.la2_backward_saved(q, k, v, decay, do, *g, block, ws)
        ref = la2.backward(q, k, v, do, decay, block)
        torch.cuda.synchronize()
    for a, r in zip(g, ref):
        assert torch.equal(a, r)


@pytest.mark.parametrize("B,H,T,seg_tiles", [(1, 8, 700, 0), (1, 3, 300, 0), (1, 2, 700, 2), (1, 8, 520, 3)])
@pytest.mark.parametrize("decay", ["heads", "none"])
def test_narrow_value_slices(B, H, T, seg_tiles, decay):
    """128-wide values run as two 64-wide slices, with (8 chains) and without (3 chains) the
    XCD-grouped block order, alone and combined with T segments."""
    x = inputs.make_random(B, H, T, 128, 128, dtype="bf16", seed=23 + T, decay=decay)
    with binding.plan_override(slice_width=64, seg_tiles=seg_tiles):
        check_full(x, 128)


@pytest.mark.parametrize("d,T,decay,seg_tiles", [(128, 700, "heads", 0), (64, 333, "none", 0),
                                                  (128, 520, "heads", 3)])
def test_separate_dkdv_scans(d, T, decay, seg_tiles):
    """The two separate reverse scans that the fused dk/dv pass replaces for d = d_v."""
    x = inputs.make_random(1, 3, T, d, d, dtype="bf16", seed=31 + T, decay=decay)
    with binding.plan_override(separate_dkdv=True, seg_tiles=seg_tiles):
        check_full(x, 128)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 191])
@pytest.mark.parametrize("seg_tiles", [1, 2])
def test_fused_dkdv_segments(T, seg_tiles):
    """Fused dk/dv pass with every split of T into 64-position segments, ragged last tile."""
    x = inputs.make_random(2, 2, T, 128, 128, dtype="bf16", seed=41 + T, decay="heads")
    with binding.plan_override(seg_tiles=seg_tiles):
        check_full(x, 128)


@pytest.mark.parametrize("B,H", [(4, 25), (8, 16)])
def test_narrow_slices_many_chains(B, H):
    """Narrow slices on 100 and 128 chains (8 x 16 chains: XCD-grouped block order)."""
    x = inputs.make_random(B, H, 200, 128, 128, dtype="bf16", seed=B * H, decay="heads")
    with binding.plan_override(slice_width=64):
        check_full(x, 128)


BLOCKS = (16, 32, 64, 128, 256)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,dv", [(64, 64), (128, 128)])
def test_tile_size_invariance(dtype, d, dv):
    """Every tile length a caller may ask for meets the bar against the oracle (the split into
    intra- and inter-tile parts is exact for any tile length), and the results agree with each
    other; ragged last tile (T = 650)."""
    x = inputs.make_random(1, 4, 650, d, dv, dtype=dtype, seed=17 + d, decay="heads")
    outs = [check_full(x, b) for b in BLOCKS]
    tol = TOL[dtype]
    for n in ("o", "dq", "dk", "dv"):
        for o in outs[1:]:
            assert rel_err(f64(o[n]), f64(outs[0][n])) <= 2 * tol


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 128, 129])
def test_edge_lengths(T):
    x = inputs.make_random(1, 2, T, 128, 128, dtype="bf16", seed=T, decay="heads")
    check_full(x, 64)
    xf = inputs.make_random(1, 2, T, 64, 64, dtype="f32", seed=T, decay="heads")
    check_full(xf, 32)


def test_zero_inputs_give_zero():
    x = inputs.make_random(1, 2, 300, 128, 128, dtype="bf16", seed=1, decay="heads")
    for n in ("q", "k", "v", "do"):
        x[n] = torch.zeros_like(x[n])
    got = run_gpu(x, 128)
    for n in ("o", "dq", "dk", "dv"):
        assert torch.count_nonzero(got[n]).item() == 0


def test_strong_decay():
    x = inputs.make_random(1, 2, 500, 64, 64, dtype="bf16", seed=3, decay=0.01)
    check_full(x, 128)


def test_causality_bitwise():
    x = inputs.make_random(1, 2, 400, 128, 128, dtype="bf16", seed=21, decay="heads")
    a = run_gpu(x, 128, backward=False)["o"]
    t = 201
    for n in ("k", "v"):
        y = dict(x)
        y[n] = x[n].clone()
        y[n][:, :, t] += 1.0
        b = run_gpu(y, 128, backward=False)["o"]
        assert torch.equal(a[:, :, :t], b[:, :, :t]), n
        assert not torch.equal(a[:, :, t:], b[:, :, t:]), n


def test_autograd_matches_backward():
    x = inputs.make_random(1, 2, 300, 64, 64, dtype="bf16", seed=4, decay="heads")
    q, k, v, do = (x[n].to(DEV).requires_grad_(n != "do") for n in ("q", "k", "v", "do"))
    decay = x["decay"].to(DEV)
    o = la2.lightning_attention(q, k, v, decay, 64)
    o.backward(do)
    dq, dk, dv = la2.backward(q.detach(), k.detach(), v.detach(), do, decay, 64)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)


@pytest.mark.parametrize("dtype,d,block", [("bf16", 128, 128), ("bf16", 64, 64), ("f32", 64, 32)])
def test_backward_saved_reuses_forward_states(dtype, d, block):
    """la2_backward_saved after la2_forward on split chains: twice in a row, bitwise equal to the
    plain backward (which recomputes the same segment states), and within the bar of the oracle."""
    x = inputs.make_random(1, 3, 700, d, d, dtype=dtype, seed=51, decay="heads")
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    decay = x["decay"].to(DEV)
    with binding.plan_override(seg_tiles=2):
        ws = la2.workspace_for(q, v, block, True)
        assert ws is not None
        o = torch.empty_like(v)
        la2.la2_forward(q, k, v, decay, o, block, ws)
        runs = []
        for _ in range(2):
            g = tuple(torch.empty_like(t) for t in (q, k, v))
            la2.la2_backward_saved(q, k, v, decay, do, *g, block, ws)
            runs.append(g)
        ref = la2.backward(q, k, v, do, decay, block)
        torch.cuda.synchronize()
    for g in runs:
        for a, r in zip(g, ref):
            assert torch.equal(a, r)
    lam = lam_of(x)
    want = oracle.backward(*(f64(x[n]) for n in ("q", "k", "v", "do")), lam)
    for a, r in zip(ref, want):
        assert rel_err(f64(a), r) <= TOL[dtype]


def test_stream_ordering_on_side_stream():
    x = inputs.make_random(1, 2, 512, 128, 128, dtype="bf16", seed=8, decay="heads")
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    decay = x["decay"].to(DEV)
    ref = la2.forward(q, k, v, decay, 128)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o = la2.forward(q, k, v, decay, 128)
    s.synchronize()
    assert torch.equal(o, ref)


# ---- the named workloads at full size --------------------------------------

def test_tiny_fp32_forward():
    x = inputs.make("tiny_fp32_fwd")
    check_full(x, x["workload"].block, backward=False)


def test_bf16_forward_t2k():
    x = inputs.make("bf16_fwd_t2k")
    check_full(x, x["workload"].block, backward=False)


def run_bench_config(x):
    """The benchmark's launch sequence for one training step: la2_forward, then la2_backward_saved on
    the same workspace (it reuses the segment start states the forward left there)."""
    w = x["workload"]
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    decay = None if x["decay"] is None else x["decay"].to(DEV)
    ws = la2.workspace_for(q, v, w.block, True)
    o = torch.empty_like(v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    la2.la2_forward(q, k, v, decay, o, w.block, ws)
    la2.la2_backward_saved(q, k, v, decay, do, dq, dk, dv, w.block, ws)
    torch.cuda.synchronize()
    out = {n: t.cpu() for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    del q, k, v, do, o, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return out


def check_whole(name, max_chain_tokens=1 << 21):
    """A named workload at full size in the benchmark's launch configuration, every output element
    compared with the oracle: the whole forward and backward token recurrences run chain by chain
    (groups of chains whose total length is at most ``max_chain_tokens``, to bound host memory),
    and max|err| / max|ref| is taken over each whole output tensor."""
    x = inputs.make(name)
    w = x["workload"]
    print(f"[{name}] B={w.B} H={w.H} T={w.T} d={w.d} block={w.block} decay={w.decay}", flush=True)
    got = run_bench_config(x)
    lam = lam_of(x)
    chains = w.B * w.H
    per = max(1, min(chains, max_chain_tokens // w.T))
    flat = {n: x[n].reshape(chains, 1, w.T, -1) for n in ("q", "k", "v", "do")}
    gflat = {n: got[n].reshape(chains, w.T, -1) for n in got}
    lams = None if lam is None else np.tile(lam, w.B)
    max_err = {n: 0.0 for n in got}
    max_ref = {n: 0.0 for n in got}
    for c0 in range(0, chains, per):
        c1 = min(chains, c0 + per)
        a = [f64(flat[n][c0:c1]).reshape(1, c1 - c0, w.T, -1) for n in ("q", "k", "v", "do")]
        lc = None if lams is None else lams[c0:c1]
        refs = {"o": oracle.forward(*a[:3], lc)}
        refs["dq"], refs["dk"], refs["dv"] = oracle.backward(*a, lc)
        for n, r in refs.items():
            r = r.reshape(c1 - c0, w.T, -1)
            max_err[n] = max(max_err[n], float(np.max(np.abs(f64(gflat[n][c0:c1]) - r))))
            max_ref[n] = max(max_ref[n], float(np.max(np.abs(r))))
        del a, refs
        print(f"[{name}] chains {c0}..{c1 - 1} compared", flush=True)
    for n in got:
        e = max_err[n] / max_ref[n]
        print(f"{name} {n}: max|err|/max|ref| = {e:.3e} over all {chains} chains x {w.T} rows "
              f"(max|ref| {max_ref[n]:.3e})", flush=True)
        assert e <= TOL[w.dtype], f"{name} {n}: {e:.3e}"


@pytest.mark.timeout(600)
def test_tnl15b_layer_whole():
    check_whole("tnl15b_layer")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", inputs.SWEEP_NAMES)
def test_length_sweep_whole(name):
    check_whole(name)


@pytest.mark.timeout(900)
def test_long_context_outliers_whole():
    check_whole("long128k_outliers")
