"""Normalized forward (numerator over denominator, feature map phi) on the GPU, through the C ABI,
against the oracle's ``forward_normalized`` (pinned by the masked-product ratio, weights that sum
to one, the running value range and the map's values).

Bars as for the plain forward: max|gpu - ref| / max|ref| <= 1e-5 for fp32 inputs, <= 2e-2 for
bf16 inputs.  With phi = elu + 1 every weight is positive, so the denominator is well away from 0;
the identity map is tested on inputs made positive (|x| + 0.1), where the same holds.
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


def positive(t):
    """|x| + 0.1, rounded to the tensor's own dtype (both sides read the rounded values)."""
    return (t.float().abs() + 0.1).to(t.dtype)


def run_case(B, H, T, d, dv, dtype, block, decay, fmap, seed):
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=seed, decay=decay, backward=False)
    if fmap == "identity":
        x["q"], x["k"] = positive(x["q"]), positive(x["k"])
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    o = la2.forward_normalized(q, k, v, dec, block, fmap)
    ref = oracle.forward_normalized(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x), fmap)
    torch.cuda.synchronize()
    err = rel_err(f64(o), ref)
    print((B, H, T, d, dv, dtype, block, decay, fmap), f"{err:.2e}", flush=True)
    assert np.isfinite(f64(o)).all()
    assert err <= TOL[dtype], err
    return o


CASES = [
    # (B, H, T, d, dv, dtype, block, decay, fmap)
    (2, 3, 333, 128, 128, "bf16", 128, "heads", "elu1"),    # split numerator and denominator, ragged tail
    (1, 2, 1000, 64, 128, "bf16", 64, "heads", "elu1"),
    (16, 16, 200, 128, 64, "bf16", 128, "none", "elu1"),   # 256 chains: nothing split
    (1, 3, 777, 64, 64, "f32", 32, "heads", "elu1"),
    (2, 2, 300, 128, 128, "f32", 64, "none", "identity"),
    (1, 4, 513, 128, 128, "bf16", 256, "heads", "identity"),
    (3, 1, 1, 64, 64, "bf16", 64, "heads", "elu1"),        # one position: o = v
    (2, 2, 65, 128, 64, "f32", 16, 0.5, "elu1"),           # strong decay
] + [
    # bf16, d = d_v = 128, no decay, chains the plan leaves unsplit: one fused launch (phi on the tiles)
    (4, 64, 300, 128, 128, "bf16", 128, "none", "elu1"),   # ragged last tile
    (16, 16, 1, 128, 128, "bf16", 128, "none", "elu1"),    # one position: o = v
    (2, 128, 130, 128, 128, "bf16", 64, "none", "identity"),
    (1, 256, 64, 128, 128, "bf16", 256, "none", "elu1"),   # one whole tile
    (2, 128, 65, 128, 128, "bf16", 64, "none", "elu1"),    # two tiles, the second with one real row
    (1, 256, 129, 128, 128, "bf16", 128, "none", "elu1"),  # three tiles: k loaded two tiles ahead
]
FUSED = CASES[-6:]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_normalized_matches_oracle(case):
    run_case(*case, seed=101 + case[2])


@pytest.mark.parametrize("seg", [64, 128, 320])
def test_normalized_forced_segments(seg):
    """Denominator segments of a forced length: the segment sums chained across up to 16 segments."""
    with binding.plan_override(norm_segment=seg):
        run_case(1, 2, 1000, 128, 128, "bf16", 128, "heads", "elu1", seed=7)
        run_case(1, 2, 1000, 64, 64, "f32", 64, "heads", "elu1", seed=8)


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "-".join(str(v) for v in c))
def test_fused_normalized_against_two_pass(case):
    """The fused launch against the denominator pass + numerator scan it replaces (forced through the
    test build): both within the bar of the oracle and of each other (their denominators differ in
    rounding: phi in bf16 against phi in fp32); and with the backward-sized workspace, where it also
    writes phi(q), phi(k) and the denominators, bitwise the same o."""
    B, H, T, d, dv, dtype, block, decay, fmap = case
    o = run_case(*case, seed=211 + T)
    with binding.plan_override(legacy_forward=True):
        o_old = run_case(*case, seed=211 + T)
    d_ = rel_err(f64(o), f64(o_old))
    print(case, f"fused vs two passes {d_:.2e}", flush=True)
    assert d_ <= TOL[dtype]
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=211 + T, decay=decay, backward=False)
    if fmap == "identity":
        x["q"], x["k"] = positive(x["q"]), positive(x["k"])
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    ws = la2.normalized_workspace_for(q, v, fmap, block, backward=True)
    o_ws = la2.forward_normalized(q, k, v, None, block, fmap, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_ws, o)


def test_normalized_ones_values_give_ones():
    """v = 1 everywhere: every output is exactly a weighted average of ones."""
    x = inputs.make_random(2, 4, 700, 128, 128, dtype="bf16", seed=3, decay="heads", backward=False)
    q, k = x["q"].to(DEV), x["k"].to(DEV)
    v = torch.ones((2, 4, 700, 128), dtype=torch.bfloat16, device=DEV)
    o = la2.forward_normalized(q, k, v, x["decay"].to(DEV), 128, "elu1")
    torch.cuda.synchronize()
    assert float((o.float() - 1.0).abs().max()) <= 2e-2


def test_normalized_full_size_whole():
    """The 1K-position length-sweep workload (128 x 16 chains, d = d_v = 128, bf16) with elu + 1,
    at full size in one launch, every output element against the oracle."""
    x = inputs.make("sweep131k_t1k")
    w = x["workload"]
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    o = la2.forward_normalized(q, k, v, dec, w.block, "elu1")
    torch.cuda.synchronize()
    ref = oracle.forward_normalized(*(f64(x[n]) for n in ("q", "k", "v")), lam_of(x), "elu1")
    err = rel_err(f64(o), ref)
    print(f"{w.name} normalized forward, all {w.B * w.H} chains: max|err|/max|ref| = {err:.2e}", flush=True)
    assert err <= TOL["bf16"]


# ---- backward ----------------------------------------------------------------------------------
#
# The bar is the one of every case: max|gpu - ref| <= 2e-2 x max|ref| (bf16), 1e-5 x max|ref| (fp32),
# per gradient.  dq and dk are d pq = S dn + dden z and d pk = R v + y (times phi'), and for the
# gradient of a ratio the two terms largely cancel (the exact dq of a one-position sequence is 0
# while each term is O(1); on random inputs the numerator term is 6-20x dq).  The bf16 dq is
# therefore computed from phi(k) = m + kap with m the chain's mean of phi(k) (la2_norm.hip, mode 7):
# only the scan over the small kap runs on bf16 MFMA operands, and the terms that cancel are formed
# in fp32.  dk's terms cancel by about 2x and keep the plain path.


def check_grads(case, got, ref, terms=None):
    dtype = case[5]
    if case[2] == 1 and terms is not None:
        # one position: dq and dk are exactly 0 (o = v_0 whatever q and k), so only an absolute bound
        # means anything; it is taken relative to the two O(1) terms that cancel
        for name, g, t in zip(("dq", "dk"), got[:2], terms):
            a, scale = float(np.max(np.abs(f64(g)))), float(np.max(np.abs(t)))
            print(case, name, f"max|gpu| {a:.2e} against terms of {scale:.2e}", flush=True)
            assert a <= TOL[dtype] * scale, (name, a, scale)
        assert rel_err(f64(got[2]), ref[2]) <= TOL[dtype]
        return
    errs = [rel_err(f64(g), r) for g, r in zip(got, ref)]
    ratio = "" if terms is None else " numerator term / ref: " + " ".join(
        f"{float(np.max(np.abs(t))) / float(np.max(np.abs(r))):.1f}" for t, r in zip(terms, ref[:2]))
    print(case, "dq dk dv max|err|/max|ref|", " ".join(f"{e:.2e}" for e in errs) + ratio, flush=True)
    for g in got:
        assert np.isfinite(f64(g)).all()
    tol = TOL[dtype]
    if dtype == "f32":
        assert max(errs) <= tol, errs
        return
    for name, e in zip(("dq", "dk", "dv"), errs):
        assert e <= tol, (name, e)


def numerator_terms(x, fmap):
    """(d pq, d pk) of the numerator alone: the oracle's plain backward on phi(q), phi(k), v with the
    normalized output's gradient dn = do / den (fp64)."""
    q, k, v, do = (f64(x[n]) for n in ("q", "k", "v", "do"))
    phi = (lambda a: np.where(a > 0, a + 1.0, np.exp(np.minimum(a, 0.0)))) if fmap == "elu1" else (lambda a: a)
    pq, pk = phi(q), phi(k)
    lam = lam_of(x)
    ones = np.ones_like(v[..., :1])
    den = oracle.forward(pq, pk, np.repeat(ones, 64, axis=-1), lam)[..., :1]   # z_t . phi(q_t)
    dq_n, dk_n, _ = oracle.backward(pq, pk, v, do / den, lam)
    return dq_n, dk_n

BN_CASES = [
    # (B, H, T, d, dv, dtype, block, decay, fmap)
    (2, 3, 333, 128, 128, "bf16", 128, "heads", "elu1"),    # split numerator and denominator, ragged tail
    (1, 2, 1000, 64, 128, "bf16", 64, "heads", "elu1"),     # d != d_v: separate reverse scans
    (16, 16, 200, 128, 64, "bf16", 128, "none", "elu1"),   # 256 chains: nothing split
    (1, 3, 777, 64, 64, "f32", 32, "heads", "elu1"),
    (2, 2, 300, 128, 128, "f32", 64, "none", "identity"),
    (1, 4, 513, 128, 128, "bf16", 256, "heads", "identity"),
    (3, 1, 1, 64, 64, "bf16", 64, "heads", "elu1"),        # one position
    (2, 2, 65, 128, 64, "f32", 16, 0.5, "elu1"),           # strong decay
    (4, 64, 300, 128, 128, "bf16", 128, "none", "elu1"),   # the fused forward's phi and denominators
    (2, 128, 130, 128, 128, "bf16", 64, "none", "identity"),
]


def run_backward_case(B, H, T, d, dv, dtype, block, decay, fmap, seed):
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=seed, decay=decay, backward=True)
    if fmap == "identity":
        x["q"], x["k"] = positive(x["q"]), positive(x["k"])
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    o = la2.forward_normalized(q, k, v, dec, block, fmap)
    dq, dk, dv_ = la2.backward_normalized(q, k, v, o, do, dec, block, fmap)
    ref = oracle.backward_normalized(*(f64(x[n]) for n in ("q", "k", "v", "do")), lam_of(x), fmap)
    torch.cuda.synchronize()
    check_grads((B, H, T, d, dv, dtype, block, decay, fmap), (dq, dk, dv_), ref,
                numerator_terms(x, fmap) if dtype == "bf16" else None)


@pytest.mark.parametrize("case", BN_CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_backward_normalized_matches_oracle(case):
    run_backward_case(*case, seed=401 + case[2])


@pytest.mark.parametrize("fmap,T", [("elu1", 200), ("elu1", 65), ("identity", 130)])
def test_normalized_dk_in_the_walk(fmap, T):
    """bf16, d = d_v = 128, no decay, unsplit chains: the dK/dV walk takes the denominator's part of dk
    and the feature map's derivative on board (dk rounded once).  Against the oracle, and against the
    separate reverse scan over dden phi(q) it replaces (the walk forced off through the test build)."""
    x = inputs.make_random(2, 128, T, 128, 128, dtype="bf16", seed=707 + T, decay="none", backward=True)
    if fmap == "identity":
        x["q"], x["k"] = positive(x["q"]), positive(x["k"])
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o = la2.forward_normalized(q, k, v, None, 128, fmap)
    dq, dk, dv_ = la2.backward_normalized(q, k, v, o, do, None, 128, fmap)
    with binding.plan_override(legacy_dkdv=True):
        dq_s, dk_s, dv_s = la2.backward_normalized(q, k, v, o, do, None, 128, fmap)
    torch.cuda.synchronize()
    ref = oracle.backward_normalized(*(f64(x[n]) for n in ("q", "k", "v", "do")), None, fmap)
    e_walk, e_scan = rel_err(f64(dk), ref[1]), rel_err(f64(dk_s), ref[1])
    print(fmap, T, f"dk max|err|/max|ref|: in the walk {e_walk:.2e}, separate scan {e_scan:.2e}", flush=True)
    assert e_walk <= TOL["bf16"] and rel_err(f64(dk), f64(dk_s)) <= TOL["bf16"]
    assert torch.equal(dq, dq_s)
    for g, r in ((dq, ref[0]), (dv_, ref[2])):
        assert rel_err(f64(g), r) <= TOL["bf16"]


@pytest.mark.parametrize("seg", [64, 128, 320])
def test_backward_normalized_forced_segments(seg):
    """Denominator scans over forced segments: forward and reverse carries across up to 16 segments,
    the reverse walk over a ragged last segment."""
    with binding.plan_override(norm_segment=seg):
        run_backward_case(1, 2, 1000, 64, 64, "f32", 64, "heads", "elu1", seed=12)
        run_backward_case(1, 2, 1000, 128, 128, "bf16", 128, "heads", "elu1", seed=11)


# ---- backward reusing the forward's workspace ----------------------------------------------------

SAVED_CASES = [
    # (B, H, T, d, dv, dtype, block, decay, fmap)
    (2, 3, 333, 128, 128, "bf16", 128, "heads", "elu1"),    # split numerator and denominator, ragged tail
    (16, 16, 200, 128, 64, "bf16", 128, "none", "elu1"),   # 256 chains: nothing split
    (1, 3, 777, 64, 64, "f32", 32, "heads", "elu1"),
    (1, 4, 513, 128, 128, "bf16", 256, "heads", "identity"),
    (4, 64, 300, 128, 128, "bf16", 128, "none", "elu1"),   # phi(q), phi(k), den from the fused forward
    (2, 128, 130, 128, 128, "bf16", 64, "none", "identity"),
]


@pytest.mark.parametrize("case", SAVED_CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_backward_normalized_saved(case):
    """la2_backward_normalized_saved after la2_forward_normalized on the backward-sized workspace:
    bitwise the gradients of la2_backward_normalized (which recomputes the denominators, phi and
    the numerator's segment states the saved call reads), twice in a row on the same workspace
    (nothing the forward left there is overwritten), and within the oracle's bar."""
    B, H, T, d, dv, dtype, block, decay, fmap = case
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=601 + T, decay=decay, backward=True)
    if fmap == "identity":
        x["q"], x["k"] = positive(x["q"]), positive(x["k"])
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    ws = la2.normalized_workspace_for(q, v, fmap, block, backward=True)
    o = la2.forward_normalized(q, k, v, dec, block, fmap, workspace=ws)
    ref = la2.backward_normalized(q, k, v, o, do, dec, block, fmap)
    for rep in range(2):
        got = la2.backward_normalized(q, k, v, o, do, dec, block, fmap, workspace=ws, saved=True)
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), (rep, name)
    oref = oracle.backward_normalized(*(f64(x[n]) for n in ("q", "k", "v", "do")), lam_of(x), fmap)
    check_grads(case, got, oref)
