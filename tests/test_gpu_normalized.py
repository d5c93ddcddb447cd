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
from causal_linear_attention_amd import inputs
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
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_normalized_matches_oracle(case):
    run_case(*case, seed=101 + case[2])


@pytest.mark.parametrize("seg", ["64", "128", "320"])
def test_normalized_forced_segments(seg, monkeypatch):
    """Denominator segments of a forced length: the segment sums chained across up to 16 segments."""
    monkeypatch.setenv("LA2_NORM_SEGMENT", seg)
    run_case(1, 2, 1000, 128, 128, "bf16", 128, "heads", "elu1", seed=7)
    run_case(1, 2, 1000, 64, 64, "f32", 64, "heads", "elu1", seed=8)


def test_normalized_ones_values_give_ones():
    """v = 1 everywhere: every output is exactly a weighted average of ones."""
    x = inputs.make_random(2, 4, 700, 128, 128, dtype="bf16", seed=3, decay="heads", backward=False)
    q, k = x["q"].to(DEV), x["k"].to(DEV)
    v = torch.ones((2, 4, 700, 128), dtype=torch.bfloat16, device=DEV)
    o = la2.forward_normalized(q, k, v, x["decay"].to(DEV), 128, "elu1")
    torch.cuda.synchronize()
    assert float((o.float() - 1.0).abs().max()) <= 2e-2


def test_normalized_full_size_sampled():
    """The 1K-position length-sweep workload (128 x 16 chains, d = d_v = 128, bf16) with elu + 1,
    at full size in one launch; the oracle on sampled whole chains."""
    x = inputs.make("sweep131k_t1k")
    w = x["workload"]
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    o = la2.forward_normalized(q, k, v, dec, w.block, "elu1")
    torch.cuda.synchronize()
    lam = lam_of(x)
    for b, h in [(0, 0), (w.B - 1, 15), (w.B // 2, 7)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        lh = None if lam is None else lam[h:h + 1]
        ref = oracle.forward_normalized(*(f64(x[n][sl]) for n in ("q", "k", "v")), lh, "elu1")
        err = rel_err(f64(o[sl]), ref)
        print("chain", b, h, f"{err:.2e}", flush=True)
        assert err <= TOL["bf16"]


# ---- backward ----------------------------------------------------------------------------------
#
# The bar for dq and dk in bf16.  They are d pq = S dn + dden z and d pk = R v + y (times phi'), and
# for the gradient of a ratio the two terms largely cancel: the exact dq of a one-position sequence
# is 0 while each term is O(1).  On the bf16 path each term carries bf16 roundings of its own size
# (phi(q), phi(k), dn and the MFMA operand S in bf16, dq stored in bf16 before the second term is
# added), so the error is bounded relative to the terms, not to their difference.  The bar is
# therefore max|gpu - ref| <= 2e-2 x max(max|ref|, max|numerator term|), the numerator term being the
# plain backward of (phi(q), phi(k), v) for the output gradient dn = do / den (oracle, fp64).  dv has
# no such cancellation and keeps 2e-2 x max|ref|; fp32 keeps 1e-5 x max|ref| throughout.


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
    if dtype == "bf16":
        terms = numerator_terms(x, fmap)
        errs = [float(np.max(np.abs(f64(g) - r))) / max(float(np.max(np.abs(r))), float(np.max(np.abs(t))))
                for g, r, t in zip((dq, dk), ref[:2], terms)] + [rel_err(f64(dv_), ref[2])]
    else:
        errs = [rel_err(f64(g), r) for g, r in zip((dq, dk, dv_), ref)]
    print((B, H, T, d, dv, dtype, block, decay, fmap), " ".join(f"{e:.2e}" for e in errs), flush=True)
    for g in (dq, dk, dv_):
        assert np.isfinite(f64(g)).all()
    assert max(errs) <= TOL[dtype], errs


@pytest.mark.parametrize("case", BN_CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_backward_normalized_matches_oracle(case):
    run_backward_case(*case, seed=401 + case[2])


@pytest.mark.parametrize("seg", ["64", "128", "320"])
def test_backward_normalized_forced_segments(seg, monkeypatch):
    """Denominator scans over forced segments: forward and reverse carries across up to 16 segments,
    the reverse walk over a ragged last segment."""
    monkeypatch.setenv("LA2_NORM_SEGMENT", seg)
    run_backward_case(1, 2, 1000, 128, 128, "bf16", 128, "heads", "elu1", seed=11)
    run_backward_case(1, 2, 1000, 64, 64, "f32", 64, "heads", "elu1", seed=12)


# ---- backward reusing the forward's workspace ----------------------------------------------------

SAVED_CASES = [
    # (B, H, T, d, dv, dtype, block, decay, fmap)
    (2, 3, 333, 128, 128, "bf16", 128, "heads", "elu1"),    # split numerator and denominator, ragged tail
    (16, 16, 200, 128, 64, "bf16", 128, "none", "elu1"),   # 256 chains: nothing split
    (1, 3, 777, 64, 64, "f32", 32, "heads", "elu1"),
    (1, 4, 513, 128, 128, "bf16", 256, "heads", "identity"),
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
    if dtype == "bf16":
        terms = numerator_terms(x, fmap)
        errs = [float(np.max(np.abs(f64(g) - r))) / max(float(np.max(np.abs(r))), float(np.max(np.abs(t))))
                for g, r, t in zip(got[:2], oref[:2], terms)] + [rel_err(f64(got[2]), oref[2])]
    else:
        errs = [rel_err(f64(g), r) for g, r in zip(got, oref)]
    print(case, " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= TOL[dtype], errs
