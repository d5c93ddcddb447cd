"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each pin takes an ``oracle.Oracle`` (so the same pins can be run against
deliberately broken copies of the oracle) and raises AssertionError when the
oracle disagrees.  None of them re-types the oracle's recurrence: they use
brute-force masked products, closed forms, library routines (numpy.cumsum,
scipy.signal.lfilter, torch.autograd), finite differences, invariants and a
hand-worked example.
"""
import json
import os

import numpy as np
import scipy.signal
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

LAMS = (1.0, 0.9, 0.42)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max|err| = {err:.3e} (scale {scale:.3e})"


def _decay_matrix(T, lam):
    """D[t, s] = lam^(t-s) for s <= t else 0 (the causal mask M when lam = 1)."""
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    return np.where(s <= t, lam ** np.clip(t - s, 0, None).astype(np.float64), 0.0)


def brute_forward(q, k, v, lam):
    """O = (Q K^T (.) D_lam) V per chain -- the masked left product over the whole sequence."""
    B, H, T, _ = q.shape
    o = np.empty(q.shape[:-1] + (v.shape[-1],))
    for b in range(B):
        for h in range(H):
            D = _decay_matrix(T, lam[h])
            o[b, h] = ((q[b, h] @ k[b, h].T) * D) @ v[b, h]
    return o


def _setup(seed, B=1, H=3, T=37, d=5, dv=4):
    q, k, v, do = (_rand((B, H, T, n), seed + i) for i, n in enumerate((d, d, dv, dv)))
    lam = np.array([LAMS[h % len(LAMS)] for h in range(H)])
    return q, k, v, do, lam


# ---- pins ------------------------------------------------------------------

def pin_golden_handworked(orc):
    """Hand-worked T = 3, lam = 1/2 example (exact dyadic values)."""
    g = json.load(open(os.path.join(GOLDEN, "handworked_t3.json")))
    q, k, v, do = (np.array(g[n], dtype=np.float64)[None, None] for n in ("q", "k", "v", "do"))
    lam = np.array([g["lam"]])
    _close(orc.forward(q, k, v, lam)[0, 0], g["o"], 0.0, "golden o")
    dq, dk, dv = orc.backward(q, k, v, do, lam)
    _close(dq[0, 0], g["dq"], 0.0, "golden dq")
    _close(dk[0, 0], g["dk"], 0.0, "golden dk")
    _close(dv[0, 0], g["dv"], 0.0, "golden dv")


def pin_bruteforce_forward(orc):
    """Recurrence == (Q K^T (.) D_lam) V for lam in {1, 0.9, 0.42}; lam = 1 is the masked product M."""
    for T in (1, 5, 37, 64):
        q, k, v, _, lam = _setup(10 + T, T=T)
        _close(orc.forward(q, k, v, lam), brute_forward(q, k, v, lam), 1e-12, f"fwd T={T}")
    q, k, v, _, _ = _setup(3, H=2, T=50)
    _close(orc.forward(q, k, v, None), brute_forward(q, k, v, np.ones(2)), 1e-12, "fwd lam=None")


def pin_closed_form_ones(orc):
    """q = k = v = 1: o_t[j] = d (1 - lam^(t+1)) / (1 - lam), and d (t+1) at lam = 1."""
    T, d, dv = 40, 6, 3
    ones_q = np.ones((1, 3, T, d))
    ones_v = np.ones((1, 3, T, dv))
    lam = np.array([1.0, 0.9, 0.42])
    o = orc.forward(ones_q, ones_q, ones_v, lam)
    t = np.arange(T, dtype=np.float64)
    for h, l in enumerate(lam):
        ref = d * (t + 1) if l == 1.0 else d * (1 - l ** (t + 1)) / (1 - l)
        _close(o[0, h], np.repeat(ref[:, None], dv, 1), 1e-13, f"ones lam={l}")


def pin_cumsum_filter(orc):
    """q_t = k_s = e_1: o = cumsum(v) at lam = 1, and the first-order IIR filter y_t = lam y_{t-1} + v_t otherwise."""
    T, d, dv = 60, 4, 5
    e1 = np.zeros((1, 3, T, d))
    e1[..., 0] = 1.0
    v = _rand((1, 3, T, dv), 7)
    lam = np.array([1.0, 0.9, 0.42])
    o = orc.forward(e1, e1, v, lam)
    _close(o[0, 0], np.cumsum(v[0, 0], axis=0), 1e-13, "cumsum")
    for h in (1, 2):
        ref = scipy.signal.lfilter([1.0], [1.0, -lam[h]], v[0, h], axis=0)
        _close(o[0, h], ref, 1e-13, f"lfilter lam={lam[h]}")


def pin_tile_invariance(orc):
    """The tile decomposition gives the same result for every tile size, including a ragged last tile."""
    for T in (37, 100):
        q, k, v, do, lam = _setup(20 + T, T=T)
        ref_o = orc.forward(q, k, v, lam)
        ref_g = orc.backward(q, k, v, do, lam)
        for blk in (1, 2, 8, 16, 32, 64, 128):
            _close(orc.tiled_forward(q, k, v, lam, blk), ref_o, 1e-12, f"tiled fwd T={T} T_B={blk}")
            for a, b, n in zip(orc.tiled_backward(q, k, v, do, lam, blk), ref_g, ("dq", "dk", "dv")):
                _close(a, b, 1e-12, f"tiled {n} T={T} T_B={blk}")


def pin_causality(orc):
    """Changing row t of k or v leaves o_s (s < t) unchanged; a NaN at row t reaches exactly rows >= t."""
    q, k, v, _, lam = _setup(31, T=30)
    o = orc.forward(q, k, v, lam)
    t = 17
    k2 = k.copy()
    k2[:, :, t] += 1.0
    v2 = v.copy()
    v2[:, :, t] -= 2.0
    for kk, vv in ((k2, v), (k, v2)):
        o2 = orc.forward(q, kk, vv, lam)
        _close(o2[:, :, :t], o[:, :, :t], 0.0, "causal prefix")
        assert np.all(np.abs(o2[:, :, t:] - o[:, :, t:]).max(axis=-1) > 0), "rows >= t must change"
    vn = v.copy()
    vn[:, :, t] = np.nan
    on = orc.forward(q, k, vn, lam)
    assert np.all(np.isfinite(on[:, :, :t])) and np.all(np.isnan(on[:, :, t:])), "NaN reach"


def _loss(orc, q, k, v, do, lam):
    return float(np.sum(orc.forward(q, k, v, lam) * do))


def pin_finite_differences(orc):
    """Backward == central finite differences of L = <o, do> in fp64."""
    q, k, v, do, lam = _setup(41, B=1, H=3, T=11, d=3, dv=2)
    grads = orc.backward(q, k, v, do, lam)
    h = 1e-6
    for idx, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            xp = x.copy()
            xp[mi] += h
            xm = x.copy()
            xm[mi] -= h
            args = [q, k, v]
            args[idx] = xp
            lp = _loss(orc, *args, do, lam)
            args[idx] = xm
            lm = _loss(orc, *args, do, lam)
            num[mi] = (lp - lm) / (2 * h)
        _close(g, num, 1e-7, f"finite differences arg {idx}")


def pin_autograd(orc):
    """Backward == torch.autograd (float64) through the brute-force masked product."""
    q, k, v, do, lam = _setup(51, B=2, H=3, T=23, d=4, dv=6)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    T = q.shape[2]
    D = torch.stack([torch.tensor(_decay_matrix(T, l)) for l in lam])     # [H, T, T]
    o = torch.matmul(torch.matmul(tq, tk.transpose(-1, -2)) * D, tv)
    o.backward(torch.tensor(do))
    dq, dk, dv = orc.backward(q, k, v, do, lam)
    _close(dq, tq.grad.numpy(), 1e-12, "autograd dq")
    _close(dk, tk.grad.numpy(), 1e-12, "autograd dk")
    _close(dv, tv.grad.numpy(), 1e-12, "autograd dv")


def pin_inner_products(orc):
    """o is linear in each of q, k, v, so <Q, dQ> = <K, dK> = <V, dV> = <O, dO>."""
    q, k, v, do, lam = _setup(61, B=2, H=3, T=45, d=7, dv=5)
    o = orc.forward(q, k, v, lam)
    dq, dk, dv = orc.backward(q, k, v, do, lam)
    ref = float(np.sum(o * do))
    for x, g, n in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        got = float(np.sum(x * g))
        assert abs(got - ref) <= 1e-11 * max(1.0, abs(ref)), f"<{n}, d{n}> = {got} vs {ref}"


def pin_backward_as_forward(orc):
    """dQ = LA(dO, V, K); dK and dV are the same attention run backwards in time."""
    q, k, v, do, lam = _setup(71, B=1, H=3, T=33, d=4, dv=6)
    dq, dk, dv = orc.backward(q, k, v, do, lam)
    f = lambda x: x[:, :, ::-1].copy()
    _close(dq, orc.forward(do, v, k, lam), 1e-12, "dq identity")
    _close(dk, f(orc.forward(f(v), f(do), f(q), lam)), 1e-12, "dk identity")
    _close(dv, f(orc.forward(f(k), f(q), f(do), lam)), 1e-12, "dv identity")


def pin_linearity_and_heads(orc):
    """o is linear in v, and chains are independent: permuting heads with their decays permutes outputs."""
    q, k, v, _, lam = _setup(81, B=2, H=3, T=29)
    v2 = _rand(v.shape, 82)
    a, b = 0.75, -1.5
    _close(orc.forward(q, k, a * v + b * v2, lam),
           a * orc.forward(q, k, v, lam) + b * orc.forward(q, k, v2, lam), 1e-12, "linearity")
    perm = [2, 0, 1]
    _close(orc.forward(q[:, perm], k[:, perm], v[:, perm], lam[perm]),
           orc.forward(q, k, v, lam)[:, perm], 0.0, "head permutation")


def pin_rows(orc):
    """Single rows from the closed sums equal the matching rows of the brute-force product."""
    q, k, v, do, lam = _setup(91, B=1, H=3, T=41, d=5, dv=3)
    rows = np.array([0, 1, 17, 39, 40])
    o = brute_forward(q, k, v, lam)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    D = torch.stack([torch.tensor(_decay_matrix(q.shape[2], l)) for l in lam])
    torch.matmul(torch.matmul(tq, tk.transpose(-1, -2)) * D, tv).backward(torch.tensor(do))
    for h in range(3):
        _close(orc.forward_rows(q[0, h], k[0, h], v[0, h], lam[h], rows), o[0, h, rows], 1e-12, "rows o")
        gq, gk, gv = orc.backward_rows(q[0, h], k[0, h], v[0, h], do[0, h], lam[h], rows)
        _close(gq, tq.grad[0, h, rows].numpy(), 1e-12, "rows dq")
        _close(gk, tk.grad[0, h, rows].numpy(), 1e-12, "rows dk")
        _close(gv, tv.grad[0, h, rows].numpy(), 1e-12, "rows dv")


def pin_state_closed_form(orc):
    """With a carried-in state S_in the outputs and the final state have closed forms:
    o_t = lam^(t+1) S_in^T q_t + (brute-force row t) and S_out = lam^T S_in + sum_s lam^(T-1-s) k_s v_s^T
    (weights built with numpy powers, the sum with einsum)."""
    B, H, T, d, dv = 2, 3, 23, 5, 4
    q, k, v, _, lam = _setup(101, B=B, H=H, T=T, d=d, dv=dv)
    s_in = _rand((B, H, d, dv), 107)
    o, s_out = orc.forward_state(q, k, v, lam, s_in)
    base = brute_forward(q, k, v, lam)
    t = np.arange(T)
    for h in range(H):
        carry = (lam[h] ** (t + 1))[None, :, None] * np.einsum("bij,bti->btj", s_in[:, h], q[:, h])
        _close(o[:, h], base[:, h] + carry, 1e-12, "o with state_in")
        w = lam[h] ** (T - 1 - t)
        want = lam[h] ** T * s_in[:, h] + np.einsum("t,bti,btj->bij", w, k[:, h], v[:, h])
        _close(s_out[:, h], want, 1e-12, "final state")
    # no state in: the final state of a single step is k v^T
    o1, s1 = orc.forward_state(q[:, :, :1], k[:, :, :1], v[:, :, :1], lam, None)
    _close(s1, np.einsum("bhi,bhj->bhij", k[:, :, 0], v[:, :, 0]), 1e-14, "one-step state")


def pin_state_split_carry(orc):
    """Cutting a sequence anywhere and carrying the state over reproduces the whole run: the state
    is the complete summary of the past (page "Lightning Attention", section 2, Memory footprint)."""
    q, k, v, _, lam = _setup(113, B=1, H=3, T=29, d=4, dv=6)
    o_all, s_all = orc.forward_state(q, k, v, lam, None)
    for cut in (0, 1, 7, 28, 29):
        oa, sa = orc.forward_state(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], lam, None)
        ob, sb = orc.forward_state(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], lam, sa)
        _close(np.concatenate([oa, ob], axis=2), o_all, 1e-12, f"split at {cut}")
        _close(sb, s_all, 1e-12, f"state after split at {cut}")


def _elu1(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def pin_normalized_bruteforce(orc):
    """Normalized form == ((Psi Phi^T (.) D) V) / ((Psi Phi^T (.) D) 1) row by row, Psi = phi(Q),
    Phi = phi(K) (the page's section 1 ratio written as one masked product; numpy)."""
    q, k, v, _, lam = _setup(131, B=2, H=3, T=31, d=5, dv=4)
    for fmap, phi in (("elu1", _elu1), ("identity", lambda x: x)):
        qq, kk = (q, k) if fmap == "elu1" else (np.abs(q) + 0.5, np.abs(k) + 0.5)   # positive denominators
        got = orc.forward_normalized(qq, kk, v, lam, fmap)
        for b in range(2):
            for h in range(3):
                A = (phi(qq[b, h]) @ phi(kk[b, h]).T) * _decay_matrix(31, lam[h])
                _close(got[b, h], (A @ v[b, h]) / A.sum(axis=1, keepdims=True), 1e-12, f"normalized {fmap}")


def pin_normalized_invariants(orc):
    """With v = 1 every output is exactly 1 (a weighted average of ones); in general each output
    lies within the range of the values seen so far (positive weights summing to 1)."""
    q, k, v, _, lam = _setup(137, B=1, H=3, T=40, d=6, dv=5)
    ones = np.ones_like(v)
    _close(orc.forward_normalized(q, k, ones, lam, "elu1"), ones, 1e-13, "weights sum to one")
    o = orc.forward_normalized(q, k, v, lam, "elu1")
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12), "outputs outside the running value range"
    # the map itself: phi(x) = x + 1 above 0, e^x at or below 0.  One position, one key: with
    # k = 0 the denominator is phi(0) . phi(q) and the output is v whatever phi is, so the map is
    # read off the two-position case instead: o_1 = (a v_0 + b v_1) / (a + b) with a = phi(k_0) phi(q_1)
    # and b = phi(k_1) phi(q_1) for d = 1, no decay.
    for k0, k1 in ((2.5, -1.0), (-0.5, 0.0), (0.25, 3.0)):
        qq = np.array([0.3, 0.7]).reshape(1, 1, 2, 1)
        kk = np.array([k0, k1]).reshape(1, 1, 2, 1)
        vv = np.array([1.0, 0.0]).reshape(1, 1, 2, 1)
        a, b_ = _elu1(np.array(k0)), _elu1(np.array(k1))
        got = orc.forward_normalized(qq, kk, vv, None, "elu1")[0, 0, 1, 0]
        _close(got, a / (a + b_), 1e-14, "elu + 1 feature values")
    _close(_elu1(np.array([2.5, -1.0, 0.0])), [3.5, np.exp(-1.0), 1.0], 1e-15, "elu + 1 values")


def pin_backward_state_finite_differences(orc):
    """backward_state == central differences of L = <o, do> + <state_out, G> with respect to q, k, v
    and the carried-in state (forward_state gives o and state_out; fp64, step 1e-6)."""
    q, k, v, do, lam = _setup(151, B=1, H=2, T=6, d=3, dv=2)
    s_in = _rand((1, 2, 3, 2), 157)
    G = _rand((1, 2, 3, 2), 163)

    def loss(q_, k_, v_, s_):
        o, s_out = orc.forward_state(q_, k_, v_, lam, s_)
        return float(np.sum(o * do) + np.sum(s_out * G))

    dq, dk, dv, ds = orc.backward_state(q, k, v, do, lam, s_in, G)
    h = 1e-6
    for name, arr, got in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("state_in", s_in, ds)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            args1 = [q, k, v, s_in]
            args2 = [q, k, v, s_in]
            pos = ("q", "k", "v", "state_in").index(name)
            args1[pos], args2[pos] = a1, a2
            num[idx] = (loss(*args1) - loss(*args2)) / (2 * h)
        _close(got, num, 1e-7, f"backward_state d{name}")


def pin_backward_state_chunks(orc):
    """Training in chunks: the backward of a sequence cut at t (second chunk from the state the first
    one left, its d(state_in) fed to the first chunk as d(state_out)) equals the whole backward, and
    with no carried states it is the plain backward with d(state_in) = sum_t lam^(t+1) q_t do_t^T."""
    q, k, v, do, lam = _setup(167, B=2, H=3, T=23, d=4, dv=3)
    s0 = _rand((2, 3, 4, 3), 171)
    G = _rand((2, 3, 4, 3), 173)
    whole = orc.backward_state(q, k, v, do, lam, s0, G)
    for t in (0, 1, 9, 22, 23):
        a, b = slice(0, t), slice(t, 23)
        _, s_mid = orc.forward_state(q[:, :, a], k[:, :, a], v[:, :, a], lam, s0) if t else (None, s0)
        if t < 23:
            g2 = orc.backward_state(q[:, :, b], k[:, :, b], v[:, :, b], do[:, :, b], lam, s_mid, G)
            ds_mid = g2[3]
        else:
            g2, ds_mid = None, G
        if t:
            g1 = orc.backward_state(q[:, :, a], k[:, :, a], v[:, :, a], do[:, :, a], lam, s0, ds_mid)
        for i, what in enumerate(("dq", "dk", "dv")):
            parts = ([g1[i]] if t else []) + ([g2[i]] if g2 is not None else [])
            _close(np.concatenate(parts, axis=2), whole[i], 1e-12, f"chunked {what} at {t}")
        _close(g1[3] if t else ds_mid, whole[3], 1e-12, f"chunked d(state_in) at {t}")
    plain = orc.backward(q, k, v, do, lam)
    zero = orc.backward_state(q, k, v, do, lam, None, None)
    for a_, b_ in zip(zero[:3], plain):
        _close(a_, b_, 1e-14, "no carried states")
    w = lam[None, :, None] ** (np.arange(23)[None, None, :] + 1)
    _close(zero[3], np.einsum("bht,bhti,bhtj->bhij", np.broadcast_to(w, (2, 3, 23)), q, do), 1e-12,
           "d(state_in) closed form")


def pin_backward_normalized(orc):
    """backward_normalized == central differences of <o, do> (elu + 1, and the identity on positive
    inputs) and == torch autograd (float64) through the masked-product ratio with the map applied."""
    import torch
    q, k, v, do, lam = _setup(181, B=1, H=2, T=6, d=3, dv=2)
    for fmap in ("elu1", "identity"):
        qq, kk = (q, k) if fmap == "elu1" else (np.abs(q) + 0.5, np.abs(k) + 0.5)
        dq, dk, dv = orc.backward_normalized(qq, kk, v, do, lam, fmap)

        def loss(q_, k_, v_):
            return float(np.sum(orc.forward_normalized(q_, k_, v_, lam, fmap) * do))

        h = 1e-6
        for name, arr, got in (("q", qq, dq), ("k", kk, dk), ("v", v, dv)):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                a1, a2 = arr.copy(), arr.copy()
                a1[idx] += h
                a2[idx] -= h
                args1, args2 = [qq, kk, v], [qq, kk, v]
                pos = ("q", "k", "v").index(name)
                args1[pos], args2[pos] = a1, a2
                num[idx] = (loss(*args1) - loss(*args2)) / (2 * h)
            _close(got, num, 1e-7, f"backward_normalized {fmap} d{name}")
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (qq, kk, v))
        phi = (lambda x: torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))) if fmap == "elu1" else (lambda x: x)
        outs = []
        for hh in range(2):
            D = torch.tensor(_decay_matrix(6, lam[hh]))
            A = (phi(tq[0, hh]) @ phi(tk[0, hh]).T) * D
            outs.append((A @ tv[0, hh]) / A.sum(dim=1, keepdim=True))
        (torch.stack(outs)[None] * torch.tensor(do)).sum().backward()
        for name, got, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad)):
            _close(got, ref.numpy(), 1e-12, f"backward_normalized {fmap} d{name} vs autograd")


ALL_PINS = [
    pin_golden_handworked,
    pin_bruteforce_forward,
    pin_closed_form_ones,
    pin_cumsum_filter,
    pin_tile_invariance,
    pin_causality,
    pin_finite_differences,
    pin_autograd,
    pin_inner_products,
    pin_backward_as_forward,
    pin_linearity_and_heads,
    pin_rows,
    pin_state_closed_form,
    pin_state_split_carry,
    pin_normalized_bruteforce,
    pin_normalized_invariants,
    pin_backward_state_finite_differences,
    pin_backward_state_chunks,
    pin_backward_normalized,
]
