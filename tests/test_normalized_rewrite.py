"""The centered form of the normalized backward's dq (the bf16 path of la2_backward_normalized,
la2_norm.hip mode 7), checked in fp64 against the oracle's chain-rule backward of the ratio (page
"Lightning Attention", section 1): with phi(k_s) = m + kap_s for any constant vector m,

    a_t = do_t . Vbar_t,   U_t = sum_{s<=t} lam^(t-s) kap_s (v_s . do_t),   zk_t = sum_{s<=t} lam^(t-s) kap_s,
    ell_t = sum_{s<=t} lam^(t-s),   sigma_t = phi(q_t) . m,   den_t = phi(q_t) . z_t,
    c_t = (sigma_t a_t + phi(q_t) . U_t) / den_t,   G_t = ((phi(q_t) . zk_t) a_t - ell_t phi(q_t) . U_t) / den_t,
    dq_t = (U_t - c_t zk_t + G_t m) / den_t (.) phi'(q_t)

is the gradient exactly (rounding of fp64 aside), whatever m is; the kernels use the chain's mean.
CPU only."""
import numpy as np
import pytest

import oracle


def phi(a, fmap):
    return np.where(a > 0, a + 1.0, np.exp(np.minimum(a, 0.0))) if fmap == "elu1" else a


def dphi(a, fmap):
    return np.where(a > 0, 1.0, np.exp(np.minimum(a, 0.0))) if fmap == "elu1" else np.ones_like(a)


def centered_dq(q, k, v, do, lam, fmap, m, with_g=True):
    T, d = q.shape
    pq, pk = phi(q, fmap), phi(k, fmap)
    kap = pk - m
    out = np.zeros_like(q)
    z = np.zeros(d)
    zk = np.zeros(d)
    vbar = np.zeros(v.shape[1])
    ell = 0.0
    # U by brute force over the causal, decayed pairs
    for t in range(T):
        z = lam * z + pk[t]
        zk = lam * zk + kap[t]
        vbar = lam * vbar + v[t]
        ell = lam * ell + 1.0
        w = lam ** (t - np.arange(t + 1))
        U = (w * (v[: t + 1] @ do[t]))[:, None] * kap[: t + 1]
        U = U.sum(0)
        den = pq[t] @ z
        a = do[t] @ vbar
        sig = pq[t] @ m
        c = (sig * a + pq[t] @ U) / den
        G = ((pq[t] @ zk) * a - ell * (pq[t] @ U)) / den
        out[t] = (U - c * zk + (G * m if with_g else 0.0)) / den * dphi(q[t], fmap)
    return out


@pytest.mark.parametrize("fmap", ["elu1", "identity"])
@pytest.mark.parametrize("lam", [1.0, 0.97, 0.5])
def test_centered_dq_is_the_gradient(fmap, lam):
    rng = np.random.default_rng(11)
    T, d, dv = 37, 16, 8
    q, k = rng.normal(size=(T, d)) / 4, rng.normal(size=(T, d)) / 4
    if fmap == "identity":
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    v, do = rng.normal(size=(T, dv)), rng.normal(size=(T, dv))
    ref = oracle.backward_normalized(q[None, None], k[None, None], v[None, None], do[None, None],
                                     np.array([lam]), fmap)[0][0, 0]
    pk = phi(k, fmap)
    for m in (pk.mean(0), np.zeros(d), rng.normal(size=d)):
        got = centered_dq(q, k, v, do, lam, fmap, m)
        assert np.abs(got - ref).max() <= 1e-10 * np.abs(ref).max()


def test_centered_dq_needs_every_term():
    """Not vacuous: leaving out the G_t m term (which vanishes only for m = 0) misses the gradient."""
    rng = np.random.default_rng(5)
    T, d, dv = 20, 8, 8
    q, k, v, do = (rng.normal(size=(T, w)) / 3 for w in (d, d, dv, dv))
    ref = oracle.backward_normalized(q[None, None], k[None, None], v[None, None], do[None, None],
                                     np.array([0.9]), "elu1")[0][0, 0]
    got = centered_dq(q, k, v, do, 0.9, "elu1", phi(k, "elu1").mean(0), with_g=False)
    assert np.abs(got - ref).max() > 1e-3 * np.abs(ref).max()
