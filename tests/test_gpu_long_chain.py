"""One chain longer than 2^32 bytes per tensor (T = 2^24 + 200, d = d_v = 128, bf16), forward and
backward, against closed forms.

Buffer resources carry a 32-bit byte count; a chain's remaining length past a tile start exceeds
it here, and the kernels must still read every tile whole.  Inputs: q_t = k_t = e_0, v_t = 1,
do_t = 1/128, lam = 1/2, so by the token recurrence
  S_t = (2 - 2^-t) e_0 1^T,  o_t = (2 - 2^-t) 1,  dq_t = (2 - 2^-t) e_0,
  R_t = c_t e_0 1^T / 128 with c_t = 2 - 2^-(T-1-t),  dk_t = c_t e_0,  dv_t = c_t / 128 1.
The values are checked on the GPU in chunks (the fp64 copies would not fit host memory); bar as
for every bf16 case, 2e-2 of the largest reference value.
"""
import pytest
import torch

import causal_linear_attention_amd as la2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
T = (1 << 24) + 200
D = 128
CHUNK = 1 << 20


def max_err(x, expected_of_t):
    """max over t of |x[t, :] - expected(t)|, x [T, n] on the GPU, expected per row."""
    worst = 0.0
    for t0 in range(0, T, CHUNK):
        t1 = min(T, t0 + CHUNK)
        t = torch.arange(t0, t1, device=DEV, dtype=torch.float64)
        ref = expected_of_t(t)
        worst = max(worst, float((x[t0:t1].double() - ref).abs().max()))
    return worst


def test_chain_over_4gib_closed_form():
    e0 = torch.zeros((1, 1, T, D), dtype=torch.bfloat16, device=DEV)
    e0[..., 0] = 1.0
    q, k = e0, e0.clone()
    v = torch.ones((1, 1, T, D), dtype=torch.bfloat16, device=DEV)
    decay = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    print("T", T, "forward", flush=True)
    o = la2.forward(q, k, v, decay, 128)
    torch.cuda.synchronize()
    geo = lambda t: (2.0 - torch.pow(2.0, -t))[:, None]
    err = max_err(o[0, 0], geo)
    print("o", err, flush=True)
    assert err <= 2e-2 * 2.0
    del o

    do = torch.full((1, 1, T, D), 1.0 / 128, dtype=torch.bfloat16, device=DEV)
    print("backward", flush=True)
    dq, dk, dv = la2.backward(q, k, v, do, decay, 128)
    torch.cuda.synchronize()
    col0 = torch.zeros(D, dtype=torch.float64, device=DEV)
    col0[0] = 1.0
    c = lambda t: (2.0 - torch.pow(2.0, -(T - 1 - t)))[:, None]
    errs = [max_err(dq[0, 0], lambda t: geo(t) * col0),
            max_err(dk[0, 0], lambda t: c(t) * col0),
            max_err(dv[0, 0], lambda t: c(t) / 128 * torch.ones(D, dtype=torch.float64, device=DEV))]
    print("dq dk dv", errs, flush=True)
    assert errs[0] <= 2e-2 * 2.0 and errs[1] <= 2e-2 * 2.0 and errs[2] <= 2e-2 * 2.0 / 128
