"""One chain longer than 2^32 bytes per tensor (T = 2^24 + 200, d = d_v = 128, bf16), forward and
backward, against references that depend on every position.

Buffer resources carry a 32-bit byte count; a chain's remaining length past a tile start exceeds
it here, and the kernels must still read every tile whole, from the right offset, and hand the
state over between the chain's segments.  Inputs: q_t = k_t = e_0, lam = 1 - 2^-10 (a memory of
about a thousand positions, so the state never settles to a constant), and position-dependent
values and output gradients with periods that are not powers of two,
  v_t[j] = ((t + 97 j) mod 1021) / 1021,   do_t[j] = ((7 t + 31 j) mod 509) / 509,
so a tile read from a wrong offset, or a segment started from a wrong state, changes the result.
By the token recurrence, S_t = e_0 y_t^T and R_t = e_0 g_t^T with the first-order filters
  y_t = lam y_{t-1} + v_t,   g_t = lam g_{t+1} + do_t,
hence o_t = y_t, dq_t = (y_t . do_t) e_0, dk_t = (g_t . v_t) e_0, dv_t = g_t.  The references are
computed on the GPU in fp64 from the stored bf16 values, chunk by chunk with the filter state
carried across chunks (the fp64 copies would not fit host memory); bar as for every bf16 case,
2e-2 of the largest reference value of each output.
"""
import pytest
import torch

import causal_linear_attention_amd as la2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
T = (1 << 24) + 200
D = 128
LAM = 1.0 - 2.0 ** -10
CHUNK = 8192          # lam^-CHUNK = e^8: the in-chunk rescaling stays well inside fp64


def pattern(mult, jmul, period):
    """[1, 1, T, D] bf16 with entry ((mult t + jmul j) mod period) / period, built in chunks."""
    x = torch.empty((1, 1, T, D), dtype=torch.bfloat16, device=DEV)
    j = torch.arange(D, device=DEV, dtype=torch.int64)[None, :]
    for t0 in range(0, T, 1 << 20):
        t = torch.arange(t0, min(T, t0 + (1 << 20)), device=DEV, dtype=torch.int64)[:, None]
        x[0, 0, t0:t0 + t.shape[0]] = (((mult * t + jmul * j) % period).float() / period).to(torch.bfloat16)
    return x


def chunk_filter(x, carry, reverse):
    """First-order filter of the fp64 rows x [L, D] with lam, continuing from `carry` (the filter value
    just before the chunk in scan order): forward y_t = lam y_{t-1} + x_t, reverse g_t = lam g_{t+1} + x_t."""
    L = x.shape[0]
    n = torch.arange(L, device=DEV, dtype=torch.float64)[:, None]
    if reverse:
        x = x.flip(0)
    y = LAM ** n * torch.cumsum(LAM ** (-n) * x, 0) + LAM ** (n + 1) * carry
    return y.flip(0) if reverse else y


class MaxRel:
    def __init__(self):
        self.err, self.ref = 0.0, 0.0

    def add(self, got, ref):
        self.err = max(self.err, float((got.double() - ref).abs().max()))
        self.ref = max(self.ref, float(ref.abs().max()))

    def value(self):
        return self.err / self.ref


def test_chain_over_4gib_position_dependent():
    e0 = torch.zeros((1, 1, T, D), dtype=torch.bfloat16, device=DEV)
    e0[..., 0] = 1.0
    q, k = e0, e0.clone()
    v = pattern(1, 97, 1021)
    do = pattern(7, 31, 509)
    decay = torch.tensor([LAM], dtype=torch.float32, device=DEV)
    assert float(decay[0]) == LAM
    print("T", T, "forward + backward", flush=True)
    o = la2.forward(q, k, v, decay, 128)
    dq, dk, dv = la2.backward(q, k, v, do, decay, 128)
    torch.cuda.synchronize()
    col0 = torch.zeros(D, dtype=torch.bool, device=DEV)
    col0[0] = True

    err = {n: MaxRel() for n in ("o", "dq", "dk", "dv")}
    off = 0.0   # largest entry of dq, dk outside column 0 (exactly zero in the reference)
    y = torch.zeros(1, D, dtype=torch.float64, device=DEV)
    for t0 in range(0, T, CHUNK):
        t1 = min(T, t0 + CHUNK)
        yc = chunk_filter(v[0, 0, t0:t1].double(), y, False)
        y = yc[-1:]
        err["o"].add(o[0, 0, t0:t1], yc)
        err["dq"].add(dq[0, 0, t0:t1, 0], (yc * do[0, 0, t0:t1].double()).sum(1))
        off = max(off, float(dq[0, 0, t0:t1, 1:].abs().max()))
    print("forward filter done", flush=True)
    g = torch.zeros(1, D, dtype=torch.float64, device=DEV)
    for t1 in range(T, 0, -CHUNK):
        t0 = max(0, t1 - CHUNK)
        gc = chunk_filter(do[0, 0, t0:t1].double(), g, True)
        g = gc[:1]
        err["dv"].add(dv[0, 0, t0:t1], gc)
        err["dk"].add(dk[0, 0, t0:t1, 0], (gc * v[0, 0, t0:t1].double()).sum(1))
        off = max(off, float(dk[0, 0, t0:t1, 1:].abs().max()))
    rel = {n: e.value() for n, e in err.items()}
    print("max|err|/max|ref|", {n: f"{r:.3e}" for n, r in rel.items()}, "off-column", off, flush=True)
    for n, r in rel.items():
        assert r <= 2e-2, (n, r)
    assert off == 0.0
