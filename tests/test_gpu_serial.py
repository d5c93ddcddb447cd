"""The token-serial recurrence kernel (la2_forward_serial, the comparison baseline of the tiled
scan) through the C ABI against the oracle's forward.  Bars: max|gpu - ref| / max|ref| <= 1e-5 for
fp32 inputs, <= 2e-2 for bf16 inputs."""
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
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(np.asarray(got) - ref))) / (scale if scale > 0 else 1.0)


@pytest.mark.parametrize("case", [
    (2, 3, 333, 128, 128, "bf16", "heads"),
    (1, 2, 17, 64, 128, "bf16", "none"),
    (3, 1, 1, 128, 64, "bf16", "heads"),
    (1, 2, 300, 64, 64, "f32", "heads"),
    (2, 2, 129, 128, 128, "f32", 0.5),
], ids=lambda c: "-".join(str(v) for v in c))
def test_serial_matches_oracle(case):
    B, H, T, d, dv, dtype, decay = case
    x = inputs.make_random(B, H, T, d, dv, dtype=dtype, seed=211 + T, decay=decay, backward=False)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    dec = None if x["decay"] is None else x["decay"].to(DEV)
    o = la2.forward_serial(q, k, v, dec)
    lam = None if x["decay"] is None else x["decay"].double().numpy()
    ref = oracle.forward(*(f64(x[n]) for n in ("q", "k", "v")), lam)
    torch.cuda.synchronize()
    err = rel_err(f64(o), ref)
    print(case, f"{err:.2e}", flush=True)
    assert err <= TOL[dtype]


def test_serial_agrees_with_tiled_scan_full_size():
    """The 1K sweep workload in one launch: serial and tiled outputs both within the bf16 bar of
    each other's scale (they round differently), and the serial one against the oracle on sampled
    whole chains."""
    x = inputs.make("sweep131k_t1k")
    w = x["workload"]
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o_ser = la2.forward_serial(q, k, v, None)
    o_tile = la2.forward(q, k, v, None, w.block)
    torch.cuda.synchronize()
    diff = float((o_ser.float() - o_tile.float()).abs().max()) / float(o_tile.float().abs().max())
    print(f"serial vs tiled: {diff:.2e}", flush=True)
    assert diff <= 2e-2
    for b, h in [(0, 0), (w.B - 1, 15)]:
        ref = oracle.forward(*(f64(x[n][b:b + 1, h:h + 1]) for n in ("q", "k", "v")), None)
        assert rel_err(f64(o_ser[b:b + 1, h:h + 1]), ref) <= 2e-2
