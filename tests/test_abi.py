"""C-ABI library on the CPU: it loads, exports what include/la2.h declares, and
rejects bad arguments before anything is enqueued (no GPU needed)."""
import ctypes
import functools
import os
import re

import pytest
import torch

import causal_linear_attention_amd as la2
from causal_linear_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = open(os.path.join(ROOT, "include", "la2.h")).read()

OK, NULLP, SHAPE, UNSUP, MISAL, ALIAS, WS = 0, 1, 2, 3, 4, 5, 6
P = 1 << 20          # fake, 16-byte aligned device addresses: validation fails before any use
MB = 1 << 26


@pytest.fixture(scope="module")
def lib():
    return la2.load_library()


def declared_functions():
    return re.findall(r"^\s*(?:int|size_t|const char \*)\s*(la2_\w+)\s*\(", HEADER, flags=re.M)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    ver = int(re.search(r"#define LA2_ABI_VERSION (\d+)", HEADER).group(1))
    assert la2.la2_abi_version() == ver
    assert binding.LA2_ABI_VERSION == ver
    for code in range(9):
        s = la2.la2_status_string(code)
        assert s and s != "unknown status"
    assert la2.la2_status_string(99) == "unknown status"


def fwd(lib, q=P, k=P + MB, v=P + 2 * MB, decay=None, o=P + 3 * MB, B=1, H=1, T=64, d=64, dv=64, block=64,
        dtype=1, ws=None, wsb=0):
    return lib.la2_forward(q, k, v, decay, o, B, H, T, d, dv, block, dtype, ws, wsb, None)


def bwd(lib, q=P, k=P + MB, v=P + 2 * MB, decay=None, do=P + 3 * MB, dq=P + 4 * MB, dk=P + 5 * MB,
        dv_=P + 6 * MB, B=1, H=1, T=64, d=64, dv=64, block=64, dtype=1, ws=None, wsb=0):
    return lib.la2_backward(q, k, v, decay, do, dq, dk, dv_, B, H, T, d, dv, block, dtype, ws, wsb, None)


def test_null_pointers(lib):
    assert fwd(lib, q=None) == NULLP
    assert fwd(lib, o=None) == NULLP
    assert bwd(lib, do=None) == NULLP
    assert bwd(lib, dv_=None) == NULLP


def test_bad_shapes(lib):
    for kw in ({"B": 0}, {"H": -1}, {"T": 0}, {"d": 0}, {"dv": -5}, {"B": 1 << 40, "H": 1 << 30}):
        assert fwd(lib, **kw) == SHAPE, kw
        assert bwd(lib, **kw) == SHAPE, kw


def test_unsupported(lib):
    assert fwd(lib, d=96) == UNSUP
    assert fwd(lib, dv=256) == UNSUP
    assert fwd(lib, dtype=7) == UNSUP
    for dtype in (0, 1):
        for block in (0, 8, 48, 100, 512, -64):
            assert fwd(lib, dtype=dtype, block=block) == UNSUP, (dtype, block)
            assert bwd(lib, dtype=dtype, block=block) == UNSUP, (dtype, block)


@pytest.mark.parametrize("dtype", [0, 1])
def test_every_tile_length_is_accepted(lib, dtype):
    """T_B in {16, 32, 64, 128, 256} for both dtypes (a request: the kernels run the nearest tile
    length they are built for, bf16 64 or 128, fp32 16, 32 or 64, and the split into segments follows
    that tile).  Checked through the workspace query, which validates like the calls do."""
    bad = ctypes.c_size_t(-1).value
    run = {16: 64, 32: 64, 64: 64, 128: 128, 256: 128} if dtype == 1 else {16: 16, 32: 32, 64: 64, 128: 64, 256: 64}
    for block, tile in run.items():
        # one chain of 64 tiles of the kernel's length: split into min(256, 64) = 64 segments
        n = lib.la2_workspace_bytes(1, 1, 64 * tile, 64, 64, block, dtype, 0)
        assert n != bad, block
        assert n == 64 * 64 * 64 * 4, (block, n)         # 64 segment states of 64 x 64 fp32
        assert lib.la2_workspace_bytes(1, 1, 64 * tile, 64, 64, block, dtype, 1) >= n


def test_misaligned(lib):
    assert fwd(lib, q=P + 2) == MISAL
    assert fwd(lib, o=P + 3 * MB + 8) == MISAL
    assert fwd(lib, decay=P + 7 * MB + 1) == MISAL
    assert bwd(lib, dk=P + 5 * MB + 4) == MISAL


def test_alias(lib):
    assert fwd(lib, o=P) == ALIAS                       # o == q
    assert fwd(lib, o=P + 2 * MB + 64) == ALIAS         # o inside v
    assert bwd(lib, dq=P + 1 * MB) == ALIAS             # dq == k
    assert bwd(lib, dk=P + 4 * MB) == ALIAS             # dk == dq


def test_workspace(lib):
    # one chain of 1024 positions is split over workgroups, so it needs segment states
    n = la2.la2_workspace_bytes(1, 1, 1024, 64, 64, 64, torch.bfloat16, False)
    assert n > 0
    assert fwd(lib, T=1024, ws=None, wsb=0) == WS
    assert fwd(lib, T=1024, ws=P + 8 * MB, wsb=n - 1) == WS
    assert bwd(lib, T=1024, ws=None, wsb=0) == WS
    assert fwd(lib, T=1024, ws=P + MB, wsb=n) == ALIAS   # workspace on top of k
    # enough chains to fill the GPU: no split, no segment states; the backward's workspace then holds only
    # each chain's final state where the one-pass backward applies (bf16, d = d_v = 128)
    assert la2.la2_workspace_bytes(16, 16, 4096, 128, 128, 128, torch.bfloat16, False) == 0
    assert la2.la2_workspace_bytes(16, 16, 4096, 128, 128, 128, torch.bfloat16, True) == 256 * 128 * 128 * 4
    assert la2.la2_workspace_bytes(16, 16, 4096, 64, 64, 64, torch.bfloat16, True) == 0
    assert la2.la2_workspace_bytes(16, 16, 4096, 128, 128, 64, torch.float32, True) == 0
    assert lib.la2_workspace_bytes(1, 1, 64, 96, 64, 64, 1, 0) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_workspace_plan_properties(lib, dtype):
    """Host plan over many shapes.  The work items are the chains (bf16) or the chains' 64-wide value
    slices (fp32); with fewer than the 256 CUs a chain is cut into min(256 // work, tiles) segments,
    so when that is below 2 there are no segment states; otherwise the workspace holds a whole number (at least 2, at most one per tile) of
    d x d_v fp32 states per chain, and the backward's is at least the forward's."""
    block = 128 if dtype == torch.bfloat16 else 64
    for B, H, T, d, dv in [(1, 1, 1024, 64, 64), (1, 16, 131072, 128, 128), (2, 40, 6144, 128, 128),
                           (1, 40, 131072, 128, 128), (8, 16, 16384, 128, 128), (3, 5, 777, 128, 64),
                           (16, 16, 4096, 128, 128), (64, 4, 100000, 64, 64), (1, 1, block, 128, 128),
                           (1, 2, block + 1, 64, 128), (255, 1, 5000, 64, 64), (128, 1, 5000, 64, 64),
                           (1, 1, 3, 64, 64)]:
        chains, tiles = B * H, -(-T // block)
        work = chains * (dv // 64 if dtype == torch.float32 else 1)
        f = la2.la2_workspace_bytes(B, H, T, d, dv, block, dtype, False)
        g = la2.la2_workspace_bytes(B, H, T, d, dv, block, dtype, True)
        unit = chains * d * dv * 4
        if min(256 // work, tiles) < 2:
            assert f == 0, (B, H, T)
        else:
            assert f % unit == 0 and 2 <= f // unit <= tiles, (B, H, T, f // unit)
        assert g >= f, (B, H, T)


def fwds(lib, q=P, k=P + MB, v=P + 2 * MB, decay=None, s_in=P + 8 * MB, o=P + 3 * MB, s_out=P + 9 * MB, B=1, H=1,
         T=64, d=64, dv=64, block=64, dtype=1, ws=None, wsb=0):
    return lib.la2_forward_state(q, k, v, decay, s_in, o, s_out, B, H, T, d, dv, block, dtype, ws, wsb, None)


def dec(lib, q=P, k=P + MB, v=P + 2 * MB, decay=None, o=P + 3 * MB, state=P + 4 * MB, B=1, H=1, d=64, dv=64,
        dtype=1):
    return lib.la2_decode_step(q, k, v, decay, o, state, B, H, d, dv, dtype, None)


def test_forward_state_validation(lib):
    assert fwds(lib, q=None) == NULLP
    assert fwds(lib, o=None) == NULLP
    assert fwds(lib, T=0) == SHAPE
    assert fwds(lib, d=96) == UNSUP
    assert fwds(lib, s_in=P + 8 * MB + 4) == MISAL
    assert fwds(lib, s_out=P + 9 * MB + 8) == MISAL
    assert fwds(lib, s_out=P) == ALIAS                         # final state on top of q
    assert fwds(lib, s_out=P + 3 * MB + 128) == ALIAS          # ... inside o
    assert fwds(lib, s_out=P + 8 * MB + 64) == ALIAS           # partly over state_in
    assert fwds(lib, s_in=P + 3 * MB) == ALIAS                 # o over state_in
    assert fwds(lib, T=1024) == WS                             # split chain, no workspace
    n = la2.la2_workspace_bytes(1, 1, 1024, 64, 64, 64, torch.bfloat16, False)
    assert fwds(lib, T=1024, ws=P + 8 * MB, wsb=n) == ALIAS    # workspace over state_in


def test_decode_step_validation(lib):
    assert dec(lib, q=None) == NULLP
    assert dec(lib, state=None) == NULLP
    assert dec(lib, B=0) == SHAPE
    assert dec(lib, d=32) == UNSUP
    assert dec(lib, dtype=5) == UNSUP
    assert dec(lib, state=P + 4 * MB + 4) == MISAL
    assert dec(lib, o=P) == ALIAS                              # o over q
    assert dec(lib, state=P + 2 * MB) == ALIAS                 # state over v
    assert dec(lib, o=P + 4 * MB + 256) == ALIAS               # o inside the state


def nrm(lib, q=P, k=P + MB, v=P + 2 * MB, decay=None, o=P + 3 * MB, B=1, H=1, T=64, d=64, dv=64, fmap=1, block=64,
        dtype=1, ws=None, wsb=0):
    return lib.la2_forward_normalized(q, k, v, decay, o, B, H, T, d, dv, fmap, block, dtype, ws, wsb, None)


def test_forward_normalized_validation(lib):
    assert nrm(lib, q=None) == NULLP
    assert nrm(lib, o=None) == NULLP
    assert nrm(lib, fmap=2) == UNSUP
    assert nrm(lib, T=0) == SHAPE
    assert nrm(lib, dv=32) == UNSUP
    assert nrm(lib, v=P + 2 * MB + 8) == MISAL
    assert nrm(lib, o=P + MB + 64) == ALIAS                    # o inside k
    assert nrm(lib) == WS                                      # elu + 1 needs phi(q), phi(k) in the workspace
    n = la2.la2_normalized_workspace_bytes(1, 1, 64, 64, 64, "elu1", 64, torch.bfloat16)
    assert n == 2 * 64 * 64 * 2 + 256                          # phi(q), phi(k) (bf16) and 64 fp32 denominators
    assert nrm(lib, ws=P + 4 * MB, wsb=n - 1) == WS
    assert nrm(lib, ws=P + 2 * MB, wsb=n) == ALIAS             # workspace over v
    assert nrm(lib, ws=P + 3 * MB - 256, wsb=n) == ALIAS       # workspace runs into o
    # identity map on a short sequence: only the denominators
    assert la2.la2_normalized_workspace_bytes(1, 1, 64, 64, 64, "identity", 64, torch.bfloat16) == 256
    # few chains, long sequences: per-segment sums of phi(k) and the numerator's segment states
    big = la2.la2_normalized_workspace_bytes(1, 2, 1 << 16, 128, 128, "identity", 128, torch.bfloat16)
    assert big >= la2.la2_workspace_bytes(1, 2, 1 << 16, 128, 128, 128, torch.bfloat16, False) + 2 * 128 * 4
    assert lib.la2_normalized_workspace_bytes(1, 1, 64, 64, 64, 3, 64, 1, 0) == ctypes.c_size_t(-1).value
    assert lib.la2_normalized_workspace_bytes(1, 1, 64, 96, 64, 1, 64, 1, 0) == ctypes.c_size_t(-1).value
    # the backward adds dden (fp32 per position) and dn (one output-sized gradient); in bf16 also the
    # segment sums of phi(k) for its mean, phi(k) - m and the scan U (two q-sized tensors) and a_t (fp32
    # per position)
    assert la2.la2_normalized_workspace_bytes(1, 1, 64, 64, 64, "elu1", 64, torch.float32, True) == (
        la2.la2_normalized_workspace_bytes(1, 1, 64, 64, 64, "elu1", 64, torch.float32) + 256 + 64 * 64 * 4)
    assert la2.la2_normalized_workspace_bytes(1, 1, 64, 64, 64, "elu1", 64, torch.bfloat16, True) == (
        n + 256 + 64 * 64 * 2 + 256 + 2 * 64 * 64 * 2 + 256)


def ser(lib, q=P, k=P + MB, v=P + 2 * MB, decay=None, o=P + 3 * MB, B=1, H=1, T=64, d=64, dv=64, dtype=1):
    return lib.la2_forward_serial(q, k, v, decay, o, B, H, T, d, dv, dtype, None)


def test_forward_serial_validation(lib):
    assert ser(lib, v=None) == NULLP
    assert ser(lib, H=0) == SHAPE
    assert ser(lib, d=32) == UNSUP
    assert ser(lib, dtype=7) == UNSUP
    assert ser(lib, o=P + 3 * MB + 2) == MISAL
    assert ser(lib, decay=P + 5 * MB + 2) == MISAL
    assert ser(lib, o=P + 2 * MB + 512) == ALIAS               # o inside v
    assert ser(lib, decay=P + 3 * MB + 64) == ALIAS            # o over the decays


def bst(lib, q=P, k=P + MB, v=P + 2 * MB, decay=None, s_in=P + 8 * MB, do=P + 3 * MB, ds_out=P + 9 * MB,
        dq=P + 4 * MB, dk=P + 5 * MB, dv_=P + 6 * MB, ds_in=P + 10 * MB, B=1, H=1, T=64, d=64, dv=64, block=64,
        dtype=1, ws=None, wsb=0):
    return lib.la2_backward_state(q, k, v, decay, s_in, do, ds_out, dq, dk, dv_, ds_in, B, H, T, d, dv, block,
                                  dtype, ws, wsb, None)


def test_backward_state_validation(lib):
    assert bst(lib, q=None) == NULLP
    assert bst(lib, dq=None) == NULLP
    assert bst(lib, T=0) == SHAPE
    assert bst(lib, d=96) == UNSUP
    assert bst(lib, s_in=P + 8 * MB + 4) == MISAL
    assert bst(lib, ds_in=P + 10 * MB + 8) == MISAL
    assert bst(lib, ds_in=P + 3 * MB) == ALIAS                # d(state_in) over dout
    assert bst(lib, ds_in=P + 9 * MB + 64) == ALIAS           # ... inside dstate_out
    assert bst(lib, ds_in=P + 4 * MB + 256) == ALIAS          # ... inside dq
    assert bst(lib, dq=P + 8 * MB) == ALIAS                   # dq over state_in
    assert bst(lib, T=1024) == WS                             # split chain, no workspace
    n = la2.la2_workspace_bytes(1, 1, 1024, 64, 64, 64, torch.bfloat16, True)
    assert bst(lib, T=1024, ws=P + 9 * MB, wsb=n) == ALIAS    # workspace over dstate_out


def bnr(lib, q=P, k=P + MB, v=P + 2 * MB, decay=None, o=P + 3 * MB, do=P + 4 * MB, dq=P + 5 * MB, dk=P + 6 * MB,
        dv_=P + 7 * MB, B=1, H=1, T=64, d=64, dv=64, fmap=1, block=64, dtype=1, ws=P + 8 * MB, wsb=1 << 24,
        saved=False):
    fn = lib.la2_backward_normalized_saved if saved else lib.la2_backward_normalized
    return fn(q, k, v, decay, o, do, dq, dk, dv_, B, H, T, d, dv, fmap, block, dtype, ws, wsb, None)


@pytest.mark.parametrize("saved", [False, True])
def test_backward_normalized_validation(lib, saved):
    bnr = functools.partial(globals()["bnr"], saved=saved)
    assert bnr(lib, o=None) == NULLP
    assert bnr(lib, dv_=None) == NULLP
    assert bnr(lib, fmap=5) == UNSUP
    assert bnr(lib, T=0) == SHAPE
    assert bnr(lib, do=P + 4 * MB + 2) == MISAL
    assert bnr(lib, ws=None, wsb=0) == WS
    assert bnr(lib, wsb=100) == WS
    assert bnr(lib, dq=P + 3 * MB) == ALIAS                  # dq over o
    assert bnr(lib, dk=P + 5 * MB + 64) == ALIAS             # dk inside dq
    assert bnr(lib, ws=P + 7 * MB) == ALIAS                  # workspace over dv


def test_binding_refuses_cpu_tensors():
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on the GPU"):
        la2.la2_forward(q, q, q, None, torch.empty_like(q), 64)
    with pytest.raises(TypeError):
        la2.forward(q.half(), q.half(), q.half())


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def test_binding_checks_every_shape_and_dtype():
    """Every low-level wrapper checks each tensor against the sizes it passes to the C ABI (shapes
    and dtypes are checked before the device, so these refusals run on the CPU): a short dout, a
    decay of the wrong length or dtype, a state of the wrong shape never reach a kernel."""
    B, H, T, d, dv = 2, 3, 40, 64, 128
    q, k, v = _t(B, H, T, d), _t(B, H, T, d), _t(B, H, T, dv)
    o, do, dq, dk, dvv = _t(B, H, T, dv), _t(B, H, T, dv), _t(B, H, T, d), _t(B, H, T, d), _t(B, H, T, dv)
    dec = torch.full((H,), 0.9)
    st = _t(B, H, d, dv, dtype=torch.float32)
    cases = [
        (lambda: la2.la2_forward(q, k[:, :, :-1], v, None, o, 64), ValueError, "k must have shape"),
        (lambda: la2.la2_forward(q, k, v[..., :64], None, o, 64), ValueError, "o must have shape"),
        (lambda: la2.la2_forward(q, k, v, None, o.float(), 64), TypeError, "o must be"),
        (lambda: la2.la2_forward(q, k, v, dec[:2], o, 64), ValueError, "decay must have shape"),
        (lambda: la2.la2_forward(q, k, v, dec.double(), o, 64), TypeError, "decay must be"),
        (lambda: la2.la2_forward(q[0], k, v, None, o, 64), ValueError, "q must have 4 dimensions"),
        (lambda: la2.la2_backward(q, k, v, None, do[:, :, :-1], dq, dk, dvv, 64), ValueError, "dout must have shape"),
        (lambda: la2.la2_backward(q, k, v, None, do, dq, dk[..., :32], dvv, 64), ValueError, "dk must have shape"),
        (lambda: la2.la2_backward(q, k, v, dec, do, dq, dk, dq, 64), ValueError, "dv must have shape"),
        (lambda: la2.la2_backward_saved(q, k, v, None, do, dq.float(), dk, dvv, 64), TypeError, "dq must be"),
        (lambda: la2.la2_forward_state(q, k, v, None, st[:1], o, st, 64), ValueError, "state_in must have shape"),
        (lambda: la2.la2_forward_state(q, k, v, None, st, o, st.double(), 64), TypeError, "state_out must be"),
        (lambda: la2.la2_backward_state(q, k, v, None, None, do, st.transpose(2, 3), dq, dk, dvv, st, 64),
         ValueError, "dstate_out must have shape"),
        (lambda: la2.la2_decode_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], None, o[:, :, 0], st[:, :2]), ValueError,
         "state must have shape"),
        (lambda: la2.la2_forward_normalized(q, k, v, dec, o[:1], "elu1", 64), ValueError, "o must have shape"),
        (lambda: la2.la2_backward_normalized(q, k, v, None, o, do, dq, dk, dvv[..., :8], "elu1", 64), ValueError,
         "dv must have shape"),
        (lambda: la2.la2_forward_serial(q, k, v, torch.ones(H, 1), o), ValueError, "decay must have shape"),
    ]
    for fn, exc, msg in cases:
        with pytest.raises(exc, match=msg):
            fn()


@pytest.mark.parametrize("bad", [0.0, -0.5, 1.5, float("nan"), float("inf")])
def test_high_level_api_rejects_decay_outside_unit_interval(bad):
    """lam must lie in (0, 1]: lam = 0 gives 0^0 on the mask diagonal, which the kernels form as
    2^(0 * log2 0) = NaN; lam > 1 grows without bound."""
    q = _t(1, 2, 16, 64)
    dec = torch.tensor([0.5, bad])
    for fn in (lambda: la2.forward(q, q, q, dec), lambda: la2.backward(q, q, q, q, dec),
               lambda: la2.lightning_attention(q, q, q, dec), lambda: la2.forward_state(q, q, q, dec),
               lambda: la2.forward_normalized(q, q, q, dec)):
        with pytest.raises(ValueError, match=r"\(0, 1\]"):
            fn()
    with pytest.raises(ValueError, match="decay must be"):
        la2.forward(q, q, q, torch.tensor([0.5]))          # one decay per head


def test_release_library_has_no_plan_overrides(lib):
    """Test knobs live only in the test build: the release library exports no override and reads no
    environment variable, so its plan depends on the arguments alone."""
    assert not any(hasattr(lib, n) for n in ("la2_test_set_plan", "la2_test_stream", "la2_test_reread"))
    import subprocess
    syms = subprocess.run(["nm", "-D", "--undefined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    assert "getenv" not in syms


def test_test_build_forces_plans():
    """The test build (libla2_testhooks.so) exports la2_test_set_plan; under binding.plan_override the
    wrappers call it and the forced plan shows in the workspace it asks for."""
    hooks = open(os.path.join(ROOT, "include", "la2_test_hooks.h")).read()
    assert "la2_test_set_plan" in hooks
    base = la2.la2_workspace_bytes(64, 4, 4096, 128, 128, 128, torch.bfloat16, False)
    assert base == 0                                  # 256 chains fill the GPU: no split
    with binding.plan_override(seg_tiles=4) as tl:
        assert hasattr(tl, "la2_test_set_plan")
        # 32 tiles per chain in segments of 4: 8 segments, a state per segment
        assert la2.la2_workspace_bytes(64, 4, 4096, 128, 128, 128, torch.bfloat16, False) == 256 * 8 * 128 * 128 * 4
    with binding.plan_override(seg_tiles=4, state_sub=2):
        assert la2.la2_workspace_bytes(64, 4, 4096, 128, 128, 128, torch.bfloat16, False) == 256 * 16 * 128 * 128 * 4
    assert la2.la2_workspace_bytes(64, 4, 4096, 128, 128, 128, torch.bfloat16, False) == 0   # restored


def test_stream_probe_validates_before_launch():
    """The test build's measurement stream refuses bad arguments before anything is enqueued."""
    tl = binding._load_test_library()
    src = (ctypes.c_void_p * 1)(0x100000)
    dst = (ctypes.c_void_p * 1)(0x200000)
    assert tl.la2_test_stream(src, 0, dst, 1, 1 << 20, 256, 256, 1, None) == SHAPE       # no source
    assert tl.la2_test_stream(src, 1, dst, 4, 1 << 20, 256, 256, 1, None) == SHAPE       # too many outputs
    assert tl.la2_test_stream(src, 1, dst, 1, (1 << 20) + 8, 256, 256, 1, None) == SHAPE
    assert tl.la2_test_stream(src, 1, dst, 1, 1 << 20, 256, 96, 1, None)  == SHAPE       # not whole waves
    bad = (ctypes.c_void_p * 1)(0x100008)
    assert tl.la2_test_stream(bad, 1, dst, 1, 1 << 20, 256, 256, 1, None) == NULLP          # misaligned


def test_reread_probe_validates_before_launch():
    """The test build's memory-side cache probe refuses bad arguments before anything is enqueued."""
    tl = binding._load_test_library()
    p = [0x100000, 0x200000, 0x300000, 0x400000]
    assert tl.la2_test_reread(*p, 1 << 20, 1 << 12, 3, 1, None) == SHAPE                 # no such mode
    assert tl.la2_test_reread(*p, 1 << 20, 24, 0, 1, None) == SHAPE                      # not 16-byte items
    assert tl.la2_test_reread(*p, 1 << 20, 3 << 10, 0, 1, None) == SHAPE                 # ragged last item
    assert tl.la2_test_reread(*p, 0, 1 << 12, 0, 1, None) == SHAPE
    assert tl.la2_test_reread(p[0], 0x200008, p[2], p[3], 1 << 20, 1 << 12, 0, 1, None) == NULLP   # misaligned
    assert tl.la2_test_reread(p[0], p[1], p[2], None, 1 << 20, 1 << 12, 0, 1, None) == NULLP


def test_noalloc_rejects_plans_beyond_its_scratch():
    """la2_forward_noalloc refuses, before anything is enqueued, sizes whose plan would need more
    segment states than its static scratch holds (reachable only through a forced plan: one tile per
    segment of a 2000-tile chain at d = d_v = 128 is 125 MiB of states), and validates like
    la2_forward otherwise."""
    SCR = 8
    assert "LA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in HEADER
    lib_ = la2.load_library()
    assert lib_.la2_forward_noalloc(None, P + MB, P + 2 * MB, None, P + 3 * MB, 1, 1, 64, 64, 64, 64, 1, None) == NULLP
    assert lib_.la2_forward_noalloc(P, P + MB, P + 2 * MB, None, P + 3 * MB, 1, 1, 64, 96, 64, 64, 1, None) == UNSUP
    assert lib_.la2_forward_noalloc(P, P + MB, P + 2 * MB, None, P + 3 * MB, 0, 1, 64, 64, 64, 64, 1, None) == SHAPE
    with binding.plan_override(seg_tiles=1) as tl:
        st = tl.la2_forward_noalloc(P, P + 4096 * MB, P + 8192 * MB, None, P + 12288 * MB, 1, 1, 128 * 2000,
                                    128, 128, 128, 1, None)
        assert st == SCR
    assert la2.la2_status_string(SCR) != "unknown status"
