"""Thin ctypes binding of ``include/la2.h``: argument marshalling only.

Every step of the computation runs in the HIP library ``lib/libla2.so``; this
module only checks tensors, passes their device pointers, sizes and torch's
current HIP stream, and turns status codes into exceptions.  There is no CPU
path: if the library is missing or a tensor is not on the GPU, it raises.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libla2.so")
LA2_ABI_VERSION = 8   # the include/la2.h version these signatures follow

LA2_F32 = 0
LA2_BF16 = 1
_DTYPES = {torch.float32: LA2_F32, torch.bfloat16: LA2_BF16}

LA2_PHI_IDENTITY = 0
LA2_PHI_ELU1 = 1
_FMAPS = {"identity": LA2_PHI_IDENTITY, "elu1": LA2_PHI_ELU1}

EXPORTS = ("la2_forward", "la2_forward_state", "la2_decode_step", "la2_forward_normalized", "la2_forward_serial",
           "la2_backward", "la2_backward_state", "la2_backward_normalized", "la2_backward_normalized_saved",
           "la2_backward_saved", "la2_workspace_bytes", "la2_normalized_workspace_bytes", "la2_status_string",
           "la2_abi_version")

_lib = None


class LA2Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({la2_status_string(status)})")


def load_library(path=LIB_PATH):
    """Load (once) and return the ctypes handle of the built HIP library."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.la2_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.la2_forward.restype = i32
    lib.la2_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.la2_backward.restype = i32
    lib.la2_backward_saved.argtypes = lib.la2_backward.argtypes
    lib.la2_backward_saved.restype = i32
    lib.la2_forward_state.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp, sz, vp]
    lib.la2_forward_state.restype = i32
    lib.la2_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.la2_decode_step.restype = i32
    lib.la2_forward_normalized.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, i32, vp, sz, vp]
    lib.la2_forward_normalized.restype = i32
    lib.la2_backward_state.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32,
                                       vp, sz, vp]
    lib.la2_backward_state.restype = i32
    lib.la2_forward_serial.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    lib.la2_forward_serial.restype = i32
    lib.la2_backward_normalized.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32,
                                            i32, vp, sz, vp]
    lib.la2_backward_normalized.restype = i32
    lib.la2_backward_normalized_saved.argtypes = lib.la2_backward_normalized.argtypes
    lib.la2_backward_normalized_saved.restype = i32
    lib.la2_normalized_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32, i32]
    lib.la2_normalized_workspace_bytes.restype = sz
    lib.la2_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32]
    lib.la2_workspace_bytes.restype = sz
    lib.la2_status_string.argtypes = [i32]
    lib.la2_status_string.restype = ctypes.c_char_p
    lib.la2_abi_version.argtypes = []
    lib.la2_abi_version.restype = i32
    if lib.la2_abi_version() != LA2_ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.la2_abi_version()}, this binding expects "
                           f"{LA2_ABI_VERSION}; rebuild it with __graft_entry__.build()")
    if path == LIB_PATH:
        _lib = lib
    return lib


def la2_status_string(status):
    return load_library().la2_status_string(int(status)).decode()


def la2_abi_version():
    return load_library().la2_abi_version()


def dtype_code(dtype):
    try:
        return _DTYPES[dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {dtype}; use torch.float32 or torch.bfloat16") from None


def la2_workspace_bytes(B, H, T, d, d_v, block, dtype, backward):
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    n = load_library().la2_workspace_bytes(B, H, T, d, d_v, block, code, 1 if backward else 0)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("unsupported sizes for la2_workspace_bytes")
    return n


def feature_map_code(feature_map):
    if isinstance(feature_map, int):
        return feature_map
    try:
        return _FMAPS[feature_map]
    except KeyError:
        raise ValueError(f"unknown feature map {feature_map!r}; use 'identity' or 'elu1'") from None


def la2_normalized_workspace_bytes(B, H, T, d, d_v, feature_map, block, dtype, backward=False):
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    n = load_library().la2_normalized_workspace_bytes(B, H, T, d, d_v, feature_map_code(feature_map), block, code,
                                                      1 if backward else 0)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("unsupported arguments for la2_normalized_workspace_bytes")
    return n


def _dev_ptr(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _decay_ptr(decay):
    if decay is None:
        return None
    if decay.dtype != torch.float32:
        raise TypeError("decay must be float32")
    return _dev_ptr(decay, "decay")


def la2_forward(q, k, v, decay, o, block, workspace=None, stream=None):
    """Enqueue o = attention(q, k, v) on ``stream`` (default: torch's current stream)."""
    B, H, T, d = q.shape
    d_v = v.shape[-1]
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().la2_forward(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _decay_ptr(decay), _dev_ptr(o, "o"),
        B, H, T, d, d_v, int(block), dtype_code(q.dtype), _dev_ptr(workspace, "workspace"), ws, _stream(stream))
    if st != 0:
        raise LA2Error(st, "la2_forward")


def _state_ptr(t, name):
    if t is None:
        return None
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return _dev_ptr(t, name)


def la2_forward_state(q, k, v, decay, state_in, o, state_out, block, workspace=None, stream=None):
    """Enqueue o = attention(q, k, v) from the carried-in fp32 state ``state_in`` ([B, H, d, d_v] or
    None) and write the final state to ``state_out`` (same shape, may be ``state_in``, or None)."""
    B, H, T, d = q.shape
    d_v = v.shape[-1]
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and tuple(t.shape) != (B, H, d, d_v):
            raise ValueError(f"{name} must be [B, H, d, d_v] = {(B, H, d, d_v)}")
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().la2_forward_state(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _decay_ptr(decay), _state_ptr(state_in, "state_in"),
        _dev_ptr(o, "o"), _state_ptr(state_out, "state_out"),
        B, H, T, d, d_v, int(block), dtype_code(q.dtype), _dev_ptr(workspace, "workspace"), ws, _stream(stream))
    if st != 0:
        raise LA2Error(st, "la2_forward_state")


def la2_decode_step(q, k, v, decay, o, state, stream=None):
    """Enqueue one token per chain: state <- lam state + k v^T (in place), o = state^T q.
    q, k: [B, H, d]; v, o: [B, H, d_v]; state: fp32 [B, H, d, d_v]."""
    B, H, d = q.shape
    d_v = v.shape[-1]
    if tuple(state.shape) != (B, H, d, d_v):
        raise ValueError(f"state must be [B, H, d, d_v] = {(B, H, d, d_v)}")
    st = load_library().la2_decode_step(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _decay_ptr(decay), _dev_ptr(o, "o"),
        _state_ptr(state, "state"), B, H, d, d_v, dtype_code(q.dtype), _stream(stream))
    if st != 0:
        raise LA2Error(st, "la2_decode_step")


def la2_forward_normalized(q, k, v, decay, o, feature_map, block, workspace=None, stream=None):
    """Enqueue the normalized output o = phi(q)^T S / phi(q)^T z (feature_map 'identity' or 'elu1')."""
    B, H, T, d = q.shape
    d_v = v.shape[-1]
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().la2_forward_normalized(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _decay_ptr(decay), _dev_ptr(o, "o"),
        B, H, T, d, d_v, feature_map_code(feature_map), int(block), dtype_code(q.dtype),
        _dev_ptr(workspace, "workspace"), ws, _stream(stream))
    if st != 0:
        raise LA2Error(st, "la2_forward_normalized")


def la2_forward_serial(q, k, v, decay, o, stream=None):
    """Enqueue o = attention(q, k, v) computed one position after another (comparison kernel)."""
    B, H, T, d = q.shape
    d_v = v.shape[-1]
    st = load_library().la2_forward_serial(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _decay_ptr(decay), _dev_ptr(o, "o"),
        B, H, T, d, d_v, dtype_code(q.dtype), _stream(stream))
    if st != 0:
        raise LA2Error(st, "la2_forward_serial")


def la2_backward_normalized(q, k, v, decay, o, dout, dq, dk, dv, feature_map, block, workspace=None, stream=None,
                            saved=False):
    """Enqueue (dq, dk, dv) = gradients of <o, dout> for the normalized forward that returned o.
    ``saved``: call la2_backward_normalized_saved, reusing what la2_forward_normalized on the same
    inputs left in ``workspace`` (which must then be the backward-sized workspace it was given)."""
    B, H, T, d = q.shape
    d_v = v.shape[-1]
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    fn = lib.la2_backward_normalized_saved if saved else lib.la2_backward_normalized
    st = fn(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _decay_ptr(decay), _dev_ptr(o, "o"),
        _dev_ptr(dout, "dout"), _dev_ptr(dq, "dq"), _dev_ptr(dk, "dk"), _dev_ptr(dv, "dv"),
        B, H, T, d, d_v, feature_map_code(feature_map), int(block), dtype_code(q.dtype),
        _dev_ptr(workspace, "workspace"), ws, _stream(stream))
    if st != 0:
        raise LA2Error(st, "la2_backward_normalized_saved" if saved else "la2_backward_normalized")


def la2_backward_normalized_saved(q, k, v, decay, o, dout, dq, dk, dv, feature_map, block, workspace=None,
                                  stream=None):
    """la2_backward_normalized reusing the forward's denominators, phi(q), phi(k) and segment states
    in ``workspace`` (see include/la2.h)."""
    la2_backward_normalized(q, k, v, decay, o, dout, dq, dk, dv, feature_map, block, workspace, stream, saved=True)


def la2_backward(q, k, v, decay, dout, dq, dk, dv, block, workspace=None, stream=None, saved=False):
    """Enqueue (dq, dk, dv) = gradients of <attention(q, k, v), dout>.  ``saved``: call
    la2_backward_saved, reusing the segment states the la2_forward call on the same inputs left in
    ``workspace``."""
    B, H, T, d = q.shape
    d_v = v.shape[-1]
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    fn = lib.la2_backward_saved if saved else lib.la2_backward
    st = fn(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _decay_ptr(decay), _dev_ptr(dout, "dout"),
        _dev_ptr(dq, "dq"), _dev_ptr(dk, "dk"), _dev_ptr(dv, "dv"),
        B, H, T, d, d_v, int(block), dtype_code(q.dtype), _dev_ptr(workspace, "workspace"), ws, _stream(stream))
    if st != 0:
        raise LA2Error(st, "la2_backward_saved" if saved else "la2_backward")


def la2_backward_state(q, k, v, decay, state_in, dout, dstate_out, dq, dk, dv, dstate_in, block, workspace=None,
                       stream=None):
    """Enqueue the backward of la2_forward_state: (dq, dk, dv) and d(state_in) (fp32 [B, H, d, d_v] or
    None) of <o, dout> + <state_out, dstate_out> (state_in, dstate_out: fp32 [B, H, d, d_v] or None)."""
    B, H, T, d = q.shape
    d_v = v.shape[-1]
    for name, t in (("state_in", state_in), ("dstate_out", dstate_out), ("dstate_in", dstate_in)):
        if t is not None and tuple(t.shape) != (B, H, d, d_v):
            raise ValueError(f"{name} must be [B, H, d, d_v] = {(B, H, d, d_v)}")
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().la2_backward_state(
        _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _decay_ptr(decay), _state_ptr(state_in, "state_in"),
        _dev_ptr(dout, "dout"), _state_ptr(dstate_out, "dstate_out"), _dev_ptr(dq, "dq"), _dev_ptr(dk, "dk"),
        _dev_ptr(dv, "dv"), _state_ptr(dstate_in, "dstate_in"),
        B, H, T, d, d_v, int(block), dtype_code(q.dtype), _dev_ptr(workspace, "workspace"), ws, _stream(stream))
    if st != 0:
        raise LA2Error(st, "la2_backward_state")


def la2_backward_saved(q, k, v, decay, dout, dq, dk, dv, block, workspace=None, stream=None):
    """la2_backward reusing the forward's segment states in ``workspace`` (see include/la2.h)."""
    la2_backward(q, k, v, decay, dout, dq, dk, dv, block, workspace, stream, saved=True)


def _check_same(q, k, v, other=None):
    for name, t in (("k", k), ("v", v)) + ((("dout", other),) if other is not None else ()):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype and device")
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B, H, T, d] and v [B, H, T, d_v]")


def workspace_for(q, v, block, backward):
    B, H, T, d = q.shape
    n = la2_workspace_bytes(B, H, T, d, v.shape[-1], block, q.dtype, backward)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def forward(q, k, v, decay=None, block=128, workspace=None):
    """Allocate o (and the workspace if none is given) and run the forward pass."""
    _check_same(q, k, v)
    o = torch.empty(q.shape[:3] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, v, block, False)
    la2_forward(q, k, v, decay, o, block, workspace)
    return o


def forward_state(q, k, v, decay=None, block=128, state_in=None, workspace=None):
    """Allocate o and the final state and run the forward from ``state_in`` (None = zero state);
    returns (o, state_out)."""
    _check_same(q, k, v)
    B, H, T, d = q.shape
    o = torch.empty(q.shape[:3] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    state_out = torch.empty((B, H, d, v.shape[-1]), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, v, block, False)
    la2_forward_state(q, k, v, decay, state_in, o, state_out, block, workspace)
    return o, state_out


def normalized_workspace_for(q, v, feature_map, block, backward=False):
    B, H, T, d = q.shape
    n = la2_normalized_workspace_bytes(B, H, T, d, v.shape[-1], feature_map, block, q.dtype, backward)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def forward_normalized(q, k, v, decay=None, block=128, feature_map="elu1", workspace=None):
    """Allocate o (and the workspace if none is given) and run the normalized forward."""
    _check_same(q, k, v)
    o = torch.empty(q.shape[:3] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = normalized_workspace_for(q, v, feature_map, block)
    la2_forward_normalized(q, k, v, decay, o, feature_map, block, workspace)
    return o


def forward_serial(q, k, v, decay=None):
    """Allocate o and run the token-serial recurrence."""
    _check_same(q, k, v)
    o = torch.empty(q.shape[:3] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    la2_forward_serial(q, k, v, decay, o)
    return o


def backward_state(q, k, v, dout, decay=None, block=128, state_in=None, dstate_out=None, workspace=None):
    """Allocate (dq, dk, dv, dstate_in) and run the backward of forward_state."""
    _check_same(q, k, v, dout)
    B, H, T, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dstate_in = torch.empty((B, H, d, v.shape[-1]), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, v, block, True)
    la2_backward_state(q, k, v, decay, state_in, dout, dstate_out, dq, dk, dv, dstate_in, block, workspace)
    return dq, dk, dv, dstate_in


def backward_normalized(q, k, v, o, dout, decay=None, block=128, feature_map="elu1", workspace=None, saved=False):
    """Allocate (dq, dk, dv) and run the normalized backward (o: the normalized forward's output;
    ``saved``: ``workspace`` is the backward-sized one the forward on the same inputs was given)."""
    _check_same(q, k, v, dout)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        if saved:
            raise ValueError("saved=True needs the workspace the normalized forward filled")
        workspace = normalized_workspace_for(q, v, feature_map, block, True)
    la2_backward_normalized(q, k, v, decay, o, dout, dq, dk, dv, feature_map, block, workspace, saved=saved)
    return dq, dk, dv


def decode_step(q, k, v, state, decay=None):
    """One token per chain from ``state`` (updated in place); q, k: [B, H, d], v: [B, H, d_v]; returns o."""
    if k.shape != q.shape or v.shape[:2] != q.shape[:2] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k must be [B, H, d] and v [B, H, d_v] of one dtype")
    o = torch.empty_like(v)
    la2_decode_step(q, k, v, decay, o, state)
    return o


def backward(q, k, v, dout, decay=None, block=128, workspace=None, saved=False):
    """Allocate (dq, dk, dv) and run the backward pass (``saved``: reuse the forward's segment states,
    which requires the workspace that forward() was given)."""
    _check_same(q, k, v, dout)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        if saved:
            raise ValueError("saved=True needs the workspace of the forward call")
        workspace = workspace_for(q, v, block, True)
    la2_backward(q, k, v, decay, dout, dq, dk, dv, block, workspace, saved=saved)
    return dq, dk, dv


class LA2Function(torch.autograd.Function):
    """autograd bridge: forward and backward both run in the HIP library."""

    @staticmethod
    def forward(ctx, q, k, v, decay=None, block=128):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        # one workspace for both passes: the backward reuses the segment states the forward leaves
        ws = workspace_for(q, v, block, True)
        ctx.save_for_backward(q, k, v, decay)
        ctx.block = block
        ctx.ws = ws
        return forward(q, k, v, decay, block, ws)

    @staticmethod
    def backward(ctx, dout):
        q, k, v, decay = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, dout.contiguous(), decay, ctx.block, ctx.ws, saved=ctx.ws is not None)
        return dq, dk, dv, None, None


def lightning_attention(q, k, v, decay=None, block=128):
    """o = attention(q, k, v) with autograd support."""
    return LA2Function.apply(q, k, v, decay, block)


class LA2StateFunction(torch.autograd.Function):
    """autograd bridge of the state-carrying forward (la2_forward_state / la2_backward_state):
    (o, state_out) from (q, k, v, state_in), differentiable in q, k, v and state_in, so a long
    sequence can be trained in chunks, each chunk started from the state the previous one left."""

    @staticmethod
    def forward(ctx, q, k, v, state_in, decay=None, block=128):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        s_in = None if state_in is None else state_in.contiguous()
        o, state_out = forward_state(q, k, v, decay, block, s_in)
        ctx.save_for_backward(q, k, v, s_in, decay)
        ctx.block = block
        return o, state_out

    @staticmethod
    def backward(ctx, dout, dstate_out):
        q, k, v, s_in, decay = ctx.saved_tensors
        if dout is None:
            dout = torch.zeros(q.shape[:3] + (v.shape[-1],), dtype=q.dtype, device=q.device)
        dq, dk, dv, dstate_in = backward_state(q, k, v, dout.contiguous(), decay, ctx.block, s_in,
                                               None if dstate_out is None else dstate_out.contiguous())
        return dq, dk, dv, (dstate_in if s_in is not None else None), None, None


def lightning_attention_state(q, k, v, state_in=None, decay=None, block=128):
    """(o, state_out) = attention(q, k, v) carried in from state_in (fp32 [B, H, d, d_v] or None),
    with autograd support through q, k, v and state_in."""
    return LA2StateFunction.apply(q, k, v, state_in, decay, block)
