"""CPU oracle for causal linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and it
never calls the HIP library; the two share no code.

Two independent formulations live here, both in fp64:

* ``forward`` / ``backward`` (C, ``la2_oracle.c``): the token recurrence
  S_t = lam S_{t-1} + k_t v_t^T, o_t = S_t^T q_t (page "Lightning Attention",
  lizeman.github.io llm-arch-kb, section 1, the numerator of the output and the
  prefix-sum recurrence, with identity feature map and no denominator), and its
  chain-rule backward with the reverse sweep R_t = lam R_{t+1} + q_t do_t^T.
  ``forward_rows`` / ``backward_rows`` evaluate single rows from the closed
  sums, for spot checks of very long sequences.  ``forward_normalized`` is
  the same section's whole output, phi(q)^T S / phi(q)^T z with the
  denominator sum z_t = lam z_{t-1} + phi(k_t) and phi = identity or elu + 1;
  ``backward_normalized`` its backward.
  ``backward_state`` is the backward of ``forward_state``: gradients of
  <o, do> + <state_out, dstate_out> including the one of the carried-in state.
* ``tiled_forward`` / ``tiled_backward`` (numpy, this file): the same page's
  section 2 derivation in its own order -- Step 1 split of each output row
  into an intra-tile and an inter-tile part, Step 2 the masked left product
  (Q_b K_b^T (.) M) V_b, Step 3 the right product Q_b S_{b-1}, Step 4 the
  state update S_b = S_{b-1} + K_b^T V_b -- with the decay weights that the
  token recurrence implies when lam < 1.

Arrays are numpy float64 in [B, H, T, d] layout (v, o, do: [B, H, T, dv]);
``lam`` is a length-H vector of per-head decays in (0, 1], or None for lam = 1.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load(path=None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.compile_oracle()
        _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


def _bind(lib):
    P = ctypes.POINTER(ctypes.c_double)
    I = ctypes.c_int64
    lib.la2_oracle_forward.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.la2_oracle_forward.restype = None
    lib.la2_oracle_forward_state.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
    lib.la2_oracle_forward_state.restype = None
    lib.la2_oracle_backward_state.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
    lib.la2_oracle_backward_state.restype = None
    lib.la2_oracle_backward_normalized.argtypes = [I, I, I, I, P, P, P, P, P, ctypes.c_int, P, P, P]
    lib.la2_oracle_backward_normalized.restype = None
    lib.la2_oracle_forward_normalized.argtypes = [I, I, I, I, P, P, P, P, ctypes.c_int, P]
    lib.la2_oracle_forward_normalized.restype = None
    lib.la2_oracle_backward.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P]
    lib.la2_oracle_backward.restype = None
    lib.la2_oracle_forward_rows.argtypes = [I, I, I, ctypes.c_double, P, P, P, I,
                                            ctypes.POINTER(ctypes.c_int64), P]
    lib.la2_oracle_forward_rows.restype = None
    lib.la2_oracle_backward_rows.argtypes = [I, I, I, ctypes.c_double, P, P, P, P, I,
                                             ctypes.POINTER(ctypes.c_int64), P, P, P]
    lib.la2_oracle_backward_rows.restype = None
    lib.la2_oracle_num_threads.argtypes = []
    lib.la2_oracle_num_threads.restype = ctypes.c_int
    lib.la2_oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.la2_oracle_set_num_threads.restype = None
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _chain_lams(lam, B, H):
    if lam is None:
        return np.ones(B * H, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64).reshape(H)
    return np.ascontiguousarray(np.tile(lam, B))


def num_threads(lib=None):
    """OpenMP threads the C oracle runs with."""
    return (lib or _load()).la2_oracle_num_threads()


def set_num_threads(n, lib=None):
    """Threads for the following C oracle calls (for timing; the results do not depend on it)."""
    (lib or _load()).la2_oracle_set_num_threads(int(n))


class Oracle:
    """Thin wrapper around one compiled copy of ``la2_oracle.c``."""

    def __init__(self, lib):
        self.lib = lib

    def forward(self, q, k, v, lam=None):
        """o for [B, H, T, d] inputs via the token recurrence."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, T, d = q.shape
        dv = v.shape[-1]
        o = np.empty((B, H, T, dv), dtype=np.float64)
        lams = _chain_lams(lam, B, H)
        self.lib.la2_oracle_forward(B * H, T, d, dv, _ptr(lams), _ptr(q), _ptr(k), _ptr(v), _ptr(o))
        return o

    def forward_state(self, q, k, v, lam=None, state_in=None):
        """(o, final state) for [B, H, T, d] inputs starting from ``state_in`` ([B, H, d, dv], None = 0)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, T, d = q.shape
        dv = v.shape[-1]
        o = np.empty((B, H, T, dv), dtype=np.float64)
        s_out = np.empty((B, H, d, dv), dtype=np.float64)
        s_in = None if state_in is None else _f64(state_in).reshape(B, H, d, dv)
        lams = _chain_lams(lam, B, H)
        self.lib.la2_oracle_forward_state(B * H, T, d, dv, _ptr(lams), _ptr(q), _ptr(k), _ptr(v),
                                          None if s_in is None else _ptr(s_in), _ptr(o), _ptr(s_out))
        return o, s_out

    def backward_normalized(self, q, k, v, do, lam=None, feature_map="elu1"):
        """(dq, dk, dv) of <o, do> for the normalized output."""
        fmap = {"identity": 0, "elu1": 1}[feature_map]
        q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
        B, H, T, d = q.shape
        dq, dk, dvo = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        lams = _chain_lams(lam, B, H)
        self.lib.la2_oracle_backward_normalized(B * H, T, d, v.shape[-1], _ptr(lams), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(do), fmap, _ptr(dq), _ptr(dk), _ptr(dvo))
        return dq, dk, dvo

    def backward_state(self, q, k, v, do, lam=None, state_in=None, dstate_out=None):
        """(dq, dk, dv, dstate_in) of <o, do> + <state_out, dstate_out> for the forward from state_in."""
        q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
        B, H, T, d = q.shape
        dv_ = v.shape[-1]
        dq, dk = np.empty_like(q), np.empty_like(k)
        dvo = np.empty_like(v)
        ds_in = np.empty((B, H, d, dv_), dtype=np.float64)
        lams = _chain_lams(lam, B, H)
        s_in = None if state_in is None else _f64(state_in)
        ds_out = None if dstate_out is None else _f64(dstate_out)
        self.lib.la2_oracle_backward_state(B * H, T, d, dv_, _ptr(lams), _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                                           None if s_in is None else _ptr(s_in),
                                           None if ds_out is None else _ptr(ds_out),
                                           _ptr(dq), _ptr(dk), _ptr(dvo), _ptr(ds_in))
        return dq, dk, dvo, ds_in

    def forward_normalized(self, q, k, v, lam=None, feature_map="elu1"):
        """Normalized output phi(q)^T S / phi(q)^T z with phi = identity or elu + 1."""
        fmap = {"identity": 0, "elu1": 1}[feature_map]
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, T, d = q.shape
        dv = v.shape[-1]
        o = np.empty((B, H, T, dv), dtype=np.float64)
        lams = _chain_lams(lam, B, H)
        self.lib.la2_oracle_forward_normalized(B * H, T, d, dv, _ptr(lams), _ptr(q), _ptr(k), _ptr(v), fmap,
                                               _ptr(o))
        return o

    def backward(self, q, k, v, do, lam=None):
        """(dq, dk, dv) of <o, do> via the forward and reverse recurrences."""
        q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
        B, H, T, d = q.shape
        dv = v.shape[-1]
        dq = np.empty_like(q)
        dk = np.empty_like(k)
        dvv = np.empty_like(v)
        lams = _chain_lams(lam, B, H)
        self.lib.la2_oracle_backward(B * H, T, d, dv, _ptr(lams), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(do), _ptr(dq), _ptr(dk), _ptr(dvv))
        return dq, dk, dvv

    def forward_rows(self, q, k, v, lam, rows):
        """o_t for t in ``rows`` of one chain ([T, d] inputs, scalar lam)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        T, d = q.shape
        dv = v.shape[-1]
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((rows.size, dv), dtype=np.float64)
        self.lib.la2_oracle_forward_rows(T, d, dv, float(1.0 if lam is None else lam), _ptr(q), _ptr(k),
                                         _ptr(v), rows.size,
                                         rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr(out))
        return out

    def backward_rows(self, q, k, v, do, lam, rows):
        """(dq_t, dk_t, dv_t) for t in ``rows`` of one chain."""
        q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
        T, d = q.shape
        dv = v.shape[-1]
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        gq = np.empty((rows.size, d))
        gk = np.empty((rows.size, d))
        gv = np.empty((rows.size, dv))
        self.lib.la2_oracle_backward_rows(T, d, dv, float(1.0 if lam is None else lam), _ptr(q), _ptr(k),
                                          _ptr(v), _ptr(do), rows.size,
                                          rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                          _ptr(gq), _ptr(gk), _ptr(gv))
        return gq, gk, gv

    def tiled_forward(self, q, k, v, lam=None, block=128):
        return tiled_forward(q, k, v, lam, block)

    def tiled_backward(self, q, k, v, do, lam=None, block=128):
        return tiled_backward(q, k, v, do, lam, block)


def load(path=None):
    """The oracle bound to ``path`` (default: the built ``liboracle.so``)."""
    return Oracle(_load(path))


def forward(q, k, v, lam=None):
    return load().forward(q, k, v, lam)


def forward_state(q, k, v, lam=None, state_in=None):
    return load().forward_state(q, k, v, lam, state_in)


def forward_normalized(q, k, v, lam=None, feature_map="elu1"):
    return load().forward_normalized(q, k, v, lam, feature_map)


def backward_state(q, k, v, do, lam=None, state_in=None, dstate_out=None):
    return load().backward_state(q, k, v, do, lam, state_in, dstate_out)


def backward_normalized(q, k, v, do, lam=None, feature_map="elu1"):
    return load().backward_normalized(q, k, v, do, lam, feature_map)


def backward(q, k, v, do, lam=None):
    return load().backward(q, k, v, do, lam)


def forward_rows(q, k, v, lam, rows):
    return load().forward_rows(q, k, v, lam, rows)


def backward_rows(q, k, v, do, lam, rows):
    return load().backward_rows(q, k, v, do, lam, rows)


# ---- tiled formulation (numpy) ---------------------------------------------

def _tiles(T, block):
    return [(s, min(s + block, T)) for s in range(0, T, block)]


def _decay_mask(n, lam, lower=True):
    """D[i, j] = lam^(i-j) for j <= i (lower) else 0; the causal mask M at lam = 1."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    e = (i - j) if lower else (j - i)
    return np.where(e >= 0, lam ** np.maximum(e, 0).astype(np.float64), 0.0)


def tiled_forward(q, k, v, lam=None, block=128):
    """Forward pass by the tile decomposition (intra left product + inter right product)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    o = np.empty((B, H, T, dv))
    lams = _chain_lams(lam, B, H).reshape(B, H)
    for b in range(B):
        for h in range(H):
            l = lams[b, h]
            S = np.zeros((d, dv))                       # state at the tile boundary
            for s, e in _tiles(T, block):
                n = e - s
                Qb, Kb, Vb = q[b, h, s:e], k[b, h, s:e], v[b, h, s:e]
                i = np.arange(n, dtype=np.float64)
                intra = ((Qb @ Kb.T) * _decay_mask(n, l)) @ Vb            # Step 2
                inter = (l ** (i + 1))[:, None] * (Qb @ S)               # Step 3
                o[b, h, s:e] = intra + inter                             # Step 1
                S = (l ** n) * S + ((l ** (n - 1 - i))[:, None] * Kb).T @ Vb   # Step 4
    return o


def tiled_backward(q, k, v, do, lam=None, block=128):
    """(dq, dk, dv) by the same tiling: a forward-order scan for dq, a reverse one for dk, dv."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    dq, dk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    lams = _chain_lams(lam, B, H).reshape(B, H)
    tiles = _tiles(T, block)
    for b in range(B):
        for h in range(H):
            l = lams[b, h]
            S = np.zeros((d, dv))
            for s, e in tiles:                                   # forward order: dq
                n = e - s
                Kb, Vb, Gb = k[b, h, s:e], v[b, h, s:e], do[b, h, s:e]
                i = np.arange(n, dtype=np.float64)
                dP = (Gb @ Vb.T) * _decay_mask(n, l)
                dq[b, h, s:e] = dP @ Kb + (l ** (i + 1))[:, None] * (Gb @ S.T)
                S = (l ** n) * S + ((l ** (n - 1 - i))[:, None] * Kb).T @ Vb
            R = np.zeros((d, dv))                                # reverse order: dk, dv
            for s, e in reversed(tiles):
                n = e - s
                Qb, Kb, Vb, Gb = q[b, h, s:e], k[b, h, s:e], v[b, h, s:e], do[b, h, s:e]
                j = np.arange(n, dtype=np.float64)
                D = _decay_mask(n, l)
                A = (Qb @ Kb.T) * D
                dP = (Gb @ Vb.T) * D
                w = (l ** (n - j))[:, None]
                dk[b, h, s:e] = dP.T @ Qb + w * (Vb @ R.T)
                dvv[b, h, s:e] = A.T @ Gb + w * (Kb @ R)
                R = (l ** n) * R + ((l ** j)[:, None] * Qb).T @ Gb
    return dq, dk, dvv
