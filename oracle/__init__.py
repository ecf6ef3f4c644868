"""fp64 CPU oracle of the Gated DeltaNet mixer core.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
cpu_baseline leg of bench.py may import this package.  It shares no code with
the HIP library under ``linear_attention_ssm_core_amd``; the two sides meet
only through the seeded input generator (``linear_attention_ssm_core_amd.workloads``),
which holds none of the method's arithmetic.

The arithmetic lives in ``gdn_oracle.c`` (token-by-token recurrence, conv1d +
SiLU, L2 norm, gated RMSNorm, all fp64).  This module marshals numpy arrays into
it and composes the decode, verify, commit and prefill chains from those steps,
in the order the pages' entry points describe them:

* decode of one token per sequence (``decode_multi_seq`` on the
  metrale_model_layers/layer/transformer_layer.rs page): conv update of one row
  with the conv state, L2, one recurrence step, optional gated norm;
* batched verify (``decode_verify_multi``, same page, and the WY pointer-table
  constants there): k rows per sequence from the state in table 0, the state
  after every row recorded; the conv state is read, not written;
* commit (``gdn_fold_accepted`` on the metrale_model_layers/layers/qwen3_ssm/
  trait_layer.rs page): the state after the last accepted row becomes the
  sequence state and the conv state advances over the accepted rows;
* varlen prefill (``prefill_gdn_full_batched_fla_varlen``, trait_layer.rs page):
  sequences packed back to back, delimited by ``cu_seqlens``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build(force=True)
        _lib = load_library(path)
    return _lib


class use_library:
    """Context manager that routes every oracle call through another build of
    ``gdn_oracle.c`` (the planted-mistake tests use it)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.prev = _lib
        _lib = load_library(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def load_library(path):
    L = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    L.orc_conv_l2norm.argtypes = [ctypes.c_int, ip, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, dp, dp, dp, ctypes.c_double, dp]
    L.orc_conv_l2norm.restype = None
    L.orc_delta_rule.argtypes = [ctypes.c_int, ip, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp,
                                 ip, ctypes.c_int, dp]
    L.orc_delta_rule.restype = None
    L.orc_gated_rmsnorm.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int, dp, dp, dp,
                                    ctypes.c_double, dp]
    L.orc_gated_rmsnorm.restype = None
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_set_num_threads.argtypes = [ctypes.c_int]
    return L


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def _d(a):
    """C-contiguous float64 copy (exact widening of fp32/bf16-valued inputs)."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def conv_dim(Hk, Hv, dk, dv):
    return 2 * Hk * dk + Hv * dv


def conv_l2norm(x, conv_w, ring, cu_seqlens, Hk, Hv, dk, dv, l2_eps=1e-6):
    """Causal conv1d + SiLU + L2(q, k) over packed rows.

    x [T, C], conv_w [C, K], ring [n, K-1, C] (oldest row first).
    Returns (y [T, C] = [q_hat | k_hat | v], new ring [n, K-1, C]).
    """
    x = _d(x)
    w = _d(conv_w)
    ring = _d(ring).copy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, C = x.shape
    K = w.shape[1]
    assert C == conv_dim(Hk, Hv, dk, dv) and w.shape[0] == C
    n = cu.shape[0] - 1
    assert ring.shape == (n, K - 1, C)
    y = np.zeros_like(x)
    lib().orc_conv_l2norm(n, _ip(cu), Hk, Hv, dk, dv, K, _p(x), _p(w), _p(ring), float(l2_eps), _p(y))
    return y, ring


def split_qkv(y, Hk, Hv, dk, dv):
    """Views q [T, Hk, dk], k [T, Hk, dk], v [T, Hv, dv] of the packed [q|k|v] rows."""
    T = y.shape[0]
    q = y[:, : Hk * dk].reshape(T, Hk, dk)
    k = y[:, Hk * dk: 2 * Hk * dk].reshape(T, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    return q, k, v


def delta_rule(q, k, v, a, b, S0, cu_seqlens, scale=1.0, heads=None, record_states=False):
    """Token-by-token gated delta rule.

    q, k [T, Hk, dk]; v [T, Hv, dv]; a, b [T, Hv]; S0 [n, Hv, dk, dv] (h = S^T).
    heads: optional list of value heads to compute (others left as S0 / zero).
    Returns (o [T, Hv, dv], S_final [n, Hv, dk, dv], states or None) where states
    is [T, nh, dk, dv], the state after each token for the computed heads.
    """
    q, k, v, a, b = _d(q), _d(k), _d(v), _d(a), _d(b)
    S = _d(S0).copy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    n = cu.shape[0] - 1
    assert S.shape == (n, Hv, dk, dv)
    assert a.shape == (T, Hv) and b.shape == (T, Hv)
    o = np.zeros((T, Hv, dv))
    if heads is None:
        hl = None
        nh = Hv
        hp = ctypes.POINTER(ctypes.c_int32)()
    else:
        hl = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        nh = hl.shape[0]
        hp = _ip(hl)
    states = np.zeros((T, nh, dk, dv)) if record_states else None
    sp = _p(states) if record_states else ctypes.POINTER(ctypes.c_double)()
    lib().orc_delta_rule(n, _ip(cu), Hk, Hv, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(b),
                         float(scale), _p(S), _p(o), hp, nh, sp)
    return o, S, states


def gated_rmsnorm(o, z, norm_w, eps=1e-6):
    """out = o / sqrt(mean(o^2) + eps) * w * SiLU(z), per (token, head) over dv.

    o, z [T, Hv, dv]; norm_w [dv].
    """
    o, z, w = _d(o), _d(z), _d(norm_w)
    T, Hv, dv = o.shape
    assert z.shape == o.shape and w.shape == (dv,)
    out = np.zeros_like(o)
    lib().orc_gated_rmsnorm(T, Hv, dv, _p(o), _p(z), _p(w), float(eps), _p(out))
    return out


# ---------------------------------------------------------------------------
# Compositions of the steps above.
# ---------------------------------------------------------------------------

def prefill(x_or_y, a, b, S0, cu_seqlens, Hk, Hv, dk, dv, *, conv_w=None, ring=None,
            scale=1.0, l2_eps=1e-6, z=None, norm_w=None, norm_eps=1e-6, heads=None):
    """Varlen prefill.  With conv_w/ring given, x_or_y is the pre-conv x and the
    conv + L2 front runs first; otherwise it is y = [q_hat | k_hat | v].
    Returns dict(o, out (gated norm, if z given), S, ring, y)."""
    res = {}
    if conv_w is not None:
        y, new_ring = conv_l2norm(x_or_y, conv_w, ring, cu_seqlens, Hk, Hv, dk, dv, l2_eps)
        res["ring"] = new_ring
    else:
        y = _d(x_or_y)
    res["y"] = y
    q, k, v = split_qkv(y, Hk, Hv, dk, dv)
    o, S, _ = delta_rule(q, k, v, a, b, S0, cu_seqlens, scale=scale, heads=heads)
    res["o"] = o
    res["S"] = S
    if z is not None:
        T = y.shape[0]
        res["out"] = gated_rmsnorm(o, _d(z).reshape(T, Hv, dv), norm_w, norm_eps)
    return res


def decode(x, conv_w, ring, a, b, S0, Hk, Hv, dk, dv, *, scale=1.0, l2_eps=1e-6, z=None,
           norm_w=None, norm_eps=1e-6, heads=None):
    """One token for each of n sequences.  x [n, C]; ring [n, K-1, C]; a, b [n, Hv];
    S0 [n, Hv, dk, dv].  Returns dict(o, out, S, ring)."""
    n = x.shape[0]
    cu = np.arange(n + 1, dtype=np.int32)
    return prefill(x, a, b, S0, cu, Hk, Hv, dk, dv, conv_w=conv_w, ring=ring, scale=scale,
                   l2_eps=l2_eps, z=z, norm_w=norm_w, norm_eps=norm_eps, heads=heads)


def verify(x, conv_w, ring, a, b, S0, cu_ks, Hk, Hv, dk, dv, *, scale=1.0, l2_eps=1e-6,
           z=None, norm_w=None, norm_eps=1e-6, heads=None):
    """k_i rows for each sequence i from state S0[i]; the conv state is only read.

    x [sum k, C]; cu_ks [n+1].  Returns dict(o, out, S_final, states) where
    states[t] is the state after packed row t (for the computed heads) and
    S_final[i] the state after the last row of sequence i."""
    y, _ = conv_l2norm(x, conv_w, ring, cu_ks, Hk, Hv, dk, dv, l2_eps)
    q, k, v = split_qkv(y, Hk, Hv, dk, dv)
    o, S, states = delta_rule(q, k, v, a, b, S0, cu_ks, scale=scale, heads=heads,
                              record_states=True)
    res = {"o": o, "S": S, "states": states, "y": y}
    if z is not None:
        T = y.shape[0]
        res["out"] = gated_rmsnorm(o, _d(z).reshape(T, Hv, dv), norm_w, norm_eps)
    return res


def commit(states, n_accepted, cu_ks, ring, x):
    """Fold the accepted prefix: for sequence i with n_i accepted rows (1..k_i) the
    new state is the state after row n_i - 1, and the conv state becomes the last
    K-1 rows of [old ring ; x rows 0..n_i-1].

    states [sum k, ...] as returned by ``verify``; ring [n, K-1, C]; x [sum k, C].
    Returns (S_new [n, ...], ring_new [n, K-1, C])."""
    cu = np.asarray(cu_ks, dtype=np.int64)
    n = cu.shape[0] - 1
    ring = _d(ring)
    x = _d(x)
    R = ring.shape[1]
    S_new = np.stack([states[cu[i] + int(n_accepted[i]) - 1] for i in range(n)])
    ring_new = np.empty_like(ring)
    for i in range(n):
        cat = np.concatenate([ring[i], x[cu[i]: cu[i] + int(n_accepted[i])]], axis=0)
        ring_new[i] = cat[cat.shape[0] - R:]
    return S_new, ring_new
