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
        # GDN_ORACLE_LIBRARY names another build of gdn_oracle.c (an instrumented
        # one, say); by default the in-tree build
        path = os.environ.get("GDN_ORACLE_LIBRARY") or _build.LIB
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
                                 ip, ctypes.c_int, dp, ctypes.c_int, dp]
    L.orc_delta_rule.restype = None
    L.orc_gated_rmsnorm.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int, dp, dp, dp,
                                    ctypes.c_double, ctypes.c_int, dp]
    L.orc_round_binary16.argtypes = [ctypes.c_double]
    L.orc_round_binary16.restype = ctypes.c_double
    L.orc_round_binary16_array.argtypes = [dp, ctypes.c_longlong]
    L.orc_round_binary16_array.restype = None
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


def round_binary16(x):
    """Nearest IEEE binary16 value of every element (ties to even), as fp64."""
    x = _d(x).copy()
    lib().orc_round_binary16_array(_p(x), x.size)
    return x


STATE_FULL, STATE_F16_EVERY_TOKEN, STATE_F16_FINAL = 0, 1, 2


def delta_rule(q, k, v, a, b, S0, cu_seqlens, scale=1.0, heads=None, record_states=False,
               state_round=STATE_FULL):
    """Token-by-token gated delta rule.

    q, k [T, Hk, dk]; v [T, Hv, dv]; a, b [T, Hv]; S0 [n, Hv, dk, dv] (h = S^T).
    heads: optional list of value heads to compute (others left as S0 / zero).
    state_round: STATE_FULL, or binary16 storage of the state rounded after every
    token (STATE_F16_EVERY_TOKEN) or only at the end (STATE_F16_FINAL).
    Returns (o [T, Hv, dv], S_final [n, Hv, dk, dv], states or None) where states
    is [T, nh, dk, dv], the state after each token for the computed heads.
    """
    r = _delta_rule(q, k, v, a, b, S0, cu_seqlens, scale, heads, record_states, state_round, False)
    return r[0], r[1], r[2]


def _delta_rule(q, k, v, a, b, S0, cu_seqlens, scale, heads, record_states, state_round, record_u):
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
    null = ctypes.POINTER(ctypes.c_double)()
    states = np.zeros((T, nh, dk, dv)) if record_states else None
    us = np.zeros((T, nh, dv)) if record_u else None
    lib().orc_delta_rule(n, _ip(cu), Hk, Hv, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(b),
                         float(scale), _p(S), _p(o), hp, nh, _p(states) if record_states else null,
                         int(state_round), _p(us) if record_u else null)
    return o, S, states, us


def gated_rmsnorm(o, z, norm_w, eps=1e-6, gate="silu"):
    """out = o / sqrt(mean(o^2) + eps) * w * g(z), per (token, head) over dv, with
    g = SiLU (gate="silu") or the logistic sigmoid (gate="sigmoid").

    o, z [T, Hv, dv]; norm_w [dv].
    """
    o, z, w = _d(o), _d(z), _d(norm_w)
    T, Hv, dv = o.shape
    assert z.shape == o.shape and w.shape == (dv,)
    assert gate in ("silu", "sigmoid")
    out = np.zeros_like(o)
    lib().orc_gated_rmsnorm(T, Hv, dv, _p(o), _p(z), _p(w), float(eps), int(gate == "sigmoid"),
                            _p(out))
    return out


# ---------------------------------------------------------------------------
# Compositions of the steps above.
#
# Options shared by the compositions:
#   gates="direct": a, b are the decay and write strength themselves;
#   gates="raw":    a holds g and b holds beta per (token, value head), and the
#                   gates are a = exp(-softplus(g)), b = sigmoid(beta).  The pages
#                   name the gate kernels (ba_gates_*, compute_gdn_gates handles on
#                   the layer_struct.rs page) without their formula; this is the
#                   construction of a and b the synthetic workloads use.
#   norm_gate:      "silu" or "sigmoid" (the gdn_norm_sigmoid model kind).
#   state="f32" or "f16": binary16 storage of the recurrent state.
# ---------------------------------------------------------------------------

def gates_from_raw(g, beta):
    """a = exp(-softplus(g)) with softplus(g) = ln(1 + e^g), b = 1 / (1 + e^-beta)."""
    g, beta = _d(g), _d(beta)
    softplus = np.maximum(g, 0.0) + np.log1p(np.exp(-np.abs(g)))
    return np.exp(-softplus), 1.0 / (1.0 + np.exp(-beta))


def _gates(a, b, gates):
    assert gates in ("direct", "raw")
    return gates_from_raw(a, b) if gates == "raw" else (_d(a), _d(b))


def _round_mode(state, every_token):
    assert state in ("f32", "f16")
    if state == "f32":
        return STATE_FULL
    return STATE_F16_EVERY_TOKEN if every_token else STATE_F16_FINAL


def prefill(x_or_y, a, b, S0, cu_seqlens, Hk, Hv, dk, dv, *, conv_w=None, ring=None,
            scale=1.0, l2_eps=1e-6, z=None, norm_w=None, norm_eps=1e-6, heads=None,
            gates="direct", norm_gate="silu", state="f32", every_token_state=False):
    """Varlen prefill.  With conv_w/ring given, x_or_y is the pre-conv x and the
    conv + L2 front runs first; otherwise it is y = [q_hat | k_hat | v].
    With state="f16" the stored state S0 is widened, the sequence runs at full
    width and the final state is narrowed (every_token_state=True rounds after
    every token instead, which is what a token-by-token decode stores).
    Returns dict(o, out (gated norm, if z given), S, ring, y)."""
    res = {}
    if conv_w is not None:
        y, new_ring = conv_l2norm(x_or_y, conv_w, ring, cu_seqlens, Hk, Hv, dk, dv, l2_eps)
        res["ring"] = new_ring
    else:
        y = _d(x_or_y)
    res["y"] = y
    a, b = _gates(a, b, gates)
    q, k, v = split_qkv(y, Hk, Hv, dk, dv)
    o, S, _ = delta_rule(q, k, v, a, b, S0, cu_seqlens, scale=scale, heads=heads,
                         state_round=_round_mode(state, every_token_state))
    res["o"] = o
    res["S"] = S
    if z is not None:
        T = y.shape[0]
        res["out"] = gated_rmsnorm(o, _d(z).reshape(T, Hv, dv), norm_w, norm_eps, gate=norm_gate)
    return res


def decode(x, conv_w, ring, a, b, S0, Hk, Hv, dk, dv, *, scale=1.0, l2_eps=1e-6, z=None,
           norm_w=None, norm_eps=1e-6, heads=None, gates="direct", norm_gate="silu", state="f32"):
    """One token for each of n sequences.  x [n, C]; ring [n, K-1, C]; a, b [n, Hv];
    S0 [n, Hv, dk, dv].  Returns dict(o, out, S, ring)."""
    n = x.shape[0]
    cu = np.arange(n + 1, dtype=np.int32)
    return prefill(x, a, b, S0, cu, Hk, Hv, dk, dv, conv_w=conv_w, ring=ring, scale=scale,
                   l2_eps=l2_eps, z=z, norm_w=norm_w, norm_eps=norm_eps, heads=heads, gates=gates,
                   norm_gate=norm_gate, state=state, every_token_state=True)


def decode_tokens(x, conv_w, ring, a, b, S0, cu_tokens, Hk, Hv, dk, dv, **kw):
    """k_i consecutive tokens of each sequence i, as k_i one-token decodes in a row
    (the decode-once-per-token default of ``decode_batched`` on the
    transformer_layer.rs page): the state and the conv state advance over all of
    them.  x [sum k, C] packed per sequence; cu_tokens [n+1].
    Returns dict(o, out, S, ring)."""
    kw.setdefault("state", "f32")
    return prefill(x, a, b, S0, cu_tokens, Hk, Hv, dk, dv, conv_w=conv_w, ring=ring,
                   every_token_state=True, **kw)


def verify(x, conv_w, ring, a, b, S0, cu_ks, Hk, Hv, dk, dv, *, scale=1.0, l2_eps=1e-6,
           z=None, norm_w=None, norm_eps=1e-6, heads=None, gates="direct", norm_gate="silu",
           state="f32", record_u=False):
    """k_i rows for each sequence i from state S0[i]; the conv state is only read.

    x [sum k, C]; cu_ks [n+1].  Returns dict(o, out, S_final, states) where
    states[t] is the state after packed row t (for the computed heads) and
    S_final[i] the state after the last row of sequence i.  Every intermediate
    state is a stored state, so with state="f16" each one is rounded."""
    y, _ = conv_l2norm(x, conv_w, ring, cu_ks, Hk, Hv, dk, dv, l2_eps)
    q, k, v = split_qkv(y, Hk, Hv, dk, dv)
    ag, bg = _gates(a, b, gates)
    o, S, states, us = _delta_rule(q, k, v, ag, bg, S0, cu_ks, scale, heads, True,
                                   _round_mode(state, True), record_u)
    res = {"o": o, "S": S, "states": states, "y": y, "a": ag, "u": us, "k": k}
    if z is not None:
        T = y.shape[0]
        res["out"] = gated_rmsnorm(o, _d(z).reshape(T, Hv, dv), norm_w, norm_eps, gate=norm_gate)
    return res


def commit(states, n_accepted, cu_ks, ring, x):
    """Fold the accepted prefix: for sequence i with n_i accepted rows (1..k_i) the
    new state is the state after row n_i - 1, and the conv state becomes the last
    K-1 rows of [old ring ; x rows 0..n_i-1].

    states [sum k, ...] as returned by ``verify``; ring [n, K-1, C]; x [sum k, C].
    Returns (S_new [n, ...], ring_new [n, K-1, C])."""
    cu = np.asarray(cu_ks, dtype=np.int64)
    n = cu.shape[0] - 1
    S_new = np.stack([states[cu[i] + int(n_accepted[i]) - 1] for i in range(n)])
    return S_new, _advance_ring(ring, x, cu, n_accepted)


def _advance_ring(ring, x, cu, n_accepted):
    ring = _d(ring)
    x = _d(x)
    R = ring.shape[1]
    ring_new = np.empty_like(ring)
    for i in range(cu.shape[0] - 1):
        cat = np.concatenate([ring[i], x[cu[i]: cu[i] + int(n_accepted[i])]], axis=0)
        ring_new[i] = cat[cat.shape[0] - R:]
    return ring_new


# ---------------------------------------------------------------------------
# Write-on-accept verify (the gdn_wy4_woa_k / gdn_wy4_fold_k handles and the
# gdn_woa_bind / gdn_fold_accepted entries: layer_struct.rs and trait_layer.rs
# pages).  The pages give the interface, not the contents of the stash; the
# reading taken here: the verify writes no state, it keeps for every row what
# the rank-1 update S_t = a_t S_{t-1} + u_t k_t^T needs -- u_t per value head,
# k_hat_t per key head and a_t per value head -- and the fold applies the updates
# of the accepted rows to the stored state, once per row in order.
# ---------------------------------------------------------------------------

def verify_woa(x, conv_w, ring, a, b, S0, cu_ks, Hk, Hv, dk, dv, **kw):
    """Outputs as ``verify``; returns dict(o, out, stash_k [T, Hk, dk],
    stash_u [T, Hv, dv], stash_a [T, Hv]) and the recorded states for checks."""
    r = verify(x, conv_w, ring, a, b, S0, cu_ks, Hk, Hv, dk, dv, record_u=True, **kw)
    r["stash_k"] = np.ascontiguousarray(r["k"])
    r["stash_u"] = r["u"]
    r["stash_a"] = r["a"]
    return r


def fold_accepted(S0, stash_k, stash_u, stash_a, cu_ks, n_accepted, ring, x, *, state="f32"):
    """For sequence i and its accepted rows t = 0..n_i-1 (1 <= n_i <= k_i), in order:
    h <- a_t h + k_t u_t^T per value head (h = S^T, so this is S <- a S + u k^T),
    rounded to binary16 after every row when state="f16".  The conv state
    advances over the accepted rows as in ``commit``.
    Returns (S_new [n, Hv, dk, dv], ring_new)."""
    S = _d(S0).copy()
    stash_k, stash_u, stash_a = _d(stash_k), _d(stash_u), _d(stash_a)
    cu = np.asarray(cu_ks, dtype=np.int64)
    n = cu.shape[0] - 1
    Hk, Hv = stash_k.shape[1], stash_u.shape[1]
    for i in range(n):
        for t in range(cu[i], cu[i] + int(n_accepted[i])):
            for h in range(Hv):
                g = h * Hk // Hv
                S[i, h] = stash_a[t, h] * S[i, h] + np.outer(stash_k[t, g], stash_u[t, h])
                if state == "f16":
                    S[i, h] = round_binary16(S[i, h])
    return S, _advance_ring(ring, x, cu, n_accepted)
