"""Pins of the oracle's variant forms (CPU only): binary16 state storage, the raw
gate inputs, the sigmoid-gated norm, the write-on-accept stash and fold, and the
decode of several consecutive tokens per sequence.

Each is checked against something other than the oracle itself: numpy's IEEE
binary16 conversion, scipy's logistic functions, torch's RMSNorm, exact rational
evaluation of the literal rule, the independent chunked form, or constructed
cases whose result is known in closed form.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as F

import oracle
from oracle.bruteforce import delta_rule_exact
from oracle.chunked import delta_rule_chunked


def _rel(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(np.asarray(b))), 1e-300)


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# binary16 state storage
# ---------------------------------------------------------------------------

def test_round_binary16_matches_numpy_float16():
    """Nearest binary16, ties to even, with subnormals and overflow: equal to
    numpy's float64 -> float16 conversion on random values over the whole range
    and on every kind of tie."""
    rng = np.random.default_rng(40)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 17, 20000))
    ties = []
    for e in range(-24, 16):  # halfway points between neighbouring binary16 values
        ulp = 2.0 ** max(e - 10, -24)
        for m in (0, 1, 2, 3, 1023):
            base = (2.0 ** e if e >= -14 else 0.0) + m * ulp
            ties += [base + 0.5 * ulp, -(base + 0.5 * ulp)]
    x = np.concatenate([x, ties, [65504.0, 65519.0, 65520.0, 7e4, 2.0 ** -25, 2.0 ** -26 * 3, 0.0]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    got = oracle.round_binary16(x)
    assert np.array_equal(got, ref)


def test_f16_state_is_rounded_where_it_is_stored():
    """a = 1, b = 0: the stored state is the binary16 rounding of S0 after one
    decode, the output of that token uses the state before rounding (o = S0 q
    exactly), and a prefill rounds only its final state."""
    rng = np.random.default_rng(41)
    T, Hk, Hv, d = 5, 1, 2, 8
    q = rng.standard_normal((T, Hk, d)); k = _unit(rng, (T, Hk, d))
    v = rng.standard_normal((T, Hv, d))
    S0 = rng.standard_normal((1, Hv, d, d)) * 0.1
    ones, zeros = np.ones((T, Hv)), np.zeros((T, Hv))
    with np.errstate(over="ignore"):
        S0_16 = S0.astype(np.float16).astype(np.float64)
    o, S, st = oracle.delta_rule(q, k, v, ones, zeros, S0, [0, T], record_states=True,
                                 state_round=oracle.STATE_F16_EVERY_TOKEN)
    assert np.array_equal(st[0], S0_16[0]) and np.array_equal(S, S0_16)
    assert _rel(o[0], np.einsum("hi,hij->hj", q[0, [0, 0]], S0[0])) < 1e-15
    o, S, _ = oracle.delta_rule(q, k, v, ones, zeros, S0, [0, T], state_round=oracle.STATE_F16_FINAL)
    assert np.array_equal(S, S0_16)
    for t in range(T):  # every token still sees the unrounded S0
        assert _rel(o[t], np.einsum("hi,hij->hj", q[t, [0, 0]], S0[0])) < 1e-15


def test_f16_every_token_equals_step_by_step_numpy_half():
    """Pure decay with binary16 storage: S_t = fp16(a_t * S_{t-1}) with numpy's
    conversion applied after every token."""
    rng = np.random.default_rng(42)
    T, Hk, Hv, d = 12, 1, 1, 4
    q = rng.standard_normal((T, Hk, d)); k = _unit(rng, (T, Hk, d)); v = rng.standard_normal((T, Hv, d))
    a = rng.uniform(0.3, 1.0, (T, Hv)); b = np.zeros((T, Hv))
    S0 = (rng.standard_normal((1, Hv, d, d))).astype(np.float16).astype(np.float64)
    _, S, st = oracle.delta_rule(q, k, v, a, b, S0, [0, T], record_states=True,
                                 state_round=oracle.STATE_F16_EVERY_TOKEN)
    ref = S0[0, 0].copy()
    for t in range(T):
        ref = (a[t, 0] * ref).astype(np.float16).astype(np.float64)
        assert np.array_equal(st[t, 0], ref)


# ---------------------------------------------------------------------------
# raw gate inputs and the sigmoid-gated norm
# ---------------------------------------------------------------------------

def test_gates_from_raw_match_scipy_logistic():
    """exp(-softplus(g)) = sigmoid(-g) and b = sigmoid(beta), against scipy's
    expit and log_expit; g = 0 gives a = 1/2."""
    rng = np.random.default_rng(43)
    g = np.concatenate([rng.standard_normal(1000) * 4, [-40.0, -5.0, 0.0, 5.0, 40.0]])
    beta = rng.standard_normal(g.shape) * 4
    a, b = oracle.gates_from_raw(g, beta)
    assert np.max(np.abs(a - sps.expit(-g)) / sps.expit(-g)) < 1e-14
    assert np.max(np.abs(np.log(a) - sps.log_expit(-g))) < 1e-14
    assert np.max(np.abs(b - sps.expit(beta))) < 1e-15
    assert oracle.gates_from_raw(np.array([0.0]), np.array([0.0]))[0][0] == 0.5


def test_decode_with_raw_gates_equals_direct_gates():
    rng = np.random.default_rng(44)
    Hk, Hv, d, K, n = 2, 4, 8, 4, 3
    C = 2 * Hk * d + Hv * d
    x = rng.standard_normal((n, C)); w = rng.standard_normal((C, K)) / 2
    ring = rng.standard_normal((n, K - 1, C)); S0 = rng.standard_normal((n, Hv, d, d)) * 0.1
    g = rng.standard_normal((n, Hv)); beta = rng.standard_normal((n, Hv))
    r1 = oracle.decode(x, w, ring, g, beta, S0, Hk, Hv, d, d, gates="raw")
    r2 = oracle.decode(x, w, ring, sps.expit(-g), sps.expit(beta), S0, Hk, Hv, d, d)
    assert _rel(r1["o"], r2["o"]) < 1e-13 and _rel(r1["S"], r2["S"]) < 1e-13


def test_sigmoid_gated_norm_library_and_closed_form():
    """torch's RMSNorm times sigmoid(z); a constant row o = c gives
    sign(c) sqrt(c^2 / (c^2 + eps)) w sigmoid(z)."""
    rng = np.random.default_rng(45)
    T, Hv, dv = 5, 3, 16
    o = rng.standard_normal((T, Hv, dv)); z = rng.standard_normal((T, Hv, dv)) * 3
    w = 1 + 0.1 * rng.standard_normal(dv)
    got = oracle.gated_rmsnorm(o, z, w, 1e-6, gate="sigmoid")
    ref = F.rms_norm(torch.from_numpy(o), (dv,), weight=torch.from_numpy(w), eps=1e-6) * torch.sigmoid(torch.from_numpy(z))
    assert _rel(got, ref.numpy()) < 1e-14
    c = -0.37
    got = oracle.gated_rmsnorm(np.full((1, 1, dv), c), z[:1, :1], w, 1e-6, gate="sigmoid")
    ref = np.sign(c) * np.sqrt(c * c / (c * c + 1e-6)) * w * sps.expit(z[0, 0])
    assert _rel(got[0, 0], ref) < 1e-14


# ---------------------------------------------------------------------------
# write-on-accept verify: the stash and the fold
# ---------------------------------------------------------------------------

def test_woa_stash_u_equals_exact_rank1_update():
    """The stashed u_t satisfies S_t = a_t S_{t-1} + u_t k_t^T for the exact
    rational states of the literal rule: u_t = (S_t - a_t S_{t-1}) k_t / (k_t . k_t)."""
    rng = np.random.default_rng(46)
    T, dk, dv, Hk, Hv = 5, 3, 4, 1, 2
    fr = lambda lo, hi, den, shape: rng.integers(lo, hi + 1, size=shape).astype(np.float64) / den
    q = fr(-8, 8, 8, (T, Hk, dk)); k = fr(1, 8, 8, (T, Hk, dk)); v = fr(-8, 8, 8, (T, Hv, dv))
    a = fr(1, 8, 8, (T, Hv)); b = fr(0, 8, 8, (T, Hv)); S0 = fr(-4, 4, 4, (1, Hv, dk, dv))
    _, _, _, u = oracle._delta_rule(q, k, v, a, b, S0, [0, T], 1.0, None, False, oracle.STATE_FULL, True)
    Fr = lambda x: Fraction(float(x))
    for h in range(Hv):
        S = [[Fr(S0[0, h, i, j]) for i in range(dk)] for j in range(dv)]
        for t in range(T):
            _, S1 = delta_rule_exact([[Fr(x) for x in q[t, 0]]], [[Fr(x) for x in k[t, 0]]],
                                     [[Fr(x) for x in v[t, h]]], [Fr(a[t, h])], [Fr(b[t, h])], S)
            kt = [Fr(x) for x in k[t, 0]]
            kk = sum(x * x for x in kt)
            u_exact = [sum((S1[j][i] - Fr(a[t, h]) * S[j][i]) * kt[i] for i in range(dk)) / kk for j in range(dv)]
            assert np.max(np.abs(u[t, h] - np.array([float(x) for x in u_exact]))) < 1e-13
            S = S1


@pytest.mark.parametrize("state", ["f32", "f16"])
def test_fold_of_stash_equals_recorded_states(state):
    """Folding the first n stashed rows into S0 gives the state the write-all
    verify records after row n-1, for every n; the conv state advances as commit."""
    rng = np.random.default_rng(47)
    Hk, Hv, d, K = 2, 4, 8, 4
    C = 2 * Hk * d + Hv * d
    ks = [3, 1, 5]
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    T = int(cu[-1])
    x = rng.standard_normal((T, C)); w = rng.standard_normal((C, K)) / 2
    ring = rng.standard_normal((3, K - 1, C))
    S0 = rng.standard_normal((3, Hv, d, d)) * 0.1
    if state == "f16":
        S0 = S0.astype(np.float16).astype(np.float64)
    a = rng.uniform(0.5, 1, (T, Hv)); b = rng.uniform(0, 1, (T, Hv))
    r = oracle.verify_woa(x, w, ring, a, b, S0, cu, Hk, Hv, d, d, state=state)
    for na in ([1, 1, 1], [2, 1, 3], [3, 1, 5]):
        S, ring_new = oracle.fold_accepted(S0, r["stash_k"], r["stash_u"], r["stash_a"], cu, na, ring, x,
                                           state=state)
        S_ref, ring_ref = oracle.commit(r["states"], na, cu, ring, x)
        assert _rel(S, S_ref) < 1e-13
        assert np.array_equal(ring_new, ring_ref)


# ---------------------------------------------------------------------------
# several consecutive tokens per sequence
# ---------------------------------------------------------------------------

def test_decode_tokens_equals_chunked_form_and_single_decodes():
    """k_i tokens per sequence == the independent chunked form on the same
    post-conv rows, and == k_i one-token decodes in a row."""
    rng = np.random.default_rng(48)
    Hk, Hv, d, K = 2, 4, 8, 4
    C = 2 * Hk * d + Hv * d
    ks = [4, 1, 17]
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    T = int(cu[-1])
    x = rng.standard_normal((T, C)); w = rng.standard_normal((C, K)) / 2
    ring = rng.standard_normal((3, K - 1, C)); S0 = rng.standard_normal((3, Hv, d, d)) * 0.1
    a = rng.uniform(0.5, 1, (T, Hv)); b = rng.uniform(0, 1, (T, Hv))
    r = oracle.decode_tokens(x, w, ring, a, b, S0, cu, Hk, Hv, d, d)
    q, k, v = oracle.split_qkv(r["y"], Hk, Hv, d, d)
    o_c, S_c = delta_rule_chunked(q, k, v, a, b, S0, cu, 5)
    assert _rel(r["o"], o_c) < 1e-12 and _rel(r["S"], S_c) < 1e-12
    S, rg = S0.copy(), ring.copy()
    for i in range(3):
        for t in range(cu[i], cu[i + 1]):
            one = oracle.decode(x[t:t + 1], w, rg[i:i + 1], a[t:t + 1], b[t:t + 1], S[i:i + 1], Hk, Hv, d, d)
            assert _rel(one["o"][0], r["o"][t]) < 1e-14
            S[i], rg[i] = one["S"][0], one["ring"][0]
    assert _rel(S, r["S"]) < 1e-14 and np.array_equal(rg, r["ring"])
