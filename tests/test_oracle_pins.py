"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test checks the oracle against what the definition of the gated delta rule
and its front/back steps fixes: exact rational brute force of the literal matrix
form, closed forms, invariants and library routines (numpy / torch / scipy).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.bruteforce import delta_rule_exact
from oracle.chunked import delta_rule_chunked


def _rand_unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rel(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(np.asarray(b))), 1e-300)


# ---------------------------------------------------------------------------
# Recurrence core
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_exact_rational(seed):
    """fp64 oracle (rank-1 order) == exact Fraction evaluation of the literal
    S_t = a S (I - b k k^T) + b v k^T with full matrix products, to 1e-13."""
    rng = np.random.default_rng(seed)
    T, dk, dv, Hk, Hv = 7, 3, 4, 1, 2
    fr = lambda lo, hi, den, shape: rng.integers(lo, hi + 1, size=shape).astype(np.float64) / den
    q = fr(-8, 8, 8, (T, Hk, dk))
    k = fr(-8, 8, 8, (T, Hk, dk))
    v = fr(-8, 8, 8, (T, Hv, dv))
    a = fr(0, 8, 8, (T, Hv))
    b = fr(0, 8, 8, (T, Hv))
    S0 = fr(-4, 4, 4, (1, Hv, dk, dv))  # h = S^T
    cu = [0, T]
    o, S, _ = oracle.delta_rule(q, k, v, a, b, S0, cu)
    F_ = lambda x: Fraction(float(x))
    for h in range(Hv):
        g = h * Hk // Hv
        outs, Sx = delta_rule_exact(
            [[F_(x) for x in q[t, g]] for t in range(T)],
            [[F_(x) for x in k[t, g]] for t in range(T)],
            [[F_(x) for x in v[t, h]] for t in range(T)],
            [F_(a[t, h]) for t in range(T)], [F_(b[t, h]) for t in range(T)],
            [[F_(S0[0, h, i, j]) for i in range(dk)] for j in range(dv)])  # S = h^T
        exact_o = np.array([[float(x) for x in row] for row in outs])
        exact_h = np.array([[float(Sx[j][i]) for j in range(dv)] for i in range(dk)])
        assert np.max(np.abs(o[:, h] - exact_o)) <= 1e-13 * max(1.0, np.abs(exact_o).max())
        assert np.max(np.abs(S[0, h] - exact_h)) <= 1e-13 * max(1.0, np.abs(exact_h).max())


def test_identity_a1_b0():
    """a = 1, b = 0 leaves S unchanged and o_t = S_0 q_t (a matmul)."""
    rng = np.random.default_rng(3)
    T, Hk, Hv, d = 20, 2, 4, 16
    q = rng.standard_normal((T, Hk, d)); k = _rand_unit(rng, (T, Hk, d))
    v = rng.standard_normal((T, Hv, d))
    S0 = rng.standard_normal((1, Hv, d, d))
    o, S, _ = oracle.delta_rule(q, k, v, np.ones((T, Hv)), np.zeros((T, Hv)), S0, [0, T])
    assert np.array_equal(S, S0)
    for h in range(Hv):
        ref = q[:, h * Hk // Hv] @ S0[0, h]          # o_j = sum_i q_i h[i][j]
        assert _rel(o[:, h], ref) < 1e-14


def test_reset_a0():
    """a = 0 forgets the past: S_t = b_t v_t k_t^T, o_t = b_t (k_t . q_t) v_t."""
    rng = np.random.default_rng(4)
    T, Hk, Hv, d = 9, 1, 2, 8
    q = rng.standard_normal((T, Hk, d)); k = _rand_unit(rng, (T, Hk, d))
    v = rng.standard_normal((T, Hv, d)); b = rng.uniform(0, 1, (T, Hv))
    S0 = rng.standard_normal((1, Hv, d, d))
    o, S, st = oracle.delta_rule(q, k, v, np.zeros((T, Hv)), b, S0, [0, T], record_states=True)
    for t in range(T):
        for h in range(Hv):
            assert _rel(st[t, h], b[t, h] * np.outer(k[t, 0], v[t, h])) < 1e-14
            assert _rel(o[t, h], b[t, h] * (k[t, 0] @ q[t, 0]) * v[t, h]) < 1e-13


def test_retrieval_b1_unit_k():
    """b = 1 and ||k|| = 1: the updated state retrieves S_t k_t = v_t for any a, S."""
    rng = np.random.default_rng(5)
    T, Hk, Hv, d = 30, 2, 4, 32
    q = rng.standard_normal((T, Hk, d)); k = _rand_unit(rng, (T, Hk, d))
    v = rng.standard_normal((T, Hv, d)); a = rng.uniform(0, 1, (T, Hv))
    S0 = rng.standard_normal((1, Hv, d, d))
    _, _, st = oracle.delta_rule(q, k, v, a, np.ones((T, Hv)), S0, [0, T], record_states=True)
    for t in range(T):
        for h in range(Hv):
            retrieved = k[t, h * Hk // Hv] @ st[t, h]  # (S k)_j = sum_i k_i h[i][j]
            assert np.max(np.abs(retrieved - v[t, h])) < 1e-12


def test_orthonormal_keys_closed_form():
    """Orthonormal keys (permuted basis vectors), T <= d_k:
    S_T = (prod a) S_0 (I - sum_t b_t k_t k_t^T) + sum_t (prod_{s>t} a_s) b_t v_t k_t^T."""
    rng = np.random.default_rng(6)
    d, T = 16, 11
    perm = rng.permutation(d)[:T]
    k = np.zeros((T, 1, d)); k[np.arange(T), 0, perm] = 1.0
    q = rng.standard_normal((T, 1, d)); v = rng.standard_normal((T, 1, d))
    a = rng.uniform(0.2, 1, (T, 1)); b = rng.uniform(0, 1, (T, 1))
    S0 = rng.standard_normal((1, 1, d, d))
    o, S, st = oracle.delta_rule(q, k, v, a, b, S0, [0, T], record_states=True)
    for t_end in range(T):
        S_mat = S0[0, 0].T  # S = h^T  (d_v x d_k)
        P = np.eye(d) - sum(b[t, 0] * np.outer(k[t, 0], k[t, 0]) for t in range(t_end + 1))
        ref = np.prod(a[: t_end + 1, 0]) * S_mat @ P
        for t in range(t_end + 1):
            ref = ref + np.prod(a[t + 1: t_end + 1, 0]) * b[t, 0] * np.outer(v[t, 0], k[t, 0])
        assert _rel(st[t_end, 0].T, ref) < 1e-13
        assert _rel(o[t_end, 0], ref @ q[t_end, 0]) < 1e-13


def test_pure_decay_b0():
    """b = 0: S_T = (prod a) S_0 and o_t = (prod_{s<=t} a_s) S_0 q_t."""
    rng = np.random.default_rng(7)
    T, d = 25, 8
    q = rng.standard_normal((T, 1, d)); k = _rand_unit(rng, (T, 1, d))
    v = rng.standard_normal((T, 1, d)); a = rng.uniform(0.5, 1, (T, 1))
    S0 = rng.standard_normal((1, 1, d, d))
    o, S, _ = oracle.delta_rule(q, k, v, a, np.zeros((T, 1)), S0, [0, T])
    assert _rel(S, np.prod(a) * S0) < 1e-14
    cum = np.cumprod(a[:, 0])
    assert _rel(o[:, 0], cum[:, None] * (q[:, 0] @ S0[0, 0])) < 1e-13


def test_single_token_from_zero():
    """From S_0 = 0 one token gives o = b (k . q) v, whatever a is."""
    rng = np.random.default_rng(8)
    d = 32
    q = rng.standard_normal((1, 1, d)); k = _rand_unit(rng, (1, 1, d)); v = rng.standard_normal((1, 1, d))
    o, _, _ = oracle.delta_rule(q, k, v, np.array([[0.37]]), np.array([[0.61]]), np.zeros((1, 1, d, d)), [0, 1])
    assert _rel(o[0, 0], 0.61 * (k[0, 0] @ q[0, 0]) * v[0, 0]) < 1e-14


def test_linearity_in_v_and_gqa_sharing():
    """From S_0 = 0 the map v -> o is linear; two value heads of one key head with
    identical (a, b, v) produce identical outputs; heads of different key heads
    do not."""
    rng = np.random.default_rng(9)
    T, Hk, Hv, d = 17, 2, 4, 8
    q = rng.standard_normal((T, Hk, d)); k = _rand_unit(rng, (T, Hk, d))
    a = rng.uniform(0, 1, (T, Hv)); b = rng.uniform(0, 1, (T, Hv))
    v1 = rng.standard_normal((T, Hv, d)); v2 = rng.standard_normal((T, Hv, d))
    Z = np.zeros((1, Hv, d, d))
    o1, _, _ = oracle.delta_rule(q, k, v1, a, b, Z, [0, T])
    o2, _, _ = oracle.delta_rule(q, k, v2, a, b, Z, [0, T])
    o12, _, _ = oracle.delta_rule(q, k, v1 + 2 * v2, a, b, Z, [0, T])
    assert _rel(o12, o1 + 2 * o2) < 1e-12
    a[:, 1] = a[:, 0]; b[:, 1] = b[:, 0]; v1[:, 1] = v1[:, 0]
    a[:, 2] = a[:, 0]; b[:, 2] = b[:, 0]; v1[:, 2] = v1[:, 0]
    o, _, _ = oracle.delta_rule(q, k, v1, a, b, Z, [0, T])
    assert np.array_equal(o[:, 0], o[:, 1])        # heads 0, 1 -> key head 0
    assert not np.allclose(o[:, 0], o[:, 2])       # head 2 -> key head 1


@pytest.mark.parametrize("chunk", [1, 7, 16, 64])
def test_chunked_form_agrees(chunk):
    """The WY/UT chunked form (scipy triangular solve) == token recurrence to 1e-12,
    varlen with partial chunks and a zero-length sequence."""
    rng = np.random.default_rng(10 + chunk)
    lens = [150, 0, 37, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, Hk, Hv, d = int(cu[-1]), 2, 4, 16
    q = _rand_unit(rng, (T, Hk, d)); k = _rand_unit(rng, (T, Hk, d))
    v = rng.standard_normal((T, Hv, d)); a = rng.uniform(0.3, 1, (T, Hv)); b = rng.uniform(0, 1, (T, Hv))
    S0 = 0.1 * rng.standard_normal((len(lens), Hv, d, d))
    o, S, _ = oracle.delta_rule(q, k, v, a, b, S0, cu, scale=0.5)
    oc, Sc = delta_rule_chunked(q, k, v, a, b, S0, cu, chunk=chunk, scale=0.5)
    assert _rel(oc, o) < 1e-12
    assert _rel(Sc, S) < 1e-12


def test_heads_subset_and_recorded_states():
    """Computing a subset of heads gives the same numbers as all heads, and the
    recorded state after the last token equals the final state."""
    rng = np.random.default_rng(11)
    T, Hk, Hv, d = 12, 2, 4, 8
    q = rng.standard_normal((T, Hk, d)); k = _rand_unit(rng, (T, Hk, d)); v = rng.standard_normal((T, Hv, d))
    a = rng.uniform(0, 1, (T, Hv)); b = rng.uniform(0, 1, (T, Hv)); S0 = rng.standard_normal((2, Hv, d, d))
    cu = [0, 5, 12]
    o, S, st = oracle.delta_rule(q, k, v, a, b, S0, cu, record_states=True)
    o2, S2, st2 = oracle.delta_rule(q, k, v, a, b, S0, cu, heads=[3, 1], record_states=True)
    assert np.array_equal(o2[:, [3, 1]], o[:, [3, 1]])
    assert np.array_equal(st2[:, 0], st[:, 3]) and np.array_equal(st2[:, 1], st[:, 1])
    assert np.array_equal(st[4], S[0]) and np.array_equal(st[11], S[1])


# ---------------------------------------------------------------------------
# Conv1d + SiLU, L2
# ---------------------------------------------------------------------------

def _silu(x):
    return x / (1.0 + np.exp(-x))


def test_conv_matches_numpy_convolve_and_torch_conv1d():
    rng = np.random.default_rng(12)
    Hk, Hv, d, K = 1, 2, 4, 4
    C = 2 * Hk * d + Hv * d
    lens = [10, 3, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    x = rng.standard_normal((T, C)); w = rng.standard_normal((C, K)); ring = rng.standard_normal((3, K - 1, C))
    y, ring_new = oracle.conv_l2norm(x, w, ring, cu, Hk, Hv, d, d, l2_eps=1e-6)
    for s in range(3):
        xe = np.concatenate([ring[s], x[cu[s]:cu[s + 1]]], axis=0)  # [K-1+len, C]
        pre = np.stack([np.convolve(xe[:, c], w[c, ::-1], mode="valid") for c in range(C)], axis=1)
        pre_t = F.conv1d(torch.from_numpy(xe.T[None]), torch.from_numpy(w[:, None, :]), groups=C)[0].numpy().T
        assert _rel(pre_t, pre) < 1e-13
        ref = _silu(pre)
        # v channels are not normalised
        assert _rel(y[cu[s]:cu[s + 1], 2 * Hk * d:], ref[:, 2 * Hk * d:]) < 1e-14
        # q, k heads: divide by sqrt(||.||^2 + eps), norm from numpy.linalg.norm
        for part in range(2):
            blk = ref[:, part * Hk * d:(part + 1) * Hk * d].reshape(-1, Hk, d)
            nrm = np.linalg.norm(blk, axis=-1, keepdims=True)
            ref_hat = blk / np.sqrt(nrm ** 2 + 1e-6)
            got = y[cu[s]:cu[s + 1], part * Hk * d:(part + 1) * Hk * d].reshape(-1, Hk, d)
            assert _rel(got, ref_hat) < 1e-14
        assert np.array_equal(ring_new[s], xe[-(K - 1):])


def test_conv_delta_tap_is_identity_and_split_calls_continue():
    rng = np.random.default_rng(13)
    Hk, Hv, d, K = 1, 1, 8, 4
    C = 3 * d
    x = rng.standard_normal((40, C))
    w = np.zeros((C, K)); w[:, K - 1] = 1.0
    y, _ = oracle.conv_l2norm(x, w, np.zeros((1, K - 1, C)), [0, 40], Hk, Hv, d, d)
    assert _rel(y[:, 2 * d:], _silu(x[:, 2 * d:])) < 1e-15
    w = rng.standard_normal((C, K)); ring = rng.standard_normal((1, K - 1, C))
    y_all, r_all = oracle.conv_l2norm(x, w, ring, [0, 40], Hk, Hv, d, d)
    y_a, r_a = oracle.conv_l2norm(x[:25], w, ring, [0, 25], Hk, Hv, d, d)
    y_b, r_b = oracle.conv_l2norm(x[25:], w, r_a, [0, 15], Hk, Hv, d, d)
    assert np.array_equal(np.concatenate([y_a, y_b]), y_all)
    assert np.array_equal(r_b, r_all)
    # a sequence shorter than K-1 shifts the ring
    y_c, r_c = oracle.conv_l2norm(x[:2], w, ring, [0, 2], Hk, Hv, d, d)
    assert np.array_equal(r_c[0], np.concatenate([ring[0, 2:], x[:2]]))


def test_l2_norm_value():
    """The L2 output of a head has norm sqrt(S / (S + eps)), S the squared norm."""
    rng = np.random.default_rng(14)
    d = 16
    C = 3 * d
    x = rng.standard_normal((5, C)) * 1e-3
    w = np.zeros((C, 4)); w[:, 3] = 1.0
    y, _ = oracle.conv_l2norm(x, w, np.zeros((1, 3, C)), [0, 5], 1, 1, d, d, l2_eps=1e-6)
    pre = _silu(x[:, :d])
    ss = np.sum(pre ** 2, axis=1)
    assert _rel(np.linalg.norm(y[:, :d], axis=1), np.sqrt(ss / (ss + 1e-6))) < 1e-14


# ---------------------------------------------------------------------------
# Gated RMSNorm
# ---------------------------------------------------------------------------

def test_gated_rmsnorm_library_and_closed_form():
    rng = np.random.default_rng(15)
    T, Hv, dv = 6, 3, 32
    o = rng.standard_normal((T, Hv, dv)); z = rng.standard_normal((T, Hv, dv)); w = 1 + 0.1 * rng.standard_normal(dv)
    out = oracle.gated_rmsnorm(o, z, w, eps=1e-6)
    ref = F.rms_norm(torch.from_numpy(o), (dv,), weight=torch.from_numpy(w), eps=1e-6) * F.silu(torch.from_numpy(z))
    assert _rel(out, ref.numpy()) < 1e-13
    # constant o = c * 1: out = c / sqrt(c^2 + eps) * w * SiLU(z)
    c = -0.003
    out_c = oracle.gated_rmsnorm(np.full((1, 1, dv), c), z[:1, :1], w, eps=1e-6)
    assert _rel(out_c[0, 0], c / np.sqrt(c * c + 1e-6) * w * z[0, 0] / (1 + np.exp(-z[0, 0]))) < 1e-14
    # z = 0 closes the gate
    assert np.array_equal(oracle.gated_rmsnorm(o, np.zeros_like(z), w), np.zeros_like(o))


# ---------------------------------------------------------------------------
# Compositions: varlen, decode, verify, commit
# ---------------------------------------------------------------------------

def test_varlen_equals_separate_sequences():
    rng = np.random.default_rng(16)
    Hk, Hv, d, K = 2, 4, 8, 4
    C = 2 * Hk * d + Hv * d
    lens = [13, 0, 70, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    x = rng.standard_normal((T, C)); z = rng.standard_normal((T, Hv * d))
    a = rng.uniform(0, 1, (T, Hv)); b = rng.uniform(0, 1, (T, Hv))
    w = rng.standard_normal((C, K)); nw = rng.standard_normal(d)
    S0 = rng.standard_normal((4, Hv, d, d)); ring = rng.standard_normal((4, K - 1, C))
    r = oracle.prefill(x, a, b, S0, cu, Hk, Hv, d, d, conv_w=w, ring=ring, z=z, norm_w=nw)
    for s in range(4):
        sl = slice(cu[s], cu[s + 1])
        rs = oracle.prefill(x[sl], a[sl], b[sl], S0[s:s + 1], [0, lens[s]], Hk, Hv, d, d, conv_w=w,
                            ring=ring[s:s + 1], z=z[sl], norm_w=nw)
        assert np.array_equal(r["out"][sl], rs["out"])
        assert np.array_equal(r["S"][s], rs["S"][0])
        assert np.array_equal(r["ring"][s], rs["ring"][0])
    assert np.array_equal(r["S"][1], S0[1])  # zero-length sequence keeps its state


def test_verify_intermediates_equal_decode_steps_and_commit():
    """Verify from S_0 over k rows records exactly the states that k one-token
    decode steps produce; commit(n) reproduces n decode steps (state and conv)."""
    rng = np.random.default_rng(17)
    Hk, Hv, d, K = 1, 2, 8, 4
    C = 2 * Hk * d + Hv * d
    ks = [3, 5]
    cu = np.array([0, 3, 8], dtype=np.int32)
    x = rng.standard_normal((8, C)); a = rng.uniform(0, 1, (8, Hv)); b = rng.uniform(0, 1, (8, Hv))
    w = rng.standard_normal((C, K)); S0 = rng.standard_normal((2, Hv, d, d)); ring = rng.standard_normal((2, K - 1, C))
    ver = oracle.verify(x, w, ring, a, b, S0, cu, Hk, Hv, d, d)
    for i, kk in enumerate(ks):
        S, rg = S0[i:i + 1], ring[i:i + 1]
        for t in range(kk):
            row = cu[i] + t
            dec = oracle.decode(x[row:row + 1], w, rg, a[row:row + 1], b[row:row + 1], S, Hk, Hv, d, d)
            S, rg = dec["S"], dec["ring"]
            assert np.array_equal(ver["states"][row], S[0])
            assert np.array_equal(ver["o"][row], dec["o"][0])
            n_acc = np.array([t + 1 if j == i else ks[j] for j in range(2)])
            S_c, ring_c = oracle.commit(ver["states"], n_acc, cu, ring, x)
            assert np.array_equal(S_c[i], S[0])
            assert np.array_equal(ring_c[i], rg[0])
