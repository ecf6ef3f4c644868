"""GPU parity of the variant forms, through the C ABI, against the fp64 oracle:
write-on-accept verify and its fold, binary16 states (decode, verify + commit,
prefill), raw gate inputs, the sigmoid-gated norm, and the decode of several
consecutive tokens per sequence."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_ssm_core_amd import binding as B
from linear_attention_ssm_core_amd import workloads as W
from tests.gpu_util import (DEV, TOL_OUT, TOL_STATE, TOL_STATE_F16, DeviceStates, act_dtype, f16_exact, host,
                            row_seq_of, slice_err, tdev)

pytestmark = pytest.mark.gpu


def _sample_rows(cu, sample):
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in sample])
    cu_s = np.concatenate([[0], np.cumsum(np.diff(cu)[sample])]).astype(np.int32)
    return rows, cu_s


def _tables(ds, ks, dims, state_dtype):
    """WY tables over ds.h (table 0) and fresh buffers for the intermediates."""
    n = len(ks)
    inter = [[torch.full((dims.Hv, dims.dk, dims.dv), float("nan"), dtype=state_dtype, device=DEV)
              for _ in range(ks[i] - 1)] for i in range(n)]
    tables = [[None] * n for _ in range(16)]
    for i in range(n):
        tables[0][i] = ds.h[i]
        for t in range(ks[i] - 1):
            tables[t + 1][i] = inter[i][t]
    return inter, B.wy_tables(tables, DEV)


def _stash_parts(stash, T, dims):
    """Split the stash rows into k_hat [T, Hk, dk], u [T, Hv, dv] and a [T, Hv]."""
    Hk, Hv, d = dims.Hk, dims.Hv, dims.dk
    row = (Hk * d + Hv * d + Hv + 3) // 4 * 4
    s = host(stash)[: T * row].reshape(T, row)
    return (s[:, : Hk * d].reshape(T, Hk, d), s[:, Hk * d: Hk * d + Hv * d].reshape(T, Hv, d),
            s[:, Hk * d + Hv * d: Hk * d + Hv * d + Hv])


def _wy_form(dims, state):
    """fp32 states at d >= 64: the write-on-accept verify takes the WY form on the
    matrix cores instead of the row-by-row recurrence."""
    return state == "f32" and dims.dk >= 64


# ---------------------------------------------------------------------------
# write-on-accept verify and fold
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case,state", [("config3", "f32"), ("config3", "f16"), ("tiny_fp32", "f32"),
                                        ("edge_k", "f32"), ("n128_k1", "f32"), ("d64_g4", "f16"),
                                        ("d64_g4", "f32"), ("extreme_raw_gates", "f32"), ("g1_f32act", "f32"),
                                        ("g4_d128_k3", "f32"), ("k2_d128", "f32"), ("repeat_keys", "f32")])
def test_woa_verify_and_fold(case, state):
    """Outputs and stash against the oracle; the fold of the accepted rows against
    the oracle and against the state the write-all verify records after the same
    row (bit for bit where both take the rows one by one: binary16 states and
    d = 32; fp32 states at d >= 64 take the WY form, whose sums associate
    differently); the conv state against the oracle's commit."""
    gates = "direct"
    if case == "config3":
        d = W.config(3)
        sample = np.arange(d["n"])
    elif case == "tiny_fp32":
        d = W.verify_inputs(3101, 5, W.TINY_DIMS, act="f32")
        sample = np.arange(5)
    elif case == "edge_k":  # k = 2 and 16 only, accepted n = 1 and n = k
        d = W.verify_inputs(3102, 6, W.QWEN_DIMS, ks=[2, 16, 2, 16, 16, 2])
        d["n_acc"] = np.array([1, 16, 2, 1, 7, 2], dtype=np.int32)
        sample = np.arange(6)
    elif case == "n128_k1":  # the widest batch, with one-row sequences among 16-row ones
        ks = np.array(([1, 16, 5, 1] * 32)[:128])
        d = W.verify_inputs(3111, 128, W.QWEN_DIMS, ks=ks)
        sample = np.arange(128)
    elif case == "extreme_raw_gates":  # raw g, beta at +-30: products of decays underflow, b saturates
        d = W.verify_inputs(3117, 6, W.QWEN_DIMS, ks=[16, 9, 2, 13, 16, 5])
        rng = np.random.default_rng(3117)
        d["a"] = rng.choice([-30.0, -3.0, 0.0, 3.0, 30.0], size=d["a"].shape).astype(np.float32)
        d["b"] = rng.choice([-30.0, 0.0, 30.0], size=d["b"].shape).astype(np.float32)
        gates = "raw"
        sample = np.arange(6)
    elif case == "repeat_keys":  # the same key in every row with a = b = 1: A's lower triangle all ones
        d = W.verify_inputs(3121, 3, W.QWEN_DIMS, ks=[16, 9, 5])
        dims0 = d["dims"]
        kc = slice(dims0.Hk * dims0.dk, 2 * dims0.Hk * dims0.dk)  # pre-conv key channels
        for i in range(3):
            r0, r1 = int(d["cu"][i]), int(d["cu"][i + 1])
            d["x"][r0:r1, kc] = d["x"][r0, kc]
            d["ring"][i][:, kc] = d["x"][r0, kc]
        d["a"][:] = 1.0
        d["b"][:] = 1.0
        sample = np.arange(3)
    elif case == "g1_f32act":  # one value head per key head, fp32 activations
        d = W.verify_inputs(3118, 5, W.Dims(Hk=4, Hv=4, dk=128, dv=128, K=4), act="f32", ks=[16, 3, 11, 1, 8])
        sample = np.arange(5)
    elif case == "k2_d128":  # a 2-tap conv: one conv-state row, read by every lane of a quad
        d = W.verify_inputs(3123, 4, W.Dims(Hk=4, Hv=8, dk=128, dv=128, K=2), act="bf16", ks=[16, 5, 2, 9])
        sample = np.arange(4)
    elif case == "g4_d128_k3":  # four value heads per key head at d = 128, a 3-tap conv
        d = W.verify_inputs(3119, 5, W.Dims(Hk=2, Hv=8, dk=128, dv=128, K=3), act="bf16", ks=[7, 16, 2, 12, 5])
        sample = np.arange(5)
    else:  # d = 64, four value heads per key head
        d = W.verify_inputs(3112, 7, W.Dims(Hk=2, Hv=8, dk=64, dv=64, K=4), act="bf16")
        sample = np.arange(7)
    sdt = torch.float16 if state == "f16" else torch.float32
    if state == "f16":
        d["S0"] = f16_exact(d["S0"])
    tol_s = TOL_STATE_F16 if state == "f16" else TOL_STATE
    dims, act = d["dims"], act_dtype(d)
    cu, ks, n_acc = d["cu"], d["ks"], d["n_acc"]
    T = int(cu[-1])
    opt = B.options(sdt, gates=gates)
    x, w = tdev(d["x"], act), tdev(d["conv_w"], act)
    a, b = tdev(d["a"], torch.float32), tdev(d["b"], torch.float32)
    z, nw = tdev(d["z"], act), tdev(d["norm_w"], act)
    cu_t = tdev(cu, torch.int32)
    max_k = int(max(2, ks.max()))

    ds = DeviceStates(d["S0"], d["ring"], act, sdt)
    S_before = [h.clone() for h in ds.h]
    ring_before = ds.ring_host()
    out = torch.empty((T, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    stash = B.gdn_verify_woa(x, w, ds.ring_ptrs, a, b, ds.h_ptrs, cu_t, max_k, out, dims, z=z, norm_w=nw, opt=opt)
    torch.cuda.synchronize()
    assert all(torch.equal(h, h0) for h, h0 in zip(ds.h, S_before))  # no state written
    assert np.array_equal(ds.ring_host(), ring_before)

    rows, cu_s = _sample_rows(cu, sample)
    ref = oracle.verify_woa(d["x"][rows], d["conv_w"], d["ring"][sample], d["a"][rows], d["b"][rows],
                            d["S0"][sample], cu_s, dims.Hk, dims.Hv, dims.dk, dims.dv, z=d["z"][rows],
                            norm_w=d["norm_w"], state=state, gates=gates)
    g = host(out)[rows].reshape(len(rows), dims.Hv, dims.dv)
    assert slice_err(g, ref["out"], row_seq_of(cu_s)) < TOL_OUT
    sk, su, sa = _stash_parts(stash, T, dims)
    assert slice_err(sk[rows], ref["stash_k"], row_seq_of(cu_s)) < 1e-5
    assert slice_err(su[rows], ref["stash_u"], row_seq_of(cu_s)) < TOL_STATE
    if gates == "raw":  # the decays the kernel derived from g (hardware exp and reciprocal)
        assert np.allclose(sa[rows], ref["stash_a"], rtol=1e-5, atol=0.0)
    else:
        assert np.array_equal(sa[rows], d["a"][rows].astype(np.float64))

    # the write-all verify on the same inputs, for the bitwise comparison
    ds2 = DeviceStates(d["S0"], d["ring"], act, sdt)
    inter, tab = _tables(ds2, ks, dims, sdt)
    out2 = torch.empty_like(out)
    B.gdn_verify_multi(x, w, ds2.ring_ptrs, a, b, tab, cu_t, max_k, out2, dims, z=z, norm_w=nw, opt=opt)
    wy = _wy_form(dims, state)
    if wy:
        assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), host(out2).reshape(T, dims.Hv, dims.dv),
                         row_seq_of(cu)) < TOL_OUT
    else:
        assert torch.equal(out, out2)

    B.gdn_fold_accepted(x, ds.ring_ptrs, ds.h_ptrs, stash, cu_t, torch.from_numpy(n_acc).to(DEV), dims,
                        opt=B.options(sdt))  # (the stash holds the decays themselves)
    torch.cuda.synchronize()
    for i in range(d["n"]):
        na = int(n_acc[i])
        recorded = inter[i][na - 1] if na < ks[i] else ds2.h[i]
        if wy:
            assert slice_err(host(ds.h[i])[None], host(recorded)[None]) < TOL_STATE, (i, na, int(ks[i]))
        else:
            assert torch.equal(ds.h[i], recorded), (i, na, int(ks[i]))
    S_ref, ring_ref = oracle.fold_accepted(d["S0"][sample], ref["stash_k"], ref["stash_u"], ref["stash_a"], cu_s,
                                           n_acc[sample], d["ring"][sample], d["x"][rows], state=state)
    assert slice_err(ds.h_host()[sample], S_ref) < tol_s
    assert np.array_equal(ds.ring_host()[sample], ring_ref)


# ---------------------------------------------------------------------------
# binary16 states
# ---------------------------------------------------------------------------

def test_decode_f16_state_config2_shapes():
    """128 sequences, binary16 states, 30 consecutive steps with the fused
    front and gated norm; outputs of every step and every final state."""
    d = W.config(2, steps=30)
    d["S0"] = f16_exact(d["S0"])
    dims = d["dims"]
    ds = DeviceStates(d["S0"], d["ring"], torch.bfloat16, torch.float16)
    idx = np.arange(d["n"])
    S, ring = d["S0"][idx].astype(np.float64), d["ring"][idx].astype(np.float64)
    worst_o = 0.0
    for step in range(d["steps"]):
        out = torch.empty((d["n"], dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
        B.gdn_decode_batched(tdev(d["x"][step], torch.bfloat16), tdev(d["conv_w"], torch.bfloat16), ds.ring_ptrs,
                             tdev(d["a"][step], torch.float32), tdev(d["b"][step], torch.float32), ds.h_ptrs, out,
                             dims, z=tdev(d["z"][step], torch.bfloat16), norm_w=tdev(d["norm_w"], torch.bfloat16),
                             opt=B.options(torch.float16))
        r = oracle.decode(d["x"][step][idx], d["conv_w"], ring, d["a"][step][idx], d["b"][step][idx], S, dims.Hk,
                          dims.Hv, dims.dk, dims.dv, z=d["z"][step][idx], norm_w=d["norm_w"], state="f16")
        S, ring = r["S"], r["ring"]
        g = host(out)[idx].reshape(len(idx), dims.Hv, dims.dv)
        worst_o = max(worst_o, slice_err(g, r["out"].reshape(len(idx), dims.Hv, dims.dv), np.arange(len(idx))))
    assert worst_o < TOL_OUT, worst_o
    gs = ds.h_host()[idx]
    assert np.array_equal(gs, f16_exact(gs))  # stored values are binary16
    assert slice_err(gs, S) < TOL_STATE_F16
    assert np.array_equal(ds.ring_host()[idx], ring)


def test_verify_f16_states_and_commit():
    d = W.verify_inputs(3103, 8, W.QWEN_DIMS)
    d["S0"] = f16_exact(d["S0"])
    dims, act = d["dims"], act_dtype(d)
    cu, ks = d["cu"], d["ks"]
    ds = DeviceStates(d["S0"], d["ring"], act, torch.float16)
    inter, tab = _tables(ds, ks, dims, torch.float16)
    T = int(cu[-1])
    out = torch.empty((T, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    opt = B.options(torch.float16)
    B.gdn_verify_multi(tdev(d["x"], act), tdev(d["conv_w"], act), ds.ring_ptrs, tdev(d["a"], torch.float32),
                       tdev(d["b"], torch.float32), tab, tdev(cu, torch.int32), int(ks.max()), out, dims,
                       z=tdev(d["z"], act), norm_w=tdev(d["norm_w"], act), opt=opt)
    ref = oracle.verify(d["x"], d["conv_w"], d["ring"], d["a"], d["b"], d["S0"], cu, dims.Hk, dims.Hv, dims.dk,
                        dims.dv, z=d["z"], norm_w=d["norm_w"], state="f16")
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["out"], row_seq_of(cu)) < TOL_OUT
    worst = 0.0
    for i in range(d["n"]):
        for t in range(ks[i]):
            gst = host(inter[i][t]) if t < ks[i] - 1 else host(ds.h[i])
            worst = max(worst, slice_err(gst[None], ref["states"][cu[i] + t][None]))
    assert worst < TOL_STATE_F16, worst
    last = [ds.h[i].clone() for i in range(d["n"])]
    B.gdn_verify_commit(tdev(d["x"], act), ds.ring_ptrs, tab, tdev(cu, torch.int32),
                        torch.from_numpy(d["n_acc"]).to(DEV), dims, opt=opt)
    torch.cuda.synchronize()
    for i in range(d["n"]):
        na = int(d["n_acc"][i])
        assert torch.equal(ds.h[i], inter[i][na - 1] if na < ks[i] else last[i])


def test_prefill_f16_state():
    """The stored binary16 state is widened at the start, the sequences run in
    fp32, and the final state is narrowed; two sequences with a ragged tail."""
    d = W.prefill_inputs(3104, [200, 77], W.QWEN_DIMS, act="bf16")
    d["S0"] = f16_exact(d["S0"])
    dims = d["dims"]
    T = int(d["cu"][-1])
    h = [tdev(d["S0"][i], torch.float16) for i in range(2)]
    ring = [tdev(d["ring"][i], torch.bfloat16) for i in range(2)]
    out = torch.empty((T, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    B.gdn_prefill_chunked(dims, tdev(d["cu"], torch.int32), tdev(d["a"], torch.float32),
                          tdev(d["b"], torch.float32), B.ptr_array(h), out, x=tdev(d["x"], torch.bfloat16),
                          conv_w=tdev(d["conv_w"], torch.bfloat16), conv_state_ptrs=B.ptr_array(ring),
                          opt=B.options(torch.float16))
    ref = oracle.prefill(d["x"], d["a"], d["b"], d["S0"], d["cu"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                         conv_w=d["conv_w"], ring=d["ring"], state="f16")
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["o"], row_seq_of(d["cu"])) < TOL_OUT
    gs = np.stack([host(t) for t in h])
    assert np.array_equal(gs, f16_exact(gs))
    assert slice_err(gs, ref["S"]) < TOL_STATE_F16


# ---------------------------------------------------------------------------
# raw gate inputs and the sigmoid-gated norm
# ---------------------------------------------------------------------------

def _raw_gates(rng, shape):
    return (rng.standard_normal(shape) * 2).astype(np.float32), (rng.standard_normal(shape) * 2).astype(np.float32)


def test_raw_gates_and_sigmoid_norm_decode_verify():
    rng = np.random.default_rng(3105)
    opt = B.options(None, gates="raw", norm_gate="sigmoid")
    # decode
    d = W.decode_inputs(3105, 16, 1, W.QWEN_DIMS)
    g, beta = _raw_gates(rng, d["a"][0].shape)
    dims = d["dims"]
    ds = DeviceStates(d["S0"], d["ring"], torch.bfloat16)
    out = torch.empty((16, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    B.gdn_decode_batched(tdev(d["x"][0], torch.bfloat16), tdev(d["conv_w"], torch.bfloat16), ds.ring_ptrs,
                         tdev(g, torch.float32), tdev(beta, torch.float32), ds.h_ptrs, out, dims,
                         z=tdev(d["z"][0], torch.bfloat16), norm_w=tdev(d["norm_w"], torch.bfloat16), opt=opt)
    r = oracle.decode(d["x"][0], d["conv_w"], d["ring"], g, beta, d["S0"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                      z=d["z"][0], norm_w=d["norm_w"], gates="raw", norm_gate="sigmoid")
    assert slice_err(host(out).reshape(16, dims.Hv, dims.dv), r["out"], np.arange(16)) < TOL_OUT
    assert slice_err(ds.h_host(), r["S"]) < TOL_STATE
    # verify
    d = W.verify_inputs(3106, 6, W.QWEN_DIMS)
    g, beta = _raw_gates(rng, d["a"].shape)
    cu, ks = d["cu"], d["ks"]
    ds = DeviceStates(d["S0"], d["ring"], torch.bfloat16)
    inter, tab = _tables(ds, ks, dims, torch.float32)
    T = int(cu[-1])
    out = torch.empty((T, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    B.gdn_verify_multi(tdev(d["x"], torch.bfloat16), tdev(d["conv_w"], torch.bfloat16), ds.ring_ptrs,
                       tdev(g, torch.float32), tdev(beta, torch.float32), tab, tdev(cu, torch.int32), int(ks.max()),
                       out, dims, z=tdev(d["z"], torch.bfloat16), norm_w=tdev(d["norm_w"], torch.bfloat16), opt=opt)
    r = oracle.verify(d["x"], d["conv_w"], d["ring"], g, beta, d["S0"], cu, dims.Hk, dims.Hv, dims.dk, dims.dv,
                      z=d["z"], norm_w=d["norm_w"], gates="raw", norm_gate="sigmoid")
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), r["out"], row_seq_of(cu)) < TOL_OUT
    assert slice_err(ds.h_host(), r["S"]) < TOL_STATE


def test_raw_gates_and_sigmoid_norm_prefill():
    """Fused front, raw gates in the chunked recurrence (ln a = -softplus(g)),
    sigmoid-gated norm epilogue; and the standalone sigmoid-gated norm."""
    rng = np.random.default_rng(3107)
    d = W.prefill_inputs(3107, [130, 64, 1], W.QWEN_DIMS, act="bf16")
    dims = d["dims"]
    T = int(d["cu"][-1])
    g, beta = _raw_gates(rng, d["a"].shape)
    h = [tdev(d["S0"][i], torch.float32) for i in range(3)]
    ring = [tdev(d["ring"][i], torch.bfloat16) for i in range(3)]
    out = torch.empty((T, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    B.gdn_prefill_chunked(dims, tdev(d["cu"], torch.int32), tdev(g, torch.float32), tdev(beta, torch.float32),
                          B.ptr_array(h), out, x=tdev(d["x"], torch.bfloat16),
                          conv_w=tdev(d["conv_w"], torch.bfloat16), conv_state_ptrs=B.ptr_array(ring),
                          z=tdev(d["z"], torch.bfloat16), norm_w=tdev(d["norm_w"], torch.bfloat16),
                          opt=B.options(None, gates="raw", norm_gate="sigmoid"))
    ref = oracle.prefill(d["x"], g, beta, d["S0"], d["cu"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                         conv_w=d["conv_w"], ring=d["ring"], z=d["z"], norm_w=d["norm_w"], gates="raw",
                         norm_gate="sigmoid")
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["out"], row_seq_of(d["cu"])) < TOL_OUT
    assert slice_err(np.stack([host(t) for t in h]), ref["S"]) < TOL_STATE
    # standalone norm on the oracle's o
    o = ref["o"].astype(np.float32)
    o_t = tdev(o.reshape(T, -1), torch.float32)
    out2 = torch.empty_like(o_t)
    B.gdn_gated_rmsnorm(o_t, tdev(d["z"], torch.bfloat16), tdev(d["norm_w"], torch.bfloat16), out2, dims,
                        opt=B.options(None, norm_gate="sigmoid"))
    ref2 = oracle.gated_rmsnorm(o, d["z"].reshape(T, dims.Hv, dims.dv), d["norm_w"], gate="sigmoid")
    assert slice_err(host(out2).reshape(T, dims.Hv, dims.dv), ref2, row_seq_of(d["cu"])) < 1e-5


# ---------------------------------------------------------------------------
# several consecutive tokens per sequence
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["mixed_bf16", "k17_tiny_fp32", "f16_state", "n128", "config3_rows",
                                  "extreme_raw_gates", "zero_decays"])
def test_decode_tokens(case):
    """k_i tokens per sequence (1..17) against the oracle's token-by-token decode;
    the final state equals, bit for bit, the last state the verify stores for the
    same rows (k_i <= 16), and the conv state advances over all the rows."""
    gates = "direct"
    if case == "mixed_bf16":
        ks = [17, 1, 5, 16, 2, 9, 17, 3]
        d = W.verify_inputs(3108, len(ks), W.QWEN_DIMS, ks=ks)
    elif case == "k17_tiny_fp32":
        ks = [17, 17, 4]
        d = W.verify_inputs(3109, len(ks), W.TINY_DIMS, act="f32", ks=ks)
    elif case == "f16_state":
        ks = [12, 7, 1, 16]
        d = W.verify_inputs(3110, len(ks), W.QWEN_DIMS, ks=ks)
        d["S0"] = f16_exact(d["S0"])
    elif case == "n128":  # the widest batch, k = 1 and 17 alternating, d = 64 heads
        ks = [1, 17] * 64
        d = W.verify_inputs(3113, len(ks), W.Dims(Hk=4, Hv=8, dk=64, dv=64, K=4), ks=ks)
    elif case == "extreme_raw_gates":  # raw g, beta at +-30: products of decays underflow, b saturates
        ks = [17, 16, 9, 2, 1, 13]
        d = W.verify_inputs(3116, len(ks), W.QWEN_DIMS, ks=ks)
        rng = np.random.default_rng(3116)
        d["a"] = rng.choice([-30.0, -3.0, 0.0, 3.0, 30.0], size=d["a"].shape).astype(np.float32)
        d["b"] = rng.choice([-30.0, 0.0, 30.0], size=d["b"].shape).astype(np.float32)
        gates = "raw"
    elif case == "zero_decays":  # a = 0 (the past forgotten) and a = 1 among ordinary decays
        ks = [5, 17, 3, 16]
        d = W.verify_inputs(3120, len(ks), W.QWEN_DIMS, ks=ks)
        rng = np.random.default_rng(3120)
        pick = rng.random(d["a"].shape)
        d["a"] = np.where(pick < 0.15, 0.0, np.where(pick > 0.85, 1.0, d["a"])).astype(np.float32)
    else:  # the launch the bench times: every row of the 64-sequence verify workload
        d = W.config(3)
        ks = list(d["ks"])
    state = "f16" if case == "f16_state" else "f32"
    sdt = torch.float16 if state == "f16" else torch.float32
    dims, act = d["dims"], act_dtype(d)
    cu = d["cu"]
    T = int(cu[-1])
    opt = B.options(sdt, gates=gates)
    ds = DeviceStates(d["S0"], d["ring"], act, sdt)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    x, w = tdev(d["x"], act), tdev(d["conv_w"], act)
    a, b = tdev(d["a"], torch.float32), tdev(d["b"], torch.float32)
    z, nw = tdev(d["z"], act), tdev(d["norm_w"], act)
    B.gdn_decode_tokens(x, w, ds.ring_ptrs, a, b, ds.h_ptrs, tdev(cu, torch.int32), int(max(ks)), out, dims,
                        z=z, norm_w=nw, opt=opt)
    r = oracle.decode_tokens(d["x"], d["conv_w"], d["ring"], d["a"], d["b"], d["S0"], cu, dims.Hk, dims.Hv,
                             dims.dk, dims.dv, z=d["z"], norm_w=d["norm_w"], state=state, gates=gates)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), r["out"], row_seq_of(cu)) < TOL_OUT
    assert slice_err(ds.h_host(), r["S"]) < (TOL_STATE_F16 if state == "f16" else TOL_STATE)
    assert np.array_equal(ds.ring_host(), r["ring"])
    # the verify's stored last state, for the sequences a verify admits
    keep = [i for i in range(len(ks)) if ks[i] <= 16]
    rows, cu_s = _sample_rows(cu, np.array(keep))
    sub = {k: d[k][rows] for k in ("x", "a", "b", "z")}
    ds2 = DeviceStates(d["S0"][keep], d["ring"][keep], act, sdt)
    _, tab = _tables(ds2, np.array(ks)[keep], dims, sdt)
    out2 = torch.empty((len(rows), dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    B.gdn_verify_multi(tdev(sub["x"], act), w, ds2.ring_ptrs, tdev(sub["a"], torch.float32),
                       tdev(sub["b"], torch.float32), tab, tdev(cu_s, torch.int32), 16, out2, dims,
                       z=tdev(sub["z"], act), norm_w=nw, opt=opt)
    torch.cuda.synchronize()
    for j, i in enumerate(keep):
        assert torch.equal(ds.h[i], ds2.h[j]), i
    assert torch.equal(out[torch.from_numpy(rows).to(DEV)], out2)


def test_extreme_raw_gates_and_f16_shapes():
    """Raw gate inputs at +-30 (a and b saturating towards 0 and 1) with binary16
    states at d = 32 and d = 64 and one or four value heads per key head."""
    for dims, seed in ((W.Dims(Hk=4, Hv=4, dk=32, dv=32, K=4), 3114), (W.Dims(Hk=2, Hv=8, dk=64, dv=64, K=3), 3115)):
        d = W.decode_inputs(seed, 6, 3, dims)
        d["S0"] = f16_exact(d["S0"])
        rng = np.random.default_rng(seed)
        ds = DeviceStates(d["S0"], d["ring"], torch.bfloat16, torch.float16)
        S, ring = d["S0"].astype(np.float64), d["ring"].astype(np.float64)
        opt = B.options(torch.float16, gates="raw", norm_gate="sigmoid")
        for step in range(3):
            g = rng.choice([-30.0, -3.0, 0.0, 3.0, 30.0], size=d["a"][step].shape).astype(np.float32)
            beta = rng.choice([-30.0, 0.0, 30.0], size=d["b"][step].shape).astype(np.float32)
            out = torch.empty((6, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
            B.gdn_decode_batched(tdev(d["x"][step], torch.bfloat16), tdev(d["conv_w"], torch.bfloat16), ds.ring_ptrs,
                                 tdev(g, torch.float32), tdev(beta, torch.float32), ds.h_ptrs, out, dims,
                                 z=tdev(d["z"][step], torch.bfloat16), norm_w=tdev(d["norm_w"], torch.bfloat16), opt=opt)
            r = oracle.decode(d["x"][step], d["conv_w"], ring, g, beta, S, dims.Hk, dims.Hv, dims.dk, dims.dv,
                              z=d["z"][step], norm_w=d["norm_w"], gates="raw", norm_gate="sigmoid", state="f16")
            S, ring = r["S"], r["ring"]
            assert slice_err(host(out).reshape(6, dims.Hv, dims.dv), r["out"], np.arange(6)) < TOL_OUT
        assert slice_err(ds.h_host(), S) < TOL_STATE_F16
        assert np.array_equal(ds.ring_host(), ring)


@pytest.mark.parametrize("case", ["config3", "d64_g4"])
def test_woa_bf16_store_and_deterministic(case):
    """The write-on-accept verify's bf16 output is the round-to-nearest-even of its fp32
    output on the same inputs (pairs of columns per store at d = 128, single columns at
    d = 64), and two runs agree bit for bit; the call writes no state."""
    if case == "config3":
        d = W.config(3)
    else:
        d = W.verify_inputs(3131, 7, W.Dims(Hk=2, Hv=8, dk=64, dv=64, K=4), act="bf16")
    dims, act = d["dims"], act_dtype(d)
    T = int(d["cu"][-1])
    x, w = tdev(d["x"], act), tdev(d["conv_w"], act)
    a, b = tdev(d["a"], torch.float32), tdev(d["b"], torch.float32)
    z, nw = tdev(d["z"], act), tdev(d["norm_w"], act)
    cu_t = tdev(d["cu"], torch.int32)
    max_k = int(max(2, d["ks"].max()))
    ds = DeviceStates(d["S0"], d["ring"], act)
    outs = []
    for dt in (torch.float32, torch.float32, torch.bfloat16):
        out = torch.empty((T, dims.Hv * dims.dv), dtype=dt, device=DEV)
        B.gdn_verify_woa(x, w, ds.ring_ptrs, a, b, ds.h_ptrs, cu_t, max_k, out, dims, z=z, norm_w=nw)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0].to(torch.bfloat16), outs[2])
