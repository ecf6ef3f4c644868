"""GPU parity with large epsilons, against the fp64 oracle fed the same values.

With the default 1e-6 the L2 and RMS epsilons barely change a result on random
inputs, so a kernel that dropped one, applied it outside the square root, or
took the other epsilon would still pass the other tests.  Here l2_eps = 0.5 and
norm_eps = 0.25, of the order of the sums they are added to: the L2 norm of each
q and k head is x (sum x^2 + l2_eps)^(-1/2), and the gated norm divides by
(mean o^2 + norm_eps)^(1/2).  Every entry point that applies them is covered:
the conv front, the chunked prefill with its fused front and norm, the one-token
decode, the k-row verify (outputs and stored states), the write-on-accept verify
in both of its forms (row loop at d = 32, WY form at d = 128), the k-token decode
and the standalone gated norm.  The multi-row modes are also run with an output
scale and no gated norm (which would cancel the scale)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_ssm_core_amd import binding as B
from linear_attention_ssm_core_amd import workloads as W
from tests.gpu_util import (DEV, TOL_OUT, TOL_STATE, DeviceStates, act_dtype, host, row_seq_of, slice_err,
                            tdev)

pytestmark = pytest.mark.gpu

L2_EPS, NORM_EPS = 0.5, 0.25
F32 = torch.float32
CASES = [(W.TINY_DIMS, "f32"), (W.Dims(Hk=2, Hv=4, dk=128, dv=128), "bf16")]


@pytest.mark.parametrize("dims,act", CASES)
def test_conv_l2norm_large_eps(dims, act):
    d = W.prefill_inputs(9000 + dims.dk, [100, 37], dims, act=act)
    T = int(d["cu"][-1])
    ds = DeviceStates(d["S0"], d["ring"], act_dtype(d))
    y = torch.empty((T, dims.conv_dim), dtype=F32, device=DEV)
    B.gdn_conv_l2norm(tdev(d["x"], act_dtype(d)), tdev(d["conv_w"], act_dtype(d)), ds.ring_ptrs,
                      tdev(d["cu"], torch.int32), y, dims, l2_eps=L2_EPS)
    ref_y, ref_ring = oracle.conv_l2norm(d["x"], d["conv_w"], d["ring"], d["cu"], dims.Hk, dims.Hv, dims.dk,
                                         dims.dv, l2_eps=L2_EPS)
    g = host(y).reshape(T, -1, dims.dk)
    r = ref_y.reshape(T, -1, dims.dk)
    assert (np.abs(g - r).max(axis=2) / np.maximum(np.abs(r).max(axis=2), 1e-30)).max() < 1e-5
    assert np.array_equal(ds.ring_host(), ref_ring)


@pytest.mark.parametrize("dims,act", CASES)
def test_prefill_large_eps(dims, act):
    d = W.prefill_inputs(9100 + dims.dk, [150, 70], dims, act=act)
    T = int(d["cu"][-1])
    a_t = act_dtype(d)
    ds = DeviceStates(d["S0"], d["ring"], a_t)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_prefill_chunked(dims, tdev(d["cu"], torch.int32), tdev(d["a"], F32), tdev(d["b"], F32), ds.h_ptrs, out,
                          x=tdev(d["x"], a_t), conv_w=tdev(d["conv_w"], a_t), conv_state_ptrs=ds.ring_ptrs,
                          z=tdev(d["z"], a_t), norm_w=tdev(d["norm_w"], a_t), l2_eps=L2_EPS, norm_eps=NORM_EPS)
    ref = oracle.prefill(d["x"], d["a"], d["b"], d["S0"], d["cu"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                         conv_w=d["conv_w"], ring=d["ring"], z=d["z"], norm_w=d["norm_w"], l2_eps=L2_EPS,
                         norm_eps=NORM_EPS)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["out"], row_seq_of(d["cu"])) < TOL_OUT
    assert slice_err(ds.h_host(), ref["S"]) < TOL_STATE


@pytest.mark.parametrize("dims,act", CASES)
def test_decode_large_eps(dims, act):
    n = 5
    dd = W.decode_inputs(9200 + dims.dk, n, 1, dims, act=act)
    a_t = torch.float32 if act == "f32" else torch.bfloat16
    ds = DeviceStates(dd["S0"], dd["ring"], a_t)
    out = torch.empty((n, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_decode_batched(tdev(dd["x"][0], a_t), tdev(dd["conv_w"], a_t), ds.ring_ptrs, tdev(dd["a"][0], F32),
                         tdev(dd["b"][0], F32), ds.h_ptrs, out, dims, z=tdev(dd["z"][0], a_t),
                         norm_w=tdev(dd["norm_w"], a_t), l2_eps=L2_EPS, norm_eps=NORM_EPS)
    ref = oracle.decode(dd["x"][0], dd["conv_w"], dd["ring"], dd["a"][0], dd["b"][0], dd["S0"], dims.Hk, dims.Hv,
                        dims.dk, dims.dv, z=dd["z"][0], norm_w=dd["norm_w"], l2_eps=L2_EPS, norm_eps=NORM_EPS)
    assert slice_err(host(out).reshape(n, dims.Hv, dims.dv), ref["out"]) < TOL_OUT
    assert slice_err(ds.h_host(), ref["S"]) < TOL_STATE


def _verify_data(dims, act, seed):
    d = W.verify_inputs(seed, 4, dims, act=act, ks=[5, 2, 16, 9])
    return d, (torch.float32 if act == "f32" else torch.bfloat16)


@pytest.mark.parametrize("dims,act", CASES)
def test_verify_large_eps(dims, act):
    d, a_t = _verify_data(dims, act, 9300 + dims.dk)
    n, ks, cu = d["n"], d["ks"], d["cu"]
    T = int(cu[-1])
    ds = DeviceStates(d["S0"], d["ring"], a_t)
    inter = [[torch.full((dims.Hv, dims.dk, dims.dv), float("nan"), device=DEV) for _ in range(ks[i] - 1)]
             for i in range(n)]
    tables = [[None] * n for _ in range(16)]
    for i in range(n):
        tables[0][i] = ds.h[i]
        for t in range(ks[i] - 1):
            tables[t + 1][i] = inter[i][t]
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_verify_multi(tdev(d["x"], a_t), tdev(d["conv_w"], a_t), ds.ring_ptrs, tdev(d["a"], F32),
                       tdev(d["b"], F32), B.wy_tables(tables, DEV), tdev(cu, torch.int32), int(ks.max()), out, dims,
                       z=tdev(d["z"], a_t), norm_w=tdev(d["norm_w"], a_t), l2_eps=L2_EPS, norm_eps=NORM_EPS)
    ref = oracle.verify(d["x"], d["conv_w"], d["ring"], d["a"], d["b"], d["S0"], cu, dims.Hk, dims.Hv, dims.dk,
                        dims.dv, z=d["z"], norm_w=d["norm_w"], l2_eps=L2_EPS, norm_eps=NORM_EPS)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["out"], row_seq_of(cu)) < TOL_OUT
    worst = 0.0
    for i in range(n):
        for t in range(ks[i]):
            g = host(inter[i][t]) if t < ks[i] - 1 else host(ds.h[i])
            worst = max(worst, slice_err(g[None], ref["states"][cu[i] + t][None]))
    assert worst < TOL_STATE, worst


@pytest.mark.parametrize("dims,act", CASES)
def test_woa_verify_large_eps(dims, act):
    d, a_t = _verify_data(dims, act, 9400 + dims.dk)
    ks, cu = d["ks"], d["cu"]
    T = int(cu[-1])
    ds = DeviceStates(d["S0"], d["ring"], a_t)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_verify_woa(tdev(d["x"], a_t), tdev(d["conv_w"], a_t), ds.ring_ptrs, tdev(d["a"], F32), tdev(d["b"], F32),
                     ds.h_ptrs, tdev(cu, torch.int32), int(ks.max()), out, dims, z=tdev(d["z"], a_t),
                     norm_w=tdev(d["norm_w"], a_t), l2_eps=L2_EPS, norm_eps=NORM_EPS)
    ref = oracle.verify_woa(d["x"], d["conv_w"], d["ring"], d["a"], d["b"], d["S0"], cu, dims.Hk, dims.Hv,
                            dims.dk, dims.dv, z=d["z"], norm_w=d["norm_w"], l2_eps=L2_EPS, norm_eps=NORM_EPS)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["out"], row_seq_of(cu)) < TOL_OUT
    assert np.array_equal(ds.h_host(), d["S0"])  # no state is written


@pytest.mark.parametrize("dims,act", CASES)
def test_decode_tokens_large_eps(dims, act):
    d, a_t = _verify_data(dims, act, 9500 + dims.dk)
    ks, cu = d["ks"], d["cu"]
    T = int(cu[-1])
    ds = DeviceStates(d["S0"], d["ring"], a_t)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_decode_tokens(tdev(d["x"], a_t), tdev(d["conv_w"], a_t), ds.ring_ptrs, tdev(d["a"], F32),
                        tdev(d["b"], F32), ds.h_ptrs, tdev(cu, torch.int32), int(ks.max()), out, dims,
                        z=tdev(d["z"], a_t), norm_w=tdev(d["norm_w"], a_t), l2_eps=L2_EPS, norm_eps=NORM_EPS)
    ref = oracle.decode_tokens(d["x"], d["conv_w"], d["ring"], d["a"], d["b"], d["S0"], cu, dims.Hk, dims.Hv,
                               dims.dk, dims.dv, z=d["z"], norm_w=d["norm_w"], l2_eps=L2_EPS, norm_eps=NORM_EPS)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["out"], row_seq_of(cu)) < TOL_OUT
    assert slice_err(ds.h_host(), ref["S"]) < TOL_STATE
    assert np.array_equal(ds.ring_host(), ref["ring"])


def test_gated_rmsnorm_large_eps():
    rng = np.random.default_rng(9600)
    T, dims = 300, W.Dims(Hk=2, Hv=4, dk=128, dv=128)
    o = (rng.standard_normal((T, dims.Hv * dims.dv)) * 0.3).astype(np.float32)
    z = rng.standard_normal((T, dims.Hv * dims.dv)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(dims.dv)).astype(np.float32)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_gated_rmsnorm(tdev(o, F32), tdev(z, F32), tdev(w, F32), out, dims, eps=NORM_EPS)
    ref = oracle.gated_rmsnorm(o.reshape(T, dims.Hv, dims.dv), z.reshape(T, dims.Hv, dims.dv), w, eps=NORM_EPS)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref, np.arange(T)) < 1e-5


# ---------------------------------------------------------------------------
# Output scale without the gated norm (the norm would cancel it): o = scale * S q
# in the row-by-row verify, both write-on-accept forms and the k-token decode.
# ---------------------------------------------------------------------------
SCALE = 0.3


@pytest.mark.parametrize("dims,act", CASES)
def test_multi_row_modes_scale_without_norm(dims, act):
    d, a_t = _verify_data(dims, act, 9700 + dims.dk)
    n, ks, cu = d["n"], d["ks"], d["cu"]
    T = int(cu[-1])
    args = lambda: (tdev(d["x"], a_t), tdev(d["conv_w"], a_t))
    ref = oracle.verify(d["x"], d["conv_w"], d["ring"], d["a"], d["b"], d["S0"], cu, dims.Hk, dims.Hv, dims.dk,
                        dims.dv, scale=SCALE)
    rows = row_seq_of(cu)

    # row-by-row verify, every state stored
    ds = DeviceStates(d["S0"], d["ring"], a_t)
    inter = [[torch.empty((dims.Hv, dims.dk, dims.dv), device=DEV) for _ in range(ks[i] - 1)] for i in range(n)]
    tables = [[None] * n for _ in range(16)]
    for i in range(n):
        tables[0][i] = ds.h[i]
        for t in range(ks[i] - 1):
            tables[t + 1][i] = inter[i][t]
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_verify_multi(*args(), ds.ring_ptrs, tdev(d["a"], F32), tdev(d["b"], F32), B.wy_tables(tables, DEV),
                       tdev(cu, torch.int32), int(ks.max()), out, dims, scale=SCALE)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["o"], rows) < TOL_OUT

    # write-on-accept verify
    ds = DeviceStates(d["S0"], d["ring"], a_t)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_verify_woa(*args(), ds.ring_ptrs, tdev(d["a"], F32), tdev(d["b"], F32), ds.h_ptrs, tdev(cu, torch.int32),
                     int(ks.max()), out, dims, scale=SCALE)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["o"], rows) < TOL_OUT

    # k-token decode (the same rows as consecutive tokens: the same outputs)
    ds = DeviceStates(d["S0"], d["ring"], a_t)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    B.gdn_decode_tokens(*args(), ds.ring_ptrs, tdev(d["a"], F32), tdev(d["b"], F32), ds.h_ptrs,
                        tdev(cu, torch.int32), int(ks.max()), out, dims, scale=SCALE)
    assert slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["o"], rows) < TOL_OUT
