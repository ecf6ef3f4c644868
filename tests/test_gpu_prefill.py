"""GPU parity of the chunked WY/UT prefill (through the C ABI) against the fp64
token-by-token oracle: the five workload shapes, ragged and empty sequences,
resumed calls and the invariants of the recurrence."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_ssm_core_amd import binding as B
from linear_attention_ssm_core_amd import workloads as W
from tests.gpu_util import (DEV, TOL_OUT, TOL_STATE, DeviceStates, act_dtype, host, row_seq_of, slice_err,
                            tdev)

pytestmark = pytest.mark.gpu


def _run(d, *, fused, epilogue, out_dtype=torch.float32, scale=1.0, y_dtype=None, ds=None):
    """Run gdn_prefill_chunked on workload d.  Unfused: gdn_conv_l2norm first
    (y in y_dtype), then the prefill on y.  Returns (out, ds, y)."""
    dims, act = d["dims"], act_dtype(d)
    T = int(d["cu"][-1])
    if ds is None:
        ds = DeviceStates(d["S0"], d["ring"], act)
    cu = tdev(d["cu"], torch.int32)
    x = tdev(d["x"], act)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=out_dtype, device=DEV)
    kw = dict(scale=scale)
    if epilogue:
        kw.update(z=tdev(d["z"], act), norm_w=tdev(d["norm_w"], act))
    y = None
    if fused:
        kw.update(x=x, conv_w=tdev(d["conv_w"], act), conv_state_ptrs=ds.ring_ptrs)
    else:
        y = torch.empty((T, dims.conv_dim), dtype=y_dtype or act, device=DEV)
        B.gdn_conv_l2norm(x, tdev(d["conv_w"], act), ds.ring_ptrs, cu, y, dims)
        kw.update(y=y)
    B.gdn_prefill_chunked(dims, cu, tdev(d["a"], torch.float32), tdev(d["b"], torch.float32), ds.h_ptrs,
                          out, **kw)
    return out, ds, y


def _ref(d, y=None, heads=None, epilogue=False, scale=1.0):
    dims = d["dims"]
    if y is None:
        return oracle.prefill(d["x"], d["a"], d["b"], d["S0"], d["cu"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                              conv_w=d["conv_w"], ring=d["ring"], scale=scale, heads=heads,
                              z=d["z"] if epilogue else None, norm_w=d["norm_w"] if epilogue else None)
    return oracle.prefill(y, d["a"], d["b"], d["S0"], d["cu"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                          scale=scale, heads=heads, z=d["z"] if epilogue else None,
                          norm_w=d["norm_w"] if epilogue else None)


def _check(d, out, ds, ref, heads=None, check_ring=True):
    dims = d["dims"]
    T = int(d["cu"][-1])
    hl = np.arange(dims.Hv) if heads is None else np.asarray(heads)
    key = "out" if "out" in ref else "o"
    g = host(out).reshape(T, dims.Hv, dims.dv)[:, hl]
    r = ref[key][:, hl]
    e_out = slice_err(g, r, row_seq_of(d["cu"]))
    e_state = slice_err(ds.h_host()[:, hl], ref["S"][:, hl])
    assert e_out < TOL_OUT, e_out
    assert e_state < TOL_STATE, e_state
    if check_ring and "ring" in ref:
        assert np.array_equal(ds.ring_host(), ref["ring"])
    return e_out, e_state


@pytest.mark.parametrize("fused,epilogue", [(True, True), (False, False), (True, False)])
def test_prefill_tiny_fp32(fused, epilogue):
    """1 sequence, T = 64, 2 key / 4 value heads, d = 32, fp32, zero state."""
    d = W.config(0)
    out, ds, y = _run(d, fused=fused, epilogue=epilogue, scale=0.5)
    ref = _ref(d, None if fused else host(y), epilogue=epilogue, scale=0.5)
    _check(d, out, ds, ref, check_ring=fused)


def test_prefill_config1_single_sequence():
    """T = 4096, 16 key / 32 value heads, d = 128, bf16 q/k/v from the conv front,
    random initial state; every head and the final state against the oracle fed
    the same bf16 y."""
    d = W.config(1)
    out, ds, y = _run(d, fused=False, epilogue=False)
    ref = _ref(d, host(y))
    _check(d, out, ds, ref)


def test_prefill_config4_varlen_fused():
    """8 sequences, log-uniform lengths in 512..32768 totalling 64,831 tokens,
    fused conv/L2 front and Z-gated RMSNorm epilogue in one call; every head,
    every output row and every final state against the oracle from the pre-conv
    rows (the front stays fp32 end to end)."""
    d = W.config(4)
    assert abs(int(d["cu"][-1]) - W.VARLEN_TARGET_TOKENS) <= 0.05 * W.VARLEN_TARGET_TOKENS
    out, ds, _ = _run(d, fused=True, epilogue=True)
    ref = _ref(d, epilogue=True)
    _check(d, out, ds, ref)


@pytest.mark.parametrize("dims,act", [(W.Dims(Hk=2, Hv=4, dk=128, dv=128), "bf16"),
                                      (W.Dims(Hk=4, Hv=4, dk=64, dv=64), "f32"),
                                      (W.Dims(Hk=1, Hv=4, dk=64, dv=64), "bf16")])
def test_prefill_ragged_and_empty(dims, act):
    """Lengths 1, 63, 64, 65, 0, 130, 3 (partial chunks, an empty sequence) and
    G = 2, 1, 4 value heads per key head."""
    lens = [1, 63, 64, 65, 0, 130, 3]
    d = W.prefill_inputs(5000 + dims.dk + dims.Hv // dims.Hk, lens, dims, act=act)
    out, ds, _ = _run(d, fused=True, epilogue=True, scale=dims.dk ** -0.5)
    ref = _ref(d, epilogue=True, scale=dims.dk ** -0.5)
    _check(d, out, ds, ref)
    assert np.array_equal(ds.h_host()[4], d["S0"][4])  # the empty sequence keeps its state


@pytest.mark.parametrize("dims,act,n,heads", [(W.TINY_DIMS, "f32", 200, None),
                                              (W.QWEN_DIMS, "bf16", 40, None)])
def test_prefill_many_short_sequences(dims, act, n, heads):
    """Batches of many short sequences (0..150 rows): the chunk table, the
    longest-first order and one spine workgroup set per sequence."""
    lens = np.random.default_rng(4321 + n).integers(0, 151, size=n)
    d = W.prefill_inputs(5000 + n, list(lens), dims, act=act)
    out, ds, y = _run(d, fused=False, epilogue=False, y_dtype=torch.float32)
    _check(d, out, ds, _ref(d, y=host(y), heads=heads), heads=heads, check_ring=False)


def test_prefill_resume_equals_one_call():
    """Prefill of rows [0, 100) then [100, 300) with the carried state equals one
    call over [0, 300) (states and conv states resume through the same buffers)."""
    dims = W.Dims(Hk=2, Hv=4, dk=128, dv=128)
    d = W.prefill_inputs(5100, [300], dims, act="bf16")
    out_all, ds_all, _ = _run(d, fused=True, epilogue=False)
    ds = DeviceStates(d["S0"], d["ring"], torch.bfloat16)
    outs = []
    for lo, hi in [(0, 100), (100, 300)]:
        part = dict(d, cu=np.array([0, hi - lo], dtype=np.int32), x=d["x"][lo:hi], z=d["z"][lo:hi],
                    a=d["a"][lo:hi], b=d["b"][lo:hi])
        o, ds, _ = _run(part, fused=True, epilogue=False, ds=ds)
        outs.append(host(o))
    e = np.abs(np.concatenate(outs) - host(out_all)).max() / np.abs(host(out_all)).max()
    assert e < 1e-4
    assert slice_err(ds.h_host(), ds_all.h_host()) < 1e-4
    assert np.array_equal(ds.ring_host(), ds_all.ring_host())


def test_prefill_invariants():
    """a = 1, b = 0 leaves the state unchanged and o_t = S_0 q_t; a = 0 forgets the
    initial state (the final state does not depend on S_0)."""
    dims = W.Dims(Hk=2, Hv=4, dk=128, dv=128)
    d = W.prefill_inputs(5200, [200], dims, act="bf16")
    d1 = dict(d, a=np.ones_like(d["a"]), b=np.zeros_like(d["b"]))
    out, ds, y = _run(d1, fused=False, epilogue=False)
    assert slice_err(ds.h_host(), d["S0"]) < 1e-6
    q = host(y)[:, : dims.Hk * dims.dk].reshape(-1, dims.Hk, dims.dk)
    ref_o = np.einsum("thi,hij->thj", q[:, [0, 0, 1, 1]], d["S0"][0].astype(np.float64))
    assert slice_err(host(out).reshape(-1, dims.Hv, dims.dv), ref_o, np.zeros(200, int)) < TOL_OUT
    d0 = dict(d, a=np.zeros_like(d["a"]))
    _, ds_a, _ = _run(d0, fused=False, epilogue=False)
    d0b = dict(d0, S0=np.zeros_like(d["S0"]))
    _, ds_b, _ = _run(d0b, fused=False, epilogue=False)
    assert slice_err(ds_a.h_host(), ds_b.h_host()) < 1e-6


def test_prefill_bf16_store_and_determinism():
    dims = W.Dims(Hk=2, Hv=4, dk=128, dv=128)
    d = W.prefill_inputs(5300, [77, 150], dims, act="bf16")
    out32, _, _ = _run(d, fused=True, epilogue=True)
    out32b, _, _ = _run(d, fused=True, epilogue=True)
    assert torch.equal(out32, out32b)
    out16, _, _ = _run(d, fused=True, epilogue=True, out_dtype=torch.bfloat16)
    assert torch.equal(out32.to(torch.bfloat16), out16)


@pytest.mark.parametrize("dims,act,lens", [
    (W.Dims(Hk=4, Hv=16, dk=128, dv=128), "bf16", [70, 1, 130, 0, 64, 200, 3, 65, 129, 17, 256, 40]),
    (W.Dims(Hk=2, Hv=8, dk=64, dv=64), "f32", [5, 64, 33, 0, 1, 97, 128, 12, 70, 2] * 4),
    (W.Dims(Hk=2, Hv=8, dk=64, dv=64), "bf16", [65, 3, 0, 130, 64, 7, 1, 90, 40, 22] * 2)])
def test_prefill_many_sequences_wide_blocks(dims, act, lens):
    """Batches with enough sequences x heads for the spine's wider column blocks
    (64 columns at d = 128 with 12 sequences, and at d = 64 with 40; 32 columns at
    d = 64 with 20), from a y in the activation type; ragged, one-row and empty
    sequences among them."""
    d = W.prefill_inputs(6100 + dims.dk + len(lens), lens, dims, act=act)
    out, ds, y = _run(d, fused=False, epilogue=True, scale=dims.dk ** -0.5)
    ref = _ref(d, host(y), epilogue=True, scale=dims.dk ** -0.5)
    _check(d, out, ds, ref, check_ring=False)
