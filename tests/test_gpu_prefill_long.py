"""GPU parity of the chunked prefill on long sequences against the fp64
token-by-token oracle: chains of 24 to 257 chunks (whole chunks, a one-row last
chunk, a ragged tail), a packed batch mixing long, short, one-row and empty
sequences, and binary16 states carried over a long chain.  Small head counts
keep the oracle within seconds while the spine's serial chain is long."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_ssm_core_amd import binding as B
from linear_attention_ssm_core_amd import workloads as W
from tests.gpu_util import (DEV, TOL_OUT, TOL_STATE, TOL_STATE_F16, DeviceStates, act_dtype, f16_exact, host,
                            row_seq_of, slice_err, tdev)

pytestmark = pytest.mark.gpu


def _run_fused(d, epilogue, scale=1.0, opt=None, state_dtype=torch.float32):
    dims, act = d["dims"], act_dtype(d)
    T = int(d["cu"][-1])
    ds = DeviceStates(d["S0"], d["ring"], act, state_dtype=state_dtype)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    kw = dict(scale=scale, x=tdev(d["x"], act), conv_w=tdev(d["conv_w"], act), conv_state_ptrs=ds.ring_ptrs)
    if epilogue:
        kw.update(z=tdev(d["z"], act), norm_w=tdev(d["norm_w"], act))
    if opt is not None:
        kw.update(opt=opt)
    B.gdn_prefill_chunked(dims, tdev(d["cu"], torch.int32), tdev(d["a"], torch.float32),
                          tdev(d["b"], torch.float32), ds.h_ptrs, out, **kw)
    torch.cuda.synchronize()
    return out, ds


def _check(d, out, ds, epilogue, scale=1.0, state="f32", tol_state=TOL_STATE):
    dims = d["dims"]
    T = int(d["cu"][-1])
    ref = oracle.prefill(d["x"], d["a"], d["b"], d["S0"], d["cu"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                         conv_w=d["conv_w"], ring=d["ring"], scale=scale, state=state,
                         z=d["z"] if epilogue else None, norm_w=d["norm_w"] if epilogue else None)
    key = "out" if epilogue else "o"
    e_out = slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref[key], row_seq_of(d["cu"]))
    e_state = slice_err(ds.h_host(), ref["S"])
    print("long prefill: T=%d lens=%s e_out=%.2e e_state=%.2e" % (T, list(np.diff(d["cu"])), e_out, e_state))
    assert e_out < TOL_OUT, e_out
    assert e_state < tol_state, e_state
    assert np.array_equal(ds.ring_host(), ref["ring"])


@pytest.mark.parametrize("T", [24 * 64, 24 * 64 + 1, 29 * 64 + 37])
@pytest.mark.parametrize("dims,act", [(W.TINY_DIMS, "f32"), (W.Dims(Hk=1, Hv=4, dk=64, dv=64), "bf16"),
                                      (W.Dims(Hk=2, Hv=4, dk=128, dv=128), "bf16")])
def test_long_single_sequence(dims, act, T):
    """One sequence of 24 chunks, 25 chunks with a one-row last chunk, and 29
    chunks + 37 rows; fused front and gated-norm epilogue, q scaled by d^-1/2."""
    d = W.prefill_inputs(7000 + T + dims.dk, [T], dims, act=act)
    scale = dims.dk ** -0.5
    out, ds = _run_fused(d, epilogue=True, scale=scale)
    _check(d, out, ds, epilogue=True, scale=scale)


@pytest.mark.parametrize("dims,act", [(W.TINY_DIMS, "f32"), (W.Dims(Hk=2, Hv=4, dk=128, dv=128), "bf16")])
def test_long_batch_mixed(dims, act):
    """A packed batch of sequences of 25, 32 and 23 chunks (the last one ragged)
    with short, one-row and empty ones between them."""
    lens = [1600, 0, 70, 2048, 1, 23 * 64 - 5, 64]
    d = W.prefill_inputs(7100 + dims.dk, lens, dims, act=act)
    out, ds = _run_fused(d, epilogue=False)
    _check(d, out, ds, epilogue=False)
    assert np.array_equal(ds.h_host()[1], d["S0"][1])  # the empty sequence keeps its state


def test_long_f16_state():
    """Binary16 states over a 27-chunk chain: the stored state is widened at the
    start and the final one narrowed at the end."""
    dims = W.Dims(Hk=2, Hv=4, dk=128, dv=128)
    d = W.prefill_inputs(7200, [26 * 64 + 11, 300], dims, act="bf16")
    d["S0"] = f16_exact(d["S0"])
    out, ds = _run_fused(d, epilogue=False, opt=B.options(torch.float16), state_dtype=torch.float16)
    gs = ds.h_host()
    assert np.array_equal(gs, f16_exact(gs))
    _check(d, out, ds, epilogue=False, state="f16", tol_state=TOL_STATE_F16)


def test_long_sequence_257_chunks():
    """A single sequence of 257 chunks (the last one 45 rows), 2 key / 4 value
    heads, d = 32, fp32, with the gated-norm epilogue."""
    d = W.prefill_inputs(7300, [256 * 64 + 45], W.TINY_DIMS, act="f32")
    out, ds = _run_fused(d, epilogue=True)
    _check(d, out, ds, epilogue=True)
