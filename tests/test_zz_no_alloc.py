"""The allocation-free prefill (gdn_prefill_chunked_noalloc) against
gdn_prefill_chunked with a caller workspace: two calls in a row on one GPU, the
second with a smaller input, each bit for bit equal to the workspace entry point
on the same inputs (same kernels); the first also against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_ssm_core_amd import binding as B
from linear_attention_ssm_core_amd import workloads as W
from tests.gpu_util import DEV, TOL_OUT, TOL_STATE, DeviceStates, act_dtype, host, row_seq_of, slice_err, tdev

pytestmark = pytest.mark.gpu


def _kw(d, ds, fused, epilogue):
    act = act_dtype(d)
    kw = {}
    if fused:
        kw.update(x=tdev(d["x"], act), conv_w=tdev(d["conv_w"], act), conv_state_ptrs=ds.ring_ptrs)
    else:
        kw.update(y=tdev(d["y"], act))
    if epilogue:
        kw.update(z=tdev(d["z"], act), norm_w=tdev(d["norm_w"], act))
    return kw


def _both(d, fused, epilogue):
    """Run both entry points on separate copies of the states; returns
    (out_ws, ds_ws, out_noalloc, ds_noalloc)."""
    dims, act = d["dims"], act_dtype(d)
    T = int(d["cu"][-1])
    cu = tdev(d["cu"], torch.int32)
    a, b = tdev(d["a"], torch.float32), tdev(d["b"], torch.float32)
    res = []
    for noalloc in (False, True):
        ds = DeviceStates(d["S0"], d["ring"], act)
        out = torch.full((T, dims.Hv * dims.dv), float("nan"), dtype=torch.float32, device=DEV)
        kw = _kw(d, ds, fused, epilogue)
        if noalloc:
            B.gdn_prefill_chunked_noalloc(dims, cu, a, b, ds.h_ptrs, out, **kw)
        else:
            need = B.gdn_prefill_workspace_bytes(dims, cu, a, b, ds.h_ptrs, out, **kw)
            assert 0 < need <= B.PREFILL_SCRATCH_BYTES
            ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)  # garbage, as a reused buffer holds
            B.gdn_prefill_chunked(dims, cu, a, b, ds.h_ptrs, out, workspace=ws, **kw)
        torch.cuda.synchronize()
        res += [out, ds]
    return res


def test_noalloc_prefill_two_calls_second_smaller():
    dims = W.QWEN_DIMS
    # call 1: three sequences (ragged tails), fused conv front and gated-norm epilogue
    d1 = W.prefill_inputs(7001, [300, 64, 129], dims, act="bf16")
    out_w, ds_w, out_n, ds_n = _both(d1, fused=True, epilogue=True)
    assert torch.equal(out_w, out_n)
    assert all(torch.equal(x, y) for x, y in zip(ds_w.h, ds_n.h))
    assert all(torch.equal(x, y) for x, y in zip(ds_w.ring, ds_n.ring))
    ref = oracle.prefill(d1["x"], d1["a"], d1["b"], d1["S0"], d1["cu"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                         conv_w=d1["conv_w"], ring=d1["ring"], z=d1["z"], norm_w=d1["norm_w"])
    T1 = int(d1["cu"][-1])
    assert slice_err(host(out_n).reshape(T1, dims.Hv, dims.dv), ref["out"], row_seq_of(d1["cu"])) < TOL_OUT
    assert slice_err(ds_n.h_host(), ref["S"]) < TOL_STATE
    assert np.array_equal(ds_n.ring_host(), ref["ring"])
    # call 2, smaller: two sequences, y given (no front), no epilogue; the scratch
    # still holds call 1's contents
    d2 = W.prefill_inputs(7002, [100, 37], dims, act="bf16")
    d2["y"] = oracle.conv_l2norm(d2["x"], d2["conv_w"], d2["ring"], d2["cu"], dims.Hk, dims.Hv, dims.dk,
                                 dims.dv)[0].astype(np.float32)
    d2["y"] = W.bf16_round(d2["y"])
    out_w, ds_w, out_n, ds_n = _both(d2, fused=False, epilogue=False)
    assert torch.equal(out_w, out_n)
    assert all(torch.equal(x, y) for x, y in zip(ds_w.h, ds_n.h))


def test_noalloc_prefill_refuses_oversized_call():
    """A call needing more than the scratch array returns GDN_ERR_WORKSPACE and
    changes nothing."""
    dims = W.QWEN_DIMS
    d = W.prefill_inputs(7003, [4096], dims, act="bf16")
    ds = DeviceStates(d["S0"], d["ring"], torch.bfloat16)
    T = 4096
    out = torch.zeros((T, dims.Hv * dims.dv), dtype=torch.float32, device=DEV)
    with pytest.raises(B.GdnError) as e:
        B.gdn_prefill_chunked_noalloc(dims, tdev(d["cu"], torch.int32), tdev(d["a"], torch.float32),
                                      tdev(d["b"], torch.float32), ds.h_ptrs, out,
                                      x=tdev(d["x"], torch.bfloat16), conv_w=tdev(d["conv_w"], torch.bfloat16),
                                      conv_state_ptrs=ds.ring_ptrs)
    assert e.value.status == B.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert np.array_equal(ds.h_host(), d["S0"])
    assert torch.count_nonzero(out).item() == 0
