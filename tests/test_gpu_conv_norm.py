"""GPU parity of the conv1d + SiLU + L2 front and the Z-gated RMSNorm against the
fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_ssm_core_amd import binding as B
from linear_attention_ssm_core_amd import workloads as W
from tests.gpu_util import DEV, TOL_OUT, DeviceStates, act_dtype, host, tdev

pytestmark = pytest.mark.gpu


def _conv_case(d, y_dtype):
    dims, act = d["dims"], act_dtype(d)
    T = int(d["cu"][-1])
    ds = DeviceStates(d["S0"], d["ring"], act)
    y = torch.empty((T, dims.conv_dim), dtype=y_dtype, device=DEV)
    B.gdn_conv_l2norm(tdev(d["x"], act), tdev(d["conv_w"], act), ds.ring_ptrs, tdev(d["cu"], torch.int32),
                      y, dims)
    ref_y, ref_ring = oracle.conv_l2norm(d["x"], d["conv_w"], d["ring"], d["cu"], dims.Hk, dims.Hv, dims.dk,
                                         dims.dv)
    return y, ds, ref_y, ref_ring


@pytest.mark.parametrize("lens,dims,act", [
    ([64], W.TINY_DIMS, "f32"),
    ([4096], W.QWEN_DIMS, "bf16"),
    ([1, 0, 2, 3, 700, 65, 0, 129], W.QWEN_DIMS, "bf16"),   # shorter than K-1, empty, ragged
    # conv widths 2 and 3 (the kernel is specialised per width): blocks wholly inside
    # a sequence, blocks at sequence starts, short and empty sequences
    ([100, 0, 37, 64, 5, 1], W.Dims(Hk=2, Hv=4, dk=32, dv=32, K=2), "f32"),
    ([100, 0, 37, 64, 5, 2], W.Dims(Hk=2, Hv=4, dk=64, dv=64, K=3), "bf16"),
])
def test_conv_l2norm(lens, dims, act):
    d = W.prefill_inputs(4000 + len(lens), lens, dims, act=act)
    y, ds, ref_y, ref_ring = _conv_case(d, torch.float32)
    g = host(y)
    # relative error per (row, head block); fp32 arithmetic on exact inputs
    blk = g.reshape(g.shape[0], -1, dims.dk)
    rb = ref_y.reshape(ref_y.shape[0], -1, dims.dk)
    err = np.abs(blk - rb).max(axis=2) / np.maximum(np.abs(rb).max(axis=2), 1e-30)
    assert err.max() < 1e-5 if g.size else True
    assert np.array_equal(ds.ring_host(), ref_ring)
    # bf16 store == round-to-nearest-even of the fp32 result
    y16, _, _, _ = _conv_case(d, torch.bfloat16)
    assert torch.equal(y.to(torch.bfloat16), y16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_rmsnorm(dtype):
    rng = np.random.default_rng(4100)
    T, Hv, dv = 777, 32, 128
    o = rng.standard_normal((T, Hv * dv)).astype(np.float32) * 0.05
    z = rng.standard_normal((T, Hv * dv)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    if dtype == "bf16":
        o, z, w = W.bf16_round(o), W.bf16_round(z), W.bf16_round(w)
    t = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty((T, Hv * dv), dtype=torch.float32, device=DEV)
    dims = W.Dims(Hk=16, Hv=Hv, dk=dv, dv=dv)
    B.gdn_gated_rmsnorm(tdev(o, t), tdev(z, t), tdev(w, t), out, dims)
    ref = oracle.gated_rmsnorm(o.reshape(T, Hv, dv), z.reshape(T, Hv, dv), w)
    g = host(out).reshape(T, Hv, dv)
    err = np.abs(g - ref).max(axis=2) / np.maximum(np.abs(ref).max(axis=2), 1e-30)
    assert err.max() < 1e-5
