"""GPU parity at the batch-size limits of the boundary, against the fp64 oracle:
prefill batches above 4,096 sequences (the chunk table then keeps the given
sequence order instead of sorting longest first), the largest batch the
boundary admits (65,535 sequences), a batch whose sequences are all empty, and
a one-token decode over 2,000 sequences.  Small head counts keep the oracle
within seconds.  States and conv states of a batch live in one device block,
reached through per-sequence pointers into it."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_ssm_core_amd import binding as B
from linear_attention_ssm_core_amd import workloads as W
from tests.gpu_util import DEV, TOL_OUT, TOL_STATE, host, row_seq_of, slice_err, tdev

pytestmark = pytest.mark.gpu

F32 = torch.float32


def _block_ptrs(block):
    """Device int64 pointers to the rows block[0], block[1], ... of one allocation."""
    n = block.shape[0]
    step = block[0].numel() * block.element_size()
    return block.data_ptr() + step * torch.arange(n, dtype=torch.int64, device=DEV)


def _prefill_batch(seed, lens, dims):
    d = W.prefill_inputs(seed, lens, dims, act="f32")
    T = int(d["cu"][-1])
    h = tdev(d["S0"], F32)
    ring = tdev(d["ring"], F32)
    out = torch.empty((T, dims.Hv * dims.dv), dtype=F32, device=DEV)
    x = tdev(d["x"], F32) if T else torch.empty((0, dims.conv_dim), dtype=F32, device=DEV)
    z = tdev(d["z"], F32) if T else torch.empty((0, dims.Hv * dims.dv), dtype=F32, device=DEV)
    a = tdev(d["a"], F32) if T else torch.empty((0, dims.Hv), dtype=F32, device=DEV)
    b = tdev(d["b"], F32) if T else torch.empty((0, dims.Hv), dtype=F32, device=DEV)
    print("batch prefill: n=%d T=%d" % (len(lens), T), flush=True)
    B.gdn_prefill_chunked(dims, tdev(d["cu"], torch.int32), a, b, _block_ptrs(h), out, x=x,
                          conv_w=tdev(d["conv_w"], F32), conv_state_ptrs=_block_ptrs(ring), z=z,
                          norm_w=tdev(d["norm_w"], F32))
    torch.cuda.synchronize()
    return d, out, h, ring


@pytest.mark.parametrize("n,max_len,seed,dims", [(5000, 40, 8100, W.TINY_DIMS),
                                                  (65535, 2, 8200, W.Dims(Hk=1, Hv=1, dk=32, dv=32))])
def test_prefill_batch_limits(n, max_len, seed, dims):
    """5,000 sequences of 0..40 rows (2 key / 4 value heads) and 65,535 sequences
    of 0..2 rows (the largest batch admitted; one key and one value head), fused
    front and gated-norm epilogue, fp32."""
    lens = list(np.random.default_rng(seed).integers(0, max_len + 1, size=n))
    d, out, h, ring = _prefill_batch(seed, lens, dims)
    T = int(d["cu"][-1])
    ref = oracle.prefill(d["x"], d["a"], d["b"], d["S0"], d["cu"], dims.Hk, dims.Hv, dims.dk, dims.dv,
                         conv_w=d["conv_w"], ring=d["ring"], z=d["z"], norm_w=d["norm_w"])
    e_out = slice_err(host(out).reshape(T, dims.Hv, dims.dv), ref["out"], row_seq_of(d["cu"]))
    e_state = slice_err(host(h), ref["S"])
    print("batch prefill: e_out=%.2e e_state=%.2e" % (e_out, e_state))
    assert e_out < TOL_OUT and e_state < TOL_STATE
    assert np.array_equal(host(ring), ref["ring"])
    empty = np.flatnonzero(np.diff(d["cu"]) == 0)
    assert np.array_equal(host(h)[empty], d["S0"][empty])  # empty sequences keep their states


def test_prefill_all_sequences_empty():
    """Three sequences, all of length 0 (T = 0): nothing changes."""
    dims = W.TINY_DIMS
    d, out, h, ring = _prefill_batch(8300, [0, 0, 0], dims)
    assert out.numel() == 0
    assert np.array_equal(host(h), d["S0"])
    assert np.array_equal(host(ring), d["ring"])


def test_decode_2000_sequences():
    """One decode step over 2,000 sequences, fp32, with the gated norm."""
    dims = W.TINY_DIMS
    n = 2000
    dd = W.decode_inputs(8400, n, 1, dims, act="f32")
    h = tdev(dd["S0"], F32)
    ring = tdev(dd["ring"], F32)
    out = torch.empty((n, dims.Hv * dims.dv), dtype=F32, device=DEV)
    print("batch decode: n=%d" % n, flush=True)
    B.gdn_decode_batched(tdev(dd["x"][0], F32), tdev(dd["conv_w"], F32), _block_ptrs(ring),
                         tdev(dd["a"][0], F32), tdev(dd["b"][0], F32), _block_ptrs(h), out, dims,
                         z=tdev(dd["z"][0], F32), norm_w=tdev(dd["norm_w"], F32))
    torch.cuda.synchronize()
    ref = oracle.decode(dd["x"][0], dd["conv_w"], dd["ring"], dd["a"][0], dd["b"][0], dd["S0"], dims.Hk, dims.Hv,
                        dims.dk, dims.dv, z=dd["z"][0], norm_w=dd["norm_w"])
    assert slice_err(host(out).reshape(n, dims.Hv, dims.dv), ref["out"]) < TOL_OUT
    assert slice_err(host(h), ref["S"]) < TOL_STATE
    assert np.array_equal(host(ring), ref["ring"])
