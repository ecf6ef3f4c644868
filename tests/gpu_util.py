"""Helpers for the GPU parity tests: moving seeded inputs to the device, building
pointer arrays, and the slice-wise error measure the tolerances are stated in."""
import numpy as np
import torch

from linear_attention_ssm_core_amd import binding as B

DEV = "cuda:0"

# Tolerances, max relative error per (sequence, value head) slice,
# max|gpu - ref| / max|ref| over that slice.
TOL_OUT = 2e-3      # outputs computed from bf16 (or fp32) inputs, compared in fp32
TOL_STATE = 1e-4    # fp32 recurrent states
# binary16 states: both sides round every stored state to nearest even, so they
# differ only where the fp32 and the fp64 value of an element fall on different
# sides of a rounding boundary -- one binary16 ulp of that element, at most
# 2^-10 of the slice's largest magnitude; two such flips are allowed.
TOL_STATE_F16 = 2.0 ** -9


def tdev(a, dtype):
    """numpy float32 array (bf16-exact when dtype is bf16) -> device tensor, exactly."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(DEV)


def act_dtype(d):
    return torch.bfloat16 if d["act"] == "bf16" else torch.float32


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def slice_err(gpu, ref, row_seq=None):
    """gpu/ref [rows, Hv, dv] (or [n, Hv, dk, dv] states when row_seq is None):
    the worst per-(sequence, head) relative error."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    if not np.all(np.isfinite(gpu)):
        return float("inf")  # a NaN or infinity anywhere fails every tolerance
    worst = 0.0
    if row_seq is None:
        diff = np.abs(gpu - ref).reshape(ref.shape[0], ref.shape[1], -1).max(axis=2)
        mag = np.abs(ref).reshape(ref.shape[0], ref.shape[1], -1).max(axis=2)
        return float(np.max(diff / np.maximum(mag, 1e-30)))
    row_seq = np.asarray(row_seq)
    if row_seq.size == 0:
        return worst
    # rows of one sequence are contiguous (packed batches): reduce each run of rows
    starts = np.flatnonzero(np.r_[True, row_seq[1:] != row_seq[:-1]])
    diff = np.maximum.reduceat(np.abs(gpu - ref).max(axis=2), starts, axis=0)
    mag = np.maximum.reduceat(np.abs(ref).max(axis=2), starts, axis=0)
    return float(np.max(diff / np.maximum(mag, 1e-30)))


def row_seq_of(cu):
    cu = np.asarray(cu)
    return np.repeat(np.arange(len(cu) - 1), np.diff(cu))


class DeviceStates:
    """Per-sequence fp32 states [Hv, dk, dv] and conv states [K-1, conv_dim] as
    separate device buffers reached through pointer arrays (pool-slot style)."""

    def __init__(self, S0, ring, act, state_dtype=torch.float32):
        self.h = [tdev(S0[i], state_dtype) for i in range(S0.shape[0])]
        self.ring = [tdev(ring[i], act) for i in range(ring.shape[0])]
        self.h_ptrs = B.ptr_array(self.h) if self.h else torch.zeros(0, dtype=torch.int64, device=DEV)
        self.ring_ptrs = B.ptr_array(self.ring) if self.ring else torch.zeros(0, dtype=torch.int64, device=DEV)

    def h_host(self):
        return np.stack([host(t) for t in self.h])

    def ring_host(self):
        return np.stack([host(t) for t in self.ring])


def f16_exact(a):
    """The nearest binary16 values of an fp32 array, as fp32 (a state stored as
    binary16 is handed to the oracle as exactly these values)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)
