"""Seeded synthetic inputs for the GDN mixer core.

This module is the only code shared by the HIP path's tests/benchmark and the
CPU oracle.  It draws random inputs and rounds them to the storage precision;
it holds none of the method's arithmetic (no conv, norm or recurrence).

Recipe (every config): ``numpy.random.default_rng(seed)`` (PCG64); values are
drawn in fp64, rounded to fp32, and, for bf16 activations, rounded to bf16 with
round-to-nearest-even.  Draw order: sequence lengths / draft lengths / accepted
counts, then x, z, g, the b logit, conv_w, norm_w, the initial state, the conv
state rows.

* x, z ~ N(0, 1)
* a = exp(-softplus(g)), g ~ N(0, 1);  b = sigmoid(N(0, 1))   (fp32, [T, Hv])
* conv_w ~ N(0, 1) / sqrt(K)   (K taps; stored in the activation dtype)
* norm_w ~ 1 + N(0, 0.1)       (activation dtype, [d_v], shared by all heads)
* initial state ~ N(0, 0.02^2) (fp32 [n, Hv, d_k, d_v]) or zero
* conv state rows ~ N(0, 1) (activation dtype) or zero

Arrays are returned as numpy float32 holding exactly the values handed to the
kernels (bf16-exact where the activation dtype is bf16).
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Dims:
    Hk: int
    Hv: int
    dk: int
    dv: int
    K: int = 4

    @property
    def conv_dim(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


QWEN_DIMS = Dims(Hk=16, Hv=32, dk=128, dv=128, K=4)
TINY_DIMS = Dims(Hk=2, Hv=4, dk=32, dv=32, K=4)


def bf16_round(x):
    """Round float32 values to the nearest bf16 (ties to even); returns float32.
    (In 32-bit words: the carry out of a finite value's top bit cannot happen, and
    for NaN/infinity patterns it wraps the same way a 64-bit sum truncated to 32
    bits would.)"""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _store(x64, act):
    x32 = np.asarray(x64, dtype=np.float32)
    return bf16_round(x32) if act == "bf16" else x32


def _normal(rng, shape, std=1.0, mean=0.0, act="f32", block=1 << 22):
    """N(mean, std^2) drawn in fp64 (in row blocks to bound memory; the stream is
    the same as one draw), stored in the activation dtype."""
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape)) if shape else 1
    out = np.empty(total, dtype=np.float32)
    pos = 0
    while pos < total:
        m = min(block, total - pos)
        out[pos: pos + m] = _store(mean + std * rng.standard_normal(m), act)
        pos += m
    return out.reshape(shape)


def _gates(rng, shape):
    g = rng.standard_normal(shape)
    a = np.exp(-np.logaddexp(0.0, g))           # exp(-softplus(g))
    blog = rng.standard_normal(shape)
    b = 1.0 / (1.0 + np.exp(-blog))             # sigmoid
    return a.astype(np.float32), b.astype(np.float32)


def _common_tail(rng, n, dims, act, rand_state, state_std):
    conv_w = _normal(rng, (dims.conv_dim, dims.K), std=1.0 / np.sqrt(dims.K), act=act)
    norm_w = _normal(rng, (dims.dv,), std=0.1, mean=1.0, act=act)
    if rand_state:
        S0 = _normal(rng, (n, dims.Hv, dims.dk, dims.dv), std=state_std, act="f32")
        ring = _normal(rng, (n, dims.K - 1, dims.conv_dim), act=act)
    else:
        S0 = np.zeros((n, dims.Hv, dims.dk, dims.dv), dtype=np.float32)
        ring = np.zeros((n, dims.K - 1, dims.conv_dim), dtype=np.float32)
    return conv_w, norm_w, S0, ring


def _rng(seed):
    return seed if isinstance(seed, np.random.Generator) else np.random.default_rng(seed)


def prefill_inputs(seed, lens, dims, act="bf16", rand_state=True, state_std=0.02):
    """Packed varlen prefill inputs for sequences of the given lengths.  ``seed``
    may also be a Generator that already drew the lengths."""
    rng = _rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.zeros(lens.shape[0] + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    n = lens.shape[0]
    x = _normal(rng, (T, dims.conv_dim), act=act)
    z = _normal(rng, (T, dims.Hv * dims.dv), act=act)
    a, b = _gates(rng, (T, dims.Hv))
    conv_w, norm_w, S0, ring = _common_tail(rng, n, dims, act, rand_state, state_std)
    return dict(dims=dims, act=act, cu=cu, x=x, z=z, a=a, b=b, conv_w=conv_w, norm_w=norm_w,
                S0=S0, ring=ring)


def decode_inputs(seed, n, steps, dims, act="bf16", rand_state=True, state_std=0.02):
    """``steps`` consecutive one-token steps for n sequences (fresh x, z, a, b per step)."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (steps, n, dims.conv_dim), act=act)
    z = _normal(rng, (steps, n, dims.Hv * dims.dv), act=act)
    a, b = _gates(rng, (steps, n, dims.Hv))
    conv_w, norm_w, S0, ring = _common_tail(rng, n, dims, act, rand_state, state_std)
    return dict(dims=dims, act=act, n=n, steps=steps, x=x, z=z, a=a, b=b, conv_w=conv_w,
                norm_w=norm_w, S0=S0, ring=ring)


def verify_inputs(seed, n, dims, kmin=2, kmax=16, act="bf16", rand_state=True, state_std=0.02,
                  ks=None):
    """Speculative verify: draft lengths k_i ~ U{kmin..kmax} (or given), accepted
    counts n_i ~ U{1..k_i}, packed rows sequence-major."""
    rng = np.random.default_rng(seed)
    if ks is None:
        ks = rng.integers(kmin, kmax + 1, size=n)
    ks = np.asarray(ks, dtype=np.int64)
    n_acc = np.array([rng.integers(1, k + 1) for k in ks], dtype=np.int32)
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ks)
    T = int(cu[-1])
    x = _normal(rng, (T, dims.conv_dim), act=act)
    z = _normal(rng, (T, dims.Hv * dims.dv), act=act)
    a, b = _gates(rng, (T, dims.Hv))
    conv_w, norm_w, S0, ring = _common_tail(rng, n, dims, act, rand_state, state_std)
    return dict(dims=dims, act=act, n=n, ks=ks.astype(np.int32), n_acc=n_acc, cu=cu, x=x, z=z,
                a=a, b=b, conv_w=conv_w, norm_w=norm_w, S0=S0, ring=ring)


def varlen_lengths(rng, n, lo=512, hi=32768):
    """Log-uniform lengths in [lo, hi]."""
    u = rng.uniform(np.log(lo), np.log(hi), size=n)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)


VARLEN_TARGET_TOKENS = 65536


def varlen_seed(first=1004, n=8, target=VARLEN_TARGET_TOKENS, rel=0.05):
    """The varlen workload's seed: the first seed from ``first`` upward whose
    log-uniform draw of n lengths totals within +-rel of ``target`` tokens (the
    workload is stated as about 65,536 tokens; seed 1004 itself draws 34,336).
    Returns 1018 (lengths 1704 .. 19204, 64,831 tokens)."""
    seed = first
    while True:
        total = int(varlen_lengths(np.random.default_rng(seed), n).sum())
        if abs(total - target) <= rel * target:
            return seed
        seed += 1


def config(idx, steps=None):
    """The five standard workloads, seed = 1000 + index.

    0: tiny fp32 case, 1 sequence, T = 64, 2 key / 4 value heads, d = 32, zero state.
    1: single-sequence chunked prefill, T = 4096, 16 / 32 heads, d = 128, bf16.
    2: batched decode, 128 sequences x 100 steps.
    3: speculative verify, 64 sequences, k ~ U{2..16}, then commit.
    4: varlen packed prefill, 8 sequences log-uniform in 512..32768 totalling about
       65,536 tokens (seed ``varlen_seed()`` = 1018, 64,831 tokens), fused front/epilogue.
    """
    seed = 1000 + idx
    if idx == 0:
        return prefill_inputs(seed, [64], TINY_DIMS, act="f32", rand_state=False)
    if idx == 1:
        return prefill_inputs(seed, [4096], QWEN_DIMS, act="bf16")
    if idx == 2:
        return decode_inputs(seed, 128, 100 if steps is None else steps, QWEN_DIMS, act="bf16")
    if idx == 3:
        return verify_inputs(seed, 64, QWEN_DIMS, 2, 16, act="bf16")
    if idx == 4:
        rng = np.random.default_rng(varlen_seed(seed))
        lens = varlen_lengths(rng, 8)
        return prefill_inputs(rng, lens, QWEN_DIMS, act="bf16")
    raise ValueError(idx)
