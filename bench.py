#!/usr/bin/env python3
"""Throughput of the GDN mixer core on one MI355X.

One step is one pass of the whole hot path over synthetic inputs resident in HBM:

  prefill  T = 4096 tokens, 16 key / 32 value heads, d = 128, bf16 activations,
           fp32 state: gdn_conv_l2norm -> gdn_prefill_chunked -> gdn_gated_rmsnorm
  decode   128 sequences x 100 consecutive steps of gdn_decode_batched (fused
           conv/L2 prologue and gated-norm epilogue, fp32 states in place); the
           100 launches cycle over DECODE_LAYERS = 4 disjoint sets of the 128
           sequences' states and conv states (the per-layer states of a 4-layer
           stack: 1 GiB of fp32 state, four times the 256 MB on-package cache), so
           every launch streams its states from HBM
  verify   64 sequences, draft lengths k ~ U{2..16}: gdn_verify_multi writing every
           intermediate state through the WY tables, then gdn_verify_commit; the
           sequence states and conv states alternate between two sets from one
           step to the next

value = tokens processed per step / step time (prefill tokens + decode
sequence-tokens + verify rows).  The JSON line also carries per-phase figures,
the roofline of the dominant kernel (from HIP events around each of its
launches) and the fp64 CPU oracle timed on a bounded sample of the same work.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --copy-calib    # plain 1 GiB copy, to scale HBM counters
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK = 8.0e12           # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15     # FLOP/s, MI355X dense bf16
VALU_FP32_PEAK = 157.3e12   # FLOP/s, MI355X fp32 vector (packed issue; half without it)

D, HK, HV, C = 128, 16, 32, 64
STATE_BYTES = HV * D * D * 4            # one sequence's fp32 state, 2 MiB
CONV_DIM = 2 * HK * D + HV * D          # 8192
DECODE_LAYERS = 4                       # disjoint state sets the decode launches cycle over
VERIFY_SETS = 2                         # state sets the verify/commit alternate between


# HBM traffic of one decode launch (recurrent_kernel<128,2,1>) in the bench step --
# cache-cold, the 100 launches cycling over DECODE_LAYERS state sets -- from two
# rocprofv3 counter runs of `bench.py --steps 1 --warmup 0 --no-cpu-baseline`
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, mean of the step's decode dispatches),
# each scaled by what the same counter reads for one 1 GiB device copy (`bench.py
# --copy-calib`: FETCH_SIZE 524302.1 KiB, WRITE_SIZE 1048576.0 KiB per copy).  The
# figures hold for the kernel sources they were taken on only (SHA-256 over the files
# below); for any other source the traffic is reported as unknown.
DECODE_TRAFFIC = {
    "sources": ["linear_attention_ssm_core_amd/csrc/recurrent_kernel.h",
                "linear_attention_ssm_core_amd/csrc/recurrent_decode.hip",
                "linear_attention_ssm_core_amd/csrc/common.h", "linear_attention_ssm_core_amd/csrc/internal.h"],
    "sha256": "a4dfcdce4b6656176b1d681c1a592f665d4198cf8b425aa59b5de7f61adc618e",
    "fetch_kib": 135901.0, "write_kib": 269524.6,
    "fetch_scale": 1048576.0 / 524302.1, "write_scale": 1048576.0 / 1048576.0,
}


def decode_traffic_bytes():
    """Measured HBM bytes of one decode launch, or None if the kernel has changed since."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in DECODE_TRAFFIC["sources"]:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != DECODE_TRAFFIC["sha256"]:
        return None
    t = DECODE_TRAFFIC
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0


def decode_bytes_per_seq():
    """Algorithmic HBM bytes of one sequence-token of batched decode."""
    return (2 * STATE_BYTES            # state read + written
            + CONV_DIM * 2             # x row (bf16)
            + 2 * 3 * CONV_DIM * 2     # conv state read + written
            + HV * D * 2               # z (bf16)
            + HV * D * 2               # out (bf16)
            + 2 * HV * 4)              # a, b


def verify_bytes(ks):
    per_seq = STATE_BYTES * (1 + ks) + 3 * CONV_DIM * 2
    per_row = CONV_DIM * 2 + HV * D * 2 + HV * D * 2 + 2 * HV * 4
    return int(np.sum(per_seq) + per_row * np.sum(ks)) + CONV_DIM * 4 * 2


def stash_row_bytes():
    """One write-on-accept stash row: k_hat of every key head, u and a of every value head."""
    return ((HK * D + HV * D + HV + 3) // 4 * 4) * 4


def woa_verify_bytes(ks):
    """Write-on-accept verify: one state read per sequence, the stash row of every row."""
    per_seq = STATE_BYTES + 3 * CONV_DIM * 2
    per_row = CONV_DIM * 2 + HV * D * 2 + HV * D * 2 + 2 * HV * 4 + stash_row_bytes()
    return int(len(ks) * per_seq + per_row * np.sum(ks)) + CONV_DIM * 4 * 2


def fold_bytes(n_acc):
    """Fold: every state read and written once, the accepted stash rows read, the
    conv state rebuilt from the accepted rows."""
    per_seq = 2 * STATE_BYTES + 2 * 3 * CONV_DIM * 2
    return int(len(n_acc) * per_seq + np.sum(n_acc) * (stash_row_bytes() + CONV_DIM * 2))


def tokens_bytes(ks, state_bytes=None):
    """k consecutive tokens per sequence: the state read and written once."""
    sb = STATE_BYTES if state_bytes is None else state_bytes
    per_seq = 2 * sb + 2 * 3 * CONV_DIM * 2
    per_row = CONV_DIM * 2 + HV * D * 2 + HV * D * 2 + 2 * HV * 4
    return int(len(ks) * per_seq + per_row * np.sum(ks)) + CONV_DIM * 4 * 2


def prefill_flops_per_token():
    return HV * (6 * D * D + C * D + 2 * C * D + C * C / 3.0) + HK * (2 * C * D)


def prefill_bytes(T):
    # q_hat, k_hat, v in (bf16), out (bf16), a, b, plus the state read and written
    return T * (CONV_DIM * 2 + HV * D * 2 + 2 * HV * 4) + 2 * STATE_BYTES


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    return ap.parse_args()


def copy_calibration(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}))


class Workloads:
    """Device buffers for the three phases, filled from the seeded generator."""

    def __init__(self, torch, B, W):
        dev = "cuda"
        bf, f32 = torch.bfloat16, torch.float32
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
        self.dims = W.QWEN_DIMS
        # prefill (T = 4096)
        p = W.config(1)
        self.p_T = int(p["cu"][-1])
        self.p_cu = t(p["cu"], torch.int32)
        self.p_x = t(p["x"], bf)
        self.p_z = t(p["z"], bf)
        self.p_a = t(p["a"], f32)
        self.p_b = t(p["b"], f32)
        self.p_w = t(p["conv_w"], bf)
        self.p_nw = t(p["norm_w"], bf)
        self.p_h = [t(p["S0"][i], f32) for i in range(p["S0"].shape[0])]
        self.p_ring = [t(p["ring"][i], bf) for i in range(p["ring"].shape[0])]
        self.p_hp, self.p_rp = B.ptr_array(self.p_h), B.ptr_array(self.p_ring)
        self.p_y = torch.empty((self.p_T, CONV_DIM), dtype=bf, device=dev)
        self.p_o = torch.empty((self.p_T, HV * D), dtype=bf, device=dev)
        self.p_out = torch.empty((self.p_T, HV * D), dtype=bf, device=dev)
        nb = B.gdn_prefill_workspace_bytes(self.dims, self.p_cu, self.p_a, self.p_b, self.p_hp, self.p_o,
                                           y=self.p_y)
        self.p_ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        # decode (128 sequences x 100 steps)
        d = W.config(2)
        self.d_n, self.d_steps = d["n"], d["steps"]
        self.d_x = t(d["x"], bf)
        self.d_z = t(d["z"], bf)
        self.d_a = t(d["a"], f32)
        self.d_b = t(d["b"], f32)
        self.d_w = t(d["conv_w"], bf)
        self.d_nw = t(d["norm_w"], bf)
        # DECODE_LAYERS disjoint sets of states and conv states (each starts from the
        # workload's initial values); launch s uses set s % DECODE_LAYERS
        self.d_h = [[t(d["S0"][i], f32) for i in range(self.d_n)] for _ in range(DECODE_LAYERS)]
        self.d_ring = [[t(d["ring"][i], bf) for i in range(self.d_n)] for _ in range(DECODE_LAYERS)]
        self.d_hp = [B.ptr_array(hs) for hs in self.d_h]
        self.d_rp = [B.ptr_array(rs) for rs in self.d_ring]
        self.d_out = torch.empty((self.d_n, HV * D), dtype=bf, device=dev)
        # verify (64 sequences, k ~ U{2..16}) and commit
        v = W.config(3)
        self.v_n, self.v_ks = v["n"], v["ks"].astype(np.int64)
        self.v_rows = int(v["cu"][-1])
        self.v_cu = t(v["cu"], torch.int32)
        self.v_x = t(v["x"], bf)
        self.v_z = t(v["z"], bf)
        self.v_a = t(v["a"], f32)
        self.v_b = t(v["b"], f32)
        self.v_w = t(v["conv_w"], bf)
        self.v_nw = t(v["norm_w"], bf)
        # VERIFY_SETS sets of sequence states (table 0) and conv states, alternating
        # per step; the intermediate-state buffers are shared (written, then read by
        # the commit of the same step)
        self.v_h = [[t(v["S0"][i], f32) for i in range(self.v_n)] for _ in range(VERIFY_SETS)]
        self.v_ring = [[t(v["ring"][i], bf) for i in range(self.v_n)] for _ in range(VERIFY_SETS)]
        self.v_rp = [B.ptr_array(rs) for rs in self.v_ring]
        self.v_inter = [[torch.empty((HV, D, D), dtype=f32, device=dev) for _ in range(k - 1)] for k in self.v_ks]
        self.v_tab = []
        for hs in self.v_h:
            tables = [[None] * self.v_n for _ in range(16)]
            for i in range(self.v_n):
                tables[0][i] = hs[i]
                for j, buf in enumerate(self.v_inter[i]):
                    tables[j + 1][i] = buf
            self.v_tab.append(B.wy_tables(tables, dev))
        self.v_out = torch.empty((self.v_rows, HV * D), dtype=bf, device=dev)
        self.v_nacc = t(v["n_acc"], torch.int32)
        self.v_maxk = int(self.v_ks.max())
        self.tokens_per_step = self.p_T + self.d_n * self.d_steps + self.v_rows


def run_step(torch, B, w, step, ev=None):
    """One pass of the hot path (step: its index, which picks the verify's state
    set).  ev: dict of lists that receives HIP events."""
    rec = (lambda key: ev[key].append(_event(torch))) if ev is not None else (lambda key: None)
    dims = w.dims
    rec("p0")
    B.gdn_conv_l2norm(w.p_x, w.p_w, w.p_rp, w.p_cu, w.p_y, dims)
    rec("p1")
    B.gdn_prefill_chunked(dims, w.p_cu, w.p_a, w.p_b, w.p_hp, w.p_o, y=w.p_y, workspace=w.p_ws)
    rec("p2")
    B.gdn_gated_rmsnorm(w.p_o, w.p_z, w.p_nw, w.p_out, dims)
    rec("p3")
    # one event pair around the back-to-back decode launches (an event pair per launch
    # would put 200 timing markers into the step): their average duration is the
    # pair's interval over the launch count
    rec("d0")
    for s in range(w.d_steps):
        L = s % DECODE_LAYERS
        B.gdn_decode_batched(w.d_x[s], w.d_w, w.d_rp[L], w.d_a[s], w.d_b[s], w.d_hp[L], w.d_out, dims,
                             z=w.d_z[s], norm_w=w.d_nw)
    rec("d1")
    vs = step % VERIFY_SETS
    rec("v0")
    B.gdn_verify_multi(w.v_x, w.v_w, w.v_rp[vs], w.v_a, w.v_b, w.v_tab[vs], w.v_cu, w.v_maxk, w.v_out, dims,
                       z=w.v_z, norm_w=w.v_nw)
    rec("v1")
    B.gdn_verify_commit(w.v_x, w.v_rp[vs], w.v_tab[vs], w.v_cu, w.v_nacc, dims)
    rec("v2")


def _timed(torch, fn, reps, warm=1):
    """Mean duration (ms) of fn() over reps back-to-back calls, one event pair
    on the launch stream, after warm untimed calls."""
    for _ in range(warm):
        fn()
    a, b = _event(torch), None
    for _ in range(reps):
        fn()
    b = _event(torch)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def variant_phases(torch, B, W, w, reps=10):
    """The variant forms on the step's workloads, timed outside the step on
    buffers of their own: write-on-accept verify + fold, binary16-state decode,
    the k-token decode, and decode with raw gates and the sigmoid-gated norm."""
    dev, bf, f32, f16 = "cuda", torch.bfloat16, torch.float32, torch.float16
    dims = w.dims
    res = {}
    v = W.config(3)
    # DECODE_LAYERS disjoint state sets, used in turn by consecutive calls, so that no
    # call finds its 128 MiB of states in the on-package cache
    nset = DECODE_LAYERS
    h = [[torch.from_numpy(v["S0"][i]).to(f32).to(dev) for i in range(w.v_n)] for _ in range(nset)]
    hp = [B.ptr_array(hs) for hs in h]
    ring = [[torch.from_numpy(v["ring"][i]).to(bf).to(dev) for i in range(w.v_n)] for _ in range(nset)]
    rp = [B.ptr_array(rs) for rs in ring]
    stash = torch.empty(max(B.gdn_woa_stash_bytes(w.v_x, w.v_cu, w.v_maxk, w.v_out, dims) // 4, 1),
                        dtype=f32, device=dev)
    turn = [0]

    def nxt():
        turn[0] += 1
        return turn[0] % nset
    woa = lambda j: B.gdn_verify_woa(w.v_x, w.v_w, rp[j], w.v_a, w.v_b, hp[j], w.v_cu, w.v_maxk, w.v_out, dims,
                                     stash=stash, z=w.v_z, norm_w=w.v_nw)
    fold = lambda j: B.gdn_fold_accepted(w.v_x, rp[j], hp[j], stash, w.v_cu, w.v_nacc, dims)
    # untimed calls first over every state set, so that the timed loops do not include
    # the first touch of freshly allocated states
    ms_v = _timed(torch, lambda: woa(nxt()), reps, warm=nset)
    ms_f = _timed(torch, lambda: fold(nxt()), reps, warm=nset)
    vb, fb = woa_verify_bytes(w.v_ks), fold_bytes(v["n_acc"])
    # k-token decode, row by row in fp32: S k and S q (2 d^2 each), S <- a S + u k^T (3 d^2)
    # per row and value head, reported as a rate against the vector-ALU peak (its bound is
    # the chain of per-row reductions; the write-on-accept verify takes the WY form on the
    # matrix cores and is bound by its bytes)
    row_flops = 7 * D * D * HV * w.v_rows
    valu = lambda ms: {"tflops": row_flops / (ms / 1e3) / 1e12,
                       "frac": row_flops / (ms / 1e3) / VALU_FP32_PEAK,
                       "frac_unpacked": row_flops / (ms / 1e3) / (VALU_FP32_PEAK / 2)}
    print("bench: write-on-accept verify and fold timed", file=sys.stderr, flush=True)
    res["verify_woa"] = {"rows": w.v_rows, "ms": ms_v, "fold_ms": ms_f, "tokens_per_s": w.v_rows / (ms_v / 1e3),
                         "gb_per_s": vb / (ms_v / 1e3) / 1e9, "hbm_frac": vb / (ms_v / 1e3) / HBM_PEAK,
                         "fold_gb_per_s": fb / (ms_f / 1e3) / 1e9, "fold_hbm_frac": fb / (ms_f / 1e3) / HBM_PEAK,
                         "bytes": vb, "fold_bytes": fb, "bound": "hbm"}
    # k consecutive tokens per sequence on the verify's rows (state written once)
    toks = lambda j: B.gdn_decode_tokens(w.v_x, w.v_w, rp[j], w.v_a, w.v_b, hp[j], w.v_cu, w.v_maxk, w.v_out,
                                         dims, z=w.v_z, norm_w=w.v_nw)
    ms_t = _timed(torch, lambda: toks(nxt()), reps, warm=nset)
    tb = tokens_bytes(w.v_ks)
    res["decode_tokens"] = {"rows": w.v_rows, "ms": ms_t, "tokens_per_s": w.v_rows / (ms_t / 1e3),
                            "gb_per_s": tb / (ms_t / 1e3) / 1e9, "hbm_frac": tb / (ms_t / 1e3) / HBM_PEAK,
                            "bound": "row chain", "valu": valu(ms_t)}
    del h, stash
    # binary16 states: the decode workload, 100 steps
    d = W.config(2)
    h16 = [[torch.from_numpy(d["S0"][i]).to(f16).to(dev) for i in range(w.d_n)] for _ in range(DECODE_LAYERS)]
    hp16 = [B.ptr_array(hs) for hs in h16]
    opt16 = B.options(f16)

    def dec16():
        for s_ in range(w.d_steps):
            L = s_ % DECODE_LAYERS
            B.gdn_decode_batched(w.d_x[s_], w.d_w, w.d_rp[L], w.d_a[s_], w.d_b[s_], hp16[L], w.d_out, dims,
                                 z=w.d_z[s_], norm_w=w.d_nw, opt=opt16)
    ms16 = _timed(torch, dec16, 1) / w.d_steps
    db16 = w.d_n * (decode_bytes_per_seq() - STATE_BYTES) + CONV_DIM * 4 * 2 + D * 2
    res["decode_f16_state"] = {"ms_per_launch": ms16, "tokens_per_s": w.d_n / (ms16 / 1e3),
                               "gb_per_s": db16 / (ms16 / 1e3) / 1e9, "hbm_frac": db16 / (ms16 / 1e3) / HBM_PEAK}
    del h16
    # raw gate inputs and the sigmoid-gated norm (the fp32-state decode otherwise,
    # cycling over the step's state sets)
    optg = B.options(None, gates="raw", norm_gate="sigmoid")

    def decg():
        for s_ in range(w.d_steps):
            L = s_ % DECODE_LAYERS
            B.gdn_decode_batched(w.d_x[s_], w.d_w, w.d_rp[L], w.d_a[s_], w.d_b[s_], w.d_hp[L], w.d_out, dims,
                                 z=w.d_z[s_], norm_w=w.d_nw, opt=optg)
    msg = _timed(torch, decg, 1) / w.d_steps
    db = w.d_n * decode_bytes_per_seq() + CONV_DIM * 4 * 2 + D * 2
    res["decode_raw_gates_sigmoid_norm"] = {"ms_per_launch": msg, "gb_per_s": db / (msg / 1e3) / 1e9,
                                            "hbm_frac": db / (msg / 1e3) / HBM_PEAK}
    # the same 128 states re-read and re-written by all 100 launches (256 MiB, about
    # the size of the on-package cache, which can serve part of the traffic): the
    # cache-warm figure, for comparison with the step's cache-cold one

    def dec_warm():
        for s_ in range(w.d_steps):
            B.gdn_decode_batched(w.d_x[s_], w.d_w, w.d_rp[0], w.d_a[s_], w.d_b[s_], w.d_hp[0], w.d_out, dims,
                                 z=w.d_z[s_], norm_w=w.d_nw)
    msw = _timed(torch, dec_warm, 1) / w.d_steps
    res["decode_cache_warm"] = {"ms_per_launch": msw, "gb_per_s": db / (msw / 1e3) / 1e9,
                                "hbm_frac": db / (msw / 1e3) / HBM_PEAK,
                                "note": "one set of 128 states (256 MiB) for all 100 launches"}
    print("bench: decode variants timed; generating the varlen prefill inputs", file=sys.stderr, flush=True)
    # the varlen packed prefill: 8 sequences, log-uniform lengths totalling about
    # 65,536 tokens, one call with the conv + L2 front and the gated-norm epilogue fused
    p = W.config(4)
    T4 = int(p["cu"][-1])
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)
    cu4, x4, z4 = t(p["cu"], torch.int32), t(p["x"], bf), t(p["z"], bf)
    a4, b4, w4, nw4 = t(p["a"], f32), t(p["b"], f32), t(p["conv_w"], bf), t(p["norm_w"], bf)
    h4 = [t(p["S0"][i], f32) for i in range(p["S0"].shape[0])]
    r4 = [t(p["ring"][i], bf) for i in range(p["ring"].shape[0])]
    hp4, rp4 = B.ptr_array(h4), B.ptr_array(r4)
    out4 = torch.empty((T4, HV * D), dtype=bf, device=dev)
    kw4 = dict(x=x4, conv_w=w4, conv_state_ptrs=rp4, z=z4, norm_w=nw4)
    ws4 = torch.empty(max(B.gdn_prefill_workspace_bytes(dims, cu4, a4, b4, hp4, out4, **kw4), 1), dtype=torch.uint8,
                      device=dev)
    ms4 = _timed(torch, lambda: B.gdn_prefill_chunked(dims, cu4, a4, b4, hp4, out4, workspace=ws4, **kw4), 3)
    fl4 = prefill_flops_per_token() * T4
    by4 = T4 * (CONV_DIM * 2 + 2 * HV * D * 2 + 2 * HV * 4) + len(h4) * 2 * STATE_BYTES
    res["prefill_varlen_fused"] = {"tokens": T4, "sequences": len(h4), "longest": int(np.max(np.diff(p["cu"]))),
                                   "ms": ms4, "tokens_per_s": T4 / (ms4 / 1e3),
                                   "tflops": fl4 / (ms4 / 1e3) / 1e12, "mfma_frac": fl4 / (ms4 / 1e3) / MFMA_BF16_PEAK,
                                   "hbm_frac": by4 / (ms4 / 1e3) / HBM_PEAK}
    return res


def copy_bandwidth(torch, nbytes=1 << 30, reps=5):
    """Attainable read+write bandwidth of a plain device copy (torch), GB/s."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2 * nbytes / (ms / 1e3) / 1e9


def gemm_tflops(torch, n=8192, reps=5):
    """Attainable dense bf16 matrix-core rate: a plain n x n x n product through
    torch (the vendor GEMM library), TFLOP/s."""
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    c = torch.mm(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return 2.0 * n ** 3 / (ms / 1e3) / 1e12


def fill_bandwidth(torch, nbytes=1 << 30, reps=5):
    """Attainable write-only bandwidth of a plain device fill (torch), GB/s."""
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.fill_(1)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.fill_(2)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del dst
    return nbytes / (ms / 1e3) / 1e9


def _event(torch):
    e = torch.cuda.Event(enable_timing=True)
    e.record(torch.cuda.current_stream())
    return e


def _pair_ms(a, b):
    return [x.elapsed_time(y) for x, y in zip(a, b)]


def cpu_baseline(W):
    """The fp64 oracle, as it stands, on a bounded sample of each phase; each
    phase's time is scaled to the step's token count."""
    import oracle
    dims = W.QWEN_DIMS
    threads = oracle.num_threads()
    t_total = 0.0
    # prefill: all 32 heads, first 1024 of the 4096 tokens
    p = W.config(1)
    Tp = 1024
    cu = np.array([0, Tp], dtype=np.int32)
    t0 = time.perf_counter()
    oracle.prefill(p["x"][:Tp], p["a"][:Tp], p["b"][:Tp], p["S0"], cu, dims.Hk, dims.Hv, dims.dk, dims.dv,
                   conv_w=p["conv_w"], ring=p["ring"], z=p["z"][:Tp], norm_w=p["norm_w"])
    t_pre = (time.perf_counter() - t0) * (4096 / Tp)
    # decode: 48 of 128 sequences, 10 of 100 steps
    d = W.config(2, steps=10)
    ns, steps = 48, 10
    S, ring = d["S0"][:ns], d["ring"][:ns]
    t0 = time.perf_counter()
    for s in range(steps):
        r = oracle.decode(d["x"][s][:ns], d["conv_w"], ring, d["a"][s][:ns], d["b"][s][:ns], S, dims.Hk,
                          dims.Hv, dims.dk, dims.dv, z=d["z"][s][:ns], norm_w=d["norm_w"])
        S, ring = r["S"], r["ring"]
    t_dec = (time.perf_counter() - t0) * (128 / ns) * (100 / steps)
    # verify: 24 of 64 sequences (all of their rows), then commit
    v = W.config(3)
    sel = np.arange(24)
    rows = np.concatenate([np.arange(v["cu"][i], v["cu"][i + 1]) for i in sel])
    cu_s = np.concatenate([[0], np.cumsum(v["ks"][sel])]).astype(np.int32)
    t0 = time.perf_counter()
    ref = oracle.verify(v["x"][rows], v["conv_w"], v["ring"][sel], v["a"][rows], v["b"][rows], v["S0"][sel],
                        cu_s, dims.Hk, dims.Hv, dims.dk, dims.dv, z=v["z"][rows], norm_w=v["norm_w"])
    oracle.commit(ref["states"], v["n_acc"][sel], cu_s, v["ring"][sel], v["x"][rows])
    t_ver = (time.perf_counter() - t0) * (int(v["cu"][-1]) / len(rows))
    t_total = t_pre + t_dec + t_ver
    tokens = 4096 + 128 * 100 + int(v["cu"][-1])
    # the same oracle on one thread, decode of 8 sequences for 2 steps (per sequence-token)
    oracle.set_num_threads(1)
    S1, ring1 = d["S0"][:8], d["ring"][:8]
    t0 = time.perf_counter()
    for s in range(2):
        r = oracle.decode(d["x"][s][:8], d["conv_w"], ring1, d["a"][s][:8], d["b"][s][:8], S1, dims.Hk, dims.Hv,
                          dims.dk, dims.dv, z=d["z"][s][:8], norm_w=d["norm_w"])
        S1, ring1 = r["S"], r["ring"]
    one_thread = 16 / (time.perf_counter() - t0)
    oracle.set_num_threads(threads)
    host = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            host = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpu": host, "decode_tokens_per_s_all_threads": 48 * 10 / (t_dec * (48 / 128) * (10 / 100)),
            "decode_tokens_per_s_one_thread": one_thread,
            "sample": "fp64 oracle (C, OpenMP over sequence x value head) on: prefill of the first 1024 of "
                      "4096 tokens (all 32 heads, conv front and gated norm), decode of 48 of 128 sequences "
                      "for 10 of 100 steps, verify + commit of 24 of 64 sequences; each phase's time scaled "
                      "to the full step (%d tokens)" % tokens,
            "phase_seconds_scaled": {"prefill": t_pre, "decode": t_dec, "verify": t_ver}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (--gpus %d refused)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    if args.copy_calib:
        copy_calibration(torch)
        return
    from linear_attention_ssm_core_amd import binding as B
    from linear_attention_ssm_core_amd import workloads as W

    torch.cuda.set_device(0)
    w = Workloads(torch, B, W)
    print("bench: inputs resident; warmup %d, timed %d steps" % (args.warmup, args.steps), file=sys.stderr,
          flush=True)
    for i in range(args.warmup):
        run_step(torch, B, w, i)
    torch.cuda.synchronize()

    keys = ["p0", "p1", "p2", "p3", "d0", "d1", "v0", "v1", "v2"]
    ev = {k: [] for k in keys}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        run_step(torch, B, w, args.warmup + i, ev)
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps

    conv_ms = np.mean(_pair_ms(ev["p0"], ev["p1"]))
    pre_ms = np.mean(_pair_ms(ev["p1"], ev["p2"]))
    norm_ms = np.mean(_pair_ms(ev["p2"], ev["p3"]))
    dec_ms = np.array(_pair_ms(ev["d0"], ev["d1"])) / w.d_steps  # mean launch duration, per step
    print("bench: decode us per launch, step by step: " + " ".join("%.1f" % (1e3 * x) for x in dec_ms),
          file=sys.stderr, flush=True)
    ver_ms = np.mean(_pair_ms(ev["v0"], ev["v1"]))
    com_ms = np.mean(_pair_ms(ev["v1"], ev["v2"]))

    dec_bytes = w.d_n * decode_bytes_per_seq() + CONV_DIM * 4 * 2 + D * 2
    dec_avg_s = float(np.mean(dec_ms)) / 1e3
    dec_gbs = dec_bytes / dec_avg_s / 1e9
    ver_bytes = verify_bytes(w.v_ks)
    pre_flops = prefill_flops_per_token() * w.p_T
    phases = {
        "prefill": {"tokens": w.p_T, "ms_chain": conv_ms + pre_ms + norm_ms, "ms_conv_l2norm": conv_ms,
                    "ms_prefill_chunked": pre_ms, "ms_gated_rmsnorm": norm_ms,
                    "tokens_per_s": w.p_T / ((conv_ms + pre_ms + norm_ms) / 1e3),
                    "prefill_chunked_tflops": pre_flops / (pre_ms / 1e3) / 1e12,
                    "mfma_frac": pre_flops / (pre_ms / 1e3) / MFMA_BF16_PEAK,
                    "hbm_frac": prefill_bytes(w.p_T) / (pre_ms / 1e3) / HBM_PEAK},
        "decode": {"seq_tokens": w.d_n * w.d_steps, "ms_per_launch": float(np.mean(dec_ms)),
                   "tokens_per_s": w.d_n / dec_avg_s, "gb_per_s": dec_gbs, "hbm_frac": dec_gbs * 1e9 / HBM_PEAK},
        "verify": {"rows": w.v_rows, "ms": ver_ms, "tokens_per_s": w.v_rows / (ver_ms / 1e3),
                   "gb_per_s": ver_bytes / (ver_ms / 1e3) / 1e9,
                   "hbm_frac": ver_bytes / (ver_ms / 1e3) / HBM_PEAK},
        "commit": {"ms": com_ms},
    }
    dec_traffic = decode_traffic_bytes()
    line = {
        "metric": "GDN tokens/s: prefill (MFMA %) + batched decode/verify (HBM GB/s %), 1 GPU",
        "value": w.tokens_per_step / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the five GDN workloads)",
        "config": {"workload": "GDN mixer core step: prefill T=4096 (16/32 heads, d=128, chunk 64) + "
                               "batched decode 128 seqs x 100 steps (over %d layers' state sets, cache-cold) + "
                               "speculative verify/commit 64 seqs k~U{2..16}" % DECODE_LAYERS,
                   "tokens_per_step": w.tokens_per_step, "verify_rows": w.v_rows,
                   "decode_state_sets": DECODE_LAYERS, "verify_state_sets": VERIFY_SETS},
        "roofline": {"bound": "hbm", "kernel": "gdn_decode_batched (recurrent_kernel<128,2,1>), cache-cold: "
                                               "%d state sets of 256 MiB cycled" % DECODE_LAYERS,
                     "achieved": dec_gbs, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": dec_gbs * 1e9 / HBM_PEAK,
                     "traffic": None if dec_traffic is None else dec_traffic / (float(np.mean(dec_ms)) / 1e3) / 1e9,
                     "traffic_bytes_per_launch": dec_traffic,
                     "bytes_per_launch": dec_bytes, "avg_launch_ms": float(np.mean(dec_ms)),
                     "launches_timed": int(dec_ms.size) * w.d_steps},
        "phases": phases,
        "variants": variant_phases(torch, B, W, w),
        "attainable": {"copy_gb_per_s": copy_bandwidth(torch), "fill_gb_per_s": fill_bandwidth(torch),
                       "bf16_gemm_tflops": gemm_tflops(torch),
                       "note": "plain 1 GiB device-to-device copy (read + write bytes / time), 1 GiB fill "
                               "(bytes written / time), and an 8192^3 bf16 product through torch.mm "
                               "(2 n^3 / time)"},
        "wall_s_timed": t_wall,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(W)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
