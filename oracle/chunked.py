"""fp64 chunked (WY / UT-transform) form of the gated delta rule.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It exists to pin the
oracle: the chunked form and the token-by-token recurrence in ``gdn_oracle.c``
are two independent evaluations of the same definition and must agree.

The chunked form is the chunkwise-parallel algorithm of Yang, Wang, Zhang, Shen
and Kim, "Parallelizing Linear Transformers with the Delta Rule over Sequence
Length" (NeurIPS 2024, section 3.2: the WY representation and the UT
transform), with the per-token decay of Yang, Kautz and Hatamizadeh, "Gated
Delta Networks" (ICLR 2025, section 3.3).  The pages name the same three steps
as the kernels `recompute_wu`, `chunk_delta_h` and `chunk_fwd_o` of the FLA
chunked prefill (metrale_model_layers/layers/qwen3_ssm/layer_struct.rs source
page, the `gdn_prefill_fla_*` handles).

Per chunk of L tokens with start state h = S^T (d_k x d_v), with
Gam_i = prod_{s<=i} a_s and R_ij = prod_{j<s<=i} a_s (= Gam_i / Gam_j, i >= j,
formed as products so that a = 0 is exact):

    A_ij  = R_ij (k_i . k_j)            for j < i, else 0
    T     = (I + diag(b) A)^-1 diag(b)  (unit lower-triangular solve)
    W     = T diag(Gam) K,   U = T V
    U'    = U - W h                     (the corrected writes u_t of every token)
    O     = diag(Gam) Q h + Mq U',      Mq_ij = R_ij (q_i . k_j) for j <= i
    h_end = Gam_{L-1} h + K^T diag(R_{L-1, :}) U'

A library triangular solve (scipy) is the only primitive; every other step is
written out as stated above.
"""
import numpy as np
from scipy.linalg import solve_triangular


def _chunk(q, k, v, a, b, h):
    """One chunk.  q, k [L, dk]; v [L, dv]; a, b [L]; h [dk, dv].  Returns (O, h_end)."""
    L = q.shape[0]
    Gam = np.cumprod(a)
    R = np.zeros((L, L))
    for i in range(L):
        R[i, i] = 1.0
        for j in range(i - 1, -1, -1):
            R[i, j] = R[i, j + 1] * a[j + 1]
    A = np.tril(R * (k @ k.T), -1)
    Lmat = np.eye(L) + b[:, None] * A
    T = solve_triangular(Lmat, np.diag(b), lower=True, unit_diagonal=True)
    W = T @ (Gam[:, None] * k)
    U = T @ v
    Up = U - W @ h
    Mq = np.tril(R * (q @ k.T))
    O = Gam[:, None] * (q @ h) + Mq @ Up
    h_end = Gam[-1] * h + k.T @ (R[-1, :][:, None] * Up)
    return O, h_end


def delta_rule_chunked(q, k, v, a, b, S0, cu_seqlens, chunk=64, scale=1.0):
    """Same contract as ``oracle.delta_rule`` (all heads, no recorded states).

    q, k [T, Hk, dk]; v [T, Hv, dv]; a, b [T, Hv]; S0 [n, Hv, dk, dv].
    Chunks restart at every sequence start; the last chunk may be partial.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    S = np.array(S0, dtype=np.float64, copy=True)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, Hk, dk = q.shape
    Hv = v.shape[1]
    o = np.zeros((T, Hv, v.shape[2]))
    for s in range(cu.shape[0] - 1):
        for h in range(Hv):
            g = h * Hk // Hv
            hs = S[s, h]
            for c0 in range(cu[s], cu[s + 1], chunk):
                c1 = min(c0 + chunk, cu[s + 1])
                O, hs = _chunk(q[c0:c1, g], k[c0:c1, g], v[c0:c1, h], a[c0:c1, h], b[c0:c1, h], hs)
                o[c0:c1, h] = scale * O
            S[s, h] = hs
    return o, S
