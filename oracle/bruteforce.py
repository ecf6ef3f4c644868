"""Exact rational evaluation of the literal gated delta rule.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Used to pin the fp64
oracle on tiny inputs (T <= 8, d <= 4): the definition is evaluated with full
matrix products over ``fractions.Fraction``, in the form the gated delta rule
is written in (Yang, Kautz and Hatamizadeh, "Gated Delta Networks", ICLR 2025,
section 3):

    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,     o_t = S_t q_t

with S of shape d_v x d_k.  Pure-Python loops; no floating point anywhere.
"""
from fractions import Fraction


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][r] * B[r][j] for r in range(m)), Fraction(0)) for j in range(p)] for i in range(n)]


def _outer(x, y):
    return [[xi * yj for yj in y] for xi in x]


def delta_rule_exact(q, k, v, a, b, S0):
    """q, k: T lists of d_k Fractions; v: T lists of d_v; a, b: T Fractions;
    S0: d_v x d_k matrix.  Returns (outputs [T][d_v], final S [d_v][d_k])."""
    dk = len(k[0])
    I = [[Fraction(int(i == j)) for j in range(dk)] for i in range(dk)]
    S = [row[:] for row in S0]
    outs = []
    for t in range(len(k)):
        kkT = _outer(k[t], k[t])
        P = [[I[i][j] - b[t] * kkT[i][j] for j in range(dk)] for i in range(dk)]
        SP = _matmul(S, P)
        vkT = _outer(v[t], k[t])
        S = [[a[t] * SP[i][j] + b[t] * vkT[i][j] for j in range(dk)] for i in range(len(S))]
        outs.append([sum((S[i][j] * q[t][j] for j in range(dk)), Fraction(0)) for i in range(len(S))])
    return outs, S
