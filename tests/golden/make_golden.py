"""Write tests/golden/bruteforce_tiny.json.

Calls only oracle/bruteforce.py (exact rational arithmetic).  The stored
outputs are the exact values of the literal gated delta rule on small rational
inputs (unit keys 3/5, 4/5 among them); the fp64 oracle must reproduce them to
rounding.
"""
import json
import os
import sys
from fractions import Fraction

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle.bruteforce import delta_rule_exact  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def case():
    # T = 4 tokens, d_k = 2, d_v = 3, one head; hand-picked dyadic inputs.
    q = [[1, Fraction(1, 2)], [0, 1], [Fraction(-3, 4), Fraction(1, 4)], [1, 1]]
    k = [[1, 0], [Fraction(3, 5), Fraction(4, 5)], [0, 1], [Fraction(-4, 5), Fraction(3, 5)]]
    v = [[1, -1, Fraction(1, 2)], [Fraction(1, 4), 2, 0], [-1, 0, 1], [Fraction(1, 8), Fraction(-1, 2), 3]]
    a = [Fraction(1, 2), 1, Fraction(3, 4), 0]
    b = [1, Fraction(1, 2), Fraction(1, 4), Fraction(3, 4)]
    S0 = [[Fraction(1, 4), 0], [0, Fraction(-1, 2)], [1, 1]]  # d_v x d_k
    return q, k, v, a, b, S0


def main():
    q, k, v, a, b, S0 = case()
    outs, S = delta_rule_exact([[Fraction(x) for x in r] for r in q], [[Fraction(x) for x in r] for r in k],
                               [[Fraction(x) for x in r] for r in v], [Fraction(x) for x in a],
                               [Fraction(x) for x in b], [[Fraction(x) for x in r] for r in S0])
    s = lambda x: str(Fraction(x))
    doc = {
        "what": "exact outputs o_t and final state S (d_v x d_k) of the literal gated delta rule",
        "source": "Gated Delta Networks (Yang, Kautz, Hatamizadeh, ICLR 2025), section 3: "
                  "S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t",
        "written_by": "tests/golden/make_golden.py (oracle/bruteforce.py only)",
        "inputs": {"q": [[s(x) for x in r] for r in q], "k": [[s(x) for x in r] for r in k],
                   "v": [[s(x) for x in r] for r in v], "a": [s(x) for x in a], "b": [s(x) for x in b],
                   "S0": [[s(x) for x in r] for r in S0]},
        "outputs": [[s(x) for x in r] for r in outs],
        "S_final": [[s(x) for x in r] for r in S],
    }
    with open(os.path.join(HERE, "bruteforce_tiny.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
