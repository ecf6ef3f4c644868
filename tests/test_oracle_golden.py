"""Stored fixtures (CPU only): exact rational results and the pages' constants."""
import json
import os
from fractions import Fraction

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_reproduces_exact_rational_fixture():
    doc = json.load(open(os.path.join(HERE, "bruteforce_tiny.json")))
    f = lambda rows: np.array([[float(Fraction(x)) for x in r] for r in rows])
    inp = doc["inputs"]
    q, k, v = f(inp["q"]), f(inp["k"]), f(inp["v"])
    a = np.array([float(Fraction(x)) for x in inp["a"]])
    b = np.array([float(Fraction(x)) for x in inp["b"]])
    S0 = f(inp["S0"])  # d_v x d_k
    T = q.shape[0]
    o, S, _ = oracle.delta_rule(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None],
                                S0.T[None, None], [0, T])
    assert np.max(np.abs(o[:, 0] - f(doc["outputs"]))) < 1e-14
    assert np.max(np.abs(S[0, 0].T - f(doc["S_final"]))) < 1e-14


def test_table_layout_constants_match_pages_and_header(root):
    doc = json.load(open(os.path.join(HERE, "wy_table_layout.json")))
    assert doc["VERIFY_WY_TABLE_STRIDE_BYTES"] == doc["VERIFY_WY_TABLE_SEQS"] * 8
    assert doc["VERIFY_WY_LAYER_STRIDE_BYTES"] == doc["VERIFY_WY_TABLES_PER_LAYER"] * doc["VERIFY_WY_TABLE_STRIDE_BYTES"]
    assert doc["verify_k_min"] <= 16 <= doc["VERIFY_WY_TABLES_PER_LAYER"] == doc["verify_k_max"]
    assert doc["VERIFY_WY_TABLE_SEQS"] >= doc["seqs_capacity_at_least"]
    hdr = open(os.path.join(root, "include", "gdn.h")).read()
    for name in ["VERIFY_WY_TABLE_SEQS", "VERIFY_WY_TABLES_PER_LAYER", "VERIFY_WY_TABLE_STRIDE_BYTES",
                 "VERIFY_WY_LAYER_STRIDE_BYTES"]:
        import re
        m = re.search(r"#define\s+GDN_%s\s+\(?(\d+)" % name, hdr)
        assert m, name
        assert int(m.group(1)) == doc[name], name
