"""Write the oracle regression fixture tests/golden/oracle_tiny.json.

Calls only oracle/ (and numpy for the seeded inputs).  The fixture freezes
the oracle's outputs on a tiny case -- a dense, an FQJL, a D-FQJL and a
P-FQJL sketch (seed 0, d = 16, m = 64), four keys and two queries -- so that
an accidental change to the oracle's arithmetic fails a test.  A deliberate
change regenerates the file:

    python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import attention as oa  # noqa: E402
from oracle import qjl as oq  # noqa: E402
from oracle import sketch as osk  # noqa: E402

CASES = [("dense", 0.0), ("fqjl", 0.0), ("fqjl", 0.5), ("dfqjl", 0.3), ("pfqjl", 0.0)]


def inputs():
    rs = np.random.default_rng(2024)
    K = np.round(rs.standard_normal((4, 16)) * 8) / 8      # exact in binary
    Q = np.round(rs.standard_normal((2, 16)) * 8) / 8
    V = np.round(rs.standard_normal((4, 8)) * 8) / 8
    return K, Q, V


def compute():
    K, Q, V = inputs()
    out = {"d": 16, "m": 64, "seed": 0, "K": K.tolist(), "Q": Q.tolist(), "V": V.tolist(),
           "cases": []}
    for variant, rho in CASES:
        sk = osk.make_sketch(0, 16, 64, variant, rho)
        bits, norms, _, _ = oq.quantize(sk, K, "f32", key_index_base=7)
        Sq = oq.project(sk, Q, "f32")
        s = oq.score(Sq, bits, norms, 64, rho, 1, 2, 4)
        att = oa.decode_attention(Sq, bits, norms, V, 64, rho, 0.25, 1, 2, 4)
        out["cases"].append({"variant": variant, "rho": rho,
                             "bits": [[int(w) for w in row] for row in bits],
                             "norms": norms.tolist(), "Sq": Sq.tolist(),
                             "scores": s[0].tolist(), "attention": att[0].tolist()})
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", os.path.join(HERE, "oracle_tiny.json"))
