"""The oracle against its frozen outputs (tests/golden/oracle_tiny.json, written
by tests/golden/make_golden.py from oracle/ alone): bits and norms exactly,
projections, scores and attention outputs to 1e-12 relative.  This guards the
oracle against accidental change; the pins of the other oracle tests say why
its values are right."""
import importlib.util
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("make_golden",
                                               os.path.join(HERE, "golden", "make_golden.py"))
mg = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(mg)


def test_oracle_matches_frozen_fixture():
    ref = json.load(open(os.path.join(HERE, "golden", "oracle_tiny.json")))
    got = mg.compute()
    assert got["K"] == ref["K"] and got["Q"] == ref["Q"] and got["V"] == ref["V"]
    assert len(got["cases"]) == len(ref["cases"])
    for g, r in zip(got["cases"], ref["cases"]):
        assert (g["variant"], g["rho"]) == (r["variant"], r["rho"])
        assert g["bits"] == r["bits"], g["variant"]
        for key in ("norms", "Sq", "scores", "attention"):
            a, b = np.array(g[key]), np.array(r[key])
            assert np.allclose(a, b, rtol=1e-12, atol=1e-12), (g["variant"], key)
