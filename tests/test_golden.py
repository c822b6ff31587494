"""The oracle against its stored tiny-workload results (regression fixture
written by tests/golden/make_golden.py, which calls only the oracle)."""
import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_oracle.json")


def test_tiny_matches_golden():
    g = json.load(open(GOLDEN))
    wl = workloads.generate("tiny")
    out, imp, lse, k, idx = oracle.run_workload(wl, want_lse=True)[0]
    assert k == g["k"] == 12
    np.testing.assert_array_equal(idx, g["idx"])
    np.testing.assert_allclose(imp, g["impact"], rtol=1e-13)
    np.testing.assert_allclose(lse, g["lse"], rtol=1e-13)
    np.testing.assert_allclose(out[:, :, :4], g["out_first4"], rtol=0, atol=1e-13)
    assert abs(sum(g["impact"]) - 16 * 4) < 1e-12
