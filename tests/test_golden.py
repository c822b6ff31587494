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



FULL = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "full_%s.npz")


def _full(name):
    return np.load(FULL % name, allow_pickle=False)


def test_full_golden_files_are_the_oracles():
    """The stored full-size results (tests/golden/make_full_golden.py) are
    the oracle's on the generated inputs: one Llama-3 layer and one ragged
    request recomputed whole; the cross-document keys at positions >= 7680
    from the rows at positions >= 7680 (the only rows that can see them);
    every stored selection equal to the oracle's top-k of the stored
    impact; every query-row impact vector summing to q_len * H."""
    import sys
    sys.path.insert(0, os.path.dirname(FULL))
    from make_full_golden import fingerprint
    for name, pi in (("llama3_8b_gqa_32l", 13), ("ragged_70b", 9)):
        g = _full(name)
        wl = workloads.generate(name, problems=[pi])
        prob = wl.problems[0]
        assert str(g["fp_%d" % pi]) == fingerprint(prob)
        _, imp, _ = oracle.attn(prob, wl.H, wl.H_kv, wl.d, wl.dtype, wl.mode)
        np.testing.assert_allclose(g["impact_%d" % pi], imp, rtol=1e-12, atol=0)
    g = _full("cross_doc")
    wl = workloads.generate("cross_doc")
    prob = wl.problems[0]
    assert str(g["fp_0"]) == fingerprint(prob)
    _, imp, _ = oracle.attn(prob, wl.H, wl.H_kv, wl.d, wl.dtype, "cross", row_lo=7680)
    np.testing.assert_allclose(g["impact_0"][7680:], imp[7680:], rtol=1e-12, atol=0)
    for name in ("llama3_8b_gqa_32l", "cross_doc", "ragged_70b"):
        g = _full(name)
        spec = workloads.CONFIGS[name]
        doc_lens, q_lens = workloads.ragged_shapes(spec)
        assert int(g["n_problems"]) == spec.n_problems
        for pi in range(spec.n_problems):
            imp = g["impact_%d" % pi]
            n_doc = sum(doc_lens[pi])
            assert len(imp) == n_doc + q_lens[pi]
            k = int(g["k_%d" % pi])
            assert k == oracle.budget(n_doc, spec.r)
            np.testing.assert_array_equal(g["idx_%d" % pi], oracle.topk(imp[:n_doc].astype(np.float32), k))
            if spec.mode == "query":
                assert abs(imp.sum() - q_lens[pi] * spec.H) < 1e-9 * q_lens[pi] * spec.H
