"""Writes tiny_oracle.json: the oracle's results on the tiny workload
(1 layer, 4 heads, d=64, fp32, 2 chunks x 64 + 16 query rows, r=0.1).

Calls only ``oracle`` and the input generator. The file is a regression fixture
for the oracle itself; the oracle's correctness is pinned separately by
``tests/oracle_pins.py``.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    wl = workloads.generate("tiny")
    out, imp, lse, k, idx = oracle.run_workload(wl, want_lse=True, n_threads=1)[0]
    doc = {
        "workload": "tiny",
        "k": int(k),
        "idx": [int(i) for i in idx],
        "impact": [float(x) for x in imp],
        "lse": [[float(x) for x in row] for row in lse],
        "out_first4": [[[float(x) for x in out[h, j, :4]] for j in range(out.shape[1])]
                       for h in range(out.shape[0])],
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
