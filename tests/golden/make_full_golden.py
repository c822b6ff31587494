"""Writes full_<workload>.npz: the oracle's impact vector (float64) and top-k
indices for EVERY problem of the three large workloads, so that the GPU tests
compare all keys of all problems without running the oracle on the box:

  * llama3_8b_gqa_32l: 32 layers x 10,100 keys, k = 1500 per layer;
  * cross_doc: 8,320 keys (every position a row, same-segment rows not
    counted), k = 409;
  * ragged_70b: 16 requests, 4,200-16,600 keys each, k = floor(0.1 N_doc).

Calls only ``oracle`` and the input generator ``workloads``. Each file also
holds a fingerprint of the inputs (lengths, q_len and a SHA-256 over Q and
the first and last segments' K and V of every problem), which the tests
check before comparing, so a change to the generator fails loudly instead
of comparing against another workload's values.

Run from the repository root:  python tests/golden/make_full_golden.py
(about 2-3 minutes on 8 cores).
"""
import hashlib
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

NAMES = ("llama3_8b_gqa_32l", "cross_doc", "ragged_70b")


def fingerprint(prob) -> str:
    h = hashlib.sha256()
    h.update(np.asarray(prob.lens, dtype=np.int64).tobytes())
    h.update(np.int64(prob.q_len).tobytes())
    for a in (prob.Q, prob.K[0], prob.V[0], prob.K[-1], prob.V[-1]):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def path_for(name: str) -> str:
    return os.path.join(HERE, "full_%s.npz" % name)


def write(name: str) -> None:
    t = time.time()
    wl = workloads.generate(name)
    arrays = {}
    for pi, prob in enumerate(wl.problems):
        _, imp, _ = oracle.attn(prob, wl.H, wl.H_kv, wl.d, wl.dtype, wl.mode)
        k = oracle.budget(prob.n_doc, wl.r)
        arrays["impact_%d" % pi] = imp
        arrays["idx_%d" % pi] = oracle.topk(imp[:prob.n_doc].astype(np.float32), k)
        arrays["k_%d" % pi] = np.int64(k)
        arrays["fp_%d" % pi] = np.array(fingerprint(prob))
        print("  %s problem %d: N %d, k %d" % (name, pi, prob.n_keys, k), flush=True)
    arrays["n_problems"] = np.int64(len(wl.problems))
    arrays["workload"] = np.array(name)
    np.savez_compressed(path_for(name), **arrays)
    print("%s: %.0f s" % (name, time.time() - t), flush=True)


def main():
    for name in (sys.argv[1:] or NAMES):
        write(name)


if __name__ == "__main__":
    main()
