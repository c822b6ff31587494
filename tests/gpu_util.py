"""Helpers shared by the GPU tests: upload a workload, run the library through
its C ABI, and compare with the oracle to the tolerances of the contract.

Tolerances (float results):
  * fp32 inputs: out within max-abs 1e-5;
  * bf16 inputs (fp32 accumulation): per (head, row), max |out - ref| <= 1e-2 * max |ref|
    (a per-element relative bound is ill-conditioned near zero);
  * impact: per element |imp - ref| <= 1e-4 * |ref|;
  * top-k: the symmetric difference of the selected sets may only hold indices
    whose oracle impact is within 1e-5 (relative) of the oracle's k-th value;
    fed the same fp32 impact, the GPU selection must equal the oracle's exactly.
"""
import os
import sys

import numpy as np
import torch

import attention_precomputed_chunk_amd as crkv

DEV = "cuda:0"


def t_dev(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def to_host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


class DeviceWorkload:
    def __init__(self, wl):
        self.wl = wl
        self.problems = []
        for p in wl.problems:
            Q = t_dev(p.Q, wl.dtype)
            K = [t_dev(k, wl.dtype) if k.size else None for k in p.K]
            V = [t_dev(v, wl.dtype) if v.size else None for v in p.V]
            out = torch.empty_like(Q)
            impact = torch.full((p.n_keys,), float("nan"), dtype=torch.float32, device=DEV)
            self.problems.append(dict(Q=Q, chunk_K=K, chunk_V=V, chunk_len=list(p.lens),
                                      q_len=p.q_len, out=out, impact=impact))

    def attn(self, **kw):
        wl = self.wl
        crkv.crkv_attn_chunks_batched(self.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode, **kw)

    def budgets(self):
        return [crkv.crkv_budget(p.n_doc, self.wl.r) for p in self.wl.problems]

    def topk(self):
        """Top-k over each problem's document slice (None where N_doc = 0:
        there is nothing to select)."""
        sel = [i for i, p in enumerate(self.wl.problems) if p.n_doc > 0]
        ks = self.budgets()
        idx = [torch.full((ks[i],), -1, dtype=torch.int32, device=DEV) if i in sel else None
               for i in range(len(ks))]
        if sel:
            crkv.crkv_topk_batched([self.problems[i]["impact"] for i in sel],
                                   [self.wl.problems[i].n_doc for i in sel], [ks[i] for i in sel],
                                   [idx[i] for i in sel])
        return idx


def check_out(out, ref, dtype, label=""):
    out = np.asarray(out, dtype=np.float64)
    assert np.isfinite(out).all(), "%s out has %d non-finite elements" % (label, int((~np.isfinite(out)).sum()))
    if dtype == "f32":
        err = np.abs(out - ref).max()
        assert err <= 1e-5, "%s out max-abs error %.3g > 1e-5" % (label, err)
        return float(err)
    else:
        err = np.abs(out - ref).max(axis=-1)
        scale = np.abs(ref).max(axis=-1)
        worst = (err / scale).max()
        assert worst <= 1e-2, "%s out row-relative error %.3g > 1e-2" % (label, worst)
        return float(worst)


def check_impact(imp, ref, label=""):
    imp = np.asarray(imp, dtype=np.float64)
    # written as "not within" so that a NaN (an unwritten element: the tests
    # pre-fill impact with NaN) counts as off
    bad = ~(np.abs(imp - ref) <= 1e-4 * np.abs(ref))
    if bad.any():
        i = int(np.argmax(np.abs(imp - ref) / np.maximum(np.abs(ref), 1e-300)))
        raise AssertionError("%s impact: %d elements off; worst at %d: %r vs %r"
                             % (label, int(bad.sum()), i, imp[i], ref[i]))
    nz = ref != 0   # keys no counted row attends to have impact 0 on both sides (checked above)
    return float((np.abs(imp - ref)[nz] / np.abs(ref[nz])).max()) if nz.any() else 0.0


def check_selection(gpu_idx, ref_idx, ref_imp_doc, label=""):
    g = set(int(x) for x in gpu_idx)
    r = set(int(x) for x in ref_idx)
    assert len(g) == len(gpu_idx), "%s duplicate indices" % label
    t = float(ref_imp_doc[ref_idx[-1]])
    for i in g ^ r:
        assert abs(ref_imp_doc[i] - t) <= 1e-5 * abs(t), \
            "%s index %d selected differently and is not a boundary tie" % (label, i)


GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name, wl):
    """The oracle's impact (float64) and top-k of every problem of workload
    `name`, stored by tests/golden/make_full_golden.py (which calls only the
    oracle and the input generator), after checking that the stored input
    fingerprints match the workload generated here."""
    sys.path.insert(0, GOLDEN_DIR)
    from make_full_golden import fingerprint
    g = np.load(os.path.join(GOLDEN_DIR, "full_%s.npz" % name), allow_pickle=False)
    assert str(g["workload"]) == name
    n = int(g["n_problems"])
    assert n == len(wl.problems), "golden has %d problems, workload %d" % (n, len(wl.problems))
    res = []
    for pi, prob in enumerate(wl.problems):
        assert str(g["fp_%d" % pi]) == fingerprint(prob), \
            "%s problem %d: inputs differ from those the golden file was written for" % (name, pi)
        res.append((g["impact_%d" % pi], g["idx_%d" % pi], int(g["k_%d" % pi])))
    return res


def check_sorted_selection(idx, imp_doc, label=""):
    """The GPU output order is (value desc, index asc) on its own impact."""
    v = imp_doc[idx]
    assert np.all(v[:-1] >= v[1:]), "%s not sorted by value" % label
    ties = v[:-1] == v[1:]
    assert np.all(idx[:-1][ties] < idx[1:][ties]), "%s ties not in index order" % label


def compare_golden(dw, gidx, golden, label=""):
    """Every problem's impact (all N keys) and selection against the stored
    oracle results; then the GPU top-k fed the oracle's own float32 impact of
    every problem must reproduce the oracle's indices exactly. Returns the
    worst impact relative error."""
    wl = dw.wl
    worst = 0.0
    for pi, (prob, (imp_ref, idx_ref, k)) in enumerate(zip(wl.problems, golden)):
        lab = "%s[problem %d]" % (label, pi)
        imp = dw.problems[pi]["impact"].cpu().numpy()
        worst = max(worst, check_impact(imp, imp_ref, lab))
        n_doc = prob.n_doc
        g = gidx[pi].cpu().numpy()
        assert len(g) == k
        check_selection(g, idx_ref, imp_ref[:n_doc], lab)
        check_sorted_selection(g, imp[:n_doc], lab)
    exact = [torch.from_numpy(imp_ref[:p.n_doc].astype(np.float32)).to(DEV)
             for p, (imp_ref, _, _) in zip(wl.problems, golden)]
    out_idx = [torch.full((k,), -1, dtype=torch.int32, device=DEV) for (_, _, k) in golden]
    crkv.crkv_topk_batched(exact, [p.n_doc for p in wl.problems], [k for (_, _, k) in golden], out_idx)
    torch.cuda.synchronize()
    for pi, (oi, (_, idx_ref, _)) in enumerate(zip(out_idx, golden)):
        np.testing.assert_array_equal(oi.cpu().numpy(), idx_ref, err_msg="%s[problem %d] top-k" % (label, pi))
    return worst
