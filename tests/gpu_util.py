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
    bad = np.abs(imp - ref) > 1e-4 * np.abs(ref)
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
