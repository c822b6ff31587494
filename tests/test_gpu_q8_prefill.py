"""GPU parity of the prefill (attention, impact, top-k) over segments in the
8-bit format, through the C ABI: the library quantises the segments, the
attention reads the codes (dtype CRKV_KV_Q8) and is compared with the
oracle's fp64 attention over the dequantised cache (oracle/q8.py), with the
contract's tolerances: out within 1e-2 of each row's largest magnitude,
impact within 1e-4 relative per element, selected sets equal up to
boundary ties."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import attention_precomputed_chunk_amd as crkv  # noqa: E402
import oracle  # noqa: E402
from oracle import q8  # noqa: E402
import workloads  # noqa: E402
from gpu_util import (DEV, DeviceWorkload, check_impact, check_out, check_selection,  # noqa: E402
                      check_sorted_selection, to_host)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib(crkv_lib):
    yield


class Q8Prefill:
    """A bf16 workload on the device, its K/V segments quantised by the
    library, and prefill problems over the 8-bit segments."""

    def __init__(self, wl):
        self.wl = wl
        self.dw = DeviceWorkload(wl)
        segs, self.q = [], []
        for pi, p in enumerate(wl.problems):
            dp = self.dw.problems[pi]
            kq, vq = [], []
            for c, n in enumerate(p.lens):
                nk = crkv.crkv_q8_bytes(wl.H_kv, n, wl.d, crkv.CRKV_Q8_K)
                nv = crkv.crkv_q8_bytes(wl.H_kv, n, wl.d, crkv.CRKV_Q8_V)
                bk = torch.full((max(nk, 16),), 0xA5, dtype=torch.uint8, device=DEV)
                bv = torch.full((max(nv, 16),), 0x5A, dtype=torch.uint8, device=DEV)
                if n:
                    segs.append((dp["chunk_K"][c], bk, n, crkv.CRKV_Q8_K))
                    segs.append((dp["chunk_V"][c], bv, n, crkv.CRKV_Q8_V))
                kq.append(bk if n else None)
                vq.append(bv if n else None)
            self.q.append((kq, vq))
        if segs:
            crkv.crkv_quantize_q8(segs, wl.H_kv, wl.d)
        torch.cuda.synchronize()
        self.problems = []
        for pi, dp in enumerate(self.dw.problems):
            kq, vq = self.q[pi]
            self.problems.append(dict(Q=dp["Q"], chunk_K=kq, chunk_V=vq, chunk_len=dp["chunk_len"],
                                      q_len=dp["q_len"], out=torch.empty_like(dp["Q"]),
                                      impact=torch.full_like(dp["impact"], float("nan"))))

    def attn(self, **kw):
        crkv.crkv_attn_chunks_batched(self.problems, self.wl.H, self.wl.H_kv, self.wl.d, mode=self.wl.mode,
                                      dtype=crkv.CRKV_KV_Q8, **kw)

    def topk(self):
        wl = self.wl
        sel = [i for i, p in enumerate(wl.problems) if p.n_doc > 0]
        ks = [crkv.crkv_budget(p.n_doc, wl.r) for p in wl.problems]
        idx = [torch.full((ks[i],), -1, dtype=torch.int32, device=DEV) if i in sel else None
               for i in range(len(ks))]
        if sel:
            crkv.crkv_topk_batched([self.problems[i]["impact"] for i in sel], [wl.problems[i].n_doc for i in sel],
                                   [ks[i] for i in sel], [idx[i] for i in sel])
        return idx

    def host_segments(self, pi):
        """(codes, scales) of every segment of problem pi, read back."""
        p = self.wl.problems[pi]
        kq, vq = self.q[pi]
        res = []
        for bufs, kind, code in ((kq, "k", crkv.CRKV_Q8_K), (vq, "v", crkv.CRKV_Q8_V)):
            segs = []
            for c, n in enumerate(p.lens):
                nb = crkv.crkv_q8_bytes(self.wl.H_kv, n, self.wl.d, code)
                buf = bufs[c][:nb].cpu().numpy() if n else np.zeros(0, np.uint8)
                segs.append(q8.unpack(buf, self.wl.H_kv, n, self.wl.d, kind))
            res.append(segs)
        return res


def compare(qp, problems=None, label=""):
    """Launch once, then compare the listed problems with the oracle over the
    codes the library wrote (which must equal the oracle's own)."""
    wl = qp.wl
    qp.attn()
    gidx = qp.topk()
    torch.cuda.synchronize()
    worst_o = worst_i = 0.0
    for pi in (range(len(wl.problems)) if problems is None else problems):
        prob = wl.problems[pi]
        lab = "%s[problem %d]" % (label, pi)
        kq, vq = qp.host_segments(pi)
        rk, rv = q8.quantize_problem(prob)
        for (gc, gs), (rc, rs) in zip(kq + vq, rk + rv):
            assert np.array_equal(gc, rc) and np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), lab
        out_ref, imp_ref, _ = q8.attn(prob, wl.H, wl.H_kv, wl.d, wl.mode, kq, vq)
        d = qp.problems[pi]
        worst_o = max(worst_o, check_out(to_host(d["out"]), out_ref, "bf16", lab))
        imp = d["impact"].cpu().numpy()
        worst_i = max(worst_i, check_impact(imp, imp_ref, lab))
        if prob.n_doc:
            k = oracle.budget(prob.n_doc, wl.r)
            ref_idx = oracle.topk(imp_ref[:prob.n_doc].astype(np.float32), k)
            g = gidx[pi].cpu().numpy()
            check_selection(g, ref_idx, imp_ref[:prob.n_doc], lab)
            check_sorted_selection(g, imp[:prob.n_doc], lab)
    say("  %s: out err %.3g, impact rel err %.3g" % (label, worst_o, worst_i))
    return gidx


SMALL = [
    # seed, doc_lens, q, H, H_kv, d, mode, outlier channels
    (1, [130, 67, 0, 5], 37, 8, 2, 128, "query", 4),
    (2, [64, 64], 16, 4, 4, 64, "query", 0),
    (3, [200, 1, 63], 100, 4, 1, 128, "query", 4),
    (4, [100, 77, 64], 20, 4, 4, 128, "cross", 4),
    (5, [33, 91], 19, 6, 2, 64, "cross", 2),
    (6, [70, 70], 12, 2, 2, 128, "all", 0),
    (7, [], 45, 4, 2, 128, "query", 0),
    (8, [511, 2], 1, 8, 8, 128, "query", 4),
    (9, [65, 0, 130], 70, 16, 2, 128, "query", 4),
]


@pytest.mark.parametrize("rt", [None, 4, 5, "4/3"], ids=["planner", "rt4", "rt5", "rt4-ranges3"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_q8_prefill_small(case, rt, monkeypatch):
    seed, doc, q, H, H_kv, d, mode, ko = SMALL[case]
    if rt == "4/3":   # keys cut into 3 ranges per row block
        rt = 4
        monkeypatch.setenv("CRKV_KEY_SPLIT", "3")
    if rt:
        monkeypatch.setenv("CRKV_ROW_TILES", str(rt))
    say("q8 prefill case", SMALL[case], "rt", rt)
    wl = workloads.custom(700 + seed, doc, q, H, H_kv, d, dtype="bf16", mode=mode, r=0.1, n_problems=2,
                          k_outliers=ko)
    qp = Q8Prefill(wl)
    plan = crkv.crkv_plan_info(qp.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode, dtype=crkv.CRKV_KV_Q8)
    assert plan["kernel"] == "bf16_wave" and plan["row_tiles"] in (4, 5), plan
    if rt:
        assert plan["row_tiles"] == rt
    compare(qp, label="q8-small%d" % case)


def test_q8_prefill_llama3_32_layers():
    """The 32-layer GQA workload over its 8-bit cache: layers 0, 17 and 31
    against the oracle (out, impact of every key, top-1500), the impact mass
    of every layer."""
    say("llama3_8b_gqa_32l over 8-bit segments: generate")
    wl = workloads.generate("llama3_8b_gqa_32l")
    qp = Q8Prefill(wl)
    say("  launch + compare")
    compare(qp, problems=[0, 17, 31], label="q8-llama3")
    for pi, d in enumerate(qp.problems):
        want = wl.problems[pi].q_len * wl.H
        assert abs(d["impact"].double().sum().item() - want) < 1e-4 * want


def test_q8_prefill_close_to_bf16_prefill():
    """How far the 8-bit cache moves the prefill from the bf16 cache's (the
    format's quantisation error, not a parity bound): reported, and bounded
    loosely."""
    wl = workloads.generate("llama3_8b_gqa_32l", problems=[3])
    qp = Q8Prefill(wl)
    qp.attn()
    qp.dw.attn()
    torch.cuda.synchronize()
    a = to_host(qp.problems[0]["out"])
    b = to_host(qp.dw.problems[0]["out"])
    rel = float((np.abs(a - b).max(axis=-1) / np.abs(b).max(axis=-1)).max())
    ia = qp.problems[0]["impact"].double().cpu().numpy()
    ib = qp.dw.problems[0]["impact"].double().cpu().numpy()
    say("  8-bit vs bf16 cache: out row-relative %.3g, impact L1 relative %.3g"
        % (rel, np.abs(ia - ib).sum() / np.abs(ib).sum()))
    assert rel < 0.1


def test_q8_prefill_static_and_plan_paths():
    """The static-scratch entry point and a prepared plan read 8-bit segments
    too, bit-identical to the per-call path."""
    wl = workloads.custom(790, [300, 129], 50, 8, 2, 128, dtype="bf16", n_problems=3, k_outliers=4)
    qp = Q8Prefill(wl)
    qp.attn()
    torch.cuda.synchronize()
    ref = [(p["out"].clone(), p["impact"].clone()) for p in qp.problems]
    for p in qp.problems:
        p["out"].zero_()
        p["impact"].zero_()
    crkv.crkv_attn_chunks_batched_static(qp.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode, dtype=crkv.CRKV_KV_Q8)
    torch.cuda.synchronize()
    for (o, i), p in zip(ref, qp.problems):
        assert torch.equal(o, p["out"]) and torch.equal(i, p["impact"])
    plan = crkv.Plan(qp.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode, dtype=crkv.CRKV_KV_Q8)
    for p in qp.problems:
        p["out"].zero_()
        p["impact"].zero_()
    plan.launch()
    torch.cuda.synchronize()
    plan.destroy()
    for (o, i), p in zip(ref, qp.problems):
        assert torch.equal(o, p["out"]) and torch.equal(i, p["impact"])
