"""Prepared plans (crkv_plan_create / crkv_plan_launch) through the C ABI:
a launch gives bit for bit what the per-call entry points give, matches the
oracle, and a launch captured into a hipGraph gives the same results on
every replay, with eager work and synchronisations between the replays."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import attention_precomputed_chunk_amd as crkv  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import DEV, DeviceWorkload, check_impact, check_out, check_selection, to_host  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib(crkv_lib):
    yield


CASES = [
    # name, workload factory
    ("tiny", lambda: workloads.generate("tiny")),
    ("llama2_7b_layer", lambda: workloads.generate("llama2_7b_layer")),
    ("gqa", lambda: workloads.custom(700, [300, 0, 77], 40, 16, 4, 128, dtype="bf16", n_problems=3,
                                     k_outliers=4)),
    ("cross", lambda: workloads.custom(701, [100, 60], 30, 8, 8, 64, dtype="bf16", mode="cross",
                                       n_problems=2)),
]


def selections(dw):
    ks = [crkv.crkv_budget(p.n_doc, dw.wl.r) if p.n_doc > 0 else 0 for p in dw.wl.problems]
    idx = [torch.full((max(k, 1),), -1, dtype=torch.int32, device=DEV) for k in ks]
    return ks, idx


def outputs(dw, idx):
    return ([p["out"].clone() for p in dw.problems], [p["impact"].clone() for p in dw.problems],
            [i.clone() for i in idx])


def clear(dw, idx):
    for p in dw.problems:
        p["out"].zero_()
        p["impact"].zero_()
    for i in idx:
        i.fill_(-1)


def same(a, b):
    for x, y in zip(a, b):
        for u, v in zip(x, y):
            assert torch.equal(u, v)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_plan_equals_per_call_path_and_oracle(case):
    name, make = CASES[case]
    say("plan case", name)
    wl = make()
    dw = DeviceWorkload(wl)
    ks, idx = selections(dw)
    # per-call entry points
    dw.attn()
    sel = [i for i, k in enumerate(ks) if k > 0]
    if sel:
        crkv.crkv_topk_batched([dw.problems[i]["impact"] for i in sel], [wl.problems[i].n_doc for i in sel],
                               [ks[i] for i in sel], [idx[i] for i in sel])
    torch.cuda.synchronize()
    ref = outputs(dw, idx)
    clear(dw, idx)
    plan = crkv.Plan(dw.problems, wl.H, wl.H_kv, wl.d, ks=ks, idxs=idx, mode=wl.mode)
    plan.launch()
    torch.cuda.synchronize()
    got = outputs(dw, idx)
    same(got, ref)
    for pi, prob in enumerate(wl.problems):
        ro, ri, _ = oracle.attn(prob, wl.H, wl.H_kv, wl.d, wl.dtype, wl.mode)
        check_out(to_host(got[0][pi]), ro, wl.dtype, "%s[%d]" % (name, pi))
        check_impact(got[1][pi].cpu().numpy(), ri, "%s[%d]" % (name, pi))
        if ks[pi] > 0:
            ref_idx = oracle.topk(ri[:prob.n_doc].astype(np.float32), ks[pi])
            check_selection(got[2][pi].cpu().numpy(), ref_idx, ri[:prob.n_doc], "%s[%d]" % (name, pi))
    plan.destroy()


@pytest.mark.parametrize("case", [0, 1, 2])
def test_plan_graph_replays(case):
    name, make = CASES[case]
    say("graph case", name)
    wl = make()
    dw = DeviceWorkload(wl)
    ks, idx = selections(dw)
    plan = crkv.Plan(dw.problems, wl.H, wl.H_kv, wl.d, ks=ks, idxs=idx, mode=wl.mode)
    plan.launch()
    torch.cuda.synchronize()
    ref = outputs(dw, idx)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # a warm launch on the capture's side stream first
        plan.launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        plan.launch()
    torch.cuda.synchronize()
    for rep in range(3):
        clear(dw, idx)                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same(outputs(dw, idx), ref)
        plan.launch()                   # and an eager launch of the same plan
        torch.cuda.synchronize()
        same(outputs(dw, idx), ref)
    del g
    plan.destroy()


def test_plan_with_workspace_and_destroy_twice():
    wl = workloads.custom(702, [90, 40], 12, 8, 2, 128, dtype="bf16", n_problems=2)
    dw = DeviceWorkload(wl)
    nbytes = crkv.crkv_workspace_size(dw.problems, wl.H, wl.H_kv, wl.d)
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device=DEV)
    plan = crkv.Plan(dw.problems, wl.H, wl.H_kv, wl.d, workspace=ws, workspace_bytes=nbytes)
    plan.launch()
    torch.cuda.synchronize()
    for pi, prob in enumerate(wl.problems):
        ro, ri, _ = oracle.attn(prob, wl.H, wl.H_kv, wl.d, "bf16", "query")
        check_out(to_host(dw.problems[pi]["out"]), ro, "bf16", "ws[%d]" % pi)
        check_impact(dw.problems[pi]["impact"].cpu().numpy(), ri, "ws[%d]" % pi)
    plan.destroy()
    plan.destroy()
    with pytest.raises(ValueError):
        plan.launch()
    with pytest.raises(crkv.CrkvError):
        crkv.Plan(dw.problems, wl.H, wl.H_kv, wl.d, workspace=ws, workspace_bytes=nbytes - 256)


def test_plan_with_more_problems_than_inline_topk():
    """70 problems: the plan keeps the top-k descriptors in device memory
    (more than fit in kernel arguments); equal to the per-call path."""
    wl = workloads.custom(703, [40, 25], 8, 4, 2, 64, dtype="bf16", n_problems=70, r=0.2)
    dw = DeviceWorkload(wl)
    ks, idx = selections(dw)
    dw.attn()
    crkv.crkv_topk_batched([p["impact"] for p in dw.problems], [p.n_doc for p in wl.problems], ks, idx)
    torch.cuda.synchronize()
    ref = outputs(dw, idx)
    clear(dw, idx)
    plan = crkv.Plan(dw.problems, wl.H, wl.H_kv, wl.d, ks=ks, idxs=idx)
    plan.launch()
    torch.cuda.synchronize()
    same(outputs(dw, idx), ref)
    ro, ri, _ = oracle.attn(wl.problems[69], wl.H, wl.H_kv, wl.d, "bf16", "query")
    check_out(to_host(dw.problems[69]["out"]), ro, "bf16", "many[69]")
    plan.destroy()
