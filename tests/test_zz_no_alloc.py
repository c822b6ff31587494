"""crkv_attn_chunks_batched_static (the entry point that allocates nothing,
for callers that cannot allocate) against crkv_attn_chunks_batched, through
the C ABI: the same kernels, so out and impact must agree bit for bit; two
calls in a row, the second with a smaller input (fewer problems, shorter
chunks), then the first shape again. (The refusals, which touch no device,
are CPU tests in test_abi.py.)"""
import sys

import pytest

torch = pytest.importorskip("torch")

import attention_precomputed_chunk_amd as crkv  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import DeviceWorkload, check_impact, check_out, to_host  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib(crkv_lib):
    yield


def _both(wl):
    """(out, impact) per problem from the per-call entry point, then from the
    static-scratch one on fresh output buffers (pre-filled with NaN)."""
    ref = DeviceWorkload(wl)
    ref.attn()
    stat = DeviceWorkload(wl)
    for p in stat.problems:
        p["out"].fill_(float("nan"))
    crkv.crkv_attn_chunks_batched_static(stat.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode)
    torch.cuda.synchronize()
    return ref, stat


CASES = [
    # label, seed, doc_lens, q, H, H_kv, d, dtype, mode, n_problems
    ("gqa-query", 501, [700, 0, 333, 64], 90, 16, 4, 128, "bf16", "query", 6),
    ("cross", 502, [257, 129, 64], 40, 8, 8, 128, "bf16", "cross", 3),
    ("f32", 503, [130, 67], 21, 4, 2, 64, "f32", "query", 2),
    # one short-query MHA layer: the planner cuts its 32 row blocks into key
    # ranges (pass-1 states and output partials in the static scratch too)
    ("mha-ranges", 504, [512, 512, 512, 512], 64, 32, 32, 128, "bf16", "query", 1),
]
SMALLER = {
    "gqa-query": (511, [200, 31], 17, 3),
    "cross": (512, [65, 40], 9, 1),
    "f32": (513, [33], 5, 1),
    "mha-ranges": (514, [300, 200], 30, 1),
}


@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[0] for c in CASES])
def test_static_matches_per_call_twice(case):
    label, seed, doc, q, H, H_kv, d, dtype, mode, n = CASES[case]
    s2, doc2, q2, n2 = SMALLER[label]
    big = workloads.custom(seed, doc, q, H, H_kv, d, dtype=dtype, mode=mode, r=0.1, n_problems=n)
    small = workloads.custom(s2, doc2, q2, H, H_kv, d, dtype=dtype, mode=mode, r=0.1, n_problems=n2)
    if label == "mha-ranges":
        st = crkv.crkv_plan_stats(DeviceWorkload(big).problems, H, H_kv, d, mode=mode)
        assert st["split_blocks"] > 0, st
    for step, wl in enumerate((big, small, big)):
        say("static scratch: %s call %d (%d problems, docs %s)" % (label, step, len(wl.problems),
                                                                  wl.problems[0].lens[:-1]))
        ref, stat = _both(wl)
        for pi, (a, b) in enumerate(zip(ref.problems, stat.problems)):
            assert torch.equal(a["out"], b["out"]), "%s call %d problem %d: out differs" % (label, step, pi)
            assert torch.equal(a["impact"], b["impact"]), "%s call %d problem %d: impact differs" % (label, step, pi)
        # and the oracle, on the first problem of each call
        p0 = wl.problems[0]
        out_ref, imp_ref, _ = oracle.attn(p0, wl.H, wl.H_kv, wl.d, wl.dtype, wl.mode)
        check_out(to_host(stat.problems[0]["out"]), out_ref, wl.dtype, "%s call %d" % (label, step))
        check_impact(stat.problems[0]["impact"].cpu().numpy(), imp_ref, "%s call %d" % (label, step))

