"""GPU parity of the decode step (q_len = 1, the newest token over a growing
last segment) and of prefill with earlier generated tokens in the query
block's segment, against the fp64 oracle, through the C ABI."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import attention_precomputed_chunk_amd as crkv  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import DEV, DeviceWorkload, check_impact, check_out, to_host  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib(crkv_lib):
    yield


def decode(dw, **kw):
    wl = dw.wl
    crkv.crkv_decode_chunks_batched(dw.problems, wl.H, wl.H_kv, wl.d, **kw)


def compare_out(dw, problems=None, label=""):
    wl = dw.wl
    sel = range(len(wl.problems)) if problems is None else problems
    worst = 0.0
    for pi in sel:
        ref, _, _ = oracle.attn(wl.problems[pi], wl.H, wl.H_kv, wl.d, wl.dtype, "query")
        worst = max(worst, check_out(to_host(dw.problems[pi]["out"]), ref, wl.dtype,
                                     "%s[problem %d]" % (label, pi)))
    return worst


DECODE = [
    # seed, doc_lens, gen_len (tokens before the current one), H, H_kv, d
    (1, [130, 67, 0, 5], 9, 8, 2, 128),
    (2, [64, 64], 0, 4, 4, 64),
    (3, [200, 1, 63], 100, 4, 1, 128),
    (4, [], 45, 16, 1, 128),
    (5, [511, 2], 300, 8, 8, 128),
    (6, [65, 0, 130], 31, 16, 2, 64),
    (7, [33], 1, 32, 2, 128),
    (8, [2048, 1000], 33, 8, 1, 128),
]


@pytest.mark.parametrize("case", range(len(DECODE)))
def test_decode_small(case):
    seed, doc, gen, H, H_kv, d = DECODE[case]
    say("decode case", DECODE[case])
    wl = workloads.custom(300 + seed, doc, 1, H, H_kv, d, dtype="bf16", n_problems=3, gen_len=gen)
    dw = DeviceWorkload(wl)
    decode(dw)
    torch.cuda.synchronize()
    say("  out err %.3g" % compare_out(dw, label="decode%d" % case))


def test_decode_32_layers():
    """The decode workload in one launch: every layer against the oracle."""
    say("llama3_8b_decode_32l")
    wl = workloads.generate("llama3_8b_decode_32l")
    dw = DeviceWorkload(wl)
    decode(dw)
    torch.cuda.synchronize()
    say("  out err %.3g" % compare_out(dw, label="decode32"))


def test_decode_deterministic_and_workspace():
    wl = workloads.custom(320, [700, 300], 1, 8, 2, 128, dtype="bf16", n_problems=2, gen_len=50)
    dw = DeviceWorkload(wl)
    decode(dw)
    first = [p["out"].clone() for p in dw.problems]
    nbytes = crkv.crkv_decode_workspace_size(dw.problems, wl.H, wl.H_kv, wl.d)
    assert nbytes > 0
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        decode(dw, workspace=ws, workspace_bytes=nbytes, stream=side)
    side.synchronize()
    for a, p in zip(first, dw.problems):
        assert torch.equal(a, p["out"])
    with pytest.raises(crkv.CrkvError):
        decode(dw, workspace=ws, workspace_bytes=nbytes - 256)


def test_decode_matches_prefill_path():
    """The same step through the prefill kernels (q_len = 1 with a longer
    last segment) agrees with the decode kernels within the bf16 bound."""
    wl = workloads.custom(321, [300, 129], 1, 8, 2, 128, dtype="bf16", n_problems=2, gen_len=77)
    dw = DeviceWorkload(wl)
    decode(dw)
    dec = [to_host(p["out"]) for p in dw.problems]
    dw.attn()
    torch.cuda.synchronize()
    for a, p in zip(dec, dw.problems):
        b = to_host(p["out"])
        assert np.all(np.abs(a - b).max(axis=-1) <= 1e-2 * np.abs(b).max(axis=-1))
    compare_out(dw, label="decode-via-prefill")


@pytest.mark.parametrize("seed,doc,q,gen,H,H_kv,d", [
    (330, [96, 40], 17, 25, 8, 2, 128),
    (331, [0, 64], 40, 100, 4, 4, 64),
    (332, [257], 1, 500, 16, 2, 128),
])
def test_prefill_after_generated_tokens(seed, doc, q, gen, H, H_kv, d):
    """Query rows at the last q_len positions of a segment that also holds
    earlier generated tokens: out and impact against the oracle."""
    wl = workloads.custom(seed, doc, q, H, H_kv, d, dtype="bf16", n_problems=2, gen_len=gen)
    dw = DeviceWorkload(wl)
    dw.attn()
    torch.cuda.synchronize()
    for pi, prob in enumerate(wl.problems):
        out_ref, imp_ref, _ = oracle.attn(prob, H, H_kv, d, "bf16", "query")
        check_out(to_host(dw.problems[pi]["out"]), out_ref, "bf16", "extend[%d]" % pi)
        check_impact(dw.problems[pi]["impact"].cpu().numpy(), imp_ref, "extend[%d]" % pi)


def test_decode_rejects_bad_arguments():
    wl = workloads.custom(322, [64], 2, 4, 2, 128, dtype="bf16")
    dw = DeviceWorkload(wl)
    with pytest.raises(crkv.CrkvError):
        decode(dw)                                   # q_len = 2
    wl = workloads.custom(323, [64], 1, 34, 2, 128, dtype="bf16")
    dw = DeviceWorkload(wl)
    with pytest.raises(crkv.CrkvError):
        decode(dw)                                   # 17 query heads per KV head


def test_library_scratch_across_streams_and_growth():
    """Without a workspace, calls share the library's per-device scratch:
    calls on two streams back to back, and calls that need it to grow, give
    the same results as one call at a time on the default stream."""
    small = DeviceWorkload(workloads.custom(324, [90, 40], 1, 8, 2, 128, dtype="bf16",
                                            n_problems=2, gen_len=20))
    big = DeviceWorkload(workloads.custom(325, [3000, 2100, 700], 1, 8, 1, 128, dtype="bf16",
                                          n_problems=4, gen_len=60))
    pre = DeviceWorkload(workloads.custom(326, [500, 260], 33, 8, 2, 128, dtype="bf16",
                                          n_problems=2))
    decode(small)
    decode(big)
    pre.attn()
    torch.cuda.synchronize()
    refs = [[p["out"].clone() for p in dw.problems] for dw in (small, big, pre)]
    ref_imp = [p["impact"].clone() for p in pre.problems]
    for dw in (small, big, pre):
        for p in dw.problems:
            p["out"].zero_()
    for p in pre.problems:
        p["impact"].zero_()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            decode(small, stream=s1)
        with torch.cuda.stream(s2):
            decode(big, stream=s2)
        with torch.cuda.stream(s1):
            pre.attn(stream=s1)
    torch.cuda.synchronize()
    for dw, ref in zip((small, big, pre), refs):
        for a, p in zip(ref, dw.problems):
            assert torch.equal(a, p["out"])
    for a, p in zip(ref_imp, pre.problems):
        assert torch.equal(a, p["impact"])
