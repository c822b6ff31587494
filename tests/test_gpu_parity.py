"""GPU parity: the HIP library, called through its C ABI, against the fp64
oracle on the same seeded inputs. Small shapes are compared element by
element; the full-size workloads run in the launch configuration the bench
times and are compared on oracle-computable samples plus invariants."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import attention_precomputed_chunk_amd as crkv  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import (DEV, DeviceWorkload, check_impact, check_out, check_selection,  # noqa: E402
                      check_sorted_selection, compare_golden, load_golden, to_host)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib(crkv_lib):
    yield


def run_and_compare(wl, problems=None, label="", oracle_rows=None):
    """Launch the whole workload once, then compare the listed problems (all
    by default) with the oracle. Returns the device workload."""
    dw = DeviceWorkload(wl)
    dw.attn()
    gidx = dw.topk()
    torch.cuda.synchronize()
    sel = range(len(wl.problems)) if problems is None else problems
    for pi in sel:
        prob = wl.problems[pi]
        lab = "%s[problem %d]" % (label, pi)
        out_ref, imp_ref, _ = oracle.attn(prob, wl.H, wl.H_kv, wl.d, wl.dtype, wl.mode)
        d = dw.problems[pi]
        e_out = check_out(to_host(d["out"]), out_ref, wl.dtype, lab)
        imp = d["impact"].cpu().numpy()
        e_imp = check_impact(imp, imp_ref, lab)
        say("  %s: out err %.3g, impact rel err %.3g" % (lab, e_out, e_imp))
        n_doc = prob.n_doc
        if n_doc:
            k = oracle.budget(n_doc, wl.r)
            ref_idx = oracle.topk(imp_ref[:n_doc].astype(np.float32), k)
            g = gidx[pi].cpu().numpy()
            check_selection(g, ref_idx, imp_ref[:n_doc], lab)
            check_sorted_selection(g, imp[:n_doc], lab)
            # bit-exact selection when both sides sort the same fp32 vector
            exact = torch.from_numpy(imp_ref[:n_doc].astype(np.float32)).to(DEV)
            out_idx = torch.full((k,), -1, dtype=torch.int32, device=DEV)
            crkv.crkv_topk(exact, n_doc, k, out_idx)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(out_idx.cpu().numpy(), ref_idx)
    return dw


# ------------------------------------------------------------------ small shapes, full compare

SMALL = [
    # seed, doc_lens, q, H, H_kv, d, dtype, mode
    (1, [130, 67, 0, 5], 37, 8, 2, 128, "bf16", "query"),
    (2, [64, 64], 16, 4, 4, 64, "bf16", "query"),
    (3, [200, 1, 63], 100, 4, 1, 128, "bf16", "query"),
    (4, [100, 77, 64], 20, 4, 4, 128, "bf16", "cross"),
    (5, [33, 91], 19, 6, 2, 64, "bf16", "cross"),
    (6, [70, 70], 12, 2, 2, 128, "bf16", "all"),
    (7, [], 45, 4, 2, 128, "bf16", "query"),
    (8, [511, 2], 1, 8, 8, 128, "bf16", "query"),
    (9, [65, 0, 130], 70, 16, 2, 128, "bf16", "query"),
    (10, [96, 31], 9, 4, 2, 128, "f32", "query"),
    (11, [64, 64], 16, 4, 4, 64, "f32", "cross"),
    (12, [17, 40], 23, 3, 1, 64, "f32", "all"),
    (13, [0, 0, 300], 3, 2, 2, 64, "f32", "query"),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_shapes(case):
    seed, doc, q, H, H_kv, d, dtype, mode = SMALL[case]
    say("small case", SMALL[case])
    wl = workloads.custom(100 + seed, doc, q, H, H_kv, d, dtype=dtype, mode=mode, r=0.1,
                          n_problems=2)
    run_and_compare(wl, label="small%d" % case)


# Every built bf16 (kernel, row tiles) configuration, forced through the
# planner's override, on shapes whose rows span several workgroups.
FORCED_BUILDS = [("wave", 1), ("wave", 2), ("wave", 4), ("wave", 5), ("wave", 7), ("pair", 2), ("pair", 4),
                 ("pair", 6)]
FORCED_CASES = [2, 3, 4, 5, 8]   # indices into SMALL: GQA query rows, cross (d=128, d=64), all rows, G=8


@pytest.mark.parametrize("build", FORCED_BUILDS, ids=["%s%d" % b for b in FORCED_BUILDS])
@pytest.mark.parametrize("case", FORCED_CASES)
def test_forced_bf16_builds(case, build, monkeypatch):
    seed, doc, q, H, H_kv, d, dtype, mode = SMALL[case]
    kernel, rt = build
    if kernel == "wave" and mode == "cross" and rt > 5:
        pytest.skip("no cross-document wave build with 7 row tiles")
    monkeypatch.setenv("CRKV_BF16_KERNEL", kernel)
    monkeypatch.setenv("CRKV_ROW_TILES", str(rt))
    say("forced", kernel, rt, "small case", SMALL[case])
    wl = workloads.custom(100 + seed, doc, q, H, H_kv, d, dtype=dtype, mode=mode, r=0.1, n_problems=2)
    dw = DeviceWorkload(wl)
    plan = crkv.crkv_plan_info(dw.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode)
    assert plan["kernel"] == "bf16_" + kernel and plan["row_tiles"] == rt, plan
    run_and_compare(wl, label="forced-%s%d-small%d" % (kernel, rt, case))


@pytest.mark.parametrize("sweep1", ["split", "fused"])
@pytest.mark.parametrize("rt", [4, 5, 7])
@pytest.mark.parametrize("case", [2, 3, 4, 8])
def test_wave_pass1_forms(case, rt, sweep1, monkeypatch):
    """The one-wave kernel with pass 1 inside it (fused) or as its own
    two-waves-per-SIMD kernel writing the row lse (split), against the
    oracle on shapes whose rows span several workgroups."""
    seed, doc, q, H, H_kv, d, dtype, mode = SMALL[case]
    if mode == "cross" and rt > 5:
        pytest.skip("no cross-document wave build with 7 row tiles")
    monkeypatch.setenv("CRKV_BF16_KERNEL", "wave")
    monkeypatch.setenv("CRKV_ROW_TILES", str(rt))
    monkeypatch.setenv("CRKV_SWEEP1", sweep1)
    say("pass 1", sweep1, "wave", rt, "small case", SMALL[case])
    wl = workloads.custom(100 + seed, doc, q, H, H_kv, d, dtype=dtype, mode=mode, r=0.1, n_problems=2)
    run_and_compare(wl, label="pass1-%s-wave%d-small%d" % (sweep1, rt, case))


# Row blocks cut into key ranges: pass 1 writes one (max, sum) state per
# range, pass 2 of every range merges them and writes fp32 output partials,
# the combine sums them. Forced range counts (100000: one range per key
# tile) on every build, and the pair kernel reading a separate pass 1
# without ranges.
SPLIT_BUILDS = [("wave", 1), ("wave", 2), ("wave", 4), ("wave", 7), ("pair", 2), ("pair", 6)]


@pytest.mark.parametrize("split", ["2", "3", "100000"])
@pytest.mark.parametrize("build", SPLIT_BUILDS, ids=["%s%d" % b for b in SPLIT_BUILDS])
@pytest.mark.parametrize("case", [0, 2, 3, 5, 8])
def test_key_ranges(case, build, split, monkeypatch):
    seed, doc, q, H, H_kv, d, dtype, mode = SMALL[case]
    kernel, rt = build
    if kernel == "wave" and mode == "cross" and rt > 5:
        pytest.skip("no cross-document wave build with 7 row tiles")
    monkeypatch.setenv("CRKV_BF16_KERNEL", kernel)
    monkeypatch.setenv("CRKV_ROW_TILES", str(rt))
    monkeypatch.setenv("CRKV_KEY_SPLIT", split)
    say("key ranges", split, kernel, rt, "small case", SMALL[case])
    wl = workloads.custom(100 + seed, doc, q, H, H_kv, d, dtype=dtype, mode=mode, r=0.1, n_problems=2)
    dw = DeviceWorkload(wl)
    st = crkv.crkv_plan_stats(dw.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode)
    assert st["kernel"] == "bf16_" + kernel and st["row_tiles"] == rt and st["split_blocks"] > 0, st
    assert st["pass1_separate"] == 1 and st["max_ranges"] >= 2
    run_and_compare(wl, label="ranges%s-%s%d-small%d" % (split, kernel, rt, case))


@pytest.mark.parametrize("rt", [2, 4, 6])
@pytest.mark.parametrize("case", [2, 3, 8])
def test_pair_separate_pass1(case, rt, monkeypatch):
    seed, doc, q, H, H_kv, d, dtype, mode = SMALL[case]
    monkeypatch.setenv("CRKV_BF16_KERNEL", "pair")
    monkeypatch.setenv("CRKV_ROW_TILES", str(rt))
    monkeypatch.setenv("CRKV_KEY_SPLIT", "off")
    monkeypatch.setenv("CRKV_SWEEP1", "split")
    say("pair, separate pass 1", rt, "small case", SMALL[case])
    wl = workloads.custom(100 + seed, doc, q, H, H_kv, d, dtype=dtype, mode=mode, r=0.1, n_problems=2)
    dw = DeviceWorkload(wl)
    st = crkv.crkv_plan_stats(dw.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode)
    assert st["pass1_separate"] == 1 and st["split_blocks"] == 0, st
    run_and_compare(wl, label="pair%d-sep-small%d" % (rt, case))


@pytest.mark.parametrize("build", [("wave", 7), ("pair", 6)], ids=["wave7", "pair6"])
def test_pass1_every_block_size(build, monkeypatch):
    """Pass 1 on its own (and pass 2 reading it) on row blocks of every size
    from 1 to 28 row tiles in one batched call: problem n has G q_len = 16 n -
    12 packed rows (G = 4), so its block holds n row tiles, the last one
    partly padded. This covers every split of a block's row tiles between
    the two waves of a SIMD, every residue of n modulo 4 (which SIMDs stage
    the key tiles), and, in the one-wave kernel, every count of the last
    wave's row tiles."""
    kernel, rt = build
    monkeypatch.setenv("CRKV_BF16_KERNEL", kernel)
    monkeypatch.setenv("CRKV_ROW_TILES", str(rt))
    monkeypatch.setenv("CRKV_SWEEP1", "split")
    monkeypatch.setenv("CRKV_KEY_SPLIT", "off")
    H, H_kv, d = 8, 2, 128
    wl = workloads.Workload(spec=None, H=H, H_kv=H_kv, d=d, dtype="bf16", mode="query", r=0.1)
    for n in range(1, 29):
        rng = np.random.default_rng(np.random.SeedSequence(7100, spawn_key=(n,)))
        wl.problems.append(workloads.make_problem(rng, [45, 38], 4 * n - 3, H, H_kv, d, "bf16", "query"))
        wl.problem_ids.append(n - 1)
    dw = DeviceWorkload(wl)
    st = crkv.crkv_plan_stats(dw.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode)
    assert st["kernel"] == "bf16_" + kernel and st["row_tiles"] == rt and st["pass1_separate"] == 1, st
    assert st["split_blocks"] == 0, st
    say("pass 1, block sizes 1..28,", kernel, rt)
    run_and_compare(wl, label="blocksizes-%s%d" % (kernel, rt))


def test_key_ranges_repeat_bit_identical(monkeypatch):
    """A split plan (the planner's own: one short-query MHA layer, whose 32
    row blocks are cut into ranges) gives the same bits on every call."""
    for v in ("CRKV_BF16_KERNEL", "CRKV_ROW_TILES", "CRKV_KEY_SPLIT", "CRKV_SWEEP1"):
        monkeypatch.delenv(v, raising=False)
    wl = workloads.custom(23, [512, 512, 512, 512], 64, 32, 32, 128, dtype="bf16", n_problems=1, k_outliers=4)
    dw = DeviceWorkload(wl)
    st = crkv.crkv_plan_stats(dw.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode)
    assert st["split_blocks"] == 32, st
    dw.attn()
    torch.cuda.synchronize()
    o1 = dw.problems[0]["out"].clone()
    i1 = dw.problems[0]["impact"].clone()
    for _ in range(3):
        dw.problems[0]["out"].zero_()
        dw.problems[0]["impact"].zero_()
        dw.attn()
        torch.cuda.synchronize()
        assert torch.equal(dw.problems[0]["out"], o1)
        assert torch.equal(dw.problems[0]["impact"], i1)


def rising_scores_workload(seed, mode):
    """Scores that climb by about 80 log2 units along the keys: channel 0 of
    every key grows with its position and channel 0 of every query row is
    in [1, 1.4], so each row's running maximum is overtaken by far more than
    the sweep-1 rescale bound many times over, while every p stays a normal
    float32."""
    wl = workloads.custom(seed, [700, 400], 48, 8, 2, 128, dtype="bf16", mode=mode, n_problems=1)
    p = wl.problems[0]
    n_keys = sum(p.lens)
    pos = 0
    for c, n in enumerate(p.lens):
        k = workloads.widen(p.K[c], "bf16").astype(np.float32)
        k[:, :, 0] += (520.0 * np.arange(pos, pos + n) / n_keys).astype(np.float32)
        p.K[c] = workloads.round_bf16(k)
        pos += n
    q = workloads.widen(p.Q, "bf16").astype(np.float32)
    q[..., 0] = 1.0 + 0.1 * np.abs(q[..., 0])
    p.Q = workloads.round_bf16(q)
    return wl


RISING_BUILDS = [None, ("wave", 4), ("wave", 7), ("pair", 6), ("wave", 7, "fused"), ("wave", 4, "3"),
                 ("pair", 6, "3")]


@pytest.mark.parametrize("build", RISING_BUILDS,
                         ids=["planner", "wave4", "wave7", "pair6", "wave7-fused", "wave4-ranges3", "pair6-ranges3"])
def test_rising_scores(build, monkeypatch):
    """Sweep 1's exact-maximum path taken again and again (a row's maximum
    keeps rising), against the oracle; also with the keys cut into ranges
    (each range's state starts from its own first tile)."""
    if build:
        monkeypatch.setenv("CRKV_BF16_KERNEL", build[0])
        monkeypatch.setenv("CRKV_ROW_TILES", str(build[1]))
        if len(build) > 2 and build[2] == "fused":
            monkeypatch.setenv("CRKV_SWEEP1", build[2])
        elif len(build) > 2:
            monkeypatch.setenv("CRKV_KEY_SPLIT", build[2])
    say("rising scores", build)
    run_and_compare(rising_scores_workload(350, "query"), label="rising-%s" % (build,))


def test_tiny_config():
    """1 layer, 4 heads, d=64, fp32; 2 chunks x 64 + 16 query rows; top-12."""
    say("tiny")
    wl = workloads.generate("tiny")
    run_and_compare(wl, label="tiny")


def test_llama2_layer_config():
    """32 heads MHA, d=128, bf16; 4 x 512 + 64 query rows; top-204."""
    say("llama2_7b_layer")
    wl = workloads.generate("llama2_7b_layer")
    run_and_compare(wl, label="llama2")


def test_llama3_gqa_32_layers():
    """32 layers in one launch (the benchmarked call): the impact of all
    10,100 keys and the top-1500 selection of every layer against the stored
    oracle results; the output of layers 0, 9, 17, 25, 31 against the oracle
    run here; the impact mass of every layer."""
    say("llama3_8b_gqa_32l: generate")
    wl = workloads.generate("llama3_8b_gqa_32l")
    golden = load_golden("llama3_8b_gqa_32l", wl)
    say("llama3_8b_gqa_32l: launch + compare")
    dw = run_and_compare(wl, problems=[0, 9, 17, 25, 31], label="llama3")
    gidx = dw.topk()
    torch.cuda.synchronize()
    say("  every layer: impact rel err %.3g" % compare_golden(dw, gidx, golden, "llama3"))
    for pi, d in enumerate(dw.problems):
        imp = d["impact"].double().sum().item()
        assert abs(imp - wl.problems[pi].q_len * wl.H) < 1e-4 * wl.problems[pi].q_len * wl.H


def test_llama3_gqa_iid_keys():
    """The other reading of 'same distributions as config 1': iid N(0,1) K."""
    say("llama3_8b_gqa_32l iid K")
    wl = workloads.generate("llama3_8b_gqa_32l", problems=[0, 1], k_outliers=0)
    run_and_compare(wl, label="llama3-iid")


def test_ragged_batch():
    """16 requests, 64 query / 8 KV heads: the impact and selection of every
    request against the stored oracle results; the output of requests 0, 4,
    7, 11, 15 against the oracle run here."""
    say("ragged_70b")
    wl = workloads.generate("ragged_70b")
    golden = load_golden("ragged_70b", wl)
    dw = run_and_compare(wl, problems=[0, 4, 7, 11, 15], label="ragged")
    gidx = dw.topk()
    torch.cuda.synchronize()
    say("  every request: impact rel err %.3g" % compare_golden(dw, gidx, golden, "ragged"))
    for pi, d in enumerate(dw.problems):
        want = wl.problems[pi].q_len * wl.H
        assert abs(d["impact"].double().sum().item() - want) < 1e-4 * want


def test_cross_doc_config():
    """Every position is a row (8 x 1024 + 128). The impact of all 8,320 keys
    and the top-409 selection against the stored oracle results; the output
    of rows >= 7680 and of 16-row blocks at the start, middle and end of
    every document against the oracle run here; the all-rows launch checks
    the impact mass."""
    say("cross_doc")
    wl = workloads.generate("cross_doc")
    golden = load_golden("cross_doc", wl)
    dw = DeviceWorkload(wl)
    dw.attn()
    gidx = dw.topk()
    torch.cuda.synchronize()
    say("  impact rel err %.3g (all keys)" % compare_golden(dw, gidx, golden, "cross"))
    prob = wl.problems[0]
    d = dw.problems[0]
    out = to_host(d["out"])
    imp = d["impact"].cpu().numpy()
    r0 = 7680
    out_ref, imp_ref, _ = oracle.attn(prob, wl.H, wl.H_kv, wl.d, wl.dtype, "cross", row_lo=r0)
    check_out(out[:, r0:], out_ref[:, r0:], "bf16", "cross late rows")
    # the row-restricted oracle is exact for keys no earlier row can see
    check_impact(imp[r0:], imp_ref[r0:], "cross late keys")
    for doc in range(prob.m):
        for lo in (1024 * doc, 1024 * doc + 504, 1024 * doc + 1008):
            o_ref, _, _ = oracle.attn(prob, wl.H, wl.H_kv, wl.d, wl.dtype, "cross", row_lo=lo,
                                      row_hi=lo + 16)
            check_out(out[:, lo:lo + 16], o_ref[:, lo:lo + 16], "bf16", "cross rows %d" % lo)
    # all-rows mode: impact sums to N * H and bounds the cross-document impact
    wl_all = workloads.Workload(spec=None, H=wl.H, H_kv=wl.H_kv, d=wl.d, dtype=wl.dtype, mode="all",
                                r=wl.r, problems=wl.problems)
    dw_all = DeviceWorkload(wl_all)
    dw_all.attn()
    torch.cuda.synchronize()
    imp_all = dw_all.problems[0]["impact"].cpu().numpy().astype(np.float64)
    assert abs(imp_all.sum() - prob.n_keys * wl.H) < 1e-4 * prob.n_keys * wl.H
    np.testing.assert_array_equal(to_host(dw_all.problems[0]["out"]), out)
    assert np.all(imp <= imp_all * (1 + 1e-5) + 1e-30)


# ------------------------------------------------------------------ behaviour

def test_repeat_calls_are_bit_identical():
    wl = workloads.custom(21, [300, 129], 50, 8, 2, 128, dtype="bf16")
    dw = DeviceWorkload(wl)
    dw.attn()
    torch.cuda.synchronize()
    o1 = dw.problems[0]["out"].clone()
    i1 = dw.problems[0]["impact"].clone()
    for _ in range(3):
        dw.attn()
        torch.cuda.synchronize()
        assert torch.equal(dw.problems[0]["out"], o1)
        assert torch.equal(dw.problems[0]["impact"], i1)


def test_workspace_and_stream():
    wl = workloads.custom(22, [150, 90], 33, 4, 2, 128, dtype="bf16", mode="cross")
    dw = DeviceWorkload(wl)
    dw.attn()
    torch.cuda.synchronize()
    o1 = dw.problems[0]["out"].clone()
    i1 = dw.problems[0]["impact"].clone()
    nbytes = crkv.crkv_workspace_size(dw.problems, wl.H, wl.H_kv, wl.d, mode=wl.mode)
    assert nbytes > 0
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=DEV)
    base = ws.data_ptr()
    aligned = (base + 255) // 256 * 256
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dw.problems[0]["out"].zero_()
        dw.problems[0]["impact"].zero_()
        dw.attn(stream=s, workspace=aligned, workspace_bytes=nbytes)
    s.synchronize()
    assert torch.equal(dw.problems[0]["out"], o1)
    assert torch.equal(dw.problems[0]["impact"], i1)
    with pytest.raises(crkv.CrkvError):
        dw.attn(workspace=aligned, workspace_bytes=nbytes - 256)


def test_partition_of_keys_into_chunks():
    """The same keys split into different chunks give the same attention
    (within tolerance: tile boundaries move)."""
    wl = workloads.custom(23, [256, 128], 40, 8, 2, 128, dtype="bf16")
    dw = DeviceWorkload(wl)
    dw.attn()
    torch.cuda.synchronize()
    out_a = to_host(dw.problems[0]["out"])
    imp_a = dw.problems[0]["impact"].cpu().numpy().astype(np.float64)
    p = wl.problems[0]
    Kc = np.concatenate(p.K[:-1], axis=1)
    Vc = np.concatenate(p.V[:-1], axis=1)
    cuts = [0, 1, 65, 65, 200, 384]
    K = [np.ascontiguousarray(Kc[:, a:b]) for a, b in zip(cuts[:-1], cuts[1:])] + [p.K[-1]]
    V = [np.ascontiguousarray(Vc[:, a:b]) for a, b in zip(cuts[:-1], cuts[1:])] + [p.V[-1]]
    lens = [b - a for a, b in zip(cuts[:-1], cuts[1:])] + [p.q_len]
    p2 = workloads.Problem(K=K, V=V, lens=lens, q_len=p.q_len, Q=p.Q)
    wl2 = workloads.Workload(spec=None, H=wl.H, H_kv=wl.H_kv, d=wl.d, dtype=wl.dtype, mode=wl.mode,
                             r=wl.r, problems=[p2])
    dw2 = DeviceWorkload(wl2)
    dw2.attn()
    torch.cuda.synchronize()
    check_out(to_host(dw2.problems[0]["out"]), out_a, "bf16", "repartition")
    check_impact(dw2.problems[0]["impact"].cpu().numpy(), imp_a, "repartition")


# ------------------------------------------------------------------ top-k alone

@pytest.mark.parametrize("n,k,kind", [
    (1, 1, "normal"), (8, 8, "normal"), (1000, 1, "normal"), (10000, 1500, "normal"),
    (16384, 1638, "normal"), (5000, 700, "ties"), (5000, 4999, "ties"), (777, 300, "signed_zeros"),
    (100000, 8192, "normal"), (4096, 409, "constant"), (3000, 17, "negative"),
    (20000, 8192, "ties"), (16385, 2, "normal"), (50, 50, "ties"), (12000, 8192, "wide"), (10000, 1500, "wide"),
    (8192, 409, "wide"),
])
def test_topk_bit_exact(n, k, kind):
    rng = np.random.default_rng(n * 31 + k)
    if kind == "normal":
        v = rng.standard_normal(n).astype(np.float32)
    elif kind == "ties":
        v = rng.integers(0, 7, size=n).astype(np.float32) * np.float32(0.125)
    elif kind == "signed_zeros":
        v = rng.choice(np.array([-0.0, 0.0, 1e-30, -1e-30, 2.0], dtype=np.float32), size=n)
    elif kind == "constant":
        v = np.full(n, 0.37, dtype=np.float32)
    elif kind == "wide":   # positive, over some 40 binades (impact-like)
        v = np.exp(4.0 * rng.standard_normal(n)).astype(np.float32)
    else:
        v = -np.abs(rng.standard_normal(n)).astype(np.float32)
    ref = oracle.topk(v, k)
    dv = torch.from_numpy(v).to(DEV)
    idx = torch.full((k,), -1, dtype=torch.int32, device=DEV)
    crkv.crkv_topk(dv, n, k, idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


def test_topk_batched_matches_single():
    rng = np.random.default_rng(5)
    vecs = [rng.standard_normal(n).astype(np.float32) for n in (10, 999, 4096, 12000)]
    ks = [3, 99, 409, 1200]
    dv = [torch.from_numpy(v).to(DEV) for v in vecs]
    idx = [torch.full((k,), -1, dtype=torch.int32, device=DEV) for k in ks]
    crkv.crkv_topk_batched(dv, [len(v) for v in vecs], ks, idx)
    torch.cuda.synchronize()
    for v, k, i in zip(vecs, ks, idx):
        np.testing.assert_array_equal(i.cpu().numpy(), oracle.topk(v, k))


@pytest.mark.parametrize("count", [2, 64, 65, 150])
def test_topk_batched_sizes(count):
    """Batches up to 64 pass their descriptors as kernel arguments, larger
    ones upload a table: both against the oracle, bit-exact."""
    rng = np.random.default_rng(40 + count)
    ns = rng.integers(1, 3000, size=count)
    vecs = [rng.standard_normal(int(n)).astype(np.float32) for n in ns]
    ks = [int(rng.integers(1, n + 1)) for n in ns]
    dv = [torch.from_numpy(v).to(DEV) for v in vecs]
    idx = [torch.full((k,), -1, dtype=torch.int32, device=DEV) for k in ks]
    crkv.crkv_topk_batched(dv, [len(v) for v in vecs], ks, idx)
    torch.cuda.synchronize()
    for v, k, i in zip(vecs, ks, idx):
        np.testing.assert_array_equal(i.cpu().numpy(), oracle.topk(v, k))
