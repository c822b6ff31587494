"""The C ABI on the CPU: the library loads, exports every function that
include/crkv.h declares, and rejects invalid arguments with status codes
before anything is enqueued (no device is touched by these calls)."""
import ctypes
import os
import re

import pytest

import attention_precomputed_chunk_amd as crkv
import workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "crkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(crkv_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(crkv_lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(crkv_lib, n), n
    assert set(names) == set(crkv.DECLARED)


def test_version_and_status_strings(crkv_lib):
    assert crkv.crkv_version() == 1
    assert crkv_lib.crkv_status_string(0) == b"ok"
    assert crkv_lib.crkv_status_string(-1) == b"invalid argument"
    assert crkv_lib.crkv_status_string(-2) == b"unsupported configuration"
    assert crkv_lib.crkv_status_string(-3) == b"HIP runtime error"
    assert crkv_lib.crkv_status_string(-4) == b"out of memory"


def test_budget(crkv_lib):
    assert crkv.crkv_budget(128, 0.1) == 12
    assert crkv.crkv_budget(2048, 0.1) == 204
    assert crkv.crkv_budget(10000, 0.15) == 1500
    assert crkv.crkv_budget(8192, 0.05) == 409
    assert crkv.crkv_budget(3, 0.1) == 1
    assert crkv.crkv_budget(-1, 0.1) == -1
    assert crkv.crkv_budget(10, 1.5) == -1


FAKE = 0x10000   # aligned, never dereferenced: validation fails first


def _call(Q=FAKE, K=None, V=None, lens=(64, 64, 16), q_len=16, H=4, H_kv=4, d=64, out=FAKE,
          impact=FAKE, dtype=crkv.CRKV_F32, mode=0, workspace=None, deterministic=1):
    L = crkv.lib()
    m = len(lens) - 1
    K = K if K is not None else [FAKE] * (m + 1)
    V = V if V is not None else [FAKE] * (m + 1)
    ka = (ctypes.c_void_p * (m + 1))(*K)
    va = (ctypes.c_void_p * (m + 1))(*V)
    la = (ctypes.c_int32 * (m + 1))(*lens)
    o = crkv.crkv_opts()
    L.crkv_opts_init(ctypes.byref(o))
    o.dtype = dtype
    o.mode = mode
    o.workspace = workspace
    assert o.deterministic == 1   # the default
    o.deterministic = deterministic
    rc = L.crkv_attn_chunks(Q, ka, va, la, m, q_len, H, H_kv, d, out, impact, ctypes.byref(o))
    return rc, L.crkv_last_error().decode()


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(Q=None), -1, "non-null"),
    (dict(out=None), -1, "non-null"),
    (dict(impact=None), -1, "non-null"),
    (dict(H=6, H_kv=4), -1, "multiple"),
    (dict(H=0), -1, ">= 1"),
    (dict(d=96), -2, "d = 96"),
    (dict(lens=(64, 64, 15)), -1, "q_len"),
    (dict(lens=(64, -3, 16)), -1, "< 0"),
    (dict(q_len=0, lens=(64, 0)), -1, "q_len"),
    (dict(K=[FAKE, 0, FAKE]), -1, "null K or V"),
    (dict(V=[FAKE, FAKE + 8, FAKE]), -1, "aligned"),
    (dict(Q=FAKE + 4), -1, "aligned"),
    (dict(impact=FAKE + 2), -1, "aligned"),
    (dict(dtype=7), -1, "dtype"),
    (dict(mode=5), -1, "mode"),
    (dict(workspace=FAKE + 16), -1, "256-byte"),
    (dict(deterministic=2), -1, "deterministic"),
])
def test_attn_rejects_invalid_arguments(crkv_lib, kwargs, status, needle):
    rc, msg = _call(**kwargs)
    assert rc == status, msg
    assert needle in msg


def test_zero_length_chunk_with_null_pointer_is_allowed_by_validation(crkv_lib):
    # a zero-length document chunk may have null K/V; the call then fails only
    # later, at the first HIP call, when there is no GPU -- so check the size query
    probs = (crkv.crkv_problem * 1)()
    k = (ctypes.c_void_p * 3)(FAKE, None, FAKE)
    v = (ctypes.c_void_p * 3)(FAKE, None, FAKE)
    lens = (ctypes.c_int32 * 3)(64, 0, 16)
    probs[0] = crkv.crkv_problem(FAKE, k, v, lens, 2, 16, FAKE, FAKE)
    o = crkv.crkv_opts()
    crkv_lib.crkv_opts_init(ctypes.byref(o))
    assert crkv_lib.crkv_workspace_size(probs, 1, 4, 4, 64, ctypes.byref(o)) > 0
    o.dtype = 9
    assert crkv_lib.crkv_workspace_size(probs, 1, 4, 4, 64, ctypes.byref(o)) == 0


def test_topk_rejects_invalid_arguments(crkv_lib):
    L = crkv_lib
    o = crkv.crkv_opts()
    L.crkv_opts_init(ctypes.byref(o))
    assert L.crkv_topk(None, 10, 3, FAKE, ctypes.byref(o)) == -1
    assert L.crkv_topk(FAKE, 10, 0, FAKE, ctypes.byref(o)) == -1
    assert L.crkv_topk(FAKE, 10, 11, FAKE, ctypes.byref(o)) == -1
    assert L.crkv_topk(FAKE, 0, 1, FAKE, ctypes.byref(o)) == -1
    assert L.crkv_topk(FAKE, 100000, 9000, FAKE, ctypes.byref(o)) == -2
    assert L.crkv_topk(FAKE + 2, 10, 3, FAKE, ctypes.byref(o)) == -1
    P = 2
    ip = (ctypes.c_void_p * P)(FAKE, FAKE)
    nn = (ctypes.c_int32 * P)(10, 10)
    kk = (ctypes.c_int32 * P)(3, 12)
    xp = (ctypes.c_void_p * P)(FAKE, FAKE)
    assert L.crkv_topk_batched(ip, nn, kk, xp, P, ctypes.byref(o)) == -1
    assert "top-k 1" in L.crkv_last_error().decode()
    assert L.crkv_topk_batched(ip, nn, kk, xp, 0, ctypes.byref(o)) == -1


def test_batched_rejects_empty_batch(crkv_lib):
    o = crkv.crkv_opts()
    crkv_lib.crkv_opts_init(ctypes.byref(o))
    assert crkv_lib.crkv_attn_chunks_batched(None, 0, 4, 4, 64, ctypes.byref(o)) == -1
    assert crkv_lib.crkv_attn_chunks_batched(None, 1, 4, 4, 64, ctypes.byref(o)) == -1


def _fake_problem(doc_lens, q_len, H, d):
    """Problem dict with placeholder device addresses (the planner never
    dereferences them)."""
    m = len(doc_lens)
    return dict(Q=0x10000, chunk_K=[0x20000 + 0x1000 * i for i in range(m + 1)],
                chunk_V=[0x40000 + 0x1000 * i for i in range(m + 1)], chunk_len=list(doc_lens) + [q_len],
                q_len=q_len, out=0x60000, impact=0x70000)


def test_plan_info_picks_kernel_by_shape(monkeypatch):
    """Host-only: 25 packed row tiles per KV head fit one one-wave workgroup
    (4 x 7 tiles); thousands of rows go to the wave-pair kernel."""
    monkeypatch.delenv("CRKV_BF16_KERNEL", raising=False)
    monkeypatch.delenv("CRKV_ROW_TILES", raising=False)
    monkeypatch.setenv("CRKV_KEY_SPLIT", "off")
    few = [_fake_problem([2500] * 4, 100, 32, 128) for _ in range(4)]
    p = crkv.crkv_plan_info(few, 32, 8, 128, mode="query", dtype=crkv.CRKV_BF16)
    assert p == {"kernel": "bf16_wave", "row_tiles": 7, "workgroups": 4 * 8}
    monkeypatch.delenv("CRKV_KEY_SPLIT")
    many = [_fake_problem([3000, 3000], 1000, 64, 128)]
    p = crkv.crkv_plan_info(many, 64, 8, 128, mode="query", dtype=crkv.CRKV_BF16)
    assert p["kernel"] == "bf16_pair" and p["row_tiles"] == 6
    p = crkv.crkv_plan_info(many, 64, 8, 128, mode="query", dtype=crkv.CRKV_F32)
    assert p["kernel"] == "f32"
    monkeypatch.setenv("CRKV_BF16_KERNEL", "wave")
    monkeypatch.setenv("CRKV_ROW_TILES", "5")
    p = crkv.crkv_plan_info(many, 64, 8, 128, mode="cross", dtype=crkv.CRKV_BF16)
    assert p["kernel"] == "bf16_wave" and p["row_tiles"] == 5


def _stats(probs, H, H_kv, mode="query"):
    return crkv.crkv_plan_stats(probs, H, H_kv, 128, mode=mode, dtype=crkv.CRKV_BF16)


def test_key_ranges_planned_where_the_model_gains(monkeypatch):
    """Host-only planner checks of the key-range split: a single short-query
    layer (32 row blocks on 256 CUs) is cut into ranges and its output rows
    summed by the combine; 256 equal blocks (the 32-layer GQA launch) are not;
    the ragged batch's modelled imbalance drops below 5 %; a forced count
    cuts every block (at most one range per key tile); the fused pass 1
    plans no ranges."""
    for v in ("CRKV_BF16_KERNEL", "CRKV_ROW_TILES", "CRKV_KEY_SPLIT", "CRKV_SWEEP1"):
        monkeypatch.delenv(v, raising=False)
    layer = [_fake_problem([512] * 4, 64, 32, 128)]
    st = _stats(layer, 32, 32)
    assert st["kernel"] == "bf16_wave" and st["row_tiles"] == 1 and st["pass1_separate"] == 1
    assert st["split_blocks"] == 32 and st["max_ranges"] >= 4
    assert st["combine_workgroups"] == 32 * 4        # 64 rows of each head: 4 row tiles
    assert st["workgroups"] >= 32 * st["max_ranges"] - 8
    assert st["imbalance"] < 0.1
    assert crkv.crkv_workspace_size(layer, 32, 32, 128, dtype=crkv.CRKV_BF16) == st["scratch_bytes"]

    layers = [_fake_problem([2500] * 4, 100, 32, 128) for _ in range(32)]
    st = _stats(layers, 32, 8)
    assert st["split_blocks"] == 0 and st["workgroups"] == 256 and st["imbalance"] < 1e-9

    lens, qs = workloads.ragged_shapes(workloads.CONFIGS["ragged_70b"])
    ragged = [_fake_problem(ln, q, 64, 128) for ln, q in zip(lens, qs)]
    monkeypatch.setenv("CRKV_KEY_SPLIT", "off")
    whole = _stats(ragged, 64, 8)
    monkeypatch.delenv("CRKV_KEY_SPLIT")
    st = _stats(ragged, 64, 8)
    assert st["imbalance"] < 0.05 < whole["imbalance"]
    assert st["model_cycles"] < whole["model_cycles"]

    monkeypatch.setenv("CRKV_KEY_SPLIT", "3")
    st = _stats(layers[:2], 32, 8)
    assert st["split_blocks"] == 16 and st["max_ranges"] == 3 and st["workgroups"] == 48
    monkeypatch.setenv("CRKV_KEY_SPLIT", "5")
    tiny = [_fake_problem([40], 8, 4, 128)]           # key tiles of 32 + 8 and 8 keys: at most 3 ranges
    st = _stats(tiny, 4, 4)
    assert st["max_ranges"] == 3
    monkeypatch.setenv("CRKV_SWEEP1", "fused")
    st = _stats(layers[:2], 32, 8)
    assert st["split_blocks"] == 0 and st["pass1_separate"] == 0


def test_plan_info_rejects_invalid():
    bad = [_fake_problem([64], 16, 6, 128)]
    with pytest.raises(crkv.CrkvError):
        crkv.crkv_plan_info(bad, 6, 4, 128, mode="query", dtype=crkv.CRKV_BF16)   # H % H_kv != 0


def test_batch_marshals_once_and_plans_the_same(monkeypatch):
    monkeypatch.delenv("CRKV_BF16_KERNEL", raising=False)
    monkeypatch.delenv("CRKV_ROW_TILES", raising=False)
    probs = [_fake_problem([700, 300], 40, 8, 128) for _ in range(3)]
    b = crkv.Batch.__new__(crkv.Batch)   # fake tensors carry no dtype: set it by hand
    b.keep, b.arr = crkv._problems(probs)
    b.dtype = crkv.CRKV_BF16
    assert len(b) == 3
    assert (crkv.crkv_plan_info(b, 8, 2, 128, mode="query", dtype=crkv.CRKV_BF16)
            == crkv.crkv_plan_info(probs, 8, 2, 128, mode="query", dtype=crkv.CRKV_BF16))
    assert (crkv.crkv_workspace_size(b, 8, 2, 128, dtype=crkv.CRKV_BF16)
            == crkv.crkv_workspace_size(probs, 8, 2, 128, dtype=crkv.CRKV_BF16))


def _sel(k=4, lens=(8, 0, 5), idx=FAKE, K_sel=FAKE, V_sel=FAKE, chunk=FAKE, m=None):
    m = len(lens) - 1 if m is None else m
    n = len(lens)
    keep = ((ctypes.c_void_p * n)(*[chunk if L else None for L in lens]),
            (ctypes.c_void_p * n)(*[chunk if L else None for L in lens]),
            (ctypes.c_int32 * n)(*lens))
    return keep, crkv.crkv_kv_select(keep[0], keep[1], keep[2], m, idx, k, K_sel, V_sel)


@pytest.mark.parametrize("field,value,status", [
    ("k", -1, -1), ("idx", None, -1), ("K_sel", None, -1), ("V_sel", FAKE + 8, -1),
    ("chunk", FAKE + 4, -1), ("lens", (8, -1, 5), -1), ("m", -1, -1),
])
def test_gather_scatter_reject_invalid_arguments(crkv_lib, field, value, status):
    kw = {field: value}
    keep, s = _sel(**kw)
    arr = (crkv.crkv_kv_select * 1)(s)
    o = crkv.crkv_opts()
    crkv_lib.crkv_opts_init(ctypes.byref(o))
    o.dtype = crkv.CRKV_BF16
    assert crkv_lib.crkv_gather_kv(arr, 1, 2, 128, ctypes.byref(o)) == status
    assert crkv_lib.crkv_scatter_kv(arr, 1, 2, 128, ctypes.byref(o)) == status


def test_gather_scatter_shape_checks_and_empty_selection(crkv_lib):
    keep, s = _sel()
    arr = (crkv.crkv_kv_select * 1)(s)
    o = crkv.crkv_opts()
    crkv_lib.crkv_opts_init(ctypes.byref(o))
    assert crkv_lib.crkv_gather_kv(arr, 1, 2, 96, ctypes.byref(o)) == -2      # d
    assert crkv_lib.crkv_gather_kv(arr, 1, 0, 128, ctypes.byref(o)) == -1     # H_kv
    assert crkv_lib.crkv_gather_kv(arr, 0, 2, 128, ctypes.byref(o)) == -1     # no selections
    o.dtype = 7
    assert crkv_lib.crkv_gather_kv(arr, 1, 2, 128, ctypes.byref(o)) == -1
    # k = 0 everywhere: valid, and nothing is enqueued (no device is touched)
    o.dtype = crkv.CRKV_F32
    keep0, s0 = _sel(k=0, idx=None, K_sel=None, V_sel=None)
    arr0 = (crkv.crkv_kv_select * 1)(s0)
    assert crkv_lib.crkv_gather_kv(arr0, 1, 2, 64, ctypes.byref(o)) == 0
    assert crkv_lib.crkv_scatter_kv(arr0, 1, 2, 64, ctypes.byref(o)) == 0


def test_rope_shift_rejects_invalid_arguments(crkv_lib):
    o = crkv.crkv_opts()
    crkv_lib.crkv_opts_init(ctypes.byref(o))
    o.dtype = crkv.CRKV_BF16
    ok = (crkv.crkv_rope_seg * 1)(crkv.crkv_rope_seg(FAKE, 16, 5))
    L = crkv_lib
    assert L.crkv_rope_shift(ok, 1, 2, 96, 10000.0, ctypes.byref(o)) == -2        # d
    assert L.crkv_rope_shift(ok, 1, 0, 128, 10000.0, ctypes.byref(o)) == -1       # H_kv
    assert L.crkv_rope_shift(ok, 1, 2, 128, 1.0, ctypes.byref(o)) == -1           # base
    assert L.crkv_rope_shift(ok, 1, 2, 128, float("inf"), ctypes.byref(o)) == -1
    assert L.crkv_rope_shift(ok, 0, 2, 128, 10000.0, ctypes.byref(o)) == -1       # n
    for seg in (crkv.crkv_rope_seg(FAKE, -1, 5), crkv.crkv_rope_seg(None, 16, 5),
                crkv.crkv_rope_seg(FAKE + 8, 16, 5)):
        bad = (crkv.crkv_rope_seg * 1)(seg)
        assert L.crkv_rope_shift(bad, 1, 2, 128, 10000.0, ctypes.byref(o)) == -1
    # nothing moves: delta 0, or an empty segment (valid; nothing is enqueued)
    idle = (crkv.crkv_rope_seg * 2)(crkv.crkv_rope_seg(None, 16, 0), crkv.crkv_rope_seg(None, 0, 7))
    assert L.crkv_rope_shift(idle, 2, 2, 128, 10000.0, ctypes.byref(o)) == 0


def test_quantize_q8_rejects_invalid_arguments(crkv_lib):
    o = crkv.crkv_opts()
    crkv_lib.crkv_opts_init(ctypes.byref(o))
    o.dtype = crkv.CRKV_BF16
    L = crkv_lib
    q_at = FAKE + (1 << 20)
    K, V = crkv.CRKV_Q8_K, crkv.CRKV_Q8_V
    ok = (crkv.crkv_q8_seg * 2)(crkv.crkv_q8_seg(FAKE, q_at, 16, K), crkv.crkv_q8_seg(FAKE, q_at + 4096, 16, V))
    assert L.crkv_quantize_q8(ok, 2, 2, 96, ctypes.byref(o)) == -2       # d
    assert L.crkv_quantize_q8(ok, 2, 0, 128, ctypes.byref(o)) == -1      # H_kv
    assert L.crkv_quantize_q8(ok, 0, 2, 128, ctypes.byref(o)) == -1      # n
    for seg in (crkv.crkv_q8_seg(FAKE, q_at, -1, V), crkv.crkv_q8_seg(None, q_at, 16, V),
                crkv.crkv_q8_seg(FAKE, None, 16, K), crkv.crkv_q8_seg(FAKE + 8, q_at, 16, K),
                crkv.crkv_q8_seg(FAKE, q_at + 4, 16, V), crkv.crkv_q8_seg(FAKE, FAKE + 256, 16, K),
                crkv.crkv_q8_seg(FAKE, q_at, 16, 2)):
        bad = (crkv.crkv_q8_seg * 1)(seg)
        assert L.crkv_quantize_q8(bad, 1, 2, 128, ctypes.byref(o)) == -1
    for dt in (crkv.CRKV_F32, crkv.CRKV_KV_Q8):   # the input is bf16
        o.dtype = dt
        assert L.crkv_quantize_q8(ok, 2, 2, 128, ctypes.byref(o)) in (-1, -2)
    o.dtype = crkv.CRKV_BF16
    idle = (crkv.crkv_q8_seg * 2)(crkv.crkv_q8_seg(None, None, 0, K), crkv.crkv_q8_seg(None, None, 0, V))
    assert L.crkv_quantize_q8(idle, 2, 2, 128, ctypes.byref(o)) == 0   # nothing to do
    assert L.crkv_q8_bytes(8, 2500, 128, V) == 8 * 2500 * 128 + 4 * 8 * 2500
    assert L.crkv_q8_bytes(8, 2500, 128, K) == 8 * 2500 * 128 + 4 * 8 * 128
    assert L.crkv_q8_bytes(8, 0, 128, K) == 0
    assert L.crkv_q8_bytes(8, 2500, 96, K) == 0 and L.crkv_q8_bytes(-1, 5, 64, V) == 0
    assert L.crkv_q8_bytes(8, 5, 64, 7) == 0


def test_q8_dtype_in_attention_and_decode(crkv_lib):
    """CRKV_KV_Q8 passes the decode step's and the prefill's validation (the
    workspace sizes are computed, the planner picks an 8-bit build of the
    wave kernel) and is refused by the entry points that move or rotate
    bf16 rows."""
    p = dict(Q=FAKE, chunk_K=[FAKE, FAKE], chunk_V=[FAKE, FAKE], chunk_len=[64, 3], q_len=1,
             out=FAKE, impact=FAKE)
    assert crkv.crkv_decode_workspace_size([p], 8, 2, 128, dtype=crkv.CRKV_KV_Q8) > 0
    for mode in ("query", "cross", "all"):
        assert crkv.crkv_workspace_size([p], 8, 2, 128, mode=mode, dtype=crkv.CRKV_KV_Q8) > 0
        plan = crkv.crkv_plan_info([p], 8, 2, 128, mode=mode, dtype=crkv.CRKV_KV_Q8)
        assert plan["kernel"] == "bf16_wave" and plan["row_tiles"] in (4, 5), plan
    with pytest.raises(crkv.CrkvError) as e:
        crkv.crkv_decode_chunks_batched([p], 8, 2, 128, dtype=5)
    assert e.value.status == -2
    with pytest.raises(crkv.CrkvError) as e:
        crkv.crkv_rope_shift([(FAKE, 64, 3)], 2, 128, crkv.CRKV_KV_Q8)
    assert e.value.status == -1


def test_plan_create_rejects_invalid_arguments(crkv_lib):
    """Validation comes before any allocation: these calls touch no device."""
    o = crkv.crkv_opts()
    crkv_lib.crkv_opts_init(ctypes.byref(o))
    o.dtype = crkv.CRKV_BF16
    p = crkv._Problem(FAKE, [FAKE, FAKE], [FAKE, FAKE], [64, 16], 16, FAKE, FAKE)
    arr = (crkv.crkv_problem * 1)(p.c)
    h = ctypes.c_void_p()
    L = crkv_lib
    assert L.crkv_plan_create(arr, 1, 8, 2, 128, None, None, ctypes.byref(o), None) == -1       # no output
    assert L.crkv_plan_create(arr, 1, 8, 3, 128, None, None, ctypes.byref(o), ctypes.byref(h)) == -1
    assert L.crkv_plan_create(arr, 1, 8, 2, 96, None, None, ctypes.byref(o), ctypes.byref(h)) == -2
    k = (ctypes.c_int32 * 1)(6)
    assert L.crkv_plan_create(arr, 1, 8, 2, 128, k, None, ctypes.byref(o), ctypes.byref(h)) == -1  # k, no idx
    idx = (ctypes.c_void_p * 1)(FAKE)
    k[0] = 65                                                                                       # k > N_doc
    assert L.crkv_plan_create(arr, 1, 8, 2, 128, k, idx, ctypes.byref(o), ctypes.byref(h)) == -1
    o.dtype = 9
    k[0] = 6
    assert L.crkv_plan_create(arr, 1, 8, 2, 128, k, idx, ctypes.byref(o), ctypes.byref(h)) == -1
    assert h.value is None
    assert L.crkv_plan_launch(None, None, None) == -1
    assert L.crkv_plan_destroy(None) == 0


def _static_call(crkv_lib, probs, H, H_kv, d, mode, workspace=None):
    arr = (crkv.crkv_problem * len(probs))()
    keep = []
    for i, p in enumerate(probs):
        m = len(p["chunk_len"]) - 1
        k = (ctypes.c_void_p * (m + 1))(*p["chunk_K"])
        v = (ctypes.c_void_p * (m + 1))(*p["chunk_V"])
        ln = (ctypes.c_int32 * (m + 1))(*p["chunk_len"])
        keep += [k, v, ln]
        arr[i] = crkv.crkv_problem(p["Q"], k, v, ln, m, p["q_len"], p["out"], p["impact"])
    o = crkv.crkv_opts()
    crkv_lib.crkv_opts_init(ctypes.byref(o))
    o.dtype = crkv.CRKV_BF16
    o.mode = mode
    o.workspace = workspace
    rc = crkv_lib.crkv_attn_chunks_batched_static(arr, len(probs), H, H_kv, d, ctypes.byref(o))
    return rc, crkv_lib.crkv_last_error().decode()


def test_static_scratch_refusals(crkv_lib):
    """crkv_attn_chunks_batched_static refuses, before touching any device, a
    call whose tables and impact partials exceed its static scratch, and a
    caller workspace; its invalid arguments fail like the per-call entry
    point's."""
    assert crkv.crkv_static_scratch_bytes() == 64 << 20
    big = [_fake_problem([8192] * 8, 128, 32, 128) for _ in range(4)]
    rc, msg = _static_call(crkv_lib, big, 32, 32, 128, 1)
    assert rc == crkv.CRKV_E_UNSUPPORTED and "static scratch" in msg, msg
    one = [_fake_problem([512] * 4, 64, 32, 128)]
    rc, msg = _static_call(crkv_lib, one, 32, 32, 128, 0, workspace=0x100000)
    assert rc == crkv.CRKV_E_INVAL and "workspace must be NULL" in msg, msg
    bad = [dict(one[0], q_len=0)]
    rc, msg = _static_call(crkv_lib, bad, 32, 32, 128, 0)
    assert rc == crkv.CRKV_E_INVAL and "q_len" in msg, msg
