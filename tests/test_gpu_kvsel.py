"""GPU parity of the selected-key K/V gather and scatter against the oracle,
bit for bit, through the C ABI."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import attention_precomputed_chunk_amd as crkv  # noqa: E402
import workloads  # noqa: E402
from gpu_util import DEV, DeviceWorkload  # noqa: E402
from oracle import kvsel  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib(crkv_lib):
    yield


def host_bits(t):
    """A device tensor's stored bits as numpy (uint16 for bf16, float32)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def dev_from_bits(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def empty_sel(H_kv, k, d, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return (torch.full((H_kv, k, d), float("nan"), dtype=tdt, device=DEV),
            torch.full((H_kv, k, d), float("nan"), dtype=tdt, device=DEV))


CASES = [
    # seed, doc_lens, q_len, H_kv, d, dtype, selected counts per problem
    (1, [130, 0, 67, 5], 9, 2, 128, "bf16", [40, 0, 17]),
    (2, [64, 64], 16, 4, 64, "bf16", [144, 1, 16]),
    (3, [0, 300], 3, 1, 128, "f32", [33, 303, 2]),
    (4, [511, 2, 1000], 100, 8, 128, "bf16", [1500, 77, 160]),
    (5, [17], 5, 3, 64, "f32", [22, 5, 13]),
]


def selection(rng, n_keys, count):
    """Distinct positions (count of them, at most n_keys + 2), with one
    past-the-end and one negative position mixed in when there is room."""
    idx = rng.permutation(n_keys)[:count].astype(np.int32)
    if count >= 4:
        idx[1] = n_keys        # gathers zeros, scatters nothing
        idx[3] = -7
    return idx


@pytest.mark.parametrize("case", range(len(CASES)))
def test_gather_and_scatter_small(case):
    seed, doc, q, H_kv, d, dtype, counts = CASES[case]
    say("kvsel case", CASES[case])
    wl = workloads.custom(400 + seed, doc, q, H_kv, H_kv, d, dtype=dtype, n_problems=len(counts))
    dw = DeviceWorkload(wl)
    rng = np.random.default_rng(seed)
    dt = crkv.CRKV_BF16 if dtype == "bf16" else crkv.CRKV_F32
    sels, idxs = [], []
    for pi, (prob, cnt) in enumerate(zip(wl.problems, counts)):
        idx = selection(rng, prob.n_keys, cnt)
        idxs.append(idx)
        Ks, Vs = empty_sel(H_kv, len(idx), d, dtype)
        pr = dw.problems[pi]
        sels.append(dict(chunk_K=pr["chunk_K"], chunk_V=pr["chunk_V"], chunk_len=prob.lens,
                         idx=torch.from_numpy(idx).to(DEV), K_sel=Ks, V_sel=Vs))
    crkv.crkv_gather_kv(sels, H_kv, d, dt)
    torch.cuda.synchronize()
    for prob, idx, s in zip(wl.problems, idxs, sels):
        Kr, Vr = kvsel.gather_kv(prob.K, prob.V, prob.lens, idx)
        assert np.array_equal(host_bits(s["K_sel"]), Kr)
        assert np.array_equal(host_bits(s["V_sel"]), Vr)

    # scatter fresh rows to the same positions, then compare every segment
    new = []
    for prob, idx, s in zip(wl.problems, idxs, sels):
        shape = (H_kv, len(idx), d)
        if dtype == "bf16":
            Kn = rng.integers(0, 1 << 15, size=shape).astype(np.uint16)   # finite bf16
            Vn = rng.integers(0, 1 << 15, size=shape).astype(np.uint16)
        else:
            Kn = rng.standard_normal(shape).astype(np.float32)
            Vn = rng.standard_normal(shape).astype(np.float32)
        s["K_sel"], s["V_sel"] = dev_from_bits(Kn, dtype), dev_from_bits(Vn, dtype)
        new.append((Kn, Vn))
    crkv.crkv_scatter_kv(sels, H_kv, d, dt)
    torch.cuda.synchronize()
    for pi, (prob, idx, (Kn, Vn)) in enumerate(zip(wl.problems, idxs, new)):
        K, V = [k.copy() for k in prob.K], [v.copy() for v in prob.V]
        kvsel.scatter_kv(K, V, prob.lens, idx, Kn, Vn)
        for c, n in enumerate(prob.lens):
            if n == 0:
                continue
            assert np.array_equal(host_bits(dw.problems[pi]["chunk_K"][c]), K[c]), (pi, c)
            assert np.array_equal(host_bits(dw.problems[pi]["chunk_V"][c]), V[c]), (pi, c)


def test_gather_topk_selection_32_layers():
    """The 32-layer GQA workload: attention, top-k, then the gather of every
    layer's selected keys, against the oracle at the GPU's own indices; a
    scatter of the gathered rows leaves every segment unchanged."""
    say("llama3_8b_gqa_32l gather")
    wl = workloads.generate("llama3_8b_gqa_32l")
    dw = DeviceWorkload(wl)
    dw.attn()
    gidx = dw.topk()
    torch.cuda.synchronize()
    sels = []
    for pi, prob in enumerate(wl.problems):
        Ks, Vs = empty_sel(wl.H_kv, int(gidx[pi].numel()), wl.d, wl.dtype)
        pr = dw.problems[pi]
        sels.append(dict(chunk_K=pr["chunk_K"], chunk_V=pr["chunk_V"], chunk_len=prob.lens,
                         idx=gidx[pi], K_sel=Ks, V_sel=Vs))
    crkv.crkv_gather_kv(sels, wl.H_kv, wl.d, crkv.CRKV_BF16)
    torch.cuda.synchronize()
    for pi, prob in enumerate(wl.problems):
        idx = gidx[pi].cpu().numpy()
        assert len(set(idx.tolist())) == len(idx) and idx.min() >= 0 and idx.max() < prob.n_doc
        Kr, Vr = kvsel.gather_kv(prob.K, prob.V, prob.lens, idx)
        assert np.array_equal(host_bits(sels[pi]["K_sel"]), Kr), pi
        assert np.array_equal(host_bits(sels[pi]["V_sel"]), Vr), pi
    crkv.crkv_scatter_kv(sels, wl.H_kv, wl.d, crkv.CRKV_BF16)
    torch.cuda.synchronize()
    for pi in (0, 13, 31):
        prob = wl.problems[pi]
        for c in range(len(prob.lens)):
            assert np.array_equal(host_bits(dw.problems[pi]["chunk_K"][c]), prob.K[c])
            assert np.array_equal(host_bits(dw.problems[pi]["chunk_V"][c]), prob.V[c])


def test_gather_rejects_misaligned_buffer():
    wl = workloads.custom(420, [64], 4, 2, 2, 64, dtype="bf16")
    dw = DeviceWorkload(wl)
    Ks, Vs = empty_sel(2, 8, 64, "bf16")
    pr = dw.problems[0]
    bad = dict(chunk_K=pr["chunk_K"], chunk_V=pr["chunk_V"], chunk_len=wl.problems[0].lens,
               idx=torch.arange(8, dtype=torch.int32, device=DEV), K_sel=Ks.data_ptr() + 2, V_sel=Vs, k=8)
    with pytest.raises(crkv.CrkvError):
        crkv.crkv_gather_kv([bad], 2, 64, crkv.CRKV_BF16)
