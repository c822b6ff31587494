"""GPU parity of the key re-positioning (rotary embedding shift) against the
oracle, through the C ABI. The rotation is done in float32 and rounded once
to the stored type; the oracle rounds its float64 result once, so bf16
results may differ by one unit in the last place where the exact value lies
within float32 rounding of a bf16 rounding boundary."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import attention_precomputed_chunk_amd as crkv  # noqa: E402
from gpu_util import DEV  # noqa: E402
from oracle import rope  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib(crkv_lib):
    yield


def make(rng, H_kv, n, d, dtype):
    if dtype == "bf16":
        x = rng.standard_normal((H_kv, n, d)).astype(np.float32)
        u = x.view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return rng.standard_normal((H_kv, n, d)).astype(np.float32)


def to_dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check(got, ref, x, dtype, label):
    if dtype == "bf16":
        # bf16 bit patterns of finite values order like sign-magnitude integers
        gi = np.where(got & 0x8000, -(got.astype(np.int32) & 0x7FFF), got.astype(np.int32) & 0x7FFF)
        ri = np.where(ref & 0x8000, -(ref.astype(np.int32) & 0x7FFF), ref.astype(np.int32) & 0x7FFF)
        ulp = np.abs(gi - ri)
        assert ulp.max() <= 1, "%s: %d ulp" % (label, ulp.max())
        assert (ulp > 0).mean() < 0.01, "%s: %.3f of elements off by one ulp" % (label, (ulp > 0).mean())
        return float((ulp > 0).mean())
    d = x.shape[-1]
    mag = np.abs(x[..., : d // 2]) + np.abs(x[..., d // 2:])
    bound = np.concatenate([mag, mag], axis=-1) * 2.0 ** -21 + 1e-30
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= bound), "%s: error %.3g over bound" % (label, (err / bound).max())
    return float((err / bound).max())


CASES = [
    # dtype, d, H_kv, lens, deltas, base
    ("bf16", 128, 8, [2500, 2500, 17, 0], [2500, 5000, -3, 9], 10000.0),
    ("bf16", 64, 2, [300, 1, 129], [40000, -40000, 1], 10000.0),
    ("bf16", 128, 1, [1000, 64], [123456, 77], 500000.0),
    ("f32", 128, 4, [257, 33], [7500, -1], 10000.0),
    ("f32", 64, 3, [100, 0, 5], [12, 99, -100000], 10000.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_rope_shift_matches_oracle(case):
    dtype, d, H_kv, lens, deltas, base = CASES[case]
    say("rope case", CASES[case])
    rng = np.random.default_rng(500 + case)
    xs = [make(rng, H_kv, n, d, dtype) for n in lens]
    dev = [to_dev(x, dtype) for x in xs]
    dt = crkv.CRKV_BF16 if dtype == "bf16" else crkv.CRKV_F32
    crkv.crkv_rope_shift([(t, n, dl) for t, n, dl in zip(dev, lens, deltas)], H_kv, d, dt, base)
    torch.cuda.synchronize()
    for x, t, dl, n in zip(xs, dev, deltas, lens):
        if n == 0:
            continue
        got = to_host(t, dtype)
        ref = rope.rope_shift(x, dl, dtype, base)
        wide = (x.astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else x
        say("  delta %d: %.3g" % (dl, check(got, ref, wide.astype(np.float64), dtype, "delta %d" % dl)))


def test_zero_shift_untouched_and_round_trip():
    rng = np.random.default_rng(510)
    x = make(rng, 4, 700, 128, "bf16")
    t = to_dev(x, "bf16")
    crkv.crkv_rope_shift([(t, 700, 0)], 4, 128, crkv.CRKV_BF16)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(t, "bf16"), x)
    # there and back: each leg rounds to bf16, so within a few ulp of the start
    crkv.crkv_rope_shift([(t, 700, 3000)], 4, 128, crkv.CRKV_BF16)
    crkv.crkv_rope_shift([(t, 700, -3000)], 4, 128, crkv.CRKV_BF16)
    torch.cuda.synchronize()
    back = (to_host(t, "bf16").astype(np.uint32) << 16).view(np.float32)
    start = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.abs(back - start).max() <= 2 ** -6 * np.abs(start).max()


def test_composition_on_device():
    """Two shifts agree with one shift by the sum (float32, tight)."""
    rng = np.random.default_rng(511)
    x = make(rng, 2, 300, 64, "f32")
    a, b = to_dev(x, "f32"), to_dev(x, "f32")
    crkv.crkv_rope_shift([(a, 300, 1500)], 2, 64, crkv.CRKV_F32)
    crkv.crkv_rope_shift([(a, 300, 2500)], 2, 64, crkv.CRKV_F32)
    crkv.crkv_rope_shift([(b, 300, 4000)], 2, 64, crkv.CRKV_F32)
    torch.cuda.synchronize()
    np.testing.assert_allclose(a.cpu().numpy(), b.cpu().numpy(), atol=1e-5 * np.abs(x).max())
