"""Pins of the 8-bit K/V format oracle against what its definition fixes, for
both groupings (K: a scale per channel over the segment's tokens; V: a scale
per token): groups with a power-of-two scale whose codes are the textbook
round-half-even of the input, a float32 tie, brute-force nearest code on tiny
inputs, the error bound, the extreme element, zero groups, sign and
power-of-two scale symmetry, the buffer layout, a decode step over a cache the
format stores exactly (equal to the decode over the original values), and
planted mistakes."""
import numpy as np
import pytest

import oracle
from oracle import q8
import workloads


def f32_to_bf16_bits(x):
    return workloads.round_bf16(np.asarray(x, dtype=np.float32))


def as_group(v, kind):
    """A 1-D group laid out as one token row (V) or one channel column (K)."""
    v = np.asarray(v, dtype=np.float32)
    return v[None, :] if kind == "v" else v[:, None]


def group_codes(codes, kind):
    return (codes[0] if kind == "v" else codes[:, 0]).tolist()


@pytest.mark.parametrize("kind", ["k", "v"])
def test_unit_scale_is_round_half_even(kind):
    """max |x| = 127 gives scale exactly 1, so the codes are the integers
    nearest to x, halves to the even one."""
    codes, scale = q8.quantize(as_group([127.0, -64.5, 32.5, 0.5, 1.5, -2.5, 3.25, 0.0], kind), kind, "f32")
    assert scale.reshape(-1)[0] == np.float32(1.0)
    assert group_codes(codes, kind) == [127, -64, 32, 0, 2, -2, 3, 0]


@pytest.mark.parametrize("kind", ["k", "v"])
def test_scale_two(kind):
    codes, scale = q8.quantize(as_group([-254.0, 5.0, 7.0, -3.0, 100.5, 2.0], kind), kind, "f32")
    assert scale.reshape(-1)[0] == np.float32(2.0)
    # x / 2 = -127, 2.5, 3.5, -1.5, 50.25, 1
    assert group_codes(codes, kind) == [-127, 2, 4, -2, 50, 1]


@pytest.mark.parametrize("kind", ["k", "v"])
def test_decision_in_float32(kind):
    """77 / 127 rounded to float32, then 38.5 divided by it, is exactly 63.5 in
    float32 (a tie, to the even code 64); the exact quotient is just below
    63.5 (code 63). The code must be the float32 one, the precision the
    kernel decides in."""
    codes, scale = q8.quantize(f32_to_bf16_bits(as_group([77.0, 38.5, -38.5, 1.0], kind)), kind, "bf16")
    s = np.float32(np.float32(77.0) / np.float32(127.0))
    assert scale.reshape(-1)[0] == s and np.float32(np.float32(38.5) / s) == np.float32(63.5)
    assert 38.5 / float(s) < 63.5
    assert group_codes(codes, kind) == [127, 64, -64, 2]


def brute_codes(x32, scale):
    """For each element, the code c in [-127, 127] nearest to x / scale computed
    in float32, found by trying all 255 (ties: the even one)."""
    out = []
    for v in x32:
        t = np.float32(v) / np.float32(scale)
        best = None
        for c in range(-127, 128):
            dist = abs(float(t) - c)
            if best is None or dist < best[0] - 1e-12 or (abs(dist - best[0]) <= 1e-12 and c % 2 == 0):
                best = (dist, c)
        out.append(best[1])
    return out


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("seed", range(4))
def test_brute_force_nearest_code(kind, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, 5, 12)).astype(np.float32) * np.float32(rng.uniform(0.01, 50))
    x[1, 3, :] = 0.0
    x[0, :, 7] = 0.0
    bits = f32_to_bf16_bits(x)
    codes, scales = q8.quantize(bits, kind, "bf16")
    xw = (bits.astype(np.uint32) << 16).view(np.float32)
    for h in range(2):
        groups = [(xw[h, t, :], codes[h, t, :], scales[h, t]) for t in range(5)] if kind == "v" else \
                 [(xw[h, :, c], codes[h, :, c], scales[h, c]) for c in range(12)]
        for g, gc, sc in groups:
            a = np.max(np.abs(g))
            assert sc == np.float32(a) / np.float32(127)
            if a > 0:
                assert gc.tolist() == brute_codes(g, sc)
            else:
                assert not gc.any()


@pytest.mark.parametrize("kind", ["k", "v"])
def test_error_bound_extreme_and_range(kind):
    wl = workloads.custom(11, [300, 7], 1, 4, 2, 128, dtype="bf16", k_outliers=4, gen_len=20)
    ax = -2 if kind == "k" else -1
    for k in wl.problems[0].K:
        codes, scales = q8.quantize(k, kind, "bf16")
        x = workloads.widen(k, "bf16")
        deq = q8.dequantize(codes, scales, kind)
        assert codes.dtype == np.int8 and int(np.abs(codes.astype(int)).max()) <= 127
        # nearest code to the float32 quotient t = (x / scale)(1 + e), |e| <= 2^-24,
        # |x / scale| <= 127: at most half a step plus 128 * 2^-24 steps
        assert np.all(np.abs(x - deq) <= (0.5 + 128 * 2.0 ** -24) * np.expand_dims(scales, ax))
        # the largest magnitude of every group lands on +-127
        arg = np.expand_dims(np.argmax(np.abs(x), axis=ax), ax)
        top = np.take_along_axis(codes.astype(int), arg, axis=ax)
        assert np.all(np.abs(top) == 127)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_zero_groups_sign_and_power_of_two_symmetry(kind):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 6, 64)).astype(np.float32)
    if kind == "v":
        x[1, 2, :] = 0.0
    else:
        x[1, :, 2] = 0.0
    c, s = q8.quantize(x, kind, "f32")
    assert s[1, 2] == 0
    zero = c[1, 2, :] if kind == "v" else c[1, :, 2]
    assert not zero.any()
    cn, sn = q8.quantize(-x, kind, "f32")
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    c8, s8 = q8.quantize(x * np.float32(8.0), kind, "f32")
    assert np.array_equal(c8, c) and np.array_equal(s8, s * np.float32(8.0))


@pytest.mark.parametrize("kind", ["k", "v"])
def test_buffer_layout(kind):
    rng = np.random.default_rng(4)
    H_kv, n, d = 3, 5, 64
    k = f32_to_bf16_bits(rng.standard_normal((H_kv, n, d)))
    codes, scales = q8.quantize(k, kind, "bf16")
    buf = q8.pack(codes, scales)
    ns = d if kind == "k" else n
    assert buf.size == q8.nbytes(H_kv, n, d, kind) == H_kv * n * d + 4 * H_kv * ns
    assert buf[:H_kv * n * d].view(np.int8).reshape(H_kv, n, d)[1, 2, 7] == codes[1, 2, 7]
    assert buf[H_kv * n * d:].view(np.float32)[1 * ns + 4] == scales[1, 4]
    c2, s2 = q8.unpack(buf, H_kv, n, d, kind)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    assert q8.nbytes(H_kv, 0, d, kind) == 0 and q8.pack(*q8.quantize(k[:, :0], kind, "bf16")).size == 0


def test_decode_over_an_exactly_stored_cache():
    """K of integers in [-127, 127] with a token of 127 in every channel, and V
    rows of integers / 16 whose largest magnitude is 127 / 16, are stored
    exactly (scales 1 and 1/16), so the decode step over the format equals the
    decode step over the original bf16 values."""
    wl = workloads.custom(5, [40, 0, 33], 1, 8, 2, 64, dtype="bf16", gen_len=6)
    p = wl.problems[0]
    rng = np.random.default_rng(9)
    for i, s in enumerate(p.K):
        v = rng.integers(-127, 128, size=s.shape).astype(np.float32)
        if v.size:
            v[:, 0, :] = 127.0
        p.K[i] = f32_to_bf16_bits(v)
    for i, s in enumerate(p.V):
        v = rng.integers(-127, 128, size=s.shape).astype(np.float32)
        if v.size:
            v[..., 0] = 127.0
        p.V[i] = f32_to_bf16_bits(v / np.float32(16.0))
    kq, vq = q8.quantize_problem(p)
    for (c, s), k in zip(kq, p.K):
        assert np.array_equal(q8.dequantize(c, s, "k"), workloads.widen(k, "bf16"))
    for (c, s), v in zip(vq, p.V):
        assert np.array_equal(q8.dequantize(c, s, "v"), workloads.widen(v, "bf16"))
    ref, _, _ = oracle.attn(p, wl.H, wl.H_kv, wl.d, "bf16", "query")
    got = q8.decode(p, wl.H, wl.H_kv, wl.d, kq, vq)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["query", "cross", "all"])
def test_attention_over_an_exactly_stored_cache(mode):
    """The same exactly stored cache (integer K with a 127 token, V in
    sixteenths): the prefill over the format (out, impact, every mode)
    equals the prefill over the original bf16 values."""
    wl = workloads.custom(6, [37, 0, 1, 50], 9, 4, 2, 64, dtype="bf16", mode=mode)
    p = wl.problems[0]
    rng = np.random.default_rng(10)
    for i, s in enumerate(p.K):
        v = rng.integers(-127, 128, size=s.shape).astype(np.float32)
        if v.size:
            v[:, 0, :] = 127.0
        p.K[i] = f32_to_bf16_bits(v / np.float32(64.0))   # scale 1/64: scores of moderate size
    for i, s in enumerate(p.V):
        v = rng.integers(-127, 128, size=s.shape).astype(np.float32)
        if v.size:
            v[..., 0] = 127.0
        p.V[i] = f32_to_bf16_bits(v / np.float32(16.0))
    kq, vq = q8.quantize_problem(p)
    for (c, s), k in zip(kq, p.K):
        assert np.array_equal(q8.dequantize(c, s, "k"), workloads.widen(k, "bf16"))
    out_ref, imp_ref, _ = oracle.attn(p, wl.H, wl.H_kv, wl.d, "bf16", mode)
    out, imp, _ = q8.attn(p, wl.H, wl.H_kv, wl.d, mode, kq, vq)
    np.testing.assert_allclose(out, out_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(imp, imp_ref, rtol=1e-12, atol=1e-15)


def test_attention_over_quantised_cache_is_attention_over_dequantised_values():
    """An ordinary (inexact) cache: the prefill over the format equals the fp64
    attention over code * scale built here by hand, and the impact still sums
    to q_len * H."""
    wl = workloads.custom(7, [70, 33], 12, 4, 2, 64, dtype="bf16", k_outliers=2)
    p = wl.problems[0]
    kq, vq = q8.quantize_problem(p)
    Ks = [c.astype(np.float64) * s[:, None, :].astype(np.float64) for c, s in kq]
    Vs = [c.astype(np.float64) * s[:, :, None].astype(np.float64) for c, s in vq]
    hand = workloads.Problem(K=Ks, V=Vs, lens=list(p.lens), q_len=p.q_len, Q=workloads.widen(p.Q, "bf16"))
    out_ref, imp_ref, _ = oracle.attn(hand, wl.H, wl.H_kv, wl.d, "f64", "query")
    out, imp, _ = q8.attn(p, wl.H, wl.H_kv, wl.d, "query")
    np.testing.assert_array_equal(out, out_ref)
    np.testing.assert_array_equal(imp, imp_ref)
    assert abs(imp.sum() - p.q_len * wl.H) < 1e-9


@pytest.mark.parametrize("mutant", ["half_away", "scale_128", "no_float32_quotient", "wrong_axis"])
def test_pins_catch_planted_mistakes(mutant, monkeypatch):
    real = q8.quantize

    def bad(x, kind, dtype="bf16"):
        if mutant == "wrong_axis":
            return real(x, "v" if kind == "k" else "k", dtype) if np.asarray(x).ndim >= 2 else real(x, kind, dtype)
        ax = -2 if kind == "k" else -1
        xf = q8._f32(x, dtype)
        amax = np.max(np.abs(xf), axis=ax)
        scale = (amax / np.float32(128 if mutant == "scale_128" else 127)).astype(np.float32)
        safe = np.expand_dims(np.where(scale > 0, scale, 1).astype(np.float32), ax)
        if mutant == "no_float32_quotient":   # quotient in float64: other ties near .5
            codes = np.rint(xf.astype(np.float64) / safe.astype(np.float64))
        else:
            t = (xf / safe).astype(np.float32)
            codes = np.sign(t) * np.floor(np.abs(t) + 0.5) if mutant == "half_away" else np.rint(t)
        codes = np.where(np.expand_dims(scale, ax) > 0, np.clip(codes, -127, 127), 0).astype(np.int8)
        return codes, scale

    monkeypatch.setattr(q8, "quantize", bad)
    with pytest.raises(AssertionError):
        for kind in ("k", "v"):
            test_unit_scale_is_round_half_even(kind)
            test_scale_two(kind)
            test_decision_in_float32(kind)
    monkeypatch.setattr(q8, "quantize", real)
