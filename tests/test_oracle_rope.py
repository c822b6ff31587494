"""Pins of the key re-positioning oracle against what the rotation fixes:
element-by-element brute force with explicit 2x2 rotations, identity,
composition, inverse, norm preservation, the relative-position property of
dot products, single rounding to bf16, and planted mistakes."""
import math

import numpy as np
import pytest

from oracle import rope


def brute(x, delta, base):
    """[..., d] float64, loops with math.cos / math.sin over pairs (i, i + d/2)."""
    d = x.shape[-1]
    h = d // 2
    flat = x.reshape(-1, d)
    out = np.empty_like(flat)
    for r in range(flat.shape[0]):
        for i in range(h):
            a = delta * math.pow(base, -2.0 * i / d)
            c, s = math.cos(a), math.sin(a)
            u, v = flat[r, i], flat[r, i + h]
            out[r, i] = u * c - v * s
            out[r, i + h] = v * c + u * s
    return out.reshape(x.shape)


@pytest.mark.parametrize("d,delta,base", [(8, 3, 10000.0), (16, -17, 10000.0), (64, 2500, 10000.0),
                                          (128, 7500, 500000.0), (128, 0, 10000.0)])
def test_brute_force(d, delta, base):
    x = np.random.default_rng(d + abs(delta)).standard_normal((2, 3, d))
    np.testing.assert_allclose(rope.rotate64(x, delta, base), brute(x, delta, base), rtol=0, atol=1e-12)


def test_identity_is_bit_exact():
    rng = np.random.default_rng(1)
    k32 = rng.standard_normal((2, 5, 64)).astype(np.float32)
    assert np.array_equal(rope.rope_shift(k32, 0, "f32"), k32)
    kb = rng.integers(0, 0x7F00, size=(2, 5, 64)).astype(np.uint16)
    assert np.array_equal(rope.rope_shift(kb, 0, "bf16"), kb)


@pytest.mark.parametrize("a,b", [(5, 7), (2500, -2500), (10000, 123), (-40, 40000)])
def test_composition_and_inverse(a, b):
    x = np.random.default_rng(abs(a * 7 + b)).standard_normal((4, 128))
    np.testing.assert_allclose(rope.rotate64(rope.rotate64(x, a), b), rope.rotate64(x, a + b), atol=1e-9)
    np.testing.assert_allclose(rope.rotate64(rope.rotate64(x, a), -a), x, atol=1e-9)


def test_pair_norms_and_relative_dot_products():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    y = rope.rotate64(k, 3333)
    np.testing.assert_allclose(y[:64] ** 2 + y[64:] ** 2, k[:64] ** 2 + k[64:] ** 2, rtol=1e-12)
    for a, b in [(100, 40), (7000, 6940), (60, 0)]:   # all with a - b = 60
        assert abs(np.dot(rope.rotate64(q, a), rope.rotate64(k, b)) - np.dot(rope.rotate64(q, 60), k)) < 1e-9


def test_bf16_store_rounds_once():
    """A float64 value just above a bf16 midpoint whose float32 rounding lands
    on the midpoint: one rounding goes up, rounding twice would go to even."""
    b = np.uint16(0x3F80)                           # 1.0, even mantissa
    mid = (np.uint32(b) << 16) | np.uint32(0x8000)  # halfway to the next bf16
    m = float(np.array([mid], dtype=np.uint32).view(np.float32)[0])
    y = np.array([m + 2.0 ** -40])                  # above the midpoint, below float32 resolution
    assert np.float32(y[0]) == np.float32(m)        # float32 alone would land on the tie
    assert rope._store(y, "bf16")[0] == b + 1
    assert rope._store(np.array([m - 2.0 ** -40]), "bf16")[0] == b
    assert rope._store(np.array([m]), "bf16")[0] == b   # an exact tie goes to even


@pytest.mark.parametrize("mutant", ["adjacent_pairs", "sign", "half_frequency"])
def test_pins_catch_planted_mistakes(mutant, monkeypatch):
    real = rope.rotate64

    def bad(x, delta, base=10000.0):
        d = x.shape[-1]
        if mutant == "adjacent_pairs":   # pairs (2i, 2i + 1)
            y = x.copy()
            a = rope.angles(d, delta, base)
            c, s = np.cos(a), np.sin(a)
            y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
            y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
            return y
        if mutant == "sign":
            return real(x, -delta, base)
        return real(x, delta, base ** 0.5)

    monkeypatch.setattr(rope, "rotate64", bad)
    with pytest.raises(AssertionError):
        test_brute_force(16, -17, 10000.0)
