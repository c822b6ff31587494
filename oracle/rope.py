"""Oracle for re-positioning cached keys under rotary position embedding.

TEST INFRASTRUCTURE ONLY: the tests, the package entry point's smoke check and
the benchmark's CPU-baseline leg may use it; the library never does. It shares
no code with the HIP library.

What it follows: the TurboRAG summary's implementation notes require, for
models with rotary position embedding, that the position IDs a chunk's cache
was computed with agree with the ones it is used at. A chunk precomputed at
positions 0 .. len-1 and placed at offset o of the concatenation therefore
needs its keys moved by o positions. The pages give no formula, so this
rests on a reading (parity unpinned against the pages): the standard rotary
embedding, pairs (i, i + d/2) (the rotate-half arrangement), frequency
theta_i = base^(-2i/d), and a key at position p rotated by angle p * theta_i
in every pair. Rotations compose, so moving a key by delta positions is one
more rotation by delta * theta_i:

    y_i       = x_i cos(a_i) - x_{i+d/2} sin(a_i)
    y_{i+d/2} = x_{i+d/2} cos(a_i) + x_i sin(a_i),    a_i = delta * theta_i

computed here in float64 from the exactly widened input and rounded once to
the stored type (bf16 round-to-nearest-even, or float32).
"""
from __future__ import annotations

import numpy as np


def angles(d: int, delta: int, base: float = 10000.0) -> np.ndarray:
    """a_i = delta * base^(-2i/d), i < d/2, in float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return float(delta) * np.power(float(base), -2.0 * i / d)


def rotate64(x: np.ndarray, delta: int, base: float = 10000.0) -> np.ndarray:
    """The rotation on float64 values ``[..., d]`` (no rounding)."""
    d = x.shape[-1]
    a = angles(d, delta, base)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _widen(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _to_f32_round_to_odd(y: np.ndarray) -> np.ndarray:
    """float64 -> float32 rounding toward zero with the last bit set when
    inexact ("round to odd"); a later round-to-nearest-even to a format with
    at least two fewer bits then equals one correct rounding of y."""
    f = y.astype(np.float32)                                    # nearest even
    inexact = f.astype(np.float64) != y
    over = np.abs(f.astype(np.float64)) > np.abs(y)
    u = f.view(np.uint32).copy()
    u[inexact & over] -= 1                                      # toward zero (same sign)
    u[inexact] |= 1
    return u.view(np.float32)


def _store(y: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 once to the stored type (round to nearest, ties to even)."""
    if dtype == "bf16":
        u = _to_f32_round_to_odd(np.ascontiguousarray(y, dtype=np.float64)).view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.ascontiguousarray(y, dtype=np.float32)


def rope_shift(K: np.ndarray, delta: int, dtype: str, base: float = 10000.0) -> np.ndarray:
    """Stored keys ``[H_kv][len][d]`` (bf16 bits or float32) moved by delta
    positions, in the stored type."""
    return _store(rotate64(_widen(K, dtype), delta, base), dtype)
