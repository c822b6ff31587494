"""Oracle for the 8-bit K/V cache format that the decode step can read.

TEST INFRASTRUCTURE ONLY: the tests, the package entry point's smoke check and
the benchmark's CPU-baseline leg may use it; the library never does. It shares
no code with the HIP library.

What it follows: the CacheGen summary observes that loading a precomputed KV
cache dominates the time to first token and that caches can be encoded into a
much smaller form (its figures: 3.5-4.3x smaller), but the page gives no codec.
The format here is this repository's own (parity unpinned against the pages);
it keeps the part of the idea that pays where the path is bound by HBM: fewer
bytes per cached key. Each row (one token of one KV head, d values x_t, bf16
widened exactly to float32) becomes a float32 scale and d signed 8-bit codes:

    a      = max_t |x_t|
    scale  = fl32(a / 127)                                  (0 when a = 0)
    code_t = clamp(round_half_even(fl32(x_t / scale)), -127, 127)

with both divisions in float32 (IEEE, round to nearest even), so the integer
decision is taken in the precision the kernel takes it. The dequantised value
is code_t * scale, exact in float64. A segment [H_kv][len][d] is stored as one
buffer: the codes [H_kv][len][d] (int8), then the scales [H_kv][len] (float32)
at byte offset H_kv * len * d.

A decode step over quantised segments is the decode step (the newest token's
row over every cached key, TurboRAG summary's generation loop) over the
dequantised cache: ``decode`` builds the dequantised segments in float64 and
runs the fp64 attention oracle on them.
"""
from __future__ import annotations

import numpy as np

CODE_MAX = 127


def _f32(x, dtype: str) -> np.ndarray:
    """Stored inputs widened exactly to float32 (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        return (np.asarray(x).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, dtype=np.float32)


def quantize(x, dtype: str = "bf16"):
    """Rows [..., d] -> (codes int8 [..., d], scales float32 [...])."""
    xf = _f32(x, dtype)
    amax = np.max(np.abs(xf), axis=-1)                         # exact
    scale = (amax / np.float32(CODE_MAX)).astype(np.float32)   # one float32 division
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (xf / safe[..., None]).astype(np.float32)              # float32 division per element
    codes = np.clip(np.rint(q), -CODE_MAX, CODE_MAX)           # rint: ties to even
    codes = np.where(scale[..., None] > 0, codes, 0.0).astype(np.int8)
    return codes, scale


def dequantize(codes, scales) -> np.ndarray:
    """code * scale in float64 (exact: at most 8 + 24 significant bits)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def nbytes(H_kv: int, n: int, d: int) -> int:
    return H_kv * n * d + 4 * H_kv * n


def pack(codes, scales) -> np.ndarray:
    """One segment buffer (uint8): codes [H_kv][len][d], then scales [H_kv][len]."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    return np.concatenate([codes.reshape(-1).view(np.uint8), scales.reshape(-1).view(np.uint8)])


def unpack(buf, H_kv: int, n: int, d: int):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    if buf.size != nbytes(H_kv, n, d):
        raise ValueError("segment buffer holds %d bytes, the format needs %d" % (buf.size, nbytes(H_kv, n, d)))
    codes = buf[: H_kv * n * d].view(np.int8).reshape(H_kv, n, d)
    scales = buf[H_kv * n * d:].view(np.float32).reshape(H_kv, n)
    return codes, scales


def widen_q(Q, dtype: str) -> np.ndarray:
    return _f32(Q, dtype).astype(np.float64)


class DequantProblem:
    """A decode problem whose segments are the dequantised cache (float64)."""

    def __init__(self, problem, kq, vq):
        self.K = [dequantize(c, s) for c, s in kq]
        self.V = [dequantize(c, s) for c, s in vq]
        self.lens = list(problem.lens)
        self.q_len = problem.q_len
        self.m = problem.m
        self.Q = widen_q(problem.Q, "bf16")


def quantize_problem(problem, dtype: str = "bf16"):
    """(codes, scales) for every segment's K and V."""
    kq = [quantize(k, dtype) for k in problem.K]
    vq = [quantize(v, dtype) for v in problem.V]
    return kq, vq


def decode(problem, H: int, H_kv: int, d: int, kq=None, vq=None):
    """out [H][1][d] float64 of the decode step over the quantised cache."""
    import oracle
    if kq is None or vq is None:
        kq, vq = quantize_problem(problem)
    dp = DequantProblem(problem, kq, vq)
    out, _, _ = oracle.attn(dp, H, H_kv, d, "f64", "query")
    return out
