"""Oracle for the 8-bit K/V cache format that the decode step can read.

TEST INFRASTRUCTURE ONLY: the tests, the package entry point's smoke check and
the benchmark's CPU-baseline leg may use it; the library never does. It shares
no code with the HIP library.

What it follows: the CacheGen summary observes that loading a precomputed KV
cache dominates the time to first token and that caches can be encoded into a
much smaller form (its figures: 3.5-4.3x smaller), but the page gives no codec.
The format here is this repository's own (parity unpinned against the pages);
it keeps the part of the idea that pays where the path is bound by HBM: fewer
bytes per cached key. Values (bf16 widened exactly to float32) become signed
8-bit codes with float32 scales, one scale per group:

    a      = max over the group of |x|
    scale  = fl32(a / 127)                                  (0 when a = 0)
    code   = clamp(round_half_even(fl32(x / scale)), -127, 127)

with both divisions in float32 (IEEE, round to nearest even), so the integer
decision is taken in the precision the kernel takes it. The dequantised value
is code * scale, exact in float64. The groups differ for K and V:

* K ("k"): one scale per (KV head, channel) over the segment's tokens. Cached
  keys carry a few channels of much larger magnitude (the synthetic workloads
  model them as outlier channels), and a scale per channel keeps them from
  coarsening the other channels' steps.
* V ("v"): one scale per (KV head, token) over the d channels.

A segment [H_kv][len][d] is stored as one buffer: the codes [H_kv][len][d]
(int8), then the scales at byte offset H_kv * len * d, float32 [H_kv][d] for
K or [H_kv][len] for V. A segment with len = 0 occupies no bytes.

A decode step over quantised segments is the decode step (the newest token's
row over every cached key, TurboRAG summary's generation loop) over the
dequantised cache: ``decode`` builds the dequantised segments in float64 and
runs the fp64 attention oracle on them; ``attn`` does the same for the
prefill (query rows, impact and the other modes).
"""
from __future__ import annotations

import numpy as np

CODE_MAX = 127


def _f32(x, dtype: str) -> np.ndarray:
    """Stored inputs widened exactly to float32 (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        return (np.asarray(x).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, dtype=np.float32)


def _axis(kind: str) -> int:
    if kind not in ("k", "v"):
        raise ValueError(kind)
    return -2 if kind == "k" else -1


def quantize(x, kind: str, dtype: str = "bf16"):
    """[H_kv][len][d] -> (codes int8 [H_kv][len][d], scales float32:
    [H_kv][d] for kind "k" (per channel), [H_kv][len] for "v" (per token))."""
    ax = _axis(kind)
    xf = _f32(x, dtype)
    if xf.shape[-2] == 0:
        sc_shape = xf.shape[:-2] + ((xf.shape[-1],) if kind == "k" else (0,))
        return np.zeros(xf.shape, dtype=np.int8), np.zeros(sc_shape, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=ax)                         # exact
    scale = (amax / np.float32(CODE_MAX)).astype(np.float32)   # one float32 division
    safe = np.expand_dims(np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32), ax)
    q = (xf / safe).astype(np.float32)                         # float32 division per element
    codes = np.clip(np.rint(q), -CODE_MAX, CODE_MAX)           # rint: ties to even
    codes = np.where(np.expand_dims(scale, ax) > 0, codes, 0.0).astype(np.int8)
    return codes, scale


def dequantize(codes, scales, kind: str) -> np.ndarray:
    """code * scale in float64 (exact: at most 8 + 24 significant bits)."""
    return np.asarray(codes, dtype=np.float64) * np.expand_dims(np.asarray(scales, dtype=np.float64), _axis(kind))


def nbytes(H_kv: int, n: int, d: int, kind: str) -> int:
    if n == 0:
        return 0
    return H_kv * n * d + 4 * H_kv * (d if kind == "k" else n)


def pack(codes, scales) -> np.ndarray:
    """One segment buffer (uint8): the codes, then the scales."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    if codes.size == 0:
        return np.zeros(0, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    return np.concatenate([codes.reshape(-1).view(np.uint8), scales.reshape(-1).view(np.uint8)])


def unpack(buf, H_kv: int, n: int, d: int, kind: str):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    if buf.size != nbytes(H_kv, n, d, kind):
        raise ValueError("segment buffer holds %d bytes, the format needs %d" % (buf.size, nbytes(H_kv, n, d, kind)))
    if n == 0:
        return quantize(np.zeros((H_kv, 0, d), dtype=np.float32), kind, "f32")
    codes = buf[: H_kv * n * d].view(np.int8).reshape(H_kv, n, d)
    scales = buf[H_kv * n * d:].view(np.float32).reshape(H_kv, d if kind == "k" else n)
    return codes, scales


def widen_q(Q, dtype: str) -> np.ndarray:
    return _f32(Q, dtype).astype(np.float64)


class DequantProblem:
    """A decode problem whose segments are the dequantised cache (float64)."""

    def __init__(self, problem, kq, vq):
        self.K = [dequantize(c, s, "k") for c, s in kq]
        self.V = [dequantize(c, s, "v") for c, s in vq]
        self.lens = list(problem.lens)
        self.q_len = problem.q_len
        self.m = problem.m
        self.Q = widen_q(problem.Q, "bf16")


def quantize_problem(problem, dtype: str = "bf16"):
    """(codes, scales) for every segment's K and V."""
    kq = [quantize(k, "k", dtype) for k in problem.K]
    vq = [quantize(v, "v", dtype) for v in problem.V]
    return kq, vq


def attn(problem, H: int, H_kv: int, d: int, mode: str, kq=None, vq=None):
    """(out, impact, lse=None) of the attention in any mode (query rows,
    cross-document, all rows) over the quantised cache: the fp64 attention
    oracle on the dequantised segments, Q widened exactly from bf16."""
    import oracle
    if kq is None or vq is None:
        kq, vq = quantize_problem(problem)
    dp = DequantProblem(problem, kq, vq)
    return oracle.attn(dp, H, H_kv, d, "f64", mode)


def decode(problem, H: int, H_kv: int, d: int, kq=None, vq=None):
    """out [H][1][d] float64 of the decode step over the quantised cache."""
    import oracle
    if kq is None or vq is None:
        kq, vq = quantize_problem(problem)
    dp = DequantProblem(problem, kq, vq)
    out, _, _ = oracle.attn(dp, H, H_kv, d, "f64", "query")
    return out
