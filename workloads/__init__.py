"""Seeded synthetic inputs for attention over precomputed per-chunk K/V caches.

This module produces input data only. It holds none of the method's
arithmetic (no scores, softmax, impact or selection), so that the fp64 oracle
under ``oracle/`` and the HIP library can both consume it without sharing any
computation.

The pages measure end-to-end serving on public QA sets (NaturalQuestions and
TriviaQA for TurboRAG; PopQA, TriviaQA, MedQA and ASQA for CacheBlend) that
need trained models. Here seeded Gaussian tensors with the shapes of those
workloads stand in for them: 4-document RAG (CacheBlend, "Background"), the
10,000-document-token / 100-query-token example (TurboRAG, "Complexity
analysis"), and recompute ratios r in [0.05, 0.15] (CacheBlend, "Recompute
ratio trade-off").

Layouts (all C-contiguous):

* segment ``c`` of a problem holds ``K[c]`` and ``V[c]`` shaped ``[H_kv][len_c][d]``;
  segments ``0..m-1`` are the document chunks, segment ``m`` is the query
  block's own K/V (TurboRAG eq. for K_combined places K^(Q) last).
* ``Q`` is ``[H][rows][d]``: ``rows = q_len`` in query-row mode, and
  ``rows = N`` (every position, N = sum of lens) in the cross-document and all-rows
  modes.
* bf16 tensors are stored as ``uint16`` bit patterns; fp32 as ``float32``.

Recipe: each problem (a layer, or a request) draws from its own PCG64 stream,
``numpy.random.default_rng(SeedSequence(seed, spawn_key=(p,)))`` with
``seed = 1000 + config index``, so any subset of problems can be regenerated
alone. Within a problem: K then V for each segment in order (documents, then
the query block), then Q, then the K outlier channels. Values are
``standard_normal`` in float32, rounded to bf16 with round-to-nearest-even
where the dtype is bf16. Outlier channels (4 distinct channels per KV head,
scaled by 8) are applied to K of every segment before rounding. Ragged lengths
(the 16-request batch) come from the root stream ``default_rng(seed)`` before
any problem is drawn.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

MODES = ("query", "cross", "all")


@dataclass(frozen=True)
class ConfigSpec:
    """One synthetic workload shape."""

    name: str
    index: int                      # seed = 1000 + index
    n_problems: int                 # layers (one launch) or requests
    H: int
    H_kv: int
    d: int
    dtype: str                      # "f32" or "bf16"
    mode: str                       # "query", "cross" or "all"
    r: float
    chunk_lens: Optional[Sequence[int]] = None   # fixed document chunk lengths
    q_len: Optional[int] = None
    ragged_m: int = 0               # ragged: chunks per request
    ragged_chunk: tuple = (0, 0)    # inclusive bounds of a chunk length
    ragged_q: tuple = (0, 0)        # inclusive bounds of q_len
    k_outliers: int = 0             # outlier channels per KV head in K
    outlier_scale: float = 8.0
    gen_len: int = 0                # earlier generated tokens in the query block's segment
    decode: bool = False            # a decode step (out only, no impact or selection)
    description: str = ""

    @property
    def seed(self) -> int:
        return 1000 + self.index


# The five workloads. Shapes follow the pages' examples: 4-document RAG at
# 2k/8k document tokens (TurboRAG Table 3), the 10,000 + 100 token example
# (TurboRAG, complexity analysis), r in [0.05, 0.15] (CacheBlend Fig. 5).
CONFIGS = {
    "tiny": ConfigSpec(
        name="tiny", index=0, n_problems=1, H=4, H_kv=4, d=64, dtype="f32",
        mode="query", r=0.1, chunk_lens=(64, 64), q_len=16,
        description="1 layer, 4 heads MHA, d=64, fp32; 2 chunks x 64 + 16 query rows"),
    "llama2_7b_layer": ConfigSpec(
        name="llama2_7b_layer", index=1, n_problems=1, H=32, H_kv=32, d=128,
        dtype="bf16", mode="query", r=0.1, chunk_lens=(512,) * 4, q_len=64,
        k_outliers=4,
        description="Llama-2-7B-shaped layer: 32 heads MHA, d=128, bf16; 4 chunks x 512 + 64 query rows"),
    "llama3_8b_gqa_32l": ConfigSpec(
        name="llama3_8b_gqa_32l", index=2, n_problems=32, H=32, H_kv=8, d=128,
        dtype="bf16", mode="query", r=0.15, chunk_lens=(2500,) * 4, q_len=100,
        k_outliers=4,
        description="Llama-3-8B-shaped GQA 32q/8kv heads, d=128, bf16, 32 layers in one launch; "
                    "4 chunks x 2500 (10,000 doc) + 100 query rows"),
    "cross_doc": ConfigSpec(
        name="cross_doc", index=3, n_problems=1, H=32, H_kv=32, d=128,
        dtype="bf16", mode="cross", r=0.05, chunk_lens=(1024,) * 8, q_len=128,
        description="cross-document impact: 32 heads MHA, d=128, bf16; 8 chunks x 1024 + 128 query rows, "
                    "every position is a row"),
    "ragged_70b": ConfigSpec(
        name="ragged_70b", index=4, n_problems=16, H=64, H_kv=8, d=128,
        dtype="bf16", mode="query", r=0.1, ragged_m=4, ragged_chunk=(1024, 4096),
        ragged_q=(32, 256),
        description="ragged batch of 16 requests, 4 chunks U[1024,4096] + q U[32,256]; "
                    "64 query / 8 KV heads, d=128, bf16 (70B-shaped layer)"),
    # A decode step after the 10,000 + 100 prefill (TurboRAG's generation
    # loop): 128 tokens generated so far, the current one is the query row.
    "llama3_8b_decode_32l": ConfigSpec(
        name="llama3_8b_decode_32l", index=5, n_problems=32, H=32, H_kv=8, d=128,
        dtype="bf16", mode="query", r=0.15, chunk_lens=(2500,) * 4, q_len=1, gen_len=227,
        k_outliers=4, decode=True,
        description="decode step of the Llama-3-8B-shaped GQA workload: 32 layers, 4 chunks x 2500 "
                    "+ 100 prompt + 127 generated + the current token (q_len = 1)"),
}
CONFIG_ORDER = ["tiny", "llama2_7b_layer", "llama3_8b_gqa_32l", "cross_doc", "ragged_70b",
                "llama3_8b_decode_32l"]


@dataclass
class Problem:
    """One (layer or request) instance: segment K/V, per-segment lengths, Q."""

    K: List[np.ndarray]
    V: List[np.ndarray]
    lens: List[int]          # m + 1 entries; the last is gen_len + q_len (the query block's segment)
    q_len: int
    Q: np.ndarray

    @property
    def m(self) -> int:
        return len(self.lens) - 1

    @property
    def n_doc(self) -> int:
        return int(sum(self.lens[:-1]))

    @property
    def n_keys(self) -> int:
        return int(sum(self.lens))


@dataclass
class Workload:
    spec: Optional[ConfigSpec]
    H: int
    H_kv: int
    d: int
    dtype: str
    mode: str
    r: float
    problems: List[Problem] = field(default_factory=list)
    problem_ids: List[int] = field(default_factory=list)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored inputs to float64 (bf16 bits or float32)."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def ragged_shapes(spec: ConfigSpec):
    """(chunk lengths per problem, q_len per problem) for a config."""
    if spec.ragged_m:
        root = np.random.default_rng(spec.seed)
        lo, hi = spec.ragged_chunk
        qlo, qhi = spec.ragged_q
        lens = root.integers(lo, hi, size=(spec.n_problems, spec.ragged_m), endpoint=True)
        qs = root.integers(qlo, qhi, size=spec.n_problems, endpoint=True)
        return [list(map(int, row)) for row in lens], [int(q) for q in qs]
    return [list(spec.chunk_lens)] * spec.n_problems, [spec.q_len] * spec.n_problems


def make_problem(rng: np.random.Generator, doc_lens: Sequence[int], q_len: int, H: int,
                 H_kv: int, d: int, dtype: str, mode: str, k_outliers: int = 0,
                 outlier_scale: float = 8.0, gen_len: int = 0) -> Problem:
    """gen_len earlier generated tokens precede the q_len query rows in the
    last segment (a decode step: q_len = 1)."""
    lens = [int(x) for x in doc_lens] + [int(gen_len) + int(q_len)]
    K32, V32 = [], []
    for n in lens:
        K32.append(rng.standard_normal((H_kv, n, d), dtype=np.float32))
        V32.append(rng.standard_normal((H_kv, n, d), dtype=np.float32))
    rows = q_len if mode == "query" else sum(lens)
    Q32 = rng.standard_normal((H, rows, d), dtype=np.float32)
    if k_outliers:
        for h in range(H_kv):
            ch = rng.choice(d, size=k_outliers, replace=False)
            for k in K32:
                k[h][:, ch] *= np.float32(outlier_scale)
    return Problem(K=[_store(k, dtype) for k in K32], V=[_store(v, dtype) for v in V32],
                   lens=lens, q_len=int(q_len), Q=_store(Q32, dtype))


def generate(name: str, problems: Optional[Sequence[int]] = None,
             k_outliers: Optional[int] = None) -> Workload:
    """Build the named workload (all problems, or the listed problem indices).

    ``k_outliers`` overrides the spec (0 gives iid N(0,1) K everywhere).
    """
    spec = CONFIGS[name]
    doc_lens, q_lens = ragged_shapes(spec)
    ids = list(range(spec.n_problems)) if problems is None else [int(p) for p in problems]
    ko = spec.k_outliers if k_outliers is None else k_outliers
    wl = Workload(spec=spec, H=spec.H, H_kv=spec.H_kv, d=spec.d, dtype=spec.dtype,
                  mode=spec.mode, r=spec.r)
    for p in ids:
        rng = np.random.default_rng(np.random.SeedSequence(spec.seed, spawn_key=(p,)))
        wl.problems.append(make_problem(rng, doc_lens[p], q_lens[p], spec.H, spec.H_kv, spec.d,
                                        spec.dtype, spec.mode, ko, spec.outlier_scale,
                                        gen_len=spec.gen_len))
        wl.problem_ids.append(p)
    return wl


def custom(seed: int, doc_lens: Sequence[int], q_len: int, H: int, H_kv: int, d: int,
           dtype: str = "f32", mode: str = "query", r: float = 0.1, n_problems: int = 1,
           k_outliers: int = 0, gen_len: int = 0) -> Workload:
    """A small workload of arbitrary shape, for tests."""
    if mode not in MODES:
        raise ValueError(mode)
    wl = Workload(spec=None, H=H, H_kv=H_kv, d=d, dtype=dtype, mode=mode, r=r)
    for p in range(n_problems):
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(p,)))
        wl.problems.append(make_problem(rng, doc_lens, q_len, H, H_kv, d, dtype, mode, k_outliers,
                                        gen_len=gen_len))
        wl.problem_ids.append(p)
    return wl


def kv_tokens(wl: Workload) -> int:
    """Keys per (layer or request), summed: the unit of the KV tokens/s metric."""
    return int(sum(p.n_keys for p in wl.problems))
