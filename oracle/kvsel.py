"""Oracle for moving the K/V rows of selected keys between the segment table
and packed buffers.

TEST INFRASTRUCTURE ONLY: the tests, the package entry point's smoke check and
the benchmark's CPU-baseline leg may use it; the library never does. It shares
no code with the HIP library.

What it follows (CacheBlend summary, the three-phase flowchart of how the
method works: after the high-impact tokens are identified, the K/V values of
exactly those tokens are recomputed, and generation then runs on the fused
cache). The recompute itself needs model weights and is not part of this
code; the data movement around it is:

  gather:  K_sel[h][j] = K_cat[h][idx[j]],  V_sel likewise,
  scatter: K_cat[h][idx[j]] = K_sel[h][j],  V_cat likewise,

where K_cat = Concat(K^(0), ..., K^(m)) along the sequence axis (TurboRAG
summary, "Precomputing the KV cache"), never formed here: an index is mapped
to (segment, offset) by walking the segment lengths in order. Readings taken
where the pages say nothing: indices are positions in the concatenation, so
the top-k indices over the document keys are used as they are; an index
outside [0, N) gathers a zero row and scatters nothing; rows are copied as
stored (bf16 bit patterns or float32), bit for bit.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def locate(lens: Sequence[int], i: int) -> Tuple[int, int]:
    """(segment, offset) of concatenated key i, or (-1, -1) outside [0, N)."""
    if i < 0:
        return -1, -1
    start = 0
    for c, n in enumerate(lens):
        if i < start + n:
            return c, i - start
        start += n
    return -1, -1


def gather_kv(K: List[np.ndarray], V: List[np.ndarray], lens: Sequence[int],
              idx: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Packed ``[H_kv][k][d]`` copies of the selected keys' K and V rows."""
    H_kv, _, d = K[0].shape
    k = len(idx)
    Ks = np.zeros((H_kv, k, d), dtype=K[0].dtype)
    Vs = np.zeros((H_kv, k, d), dtype=V[0].dtype)
    for j, i in enumerate(idx):
        c, off = locate(lens, int(i))
        if c < 0:
            continue
        Ks[:, j, :] = K[c][:, off, :]
        Vs[:, j, :] = V[c][:, off, :]
    return Ks, Vs


def scatter_kv(K: List[np.ndarray], V: List[np.ndarray], lens: Sequence[int],
               idx: Sequence[int], K_sel: np.ndarray, V_sel: np.ndarray) -> None:
    """Write the packed rows back into the segments in place (distinct
    indices; indices outside [0, N) are skipped)."""
    for j, i in enumerate(idx):
        c, off = locate(lens, int(i))
        if c < 0:
            continue
        K[c][:, off, :] = K_sel[:, j, :]
        V[c][:, off, :] = V_sel[:, j, :]
