"""fp64 CPU oracle for attention over precomputed per-chunk K/V caches.

TEST INFRASTRUCTURE ONLY: the tests, the package entry point's smoke check and
the benchmark's CPU-baseline leg may use it; the library never does. The
arithmetic lives in ``oracle.c`` (plain C, float64 loops). This module only
builds that file with gcc and marshals arguments through ctypes; it shares no
code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

MODE_CODE = {"query": 0, "cross": 1, "all": 2}
DTYPE_CODE = {"f32": 0, "bf16": 1, "f64": 2}


def _stale() -> bool:
    return not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP, -O2); without
    ``force``, only when the library is missing or older than the source."""
    if force or _stale():
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _stale():
            build()
        lib = ctypes.CDLL(_LIB)
        vp = ctypes.c_void_p
        lib.oracle_attn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                    ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, vp, vp, vp, ctypes.c_int]
        lib.oracle_attn.restype = ctypes.c_int
        lib.oracle_budget.argtypes = [ctypes.c_long, ctypes.c_double]
        lib.oracle_budget.restype = ctypes.c_long
        lib.oracle_topk.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
        lib.oracle_topk.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def attn(problem, H: int, H_kv: int, d: int, dtype: str, mode: str, causal: bool = True,
         row_lo: int = 0, row_hi: int = 0, want_lse: bool = False, n_threads: int = 0):
    """Run the oracle on one ``workloads.Problem``.

    Returns ``(out, impact, lse)``: out ``[H][rows][d]`` float64, impact ``[N]``
    float64, lse ``[H][rows]`` float64 or None.
    """
    lib = _load()
    m = problem.m
    Ks = [np.ascontiguousarray(k) for k in problem.K]
    Vs = [np.ascontiguousarray(v) for v in problem.V]
    Q = np.ascontiguousarray(problem.Q)
    lens = np.asarray(problem.lens, dtype=np.int32)
    N = int(lens.sum())
    rows = problem.q_len if mode == "query" else N
    kp = (ctypes.c_void_p * (m + 1))(*[k.ctypes.data for k in Ks])
    vp = (ctypes.c_void_p * (m + 1))(*[v.ctypes.data for v in Vs])
    out = np.zeros((H, rows, d), dtype=np.float64)
    impact = np.zeros(N, dtype=np.float64)
    lse = np.zeros((H, rows), dtype=np.float64) if want_lse else None
    rc = lib.oracle_attn(DTYPE_CODE[dtype], MODE_CODE[mode], int(bool(causal)), Q.ctypes.data,
                         kp, vp, lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), m,
                         problem.q_len, H, H_kv, d, row_lo, row_hi, out.ctypes.data,
                         impact.ctypes.data, lse.ctypes.data if lse is not None else None,
                         n_threads)
    if rc != 0:
        raise ValueError("oracle_attn failed with %d" % rc)
    return out, impact, lse


def budget(n_doc: int, r: float) -> int:
    return int(_load().oracle_budget(int(n_doc), float(r)))


def topk(values, k: int) -> np.ndarray:
    """Top-k of a float32 vector (ties to the lower index), sorted (desc, asc)."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    idx = np.zeros(k, dtype=np.int32)
    rc = _load().oracle_topk(v.ctypes.data, int(v.size), int(k), idx.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_topk failed with %d" % rc)
    return idx


def run_workload(wl, want_lse: bool = False, n_threads: int = 0, problems: Optional[list] = None):
    """Oracle over every problem of a ``workloads.Workload``: list of
    ``(out, impact, lse, k, idx)`` with idx from the fp32-rounded impact."""
    res = []
    for pi, prob in enumerate(wl.problems):
        if problems is not None and pi not in problems:
            res.append(None)
            continue
        out, imp, lse = attn(prob, wl.H, wl.H_kv, wl.d, wl.dtype, wl.mode, want_lse=want_lse,
                             n_threads=n_threads)
        n_doc = prob.n_doc
        k = budget(n_doc, wl.r) if n_doc > 0 else 0
        idx = topk(imp[:n_doc].astype(np.float32), k) if n_doc > 0 else np.zeros(0, np.int32)
        res.append((out, imp, lse, k, idx))
    return res
