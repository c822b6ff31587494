"""Python binding of the crkv C ABI (``include/crkv.h``).

Argument marshalling only: every step of the attention, impact and top-k path
runs in the HIP kernels of ``libcrkv.so``. torch supplies device memory and
the current stream; nothing here computes. If the library has not been built
the import of a function raises; there is no fallback.

Functions carry the C names:

* ``crkv_attn_chunks(Q, chunk_K, chunk_V, chunk_len, m, q_len, H, H_kv, d, out, impact, ...)``
* ``crkv_attn_chunks_batched(problems, H, H_kv, d, ...)``
* ``crkv_topk(impact, n, k, idx, ...)`` and ``crkv_topk_batched(...)``
* ``crkv_decode_chunks_batched(problems, H, H_kv, d, ...)`` (one decode step)
* ``crkv_quantize_q8(...)``, ``crkv_q8_bytes(...)`` (the 8-bit K/V segment format;
  ``crkv_decode_chunks_batched(..., dtype=CRKV_KV_Q8)`` reads it)
* ``crkv_budget(n_doc, r)``, ``crkv_workspace_size(...)``, ``crkv_plan_info(...)``,
  ``crkv_version()``
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcrkv.so")

CRKV_OK = 0
CRKV_E_INVAL = -1
CRKV_E_UNSUPPORTED = -2
CRKV_E_HIP = -3
CRKV_E_NOMEM = -4
CRKV_F32 = 0
CRKV_BF16 = 1
CRKV_KV_Q8 = 2
MODES = {"query": 0, "cross": 1, "all": 2}


class CrkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("crkv status %d: %s" % (status, message))
        self.status = status


class crkv_opts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("mode", ctypes.c_int), ("stream", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("timing_events", ctypes.c_void_p * 2), ("deterministic", ctypes.c_int)]


class crkv_problem(ctypes.Structure):
    _fields_ = [("Q", ctypes.c_void_p), ("chunk_K", ctypes.POINTER(ctypes.c_void_p)),
                ("chunk_V", ctypes.POINTER(ctypes.c_void_p)),
                ("chunk_len", ctypes.POINTER(ctypes.c_int32)), ("m", ctypes.c_int),
                ("q_len", ctypes.c_int), ("out", ctypes.c_void_p), ("impact", ctypes.c_void_p)]


class crkv_kv_select(ctypes.Structure):
    _fields_ = [("chunk_K", ctypes.POINTER(ctypes.c_void_p)), ("chunk_V", ctypes.POINTER(ctypes.c_void_p)),
                ("chunk_len", ctypes.POINTER(ctypes.c_int32)), ("m", ctypes.c_int),
                ("idx", ctypes.c_void_p), ("k", ctypes.c_int), ("K_sel", ctypes.c_void_p),
                ("V_sel", ctypes.c_void_p)]


class crkv_rope_seg(ctypes.Structure):
    _fields_ = [("K", ctypes.c_void_p), ("len", ctypes.c_int), ("delta", ctypes.c_int)]


CRKV_Q8_K = 0
CRKV_Q8_V = 1


class crkv_q8_seg(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("q8", ctypes.c_void_p), ("len", ctypes.c_int), ("kind", ctypes.c_int)]


class crkv_plan_stat(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("row_tiles", ctypes.c_int), ("workgroups", ctypes.c_int),
                ("pass1_separate", ctypes.c_int), ("split_blocks", ctypes.c_int), ("max_ranges", ctypes.c_int),
                ("combine_workgroups", ctypes.c_int), ("pad", ctypes.c_int), ("model_cycles", ctypes.c_double),
                ("work_cycles", ctypes.c_double), ("scratch_bytes", ctypes.c_size_t)]


_lib = None

DECLARED = ["crkv_plan_create", "crkv_plan_launch", "crkv_plan_destroy", "crkv_q8_bytes", "crkv_quantize_q8", "crkv_opts_init", "crkv_attn_chunks", "crkv_topk", "crkv_attn_chunks_batched",
            "crkv_attn_chunks_batched_static", "crkv_static_scratch_bytes",
            "crkv_topk_batched", "crkv_budget", "crkv_workspace_size", "crkv_plan_info", "crkv_plan_stats",
            "crkv_decode_chunks_batched", "crkv_decode_workspace_size", "crkv_gather_kv",
            "crkv_scatter_kv", "crkv_rope_shift",
            "crkv_status_string", "crkv_last_error", "crkv_version"]


def lib():
    """The loaded libcrkv.so (torch is imported first so that the library
    binds to the same HIP runtime as torch's tensors and streams)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcrkv.so is not built: run `python -m attention_precomputed_chunk_amd.build`")
        try:
            import torch  # noqa: F401  (shares its HIP runtime with the library)
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, c_int = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
        L.crkv_opts_init.argtypes = [ctypes.POINTER(crkv_opts)]
        L.crkv_opts_init.restype = None
        L.crkv_attn_chunks.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(i32),
                                       c_int, c_int, c_int, c_int, c_int, vp, vp,
                                       ctypes.POINTER(crkv_opts)]
        L.crkv_attn_chunks.restype = c_int
        L.crkv_attn_chunks_batched.argtypes = [ctypes.POINTER(crkv_problem), c_int, c_int, c_int, c_int,
                                               ctypes.POINTER(crkv_opts)]
        L.crkv_attn_chunks_batched.restype = c_int
        L.crkv_attn_chunks_batched_static.argtypes = [ctypes.POINTER(crkv_problem), c_int, c_int, c_int, c_int,
                                                      ctypes.POINTER(crkv_opts)]
        L.crkv_attn_chunks_batched_static.restype = c_int
        L.crkv_static_scratch_bytes.argtypes = []
        L.crkv_static_scratch_bytes.restype = ctypes.c_size_t
        L.crkv_topk.argtypes = [vp, c_int, c_int, vp, ctypes.POINTER(crkv_opts)]
        L.crkv_topk.restype = c_int
        L.crkv_topk_batched.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i32), ctypes.POINTER(i32),
                                        ctypes.POINTER(vp), c_int, ctypes.POINTER(crkv_opts)]
        L.crkv_topk_batched.restype = c_int
        L.crkv_budget.argtypes = [ctypes.c_int64, ctypes.c_double]
        L.crkv_budget.restype = ctypes.c_int64
        L.crkv_workspace_size.argtypes = [ctypes.POINTER(crkv_problem), c_int, c_int, c_int, c_int,
                                          ctypes.POINTER(crkv_opts)]
        L.crkv_workspace_size.restype = ctypes.c_size_t
        L.crkv_plan_info.argtypes = [ctypes.POINTER(crkv_problem), c_int, c_int, c_int, c_int,
                                     ctypes.POINTER(crkv_opts), ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                     ctypes.POINTER(c_int)]
        L.crkv_plan_info.restype = c_int
        L.crkv_plan_stats.argtypes = [ctypes.POINTER(crkv_problem), c_int, c_int, c_int, c_int,
                                      ctypes.POINTER(crkv_opts), ctypes.POINTER(crkv_plan_stat)]
        L.crkv_plan_stats.restype = c_int
        L.crkv_decode_chunks_batched.argtypes = [ctypes.POINTER(crkv_problem), c_int, c_int, c_int, c_int,
                                                 ctypes.POINTER(crkv_opts)]
        L.crkv_decode_chunks_batched.restype = c_int
        L.crkv_decode_workspace_size.argtypes = [ctypes.POINTER(crkv_problem), c_int, c_int, c_int, c_int,
                                                 ctypes.POINTER(crkv_opts)]
        L.crkv_decode_workspace_size.restype = ctypes.c_size_t
        for name in ("crkv_gather_kv", "crkv_scatter_kv"):
            f = getattr(L, name)
            f.argtypes = [ctypes.POINTER(crkv_kv_select), c_int, c_int, c_int, ctypes.POINTER(crkv_opts)]
            f.restype = c_int
        L.crkv_rope_shift.argtypes = [ctypes.POINTER(crkv_rope_seg), c_int, c_int, c_int, ctypes.c_double,
                                      ctypes.POINTER(crkv_opts)]
        L.crkv_rope_shift.restype = c_int
        L.crkv_plan_create.argtypes = [ctypes.POINTER(crkv_problem), c_int, c_int, c_int, c_int,
                                       ctypes.POINTER(i32), ctypes.POINTER(vp), ctypes.POINTER(crkv_opts),
                                       ctypes.POINTER(vp)]
        L.crkv_plan_create.restype = c_int
        L.crkv_plan_launch.argtypes = [vp, vp, ctypes.POINTER(vp)]
        L.crkv_plan_launch.restype = c_int
        L.crkv_plan_destroy.argtypes = [vp]
        L.crkv_plan_destroy.restype = c_int
        L.crkv_q8_bytes.argtypes = [c_int, c_int, c_int, c_int]
        L.crkv_q8_bytes.restype = ctypes.c_size_t
        L.crkv_quantize_q8.argtypes = [ctypes.POINTER(crkv_q8_seg), c_int, c_int, c_int, ctypes.POINTER(crkv_opts)]
        L.crkv_quantize_q8.restype = c_int
        L.crkv_status_string.argtypes = [c_int]
        L.crkv_status_string.restype = ctypes.c_char_p
        L.crkv_last_error.argtypes = []
        L.crkv_last_error.restype = ctypes.c_char_p
        L.crkv_version.argtypes = []
        L.crkv_version.restype = c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != CRKV_OK:
        raise CrkvError(status, lib().crkv_last_error().decode(errors="replace"))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CRKV_BF16
    if t.dtype == torch.float32:
        return CRKV_F32
    raise TypeError("Q must be bfloat16 or float32, got %s" % t.dtype)


def make_opts(dtype: int = CRKV_F32, mode: str = "query", stream=None, workspace=None,
              workspace_bytes: int = 0, timing_events=None) -> crkv_opts:
    o = crkv_opts()
    lib().crkv_opts_init(ctypes.byref(o))
    o.dtype = dtype
    o.mode = MODES[mode] if isinstance(mode, str) else int(mode)
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    o.stream = stream or None
    o.workspace = _ptr(workspace)
    o.workspace_bytes = int(workspace_bytes)
    if timing_events is not None:
        o.timing_events[0] = timing_events[0]
        o.timing_events[1] = timing_events[1]
    return o


class _Problem:
    """Keeps the ctypes arrays of one crkv_problem alive."""

    def __init__(self, Q, chunk_K, chunk_V, chunk_len, q_len, out, impact):
        m = len(chunk_len) - 1
        if len(chunk_K) != m + 1 or len(chunk_V) != m + 1:
            raise ValueError("chunk_K, chunk_V and chunk_len need m + 1 entries")
        self.k = (ctypes.c_void_p * (m + 1))(*[_ptr(x) for x in chunk_K])
        self.v = (ctypes.c_void_p * (m + 1))(*[_ptr(x) for x in chunk_V])
        self.lens = (ctypes.c_int32 * (m + 1))(*[int(x) for x in chunk_len])
        self.c = crkv_problem(_ptr(Q), self.k, self.v, self.lens, m, int(q_len), _ptr(out), _ptr(impact))


def crkv_attn_chunks(Q, chunk_K: Sequence, chunk_V: Sequence, chunk_len: Sequence[int], m: int,
                     q_len: int, H: int, H_kv: int, d: int, out, impact, mode: str = "query",
                     stream=None, workspace=None, workspace_bytes: int = 0, timing_events=None,
                     dtype: Optional[int] = None):
    p = _Problem(Q, chunk_K, chunk_V, chunk_len, q_len, out, impact)
    if p.c.m != m:
        raise ValueError("m = %d but chunk_len has %d entries" % (m, len(chunk_len)))
    o = make_opts(_dtype_code(Q) if dtype is None else dtype, mode, stream, workspace,
                  workspace_bytes, timing_events)
    _check(lib().crkv_attn_chunks(p.c.Q, p.k, p.v, p.lens, m, int(q_len), H, H_kv, d,
                                  p.c.out, p.c.impact, ctypes.byref(o)))


def _problems(problems):
    if isinstance(problems, Batch):
        return problems.keep, problems.arr
    ps = [_Problem(pr["Q"], pr["chunk_K"], pr["chunk_V"], pr["chunk_len"], pr["q_len"], pr["out"],
                   pr.get("impact")) for pr in problems]
    arr = (crkv_problem * len(ps))(*[p.c for p in ps])
    return ps, arr


class Batch:
    """Problems marshalled once into their C structures, for repeated calls on
    the same tensors (a decode loop, a benchmark): every batched function takes
    a Batch in place of the list of dicts."""

    def __init__(self, problems: Sequence[dict]):
        self.keep, self.arr = _problems(problems)
        self.dtype = _dtype_code(problems[0]["Q"])

    def __len__(self):
        return len(self.keep)


def _batch_dtype(problems):
    return problems.dtype if isinstance(problems, Batch) else _dtype_code(problems[0]["Q"])


def crkv_attn_chunks_batched(problems: Sequence[dict], H: int, H_kv: int, d: int,
                             mode: str = "query", stream=None, workspace=None,
                             workspace_bytes: int = 0, timing_events=None,
                             dtype: Optional[int] = None):
    """problems: dicts with keys Q, chunk_K, chunk_V, chunk_len, q_len, out, impact
    (or a Batch of them)."""
    keep, arr = _problems(problems)
    o = make_opts(_batch_dtype(problems) if dtype is None else dtype, mode, stream,
                  workspace, workspace_bytes, timing_events)
    _check(lib().crkv_attn_chunks_batched(arr, len(keep), H, H_kv, d, ctypes.byref(o)))


def crkv_attn_chunks_batched_static(problems: Sequence[dict], H: int, H_kv: int, d: int,
                                    mode: str = "query", stream=None, timing_events=None,
                                    dtype: Optional[int] = None):
    """crkv_attn_chunks_batched with the library's static device scratch (no
    device allocation; for callers that cannot allocate)."""
    keep, arr = _problems(problems)
    o = make_opts(_batch_dtype(problems) if dtype is None else dtype, mode, stream, None, 0, timing_events)
    _check(lib().crkv_attn_chunks_batched_static(arr, len(keep), H, H_kv, d, ctypes.byref(o)))


def crkv_static_scratch_bytes() -> int:
    return int(lib().crkv_static_scratch_bytes())


class Plan:
    """A batched attention (+ top-k) call planned once (crkv_plan_create):
    launch() only enqueues kernels, so it can be captured into a graph.
    problems as for crkv_attn_chunks_batched; ks / idxs: per-problem top-k
    budgets (0 = none) and int32 device tensors, or None for no selection."""

    def __init__(self, problems: Sequence[dict], H: int, H_kv: int, d: int, ks: Optional[Sequence[int]] = None,
                 idxs: Optional[Sequence] = None, mode: str = "query", dtype: Optional[int] = None,
                 workspace=None, workspace_bytes: int = 0):
        self._keep, self._arr = _problems(problems)
        n = len(self._keep)
        o = make_opts(_batch_dtype(problems) if dtype is None else dtype, mode, stream=0, workspace=workspace,
                      workspace_bytes=workspace_bytes)
        self._workspace = workspace   # must outlive the plan
        self._k = self._idx = None
        if ks is not None:
            self._k = (ctypes.c_int32 * n)(*[int(k) for k in ks])
            self._idx = (ctypes.c_void_p * n)(*[_ptr(x) for x in idxs])
        h = ctypes.c_void_p()
        _check(lib().crkv_plan_create(self._arr, n, H, H_kv, d, self._k, self._idx, ctypes.byref(o),
                                      ctypes.byref(h)))
        self.handle = h.value

    def launch(self, stream=None, timing_events=None):
        if not self.handle:
            raise ValueError("plan destroyed")
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        elif hasattr(stream, "cuda_stream"):
            stream = stream.cuda_stream
        ev = None
        if timing_events is not None:
            ev = (ctypes.c_void_p * 2)(timing_events[0], timing_events[1])
        _check(lib().crkv_plan_launch(self.handle, stream or None, ev))

    def destroy(self):
        if self.handle:
            h, self.handle = self.handle, None
            _check(lib().crkv_plan_destroy(h))

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def crkv_workspace_size(problems: Sequence[dict], H: int, H_kv: int, d: int, mode: str = "query",
                        dtype: Optional[int] = None) -> int:
    keep, arr = _problems(problems)
    o = make_opts(_batch_dtype(problems) if dtype is None else dtype, mode, stream=0)
    return int(lib().crkv_workspace_size(arr, len(keep), H, H_kv, d, ctypes.byref(o)))


def crkv_decode_chunks_batched(problems: Sequence[dict], H: int, H_kv: int, d: int, stream=None,
                               workspace=None, workspace_bytes: int = 0, timing_events=None,
                               dtype: int = CRKV_BF16):
    """One decode step (q_len = 1 per problem); dicts as for crkv_attn_chunks_batched,
    'impact' may be None. dtype=CRKV_KV_Q8: chunk_K / chunk_V are segment
    buffers in the 8-bit format (crkv_quantize_q8)."""
    keep, arr = _problems(problems)
    o = make_opts(dtype, "query", stream, workspace, workspace_bytes, timing_events)
    _check(lib().crkv_decode_chunks_batched(arr, len(keep), H, H_kv, d, ctypes.byref(o)))


def crkv_decode_workspace_size(problems: Sequence[dict], H: int, H_kv: int, d: int,
                               dtype: int = CRKV_BF16) -> int:
    keep, arr = _problems(problems)
    o = make_opts(dtype, "query", stream=0)
    return int(lib().crkv_decode_workspace_size(arr, len(keep), H, H_kv, d, ctypes.byref(o)))


PLAN_KERNELS = {0: "f32", 1: "bf16_wave", 2: "bf16_pair"}


def crkv_plan_info(problems: Sequence[dict], H: int, H_kv: int, d: int, mode: str = "query",
                   dtype: Optional[int] = None) -> dict:
    """Launch configuration the planner picks: kernel name, row tiles, workgroups."""
    keep, arr = _problems(problems)
    o = make_opts(_batch_dtype(problems) if dtype is None else dtype, mode, stream=0)
    k, rt, wg = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().crkv_plan_info(arr, len(keep), H, H_kv, d, ctypes.byref(o), ctypes.byref(k),
                                ctypes.byref(rt), ctypes.byref(wg)))
    return {"kernel": PLAN_KERNELS[k.value], "row_tiles": rt.value, "workgroups": wg.value}


def crkv_plan_stats(problems: Sequence[dict], H: int, H_kv: int, d: int, mode: str = "query",
                    dtype: Optional[int] = None) -> dict:
    """The planner's plan in detail: kernel, row tiles, workgroups, whether
    pass 1 runs on its own, blocks split into key ranges (and the most ranges
    of one block), combine workgroups, the modelled duration and work (shader
    cycles; imbalance = duration * 256 / work - 1), and the scratch size."""
    keep, arr = _problems(problems)
    o = make_opts(_batch_dtype(problems) if dtype is None else dtype, mode, stream=0)
    st = crkv_plan_stat()
    _check(lib().crkv_plan_stats(arr, len(keep), H, H_kv, d, ctypes.byref(o), ctypes.byref(st)))
    out = {f: getattr(st, f) for f, _ in crkv_plan_stat._fields_ if f != "pad"}
    out["kernel"] = PLAN_KERNELS[st.kernel]
    out["imbalance"] = st.model_cycles * 256 / st.work_cycles - 1 if st.work_cycles else 0.0
    return out


def crkv_topk(impact, n: int, k: int, idx, stream=None):
    o = make_opts(stream=stream)
    _check(lib().crkv_topk(_ptr(impact), int(n), int(k), _ptr(idx), ctypes.byref(o)))


def crkv_topk_batched(impacts: Sequence, ns: Sequence[int], ks: Sequence[int], idxs: Sequence,
                      stream=None):
    P = len(impacts)
    ip = (ctypes.c_void_p * P)(*[_ptr(x) for x in impacts])
    nn = (ctypes.c_int32 * P)(*[int(x) for x in ns])
    kk = (ctypes.c_int32 * P)(*[int(x) for x in ks])
    xp = (ctypes.c_void_p * P)(*[_ptr(x) for x in idxs])
    o = make_opts(stream=stream)
    _check(lib().crkv_topk_batched(ip, nn, kk, xp, P, ctypes.byref(o)))


class _Select:
    """Keeps the ctypes arrays of one crkv_kv_select alive."""

    def __init__(self, sel: dict):
        lens = sel["chunk_len"]
        m = len(lens) - 1
        if len(sel["chunk_K"]) != m + 1 or len(sel["chunk_V"]) != m + 1:
            raise ValueError("chunk_K, chunk_V and chunk_len need m + 1 entries")
        self.k = (ctypes.c_void_p * (m + 1))(*[_ptr(x) for x in sel["chunk_K"]])
        self.v = (ctypes.c_void_p * (m + 1))(*[_ptr(x) for x in sel["chunk_V"]])
        self.lens = (ctypes.c_int32 * (m + 1))(*[int(x) for x in lens])
        idx = sel["idx"]
        n_sel = int(sel["k"]) if "k" in sel else (0 if idx is None else int(idx.numel()))
        self.c = crkv_kv_select(self.k, self.v, self.lens, m, _ptr(idx), n_sel, _ptr(sel["K_sel"]),
                                _ptr(sel["V_sel"]))


def _selections(sels):
    if isinstance(sels, SelectBatch):
        return sels.keep, sels.arr
    keep = [_Select(s) for s in sels]
    return keep, (crkv_kv_select * len(keep))(*[s.c for s in keep])


class SelectBatch:
    """Selections marshalled once into their C structures, for repeated
    gather/scatter calls on the same tensors: both functions take a
    SelectBatch in place of the list of dicts."""

    def __init__(self, sels: Sequence[dict]):
        self.keep, self.arr = _selections(list(sels))

    def __len__(self):
        return len(self.keep)


def crkv_gather_kv(sels: Sequence[dict], H_kv: int, d: int, dtype: int, stream=None, timing_events=None):
    """Gather the selected keys' K/V rows into packed buffers. Each dict:
    chunk_K, chunk_V (m + 1 tensors or None), chunk_len, idx (int32 device
    tensor), K_sel, V_sel ([H_kv][k][d]); optional k (default idx.numel())."""
    keep, arr = _selections(sels)
    o = make_opts(dtype, "query", stream, timing_events=timing_events)
    _check(lib().crkv_gather_kv(arr, len(keep), H_kv, d, ctypes.byref(o)))


def crkv_scatter_kv(sels: Sequence[dict], H_kv: int, d: int, dtype: int, stream=None, timing_events=None):
    """Write packed K/V rows back to the selected positions of the segments."""
    keep, arr = _selections(sels)
    o = make_opts(dtype, "query", stream, timing_events=timing_events)
    _check(lib().crkv_scatter_kv(arr, len(keep), H_kv, d, ctypes.byref(o)))


class RopeBatch:
    """Segments marshalled once for repeated crkv_rope_shift calls."""

    def __init__(self, segs: Sequence[tuple]):
        self.n = len(segs)
        self.arr = (crkv_rope_seg * self.n)(*[crkv_rope_seg(_ptr(k), int(n), int(dl)) for k, n, dl in segs])


def crkv_rope_shift(segs, H_kv: int, d: int, dtype: int, base: float = 10000.0,
                    stream=None, timing_events=None):
    """Rotate cached keys in place to new positions: segs is a list of
    (K tensor [H_kv][len][d], len, delta), or a RopeBatch."""
    b = segs if isinstance(segs, RopeBatch) else RopeBatch(segs)
    o = make_opts(dtype, "query", stream, timing_events=timing_events)
    _check(lib().crkv_rope_shift(b.arr, b.n, H_kv, d, float(base), ctypes.byref(o)))


def crkv_q8_bytes(H_kv: int, n: int, d: int, kind: int) -> int:
    """Bytes of one segment of n keys in the 8-bit format (kind CRKV_Q8_K or CRKV_Q8_V)."""
    return int(lib().crkv_q8_bytes(H_kv, n, d, kind))


class Q8Batch:
    """Segments marshalled once for repeated crkv_quantize_q8 calls."""

    def __init__(self, segs: Sequence[tuple]):
        self.n = len(segs)
        self.arr = (crkv_q8_seg * self.n)(*[crkv_q8_seg(_ptr(x), _ptr(q), int(n), int(k))
                                            for x, q, n, k in segs])


def crkv_quantize_q8(segs, H_kv: int, d: int, stream=None, timing_events=None):
    """Quantise bf16 segments into the 8-bit format: segs is a list of
    (x bf16 tensor [H_kv][len][d], q8 uint8 tensor of crkv_q8_bytes bytes, len,
    kind CRKV_Q8_K or CRKV_Q8_V), or a Q8Batch."""
    b = segs if isinstance(segs, Q8Batch) else Q8Batch(segs)
    o = make_opts(CRKV_BF16, "query", stream, timing_events=timing_events)
    _check(lib().crkv_quantize_q8(b.arr, b.n, H_kv, d, ctypes.byref(o)))


def crkv_budget(n_doc: int, r: float) -> int:
    return int(lib().crkv_budget(int(n_doc), float(r)))


def crkv_version() -> int:
    return int(lib().crkv_version())
