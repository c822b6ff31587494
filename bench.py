"""Benchmark: KV tokens/s through attention + impact + top-k on one MI355X.

One step = one batched attention call over every problem of the workload
(per-layer or per-request segment tables, impact combine included) plus one
batched top-k call. Inputs are resident in HBM before timing starts.

Default workload: the Llama-3-8B-shaped GQA configuration (32 query / 8 KV
heads, d=128, bf16, 32 layers in one launch, 4 chunks x 2500 = 10,000
document tokens + 100 query tokens, r = 0.15), the shape of TurboRAG's
10,000 + 100 token example.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

(defaults: 100 timed steps after 10 warm-up steps)

With --config llama3_8b_decode_32l a step is one decode call (the newest
token of every layer over its 10,000 + 228 keys; out only), timed the same way.

With --config llama3_8b_select_kv_32l a step moves the K/V rows of every
layer's selected keys (the top-1500 of the default workload's impact, found
once before timing): one gather launch into packed buffers and one scatter
launch back into the segments.

With --config llama3_8b_decode_q8_32l a step is the same decode step over the
cache stored in the 8-bit format (codes + one float32 scale per row; the
cache is quantised once before timing, as it is when the chunk caches are
precomputed).

With --config llama3_8b_rope_shift_32l a step moves the cached keys of every
document chunk of the 32 layers from positions 0 .. 2499 to their place in the
concatenation (offsets 2500, 5000, 7500; the first chunk stays): one
rotary re-positioning launch over all of them.

For the attention workloads the line also holds `graph`: the same step
planned once (crkv_plan_create) and replayed from a captured graph, which
removes the per-call host planning and launch gaps (most visible on the
launch-bound tiny and llama2_7b_layer shapes).

Prints one JSON line. The roofline object is for the attention kernel alone,
timed with HIP events recorded on its stream around every launch (mean, and
the median / p10 / p90 over the timed steps).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV tokens/s through attention+impact+top-k; % of HBM / MFMA roofline"
METRIC_DECODE = "KV tokens/s through one decode step; % of HBM roofline"
METRIC_SELECT = "selected token-layers/s through K/V gather + scatter; % of HBM roofline"
SELECT_CONFIGS = {"llama3_8b_select_kv_32l": "llama3_8b_gqa_32l"}
METRIC_ROPE = "re-positioned key-layers/s (rotary shift of cached keys); % of HBM roofline"
ROPE_CONFIGS = {"llama3_8b_rope_shift_32l": "llama3_8b_gqa_32l"}
Q8_CONFIGS = {"llama3_8b_decode_q8_32l": "llama3_8b_decode_32l"}
# the prefill over the same workload's cache stored in the 8-bit format
# (quantised once before timing)
Q8_ATTN_CONFIGS = {"llama3_8b_gqa_32l_q8": "llama3_8b_gqa_32l"}
SMALL_CONFIGS = ("tiny", "llama2_7b_layer")
DEFAULT_CONFIG = "llama3_8b_gqa_32l"
# timed after the headline in the default run and reported under "configs"
OTHER_ATTN_CONFIGS = ("ragged_70b", "cross_doc", "llama2_7b_layer", "tiny")   # single small problems: the oracle is also timed on one core
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(wl):
    """Bytes and FLOPs a perfect kernel must move / do for one launch:
    K and V of every key once (2 * H_kv * d * s per key), Q and out once
    (2 * H * d * s per row), the impact vector once (4 B per key; not in a
    decode step); FLOPs 4 * H * d per visible (row, key) pair (Q.K^T and P.V)."""
    s = 2 if wl.dtype == "bf16" else 4
    decode = bool(wl.spec and wl.spec.decode)
    nbytes = 0
    pairs = 0
    for p in wl.problems:
        N = p.n_keys
        rows = p.q_len if wl.mode == "query" else N
        nbytes += N * 2 * wl.H_kv * wl.d * s + rows * 2 * wl.H * wl.d * s + (0 if decode else N * 4)
        if wl.mode == "query":   # the q_len rows are the last positions
            pairs += p.q_len * (N - p.q_len) + p.q_len * (p.q_len + 1) // 2
        else:
            pairs += N * (N + 1) // 2
    return nbytes, 4 * pairs * wl.H * wl.d, pairs


# Sources each timed kernel is built from; a counter summary stays valid while
# their hash matches.
KERNEL_SOURCES = {
    "attn": ("attn_bf16_wave.hip", "attn_bf16_pair.hip", "attn_lse.hip", "attn_bf16_common.h", "device_util.h",
             "crkv_internal.h", "crkv_api.hip"),
    "decode": ("decode_bf16.hip", "attn_bf16_common.h", "device_util.h", "crkv_internal.h", "crkv_api.hip"),
    "kvsel": ("kvsel.hip", "device_util.h", "crkv_internal.h", "crkv_api.hip"),
    "rope": ("rope.hip", "device_util.h", "crkv_internal.h", "crkv_api.hip"),
    "q8": ("q8.hip", "decode_bf16.hip", "attn_bf16_common.h", "device_util.h", "crkv_internal.h",
           "crkv_api.hip"),
}


def kernel_source_sha(kind="attn"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "attention_precomputed_chunk_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config, kind="attn"):
    """HBM bytes per launch of the timed kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kind, config))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_source_sha(kind):
        return None
    return t.get("bytes_per_launch")


def measured_mfma(config):
    """Executed bf16 MFMA FLOPs, matrix-core busy share and clock of the timed
    attention kernel from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "attn_%s_mfma.json" % config)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_source_sha("attn"):
        return None
    return {k: t[k] for k in ("executed_flops_per_launch", "mfma_busy_pct", "clock_ghz")}


class HipEvents:
    """hipEvent_t pairs from the HIP runtime torch has loaded."""

    def __init__(self):
        import torch
        self.rt = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.rt.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, ev):
        self.rt.hipEventDestroy(ev)


def cpu_baseline(wl, budget_s=15.0):
    """The fp64 oracle as it stands, on the first problems of the same
    workload, using every host core; scaled to KV tokens/s."""
    import oracle
    oracle.build(force=False)
    t0 = time.perf_counter()
    oracle.run_workload(wl, problems=[0])
    t1 = time.perf_counter() - t0
    n = int(max(1, min(len(wl.problems), round(budget_s / max(t1, 1e-3)))))
    if n > 1:
        t0 = time.perf_counter()
        oracle.run_workload(wl, problems=list(range(n)))
        elapsed = time.perf_counter() - t0
    else:
        elapsed = t1
    tokens = sum(p.n_keys for p in wl.problems[:n])
    rec = {"value": tokens / elapsed, "unit": "KV tokens/s", "cores": oracle.max_threads(),
           "kind": "oracle", "sample": "problems 0..%d of %d (%s), %.1f s of CPU time"
           % (n - 1, len(wl.problems), wl.spec.name if wl.spec else "custom", elapsed)}
    if wl.spec and wl.spec.name in SMALL_CONFIGS:
        t0 = time.perf_counter()
        oracle.run_workload(wl, problems=[0], n_threads=1)
        rec["single_thread_value"] = wl.problems[0].n_keys / (time.perf_counter() - t0)
    return rec


def cpu_baseline_q8(wl, budget_s=15.0):
    """The oracle of the 8-bit prefill (quantise, dequantise, fp64 attention)
    on the first layers of the workload, every host core."""
    import oracle
    from oracle import q8
    t0 = time.perf_counter()
    done = 0
    for p in wl.problems:
        q8.attn(p, wl.H, wl.H_kv, wl.d, wl.mode)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": sum(p.n_keys for p in wl.problems[:done]) / el, "unit": "KV tokens/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "layers 0..%d of %d (quantise + dequantise + fp64 attention), %.1f s"
            % (done - 1, len(wl.problems), el)}


def bench_q8_decode(args, torch, crkv, workloads):
    """One decode step over the 8-bit cache (all layers, one launch of the
    split kernel and one of the merge); the roofline is the pair's."""
    from_cfg = Q8_CONFIGS[args.config]
    log("generating %s" % from_cfg)
    wl = workloads.generate(from_cfg)
    dev = "cuda:0"
    up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    problems, segs, keep = [], [], []
    q8_bytes = 0
    for p in wl.problems:
        Q = up(p.Q)
        kq, vq = [], []
        for k, v, n in zip(p.K, p.V, p.lens):
            nk = crkv.crkv_q8_bytes(wl.H_kv, n, wl.d, crkv.CRKV_Q8_K)
            nv = crkv.crkv_q8_bytes(wl.H_kv, n, wl.d, crkv.CRKV_Q8_V)
            q8_bytes += nk + nv
            bk = torch.empty(max(nk, 16), dtype=torch.uint8, device=dev)
            bv = torch.empty(max(nv, 16), dtype=torch.uint8, device=dev)
            kd, vd = up(k), up(v)
            segs += [(kd, bk, n, crkv.CRKV_Q8_K), (vd, bv, n, crkv.CRKV_Q8_V)]
            keep += [kd, vd]
            kq.append(bk)
            vq.append(bv)
        problems.append(dict(Q=Q, chunk_K=kq, chunk_V=vq, chunk_len=list(p.lens), q_len=1,
                             out=torch.empty_like(Q), impact=None))
    qev = HipEvents()
    qa, qb = qev.create(), qev.create()
    qbatch = crkv.Q8Batch(segs)
    crkv.crkv_quantize_q8(qbatch, wl.H_kv, wl.d)   # the stored cache (the first launch also loads the code)
    crkv.crkv_quantize_q8(qbatch, wl.H_kv, wl.d, timing_events=(qa, qb))   # the same again, timed
    torch.cuda.synchronize()
    q_ms = qev.elapsed_ms(qa, qb)
    del segs, keep, qbatch
    torch.cuda.empty_cache()
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    batch = crkv.Batch(problems)

    def step(events=None):
        crkv.crkv_decode_chunks_batched(batch, wl.H, wl.H_kv, wl.d, timing_events=events,
                                        dtype=crkv.CRKV_KV_Q8)

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(pairs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs]))
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    tokens = workloads.kv_tokens(wl)
    # algorithmic bytes: every key's K and V codes and scales once, Q and out (bf16)
    nbytes = q8_bytes + sum(2 * wl.H * wl.d * 2 for _ in wl.problems)
    achieved = nbytes / (k_ms * 1e-3) / 1e9
    spec = wl.spec
    cfg = {"workload": args.config, "problems": len(wl.problems), "H": wl.H, "H_kv": wl.H_kv, "d": wl.d,
           "chunks": len(spec.chunk_lens), "chunk_len": spec.chunk_lens[0], "n_doc": int(sum(spec.chunk_lens)),
           "gen_len": spec.gen_len, "q_len": 1, "step": "decode", "kv_format": "int8 codes; fp32 scales per (KV head, channel) for K, per (KV head, token) for V"}
    rec = {"metric": METRIC_DECODE, "value": round(tokens / (wall / args.steps), 1), "unit": "KV tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": cfg,
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config, "q8"),
                        "kernel": "decode_q8_split+merge", "kernel_ms": round(k_ms, 4),
                        "alg_bytes_per_launch": nbytes},
           "quantize_once": {"kernels": "quantize_q8_token_kernel + quantize_q8_channel_kernel", "ms": round(q_ms, 4),
                             "bytes": int(sum(k.size + v.size for p in wl.problems for k, v in zip(p.K, p.V))) * 2 + q8_bytes},
           "kv_tokens_per_step": tokens}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        from oracle import q8
        t0 = time.perf_counter()
        done = 0
        for p in wl.problems:
            q8.decode(p, wl.H, wl.H_kv, wl.d)
            done += 1
            if time.perf_counter() - t0 > 10.0:
                break
        el = time.perf_counter() - t0
        import oracle
        rec["cpu_baseline"] = {"value": sum(p.n_keys for p in wl.problems[:done]) / el, "unit": "KV tokens/s",
                               "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": "layers 0..%d of %d (quantise + dequantise + fp64 decode), %.1f s"
                               % (done - 1, len(wl.problems), el)}
    print(json.dumps(rec), flush=True)


def bench_select(args, torch, crkv, workloads):
    """Gather + scatter of the selected keys' K/V rows (all layers, one launch
    each); the roofline is the gather kernel's."""
    base = SELECT_CONFIGS[args.config]
    log("generating %s" % base)
    wl = workloads.generate(base)
    dev = "cuda:0"
    up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    problems = []
    for p in wl.problems:
        Q = up(p.Q)
        problems.append(dict(Q=Q, chunk_K=[up(k) for k in p.K], chunk_V=[up(v) for v in p.V],
                             chunk_len=list(p.lens), q_len=p.q_len, out=torch.empty_like(Q),
                             impact=torch.empty(p.n_keys, dtype=torch.float32, device=dev)))
    ks = [crkv.crkv_budget(p.n_doc, wl.r) for p in wl.problems]
    idx = [torch.empty(k, dtype=torch.int32, device=dev) for k in ks]
    crkv.crkv_attn_chunks_batched(problems, wl.H, wl.H_kv, wl.d, mode=wl.mode)
    crkv.crkv_topk_batched([pr["impact"] for pr in problems], [p.n_doc for p in wl.problems], ks, idx)
    sels = [dict(chunk_K=pr["chunk_K"], chunk_V=pr["chunk_V"], chunk_len=pr["chunk_len"], idx=ix,
                 K_sel=torch.empty((wl.H_kv, k, wl.d), dtype=torch.bfloat16, device=dev),
                 V_sel=torch.empty((wl.H_kv, k, wl.d), dtype=torch.bfloat16, device=dev))
            for pr, ix, k in zip(problems, idx, ks)]
    torch.cuda.synchronize()
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    batch = crkv.SelectBatch(sels)   # marshalled once: the same tensors every step

    def step(events=None):
        crkv.crkv_gather_kv(batch, wl.H_kv, wl.d, crkv.CRKV_BF16, timing_events=events)
        crkv.crkv_scatter_kv(batch, wl.H_kv, wl.d, crkv.CRKV_BF16)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(pairs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs]))
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    selected = int(sum(ks))
    row_bytes = wl.d * 2
    gather_bytes = selected * wl.H_kv * 2 * row_bytes * 2     # K and V rows, read once and written once
    achieved = gather_bytes / (k_ms * 1e-3) / 1e9
    ms_per_step = wall * 1e3 / args.steps
    rec = {"metric": METRIC_SELECT, "value": round(selected / (wall / args.steps), 1),
           "unit": "selected token-layers/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": args.config, "layers": len(wl.problems), "H_kv": wl.H_kv, "d": wl.d,
                      "selected_per_layer": ks[0], "chunks": len(wl.spec.chunk_lens),
                      "chunk_len": wl.spec.chunk_lens[0], "q_len": wl.spec.q_len,
                      "selection": "top-k of the attention impact, r = %g" % wl.r},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(args.config, "kvsel"),
                        "kernel": "kvsel_kernel<gather>", "kernel_ms": round(k_ms, 4),
                        "alg_bytes_per_launch": gather_bytes}}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        from oracle import kvsel
        host_idx = [ix.cpu().numpy() for ix in idx]
        reps = 0
        t0 = time.perf_counter()
        while True:
            for p, ix in zip(wl.problems, host_idx):
                Kp, Vp = kvsel.gather_kv(p.K, p.V, p.lens, ix)
                kvsel.scatter_kv(p.K, p.V, p.lens, ix, Kp, Vp)
            reps += 1
            if time.perf_counter() - t0 > 10.0:
                break
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": reps * selected / el, "unit": "selected token-layers/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "all %d layers, gather + scatter repeated %d times, %.1f s"
                               % (len(wl.problems), reps, el)}
    print(json.dumps(rec), flush=True)


def bench_rope(args, torch, crkv, workloads):
    """Rotary re-positioning of every document chunk's cached keys (all layers,
    one launch)."""
    base = ROPE_CONFIGS[args.config]
    log("generating %s" % base)
    wl = workloads.generate(base)
    dev = "cuda:0"
    segs = []
    for p in wl.problems:
        off = 0
        for c in range(len(p.lens) - 1):   # document chunks; each was built at positions 0 ..
            K = torch.from_numpy(p.K[c].view(np.int16)).to(dev).view(torch.bfloat16)
            segs.append((K, p.lens[c], off))
            off += p.lens[c]
    torch.cuda.synchronize()
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]

    batch = crkv.RopeBatch(segs)   # marshalled once: the same tensors every step

    def step(events=None):
        crkv.crkv_rope_shift(batch, wl.H_kv, wl.d, crkv.CRKV_BF16, timing_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(pairs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs]))
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    moved = int(sum(n for _, n, dl in segs if dl != 0))
    nbytes = moved * wl.H_kv * wl.d * 2 * 2     # every moved key row read once and written once
    achieved = nbytes / (k_ms * 1e-3) / 1e9
    rec = {"metric": METRIC_ROPE, "value": round(moved / (wall / args.steps), 1),
           "unit": "key-layers/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": args.config, "layers": len(wl.problems), "H_kv": wl.H_kv, "d": wl.d,
                      "chunks": len(wl.spec.chunk_lens), "chunk_len": wl.spec.chunk_lens[0],
                      "shifts": sorted(set(dl for _, _, dl in segs)), "base": 10000.0},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config, "rope"),
                        "kernel": "rope_shift_kernel", "kernel_ms": round(k_ms, 4), "alg_bytes_per_launch": nbytes}}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        from oracle import rope
        done, t0 = 0, time.perf_counter()
        for p in wl.problems:
            off = 0
            for c in range(len(p.lens) - 1):
                if off:
                    rope.rope_shift(p.K[c], off, "bf16")
                    done += p.lens[c]
                off += p.lens[c]
            if time.perf_counter() - t0 > 10.0:
                break
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": done / el, "unit": "key-layers/s", "cores": 1, "kind": "oracle",
                               "sample": "%d moved chunks' keys of the first layers, %.1f s" % (done // 2500, el)}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="with the default workload, skip timing the other attention workloads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB "
                         "(the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_precomputed_chunk_amd as crkv
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "launches": 3}), flush=True)
        return
    if not os.path.exists(crkv.LIB_PATH):
        from attention_precomputed_chunk_amd import build as crkv_build
        crkv_build.build()
    if args.config in SELECT_CONFIGS:
        bench_select(args, torch, crkv, workloads)
        return
    if args.config in ROPE_CONFIGS:
        bench_rope(args, torch, crkv, workloads)
        return
    if args.config in Q8_CONFIGS:
        bench_q8_decode(args, torch, crkv, workloads)
        return

    rec = bench_attention(args, torch, crkv, workloads, args.config, args.steps, args.warmup,
                          with_cpu=not args.no_cpu_baseline)
    if args.config == DEFAULT_CONFIG and not args.no_other_configs:
        # the other attention workloads of the contract, timed in the same
        # process after the headline (their own lines of the record)
        rec["configs"] = {}
        for name in OTHER_ATTN_CONFIGS:
            sub = bench_attention(args, torch, crkv, workloads, name, args.steps, args.warmup, with_cpu=False)
            rec["configs"][name] = {k: sub[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                                        "roofline", "roofline_other", "graph",
                                                        "kv_tokens_per_step")}
    print(json.dumps(rec), flush=True)


def bench_attention(args, torch, crkv, workloads, name, steps, warmup, with_cpu):
    """Attention + impact combine + top-k of one workload: `steps` timed
    steps after `warmup`, the attention kernel bracketed by HIP events on the
    library's launch stream; returns the record (not printed). For an 8-bit
    workload the segments are quantised by the library once, before timing,
    and the attention reads the codes."""
    q8 = name in Q8_ATTN_CONFIGS
    base = Q8_ATTN_CONFIGS.get(name, name)
    log("generating %s" % base)
    wl = workloads.generate(base)
    dev = "cuda:0"

    def up(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    problems = []
    for p in wl.problems:
        Q = up(p.Q)
        problems.append(dict(Q=Q, chunk_K=[up(k) for k in p.K], chunk_V=[up(v) for v in p.V],
                             chunk_len=list(p.lens), q_len=p.q_len, out=torch.empty_like(Q),
                             impact=torch.empty(p.n_keys, dtype=torch.float32, device=dev)))
    ks = [crkv.crkv_budget(p.n_doc, wl.r) for p in wl.problems]
    idx = [torch.empty(k, dtype=torch.int32, device=dev) for k in ks]
    ns = [p.n_doc for p in wl.problems]
    imps = [pr["impact"] for pr in problems]
    dtype = crkv.CRKV_KV_Q8 if q8 else None
    q8_bytes = 0
    if q8:   # the stored cache: every segment quantised once, the bf16 copies dropped
        segs = []
        for pr, p in zip(problems, wl.problems):
            kq, vq = [], []
            for k, v, n in zip(pr["chunk_K"], pr["chunk_V"], p.lens):
                nk = crkv.crkv_q8_bytes(wl.H_kv, n, wl.d, crkv.CRKV_Q8_K)
                nv = crkv.crkv_q8_bytes(wl.H_kv, n, wl.d, crkv.CRKV_Q8_V)
                q8_bytes += nk + nv
                bk = torch.empty(max(nk, 16), dtype=torch.uint8, device=dev)
                bv = torch.empty(max(nv, 16), dtype=torch.uint8, device=dev)
                segs += [(k, bk, n, crkv.CRKV_Q8_K), (v, bv, n, crkv.CRKV_Q8_V)]
                kq.append(bk)
                vq.append(bv)
            pr["chunk_K"], pr["chunk_V"] = kq, vq
        crkv.crkv_quantize_q8(segs, wl.H_kv, wl.d)
        torch.cuda.synchronize()
        del segs
        torch.cuda.empty_cache()
    torch.cuda.synchronize()

    if wl.spec.decode:
        plan = {"kernel": "decode_split+merge", "row_tiles": 1, "workgroups": None}
    else:
        plan = crkv.crkv_plan_stats(problems, wl.H, wl.H_kv, wl.d, mode=wl.mode, dtype=dtype)
    log("plan: %s" % plan)
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(steps)]

    decode = bool(wl.spec.decode)
    batch = crkv.Batch(problems)   # marshalled once: the same tensors every step

    def step(events=None):
        if decode:   # one decode step: out only
            crkv.crkv_decode_chunks_batched(batch, wl.H, wl.H_kv, wl.d, timing_events=events)
            return
        crkv.crkv_attn_chunks_batched(batch, wl.H, wl.H_kv, wl.d, mode=wl.mode,
                                      timing_events=events, dtype=dtype)
        crkv.crkv_topk_batched(imps, ns, ks, idx)

    log("warmup %d" % warmup)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log("timing %d steps" % steps)
    t0 = time.perf_counter()
    for i in range(steps):
        step(pairs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)

    ms_per_step = wall * 1e3 / steps
    tokens = workloads.kv_tokens(wl)
    value = tokens / (wall / steps)
    nbytes, flops, npairs = algorithmic_work(wl)
    if q8:   # the codes and scales replace the bf16 K/V bytes
        nbytes += q8_bytes - sum(p.n_keys * 2 * wl.H_kv * wl.d * 2 for p in wl.problems)
    k_ms = float(np.mean(kern_ms))
    achieved_gbs = nbytes / (k_ms * 1e-3) / 1e9
    achieved_tf = flops / (k_ms * 1e-3) / 1e12
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    traffic = measured_traffic(name, "decode" if decode else "attn")
    p10, p50, p90 = (float(x) for x in np.percentile(kern_ms, [10, 50, 90]))
    hbm = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
           "kernel": plan["kernel"] if decode else "attn_%s_kernel" % plan["kernel"],
           "row_tiles": plan["row_tiles"],
           "workgroups": plan["workgroups"],
           "kernel_ms": round(k_ms, 4), "kernel_ms_p50": round(p50, 4), "kernel_ms_p10": round(p10, 4),
           "kernel_ms_p90": round(p90, 4), "alg_bytes_per_launch": nbytes}
    if not decode:
        # the timed region holds every attention kernel of the launch
        # (kernel_ms is their sum): pass 1 on its own where the plan runs it
        # so, pass 2, and the sum of output partials where blocks are cut
        # into key ranges
        hbm["kernels"] = ((["attn_lse_kernel"] if plan["pass1_separate"] else []) + [hbm["kernel"]] +
                          (["attn_out_combine_kernel"] if plan["split_blocks"] else []))
        hbm["split_blocks"] = plan["split_blocks"]
        hbm["max_ranges"] = plan["max_ranges"]
        hbm["model_imbalance"] = round(plan["imbalance"], 4)
    mfma = {"bound": "mfma", "achieved": round(achieved_tf, 2), "peak": mfma_peak,
            "unit": "TFLOP/s", "frac": round(achieved_tf / mfma_peak, 4),
            "alg_flops_per_launch": flops, "visible_pairs": npairs,
            "counters": None if decode else measured_mfma(name)}
    # the short-query workloads are reported against HBM first, the large
    # row-count ones (ragged batch, cross-document) against the matrix cores
    primary, secondary = (mfma, hbm) if name in ("ragged_70b", "cross_doc") else (hbm, mfma)
    spec = wl.spec
    cfg = {"workload": name, "problems": len(wl.problems), "H": wl.H, "H_kv": wl.H_kv,
           "d": wl.d, "mode": wl.mode, "r": wl.r}
    if q8:
        cfg["kv_format"] = ("int8 codes; fp32 scales per (KV head, channel) for K, per (KV head, token) for V; "
                            "quantised once before timing")
    if spec.chunk_lens:
        cfg.update({"chunks": len(spec.chunk_lens), "chunk_len": spec.chunk_lens[0],
                    "q_len": spec.q_len, "n_doc": int(sum(spec.chunk_lens))})
    else:
        cfg.update({"chunks": spec.ragged_m, "chunk_len": list(spec.ragged_chunk),
                    "q_len": list(spec.ragged_q)})
    if spec.gen_len:
        cfg["gen_len"] = spec.gen_len
    if decode:
        cfg["step"] = "decode"
    rec = {"metric": METRIC_DECODE if decode else METRIC, "value": round(value, 1), "unit": "KV tokens/s", "n_gpus": 1,
           "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
           "data": "synthetic", "config": cfg, "roofline": primary, "roofline_other": secondary,
           "kv_tokens_per_step": tokens}
    if not decode:
        rec["graph"] = graph_replay(steps, warmup, torch, crkv, wl, problems, ks, idx, tokens, dtype)
    if with_cpu:
        log("cpu baseline (oracle)")
        rec["cpu_baseline"] = cpu_baseline_q8(wl) if q8 else cpu_baseline(wl)
    del problems, batch, imps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def graph_replay(steps, warmup, torch, crkv, wl, problems, ks, idx, tokens, dtype=None):
    """The step (attention + impact combine + top-k) planned once and captured
    into a graph; W replays untimed, then K timed between synchronisations."""
    plan = crkv.Plan(problems, wl.H, wl.H_kv, wl.d, ks=ks, idxs=idx, mode=wl.mode, dtype=dtype)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.launch()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del g
    plan.destroy()
    return {"value": round(tokens / (wall / steps), 1), "unit": "KV tokens/s",
            "ms_per_step": round(wall * 1e3 / steps, 4),
            "how": "crkv_plan_create once; one captured crkv_plan_launch replayed per step"}


if __name__ == "__main__":
    main()
