"""Builds libcrkv.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m attention_precomputed_chunk_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcrkv.so")
SOURCES = ["crkv_api.hip", "attn_bf16_wave.hip", "attn_lse.hip", "attn_bf16_pair.hip", "decode_bf16.hip", "attn_f32.hip",
           "topk.hip", "kvsel.hip", "rope.hip", "q8.hip"]
# Device-code files. They never meet a NaN on the contract's inputs (masked
# scores are -inf), so maxima need no NaN canonicalisation; and matrix-core
# results are kept in ordinary VGPRs, which the vector ALU reads directly
# (the default AGPR form costs a v_accvgpr_read per score).
KERNEL_SOURCES = {"attn_bf16_wave.hip", "attn_lse.hip", "attn_bf16_pair.hip", "decode_bf16.hip", "attn_f32.hip", "topk.hip",
                  "kvsel.hip", "rope.hip", "q8.hip"}
KERNEL_FLAGS = ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
ARCH = os.environ.get("CRKV_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (res.stderr or "").splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, src.replace(".hip", ".o")) for src in SOURCES]
    cmds = [[hipcc()] + HIPCC_FLAGS + (KERNEL_FLAGS if src in KERNEL_SOURCES else []) +
            ["-c", os.path.join(CSRC, src), "-o", obj] for src, obj in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
