"""Planted mistakes: each is a plausible slip in the oracle (a dropped term, a
wrong sign, index or operand). A mutated copy of the oracle source is built on
the CPU in a temporary directory; at least one pin must reject it. This shows
that the pins constrain every part of the oracle, not that the oracle matches
itself."""
import os
import shutil
import subprocess
import sys

import pytest
import oracle

SRC_DIR = os.path.dirname(os.path.abspath(oracle.__file__))

MUTATIONS = {
    "scale_by_d": ("1.0 / sqrt((double)d)", "1.0 / (double)d"),
    "mask_off_by_one": ("causal ? pos + 1 : N", "causal ? (pos + 2 < N ? pos + 2 : N) : N"),
    "query_rows_at_start": ("(mode == OR_QUERY_ROWS) ? N - q_len + j : j", "j"),
    "query_rows_after_documents": ("(mode == OR_QUERY_ROWS) ? N - q_len + j : j", "(mode == OR_QUERY_ROWS) ? n_doc + j : j"),
    "gqa_modulo_groups": ("const int hk = h / G;", "const int hk = h % H_kv;"),
    "lse_sign": ("mx + log(l)", "mx - log(l)"),
    "unnormalised_weights": ("exp(s[i] - row_lse)", "exp(s[i] - mx)"),
    "value_from_keys": ("acc[t] += p * widen(V[c]", "acc[t] += p * widen(K[c]"),
    "cross_doc_exclusion_dropped": ("(seg_row != c)", "(1)"),
    "cross_doc_exclusion_inverted": ("(seg_row != c)", "(seg_row == c)"),
    "impact_one_head": ("if (counted)", "if (counted && h == 0)"),
    "impact_mask_all_modes": ("(mode != OR_CROSS_DOC) || (seg_row != c)", "(seg_row != c)"),
    "topk_ties_high_index": ("(x->idx > y->idx) - (x->idx < y->idx)", "(x->idx < y->idx) - (x->idx > y->idx)"),
    "topk_negative_order": ("(u >> 31) ? ~u : (u | 0x80000000u)", "u ^ 0x80000000u"),
    "budget_ceil": ("floor(r * (double)n_doc)", "ceil(r * (double)n_doc)"),
    "budget_no_minimum": ("k < 1 ? 1 : k", "k"),
    "query_keys_dropped": ("causal ? pos + 1 : N", "causal ? (pos + 1 < n_doc ? pos + 1 : n_doc) : n_doc"),
}


RUNNER = r"""
import importlib.util, json, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import torch
torch.set_default_dtype(torch.float64)
spec = importlib.util.spec_from_file_location({pkg!r}, {init!r}, submodule_search_locations=[{pkgdir!r}])
mod = importlib.util.module_from_spec(spec); sys.modules[{pkg!r}] = mod; spec.loader.exec_module(mod)
mod.build()
from oracle_pins import PINS
for name, pin in sorted(PINS.items()):
    try:
        pin(mod)
    except Exception:
        print("CAUGHT", name, flush=True)
"""


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(os.path.join(SRC_DIR, "oracle.c")).read()
    assert src.count(old) >= 1, "mutation anchor not found: %s" % name
    pkg = "oracle_mutant_" + name
    d = tmp_path / pkg
    d.mkdir()
    (d / "oracle.c").write_text(src.replace(old, new, 1))
    shutil.copy(os.path.join(SRC_DIR, "__init__.py"), d / "__init__.py")
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    code = RUNNER.format(root=os.path.dirname(tests_dir), tests=tests_dir, pkg=pkg,
                         init=str(d / "__init__.py"), pkgdir=str(d))
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600)
    caught = [ln.split()[1] for ln in proc.stdout.splitlines() if ln.startswith("CAUGHT")]
    # a mutant that crashes its process is rejected too
    assert caught or proc.returncode != 0, "no pin rejects the planted mistake %r" % name
