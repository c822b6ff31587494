"""Pins for the fp64 oracle, checked against things other than itself.

Each pin ties the oracle to something the pages or the mathematics fix:
torch's float64 scaled-dot-product attention on explicitly concatenated K/V
(TurboRAG K_combined equation and causal attention equation; CacheBlend
full-prefill formulation), the CacheBlend listing's unmasked softmax, closed
forms for uniform attention, row-stochastic softmax, the impact mass, the
invariance of concatenation under re-partitioning, GQA as MHA with repeated
K/V heads, textbook causal attention when there are no documents, a single
softmax row, a dominant key, decode steps (the newest token over a growing
last segment) against torch and against the query block's rows, a
brute-force top-k on tiny inputs and the budget k = max(1, int(N_doc * r)).

Every pin is a function of an oracle module (``orc``), so that the
planted-mistake test can run the same pins against a mutated copy of the
oracle and require that each plausible mistake fails at least one of them.
"""
import itertools
import math

import numpy as np
import torch
import torch.nn.functional as F

import workloads


def _t(arr, dtype):
    """Stored input -> torch float64, using torch's own bf16 conversion."""
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(arr.astype(np.float32)).to(torch.float64)


def torch_reference(prob, H, H_kv, d, dtype, mode, causal=True):
    """Full score matrix in torch float64: (out, impact)."""
    G = H // H_kv
    Q = _t(prob.Q, dtype)
    K = torch.cat([_t(k, dtype) for k in prob.K], dim=1).repeat_interleave(G, dim=0)
    V = torch.cat([_t(v, dtype) for v in prob.V], dim=1).repeat_interleave(G, dim=0)
    N = prob.n_keys
    seg_key = torch.cat([torch.full((n,), c) for c, n in enumerate(prob.lens)])
    if mode == "query":   # the q_len rows are the last positions of the concatenation
        row_pos = N - prob.q_len + torch.arange(prob.q_len)
    else:
        row_pos = torch.arange(N)
    seg_row = seg_key[row_pos]
    key_pos = torch.arange(N)
    if causal:
        vis = key_pos[None, :] <= row_pos[:, None]
    else:
        vis = torch.ones(len(row_pos), N, dtype=torch.bool)
    out = F.scaled_dot_product_attention(Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0),
                                         attn_mask=vis).squeeze(0)
    scores = torch.matmul(Q, K.transpose(1, 2).contiguous()) / math.sqrt(d)
    P = torch.softmax(scores.masked_fill(~vis, float("-inf")), dim=-1)
    counted = (seg_row[:, None] != seg_key[None, :]) if mode == "cross" else torch.ones_like(vis)
    impact = (P * counted).sum(dim=(0, 1))
    return out.numpy(), impact.numpy()


def close(a, b, rtol=0.0, atol=0.0):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


SHAPES = [
    # doc_lens, q_len, H, H_kv, d
    ([7, 0, 13], 5, 4, 2, 16),
    ([16, 16], 8, 2, 2, 8),
    ([1, 3, 2, 9], 6, 6, 3, 12),
    ([], 7, 2, 1, 8),
]


def pin_matches_torch_sdpa(orc):
    for si, (doc_lens, q, H, H_kv, d) in enumerate(SHAPES):
        for dtype in ("f32", "bf16"):
            for mode in ("query", "cross", "all"):
                wl = workloads.custom(11 + si, doc_lens, q, H, H_kv, d, dtype=dtype, mode=mode)
                prob = wl.problems[0]
                out, imp, _ = orc.attn(prob, H, H_kv, d, dtype, mode)
                ref_out, ref_imp = torch_reference(prob, H, H_kv, d, dtype, mode)
                close(out, ref_out, atol=1e-12)
                close(imp, ref_imp, rtol=1e-12, atol=1e-13)


def pin_unmasked_listing(orc):
    """causal off gives the CacheBlend listing's softmax over every key."""
    for mode in ("query", "all"):
        wl = workloads.custom(5, [9, 4], 6, 2, 2, 8, mode=mode)
        prob = wl.problems[0]
        out, imp, _ = orc.attn(prob, 2, 2, 8, "f32", mode, causal=False)
        ref_out, ref_imp = torch_reference(prob, 2, 2, 8, "f32", mode, causal=False)
        close(out, ref_out, atol=1e-12)
        close(imp, ref_imp, rtol=1e-12)
        rows = prob.q_len if mode == "query" else prob.n_keys
        close(imp.sum(), rows * 2, rtol=1e-13)


def pin_rows_are_stochastic(orc):
    """softmax rows sum to one: with V == 1 every output element is 1."""
    for mode in ("query", "cross", "all"):
        wl = workloads.custom(3, [5, 11, 2], 4, 4, 2, 16, mode=mode)
        prob = wl.problems[0]
        for v in prob.V:
            v[...] = np.float32(1.0)
        out, _, _ = orc.attn(prob, 4, 2, 16, "f32", mode)
        close(out, 1.0, atol=1e-13)


def pin_impact_mass(orc):
    """Summed over all N columns, impact is rows * H (each row's weights sum to 1)."""
    for mode in ("query", "all"):
        wl = workloads.custom(4, [6, 2, 9], 5, 6, 2, 8, dtype="bf16", mode=mode)
        prob = wl.problems[0]
        _, imp, _ = orc.attn(prob, 6, 2, 8, "bf16", mode)
        rows = prob.q_len if mode == "query" else prob.n_keys
        close(imp.sum(), rows * 6, rtol=1e-13)


def _harm(n):
    return sum(1.0 / t for t in range(1, n + 1))


def pin_uniform_query_rows_closed_form(orc):
    """Q = 0: every visible key gets weight 1/n_vis; impact is a harmonic sum
    and each output row is the mean of the visible V rows."""
    doc, q, H, d = [5, 7], 4, 3, 8
    wl = workloads.custom(6, doc, q, H, H, d)
    prob = wl.problems[0]
    prob.Q[...] = 0
    out, imp, _ = orc.attn(prob, H, H, d, "f32", "query")
    n_doc = prob.n_doc
    for i in range(n_doc):
        close(imp[i], H * (_harm(n_doc + q) - _harm(n_doc)), rtol=1e-13)
    for t in range(q):
        close(imp[n_doc + t], H * sum(1.0 / (n_doc + j + 1) for j in range(t, q)), rtol=1e-13)
    Vcat = np.concatenate([v.astype(np.float64) for v in prob.V], axis=1)
    for h in range(H):
        for j in range(q):
            close(out[h, j], Vcat[h, : n_doc + j + 1].mean(axis=0), atol=1e-13)


def pin_uniform_cross_doc_closed_form(orc):
    """Q = 0 in cross-document mode: impact_i = H * sum_{j>=i, seg(j)!=seg(i)} 1/(j+1)."""
    doc, q, H, d = [4, 3, 5], 2, 2, 8
    wl = workloads.custom(7, doc, q, H, H, d, mode="cross")
    prob = wl.problems[0]
    prob.Q[...] = 0
    _, imp, _ = orc.attn(prob, H, H, d, "f32", "cross")
    seg = np.concatenate([np.full(n, c) for c, n in enumerate(prob.lens)])
    N = prob.n_keys
    for i in range(N):
        expect = H * sum(1.0 / (j + 1) for j in range(i, N) if seg[j] != seg[i])
        close(imp[i], expect, rtol=1e-13, atol=1e-15)


def repartition(prob, new_doc_lens):
    Kc = np.concatenate(prob.K[:-1], axis=1)
    Vc = np.concatenate(prob.V[:-1], axis=1)
    assert sum(new_doc_lens) == Kc.shape[1]
    K, V, o = [], [], 0
    for n in new_doc_lens:
        K.append(np.ascontiguousarray(Kc[:, o:o + n]))
        V.append(np.ascontiguousarray(Vc[:, o:o + n]))
        o += n
    K.append(prob.K[-1])
    V.append(prob.V[-1])
    return workloads.Problem(K=K, V=V, lens=list(new_doc_lens) + [prob.q_len], q_len=prob.q_len,
                             Q=prob.Q)


def pin_concat_is_partition_invariant(orc):
    """Any split of the same keys into chunks (empty and length-1 chunks
    included, and m=1 as the single-sequence prefill) gives the same result."""
    for mode in ("query", "all"):
        wl = workloads.custom(8, [10, 6], 5, 4, 2, 8, dtype="bf16", mode=mode)
        prob = wl.problems[0]
        base_out, base_imp, _ = orc.attn(prob, 4, 2, 8, "bf16", mode)
        for split in ([16], [0, 16], [1, 0, 15], [3, 3, 3, 3, 4], [15, 1, 0]):
            out, imp, _ = orc.attn(repartition(prob, split), 4, 2, 8, "bf16", mode)
            np.testing.assert_array_equal(out, base_out)
            np.testing.assert_array_equal(imp, base_imp)


def pin_cross_doc_split_moves_only_exclusions(orc):
    """In cross mode the output does not depend on the split; the impact does,
    and it never exceeds the all-rows impact."""
    wl = workloads.custom(9, [6, 6], 3, 2, 2, 8, mode="cross")
    prob = wl.problems[0]
    out_a, imp_a, _ = orc.attn(prob, 2, 2, 8, "f32", "cross")
    out_b, imp_b, _ = orc.attn(repartition(prob, [12]), 2, 2, 8, "f32", "cross")
    np.testing.assert_array_equal(out_a, out_b)
    assert not np.allclose(imp_a, imp_b)
    _, imp_all, _ = orc.attn(prob, 2, 2, 8, "f32", "all")
    assert np.all(imp_a <= imp_all + 1e-15)


def pin_gqa_equals_mha_with_repeated_heads(orc):
    H, H_kv, d = 6, 2, 8
    for mode in ("query", "cross"):
        wl = workloads.custom(10, [5, 4], 3, H, H_kv, d, dtype="bf16", mode=mode)
        prob = wl.problems[0]
        out, imp, _ = orc.attn(prob, H, H_kv, d, "bf16", mode)
        G = H // H_kv
        rep = workloads.Problem(K=[np.repeat(k, G, axis=0) for k in prob.K],
                                V=[np.repeat(v, G, axis=0) for v in prob.V],
                                lens=prob.lens, q_len=prob.q_len, Q=prob.Q)
        out2, imp2, _ = orc.attn(rep, H, H, d, "bf16", mode)
        np.testing.assert_array_equal(out, out2)
        np.testing.assert_array_equal(imp, imp2)


def pin_no_documents_is_textbook_causal_attention(orc):
    H, d, q = 3, 16, 9
    wl = workloads.custom(12, [], q, H, H, d)
    prob = wl.problems[0]
    out, imp, _ = orc.attn(prob, H, H, d, "f32", "query")
    Q = torch.from_numpy(prob.Q.astype(np.float64))
    K = torch.from_numpy(prob.K[0].astype(np.float64))
    V = torch.from_numpy(prob.V[0].astype(np.float64))
    ref = F.scaled_dot_product_attention(Q, K, V, is_causal=True).numpy()
    close(out, ref, atol=1e-12)
    close(imp.sum(), q * H, rtol=1e-13)


def pin_single_query_row_is_one_softmax(orc):
    H, d = 2, 8
    wl = workloads.custom(13, [4, 3], 1, H, H, d)
    prob = wl.problems[0]
    out, imp, lse = orc.attn(prob, H, H, d, "f32", "query", want_lse=True)
    Kc = np.concatenate([k.astype(np.float64) for k in prob.K], axis=1)
    Vc = np.concatenate([v.astype(np.float64) for v in prob.V], axis=1)
    for h in range(H):
        s = Kc[h] @ prob.Q[h, 0].astype(np.float64) / math.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        close(out[h, 0], p @ Vc[h], atol=1e-13)
        close(lse[h, 0], s.max() + math.log(np.exp(s - s.max()).sum()), rtol=1e-14)
    close(imp.sum(), H, rtol=1e-14)


def pin_decode_step_matches_torch_sdpa(orc):
    """A decode step (TurboRAG summary, the generation loop that appends each
    token's K/V): the last segment holds earlier generated tokens and the one
    query row is the newest position, which sees every key."""
    for seed, doc, gen, H, H_kv, d, dtype in [(31, [9, 0, 6], 5, 4, 2, 16, "f32"),
                                              (32, [12], 3, 2, 1, 8, "bf16"),
                                              (33, [], 7, 2, 2, 8, "f32")]:
        wl = workloads.custom(seed, doc, 1, H, H_kv, d, dtype=dtype, gen_len=gen)
        prob = wl.problems[0]
        assert prob.lens[-1] == gen + 1
        out, imp, _ = orc.attn(prob, H, H_kv, d, dtype, "query")
        ref_out, ref_imp = torch_reference(prob, H, H_kv, d, dtype, "query")
        close(out, ref_out, atol=1e-12)
        close(imp, ref_imp, atol=1e-12)


def pin_uniform_decode_closed_form(orc):
    """Q = 0 in a decode step: every key gets weight 1/N, so the output is the
    mean of all V rows of the head's KV head and every impact is H / N."""
    doc, gen, H, H_kv, d = [5, 3], 4, 4, 2, 8
    wl = workloads.custom(34, doc, 1, H, H_kv, d, gen_len=gen)
    prob = wl.problems[0]
    prob.Q[...] = 0
    out, imp, _ = orc.attn(prob, H, H_kv, d, "f32", "query")
    N = prob.n_keys
    close(imp, np.full(N, H / N), rtol=1e-13)
    Vcat = np.concatenate([v.astype(np.float64) for v in prob.V], axis=1)
    for h in range(H):
        close(out[h, 0], Vcat[h // (H // H_kv)].mean(axis=0), atol=1e-13)


def pin_prefill_rows_equal_decode_steps(orc):
    """Causality: row j of a T-row query block sees exactly the keys a decode
    step sees when the last segment stops at that row's own key."""
    doc, T, H, d = [6, 4], 5, 2, 8
    wl = workloads.custom(35, doc, T, H, H, d)
    prob = wl.problems[0]
    out, _, _ = orc.attn(prob, H, H, d, "f32", "query")
    for j in range(T):
        step = workloads.Problem(K=prob.K[:-1] + [np.ascontiguousarray(prob.K[-1][:, : j + 1])],
                                 V=prob.V[:-1] + [np.ascontiguousarray(prob.V[-1][:, : j + 1])],
                                 lens=prob.lens[:-1] + [j + 1], q_len=1,
                                 Q=np.ascontiguousarray(prob.Q[:, j : j + 1]))
        o1, _, _ = orc.attn(step, H, H, d, "f32", "query")
        close(o1[:, 0], out[:, j], atol=1e-14)


def pin_dominant_key_takes_all_impact(orc):
    """k_i = c * q with large c puts (almost) all of each row's weight on key i."""
    H, d = 4, 8
    wl = workloads.custom(14, [6, 5], 1, H, H, d)
    prob = wl.problems[0]
    star_seg, star_off = 1, 2
    for h in range(H):
        prob.K[star_seg][h, star_off] = np.float32(40.0) * prob.Q[h, 0]
    _, imp, _ = orc.attn(prob, H, H, d, "f32", "query")
    star = prob.lens[0] + star_off
    close(imp[star], H, rtol=1e-6)
    assert int(np.argmax(imp)) == star


def pin_row_range_is_exact_for_late_keys(orc):
    """Computing only rows at positions >= r0 gives the exact impact of keys at
    positions >= r0 (earlier rows cannot see them under the causal mask)."""
    for mode in ("cross", "all"):
        wl = workloads.custom(15, [7, 9, 4], 3, 2, 1, 8, dtype="bf16", mode=mode)
        prob = wl.problems[0]
        out, imp, lse = orc.attn(prob, 2, 1, 8, "bf16", mode, want_lse=True)
        r0 = 13
        out2, imp2, lse2 = orc.attn(prob, 2, 1, 8, "bf16", mode, row_lo=r0, want_lse=True)
        close(imp2[r0:], imp[r0:], rtol=1e-14)
        np.testing.assert_array_equal(out2[:, r0:], out[:, r0:])
        np.testing.assert_array_equal(lse2[:, r0:], lse[:, r0:])


# ---------------------------------------------------------------- top-k and budget

def _order_key(x):
    """Total order on float32 values used by the selection: value, then -0 < +0."""
    return (float(x), math.copysign(1.0, float(x)))


def pin_topk_brute_force_small_alphabet(orc):
    """Every selected element >= every unselected one; among equal keys the
    lower indices are chosen; output sorted (value desc, index asc)."""
    rng = np.random.default_rng(0)
    alphabet = np.array([-1.5, -0.0, 0.0, 0.25, 1.0, 3.0], dtype=np.float32)
    for n in range(1, 8):
        for _ in range(12):
            vals = alphabet[rng.integers(0, len(alphabet), size=n)]
            keys = [_order_key(v) for v in vals]
            for k in range(1, n + 1):
                idx = orc.topk(vals, k)
                valid = []
                for sub in itertools.combinations(range(n), k):
                    ins = set(sub)
                    if all(not (keys[a] < keys[b] or (keys[a] == keys[b] and a > b))
                           for a in ins for b in range(n) if b not in ins):
                        valid.append(ins)
                assert len(valid) == 1
                assert set(idx.tolist()) == valid[0]
                order = sorted(valid[0], key=lambda i: (tuple(-x for x in keys[i]), i))
                assert idx.tolist() == order


def pin_topk_matches_lexsort(orc):
    rng = np.random.default_rng(1)
    for n in (5, 100, 3000):
        vals = rng.standard_normal(n).astype(np.float32)
        vals[rng.integers(0, n, size=n // 5)] = vals[0]        # plenty of ties
        k = max(1, n // 7)
        u = vals.view(np.uint32).astype(np.int64)
        keys = np.where(u >> 31, (~u) & 0xFFFFFFFF, u | 0x80000000)
        ref = np.lexsort((np.arange(n), -keys))[:k]
        np.testing.assert_array_equal(orc.topk(vals, k), ref)


def pin_budget_values(orc):
    """k = max(1, int(N_doc * r)) (CacheBlend listing; the budget r * sum |D_i|)."""
    assert orc.budget(128, 0.1) == 12
    assert orc.budget(2048, 0.1) == 204
    assert orc.budget(10000, 0.15) == 1500
    assert orc.budget(8192, 0.05) == 409
    assert orc.budget(5, 0.1) == 1
    assert orc.budget(0, 0.1) == 1
    lens, _ = workloads.ragged_shapes(workloads.CONFIGS["ragged_70b"])
    for row in lens:
        assert orc.budget(sum(row), 0.1) == int(sum(row) * 0.1)


PINS = {name[4:]: fn for name, fn in sorted(globals().items())
        if name.startswith("pin_") and callable(fn)}
