"""Pins for the CPU oracle: each check ties it to something other than itself.

* the hand-worked example in tests/golden/hand_example.json (values derived by hand);
* the constants the pages print (tests/golden/page_constants.json);
* closed forms (block sums of an arithmetic sequence, the 8x candidate-count ratio);
* special cases that reduce to a library routine (dense causal attention = torch SDPA in fp64
  with an explicit bottom-right causal mask; B = 1 = token-level top-k via heapq.nlargest);
* brute force on tiny inputs (an O(n^2) rank count for the selection, independent of sorting);
* invariants (nesting in k, permutation of index dims, positive scaling, constant values).
"""
import heapq
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from sgqa_inputs import generate_small, get_workload


# ----------------------------------------------------------------------------------------------
# hand-worked example
# ----------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def hand(golden_dir):
    with open(os.path.join(golden_dir, "hand_example.json")) as f:
        return json.load(f)


def test_hand_compress(hand):
    k_idx = np.array(hand["k_idx"], dtype=np.float64)[None]
    kb = oracle.compress(k_idx, hand["block"])
    assert kb.shape == (1, 5, 2)
    np.testing.assert_array_equal(kb[0], np.array(hand["k_blk_by_hand"], dtype=np.float64))


def test_hand_scores_and_selection(hand):
    kb = oracle.compress(np.array(hand["k_idx"], dtype=np.float64)[None], hand["block"])[0]
    for qd in hand["queries"]:
        p = qd["position"]
        o = p // hand["block"]
        s = oracle.block_scores(qd["q_idx"], kb, o)
        np.testing.assert_array_equal(s, np.array(qd["scores_by_hand"], dtype=np.float64))
        sel = oracle.select_blocks(s, o, hand["n_sel"])
        assert sel.tolist() == qd["sel"]
        toks = oracle.attended_tokens(sel, hand["block"], p, hand["t_kv"])
        assert toks.tolist() == qd["tokens"]


@pytest.mark.parametrize("which", ["attention_uniform", "attention_weighted"])
def test_hand_attention(hand, which):
    t_kv = hand["t_kv"]
    v = np.arange(t_kv, dtype=np.float64)[:, None]
    if which == "attention_uniform":
        q = np.zeros((1, 1))
        k = np.ones((t_kv, 1))
    else:
        q = np.ones((1, 1))
        k = np.log(np.arange(t_kv, dtype=np.float64) + 1.0)[:, None]
    for qd in hand["queries"]:
        num, den = hand[which]["expected"][str(qd["position"])]
        out = oracle.gated_attention(q, k, v, np.zeros((1, 1)), np.array(qd["tokens"]), 1.0)
        assert out.shape == (1, 1)
        assert abs(out[0, 0] - num / den) < 1e-14


def test_hand_forward_end_to_end(hand):
    """The whole path on the hand example, through forward_rows."""
    t_kv = hand["t_kv"]
    pos = [q["position"] for q in hand["queries"]]
    t_q = t_kv  # every position is a query; only the hand-worked ones are checked
    q_idx = np.zeros((1, t_q, 1, 2))
    for qd in hand["queries"]:
        q_idx[0, qd["position"], 0] = qd["q_idx"]
    inputs = {
        "q_idx": q_idx,
        "k_idx": np.array(hand["k_idx"], dtype=np.float64)[None],
        "q": np.ones((1, t_q, 1, 1, 1)),
        "k": np.log(np.arange(t_kv, dtype=np.float64) + 1.0)[None, None, :, None],
        "v": np.arange(t_kv, dtype=np.float64)[None, None, :, None],
        "gate": np.zeros((1, t_q, 1, 1, 1)),
    }
    sel, out, _ = oracle.forward_rows(inputs, hand["block"], hand["topk_tokens"], 1.0,
                                      [(0, p) for p in pos])
    for r, qd in enumerate(hand["queries"]):
        assert sel[r, 0].tolist() == qd["sel"]
        num, den = hand["attention_weighted"]["expected"][str(qd["position"])]
        assert abs(out[r, 0, 0, 0] - num / den) < 1e-14


# ----------------------------------------------------------------------------------------------
# constants the pages print
# ----------------------------------------------------------------------------------------------
def test_page_constants(golden_dir):
    with open(os.path.join(golden_dir, "page_constants.json")) as f:
        c = json.load(f)
    B, k = c["final_block_size"]["value"], c["final_topk_tokens"]["value"]
    assert oracle.n_selected_blocks(k, B) == c["selected_blocks"]["value"]
    # the workloads carry the pages' setting
    for name in ("32k", "128k", "decode", "1m"):
        w = get_workload(name)
        assert (w.block, w.topk, w.n_sel) == (B, k, c["selected_blocks"]["value"])
    assert get_workload("1m").t_kv == c["max_context_tokens"]["value"]


def test_eightfold_candidate_reduction(golden_dir):
    """Indexer/top-k work is the number of scored candidates; B=8 cuts it ~8x (pages' claim).

    Closed form over a full 128K prefill: sum_p p / sum_p floor(p/8) = (N-1)/(N/8-1).
    """
    with open(os.path.join(golden_dir, "page_constants.json")) as f:
        c = json.load(f)
    N = 131072
    b1 = sum(oracle.scored_candidates(p, c["reference_block_size"]["value"]) for p in range(N))
    b8 = sum(oracle.scored_candidates(p, c["final_block_size"]["value"]) for p in range(N))
    assert Fraction(b1, b8) == Fraction(N - 1, N // 8 - 1)
    assert abs(b1 / b8 - c["indexer_topk_cost_reduction"]["value"]) < 1e-3


# ----------------------------------------------------------------------------------------------
# compression: closed forms and invariants
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("B,T", [(8, 64), (8, 61), (3, 20), (1, 7), (16, 40)])
def test_compress_arithmetic_sequence(B, T):
    """k_idx[t] = (t, 1): block j sums to (sum of its token indices, its token count)."""
    k_idx = np.stack([np.arange(T, dtype=np.float64), np.ones(T)], axis=1)[None]
    kb = oracle.compress(k_idx, B)[0]
    assert kb.shape[0] == math.ceil(T / B)
    for j in range(kb.shape[0]):
        lo, hi = j * B, min(j * B + B, T) - 1
        n = hi - lo + 1
        assert kb[j, 0] == (lo + hi) * n / 2      # arithmetic series
        assert kb[j, 1] == n


def test_compress_invariants():
    rng = np.random.default_rng(1)
    k_idx = rng.integers(-4, 5, size=(2, 53, 6)).astype(np.float64)
    for B in (1, 2, 5, 8):
        kb = oracle.compress(k_idx, B)
        np.testing.assert_array_equal(kb.sum(axis=1), k_idx.sum(axis=1))
    np.testing.assert_array_equal(oracle.compress(k_idx, 1), k_idx)


# ----------------------------------------------------------------------------------------------
# scores
# ----------------------------------------------------------------------------------------------
def test_scores_unit_queries_pick_columns():
    rng = np.random.default_rng(2)
    k_idx = rng.integers(-4, 5, size=(1, 40, 5)).astype(np.float64)
    kb = oracle.compress(k_idx, 8)[0]
    for c in range(5):
        e = np.zeros(5)
        e[c] = 1.0
        s = oracle.block_scores(e, kb, 5)
        # column c of the block sums of the raw keys
        expect = [k_idx[0, 8 * j:8 * j + 8, c].sum() for j in range(5)]
        np.testing.assert_array_equal(s, expect)


def test_scores_bilinear_and_permutation_invariant():
    rng = np.random.default_rng(3)
    kb = rng.integers(-32, 33, size=(30, 7)).astype(np.float64)
    a = rng.integers(-4, 5, size=7).astype(np.float64)
    b = rng.integers(-4, 5, size=7).astype(np.float64)
    np.testing.assert_array_equal(oracle.block_scores(a + 2 * b, kb, 30),
                                  oracle.block_scores(a, kb, 30) + 2 * oracle.block_scores(b, kb, 30))
    perm = rng.permutation(7)
    np.testing.assert_array_equal(oracle.block_scores(a[perm], kb[:, perm], 30),
                                  oracle.block_scores(a, kb, 30))


# ----------------------------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------------------------
def _brute_force_selection(s, o, n_sel):
    """Independent O(n^2) definition: j is chosen iff j == o, or fewer than n_sel-1 candidates beat
    it, where j' beats j when s[j'] > s[j] or (s[j'] == s[j] and j' < j)."""
    if o + 1 <= n_sel:
        return list(range(o + 1))
    chosen = [o]
    for j in range(o):
        beaten_by = sum(1 for jj in range(o) if s[jj] > s[j] or (s[jj] == s[j] and jj < j))
        if beaten_by < n_sel - 1:
            chosen.append(j)
    return sorted(chosen)


@pytest.mark.parametrize("B", [1, 2, 3, 8])
def test_selection_brute_force(B):
    rng = np.random.default_rng(10 + B)
    T = 64
    k_idx = rng.integers(-1, 2, size=(1, T, 3)).astype(np.float64)   # tiny range: many ties
    kb = oracle.compress(k_idx, B)[0]
    for p in range(T):
        o = p // B
        q = rng.integers(-1, 2, size=3).astype(np.float64)
        s = oracle.block_scores(q, kb, o)
        for n_sel in range(1, oracle.num_blocks(T, B) + 2):
            sel = oracle.select_blocks(s, o, n_sel)
            got = [j for j in sel.tolist() if j >= 0]
            assert got == _brute_force_selection(s.tolist(), o, n_sel)
            assert sel.tolist()[len(got):] == [-1] * (n_sel - len(got))


def test_selection_b1_is_token_level_topk():
    """B=1: own token plus the top k-1 past tokens, ties to the lower token (heapq, no sort)."""
    rng = np.random.default_rng(4)
    T, k = 300, 64
    k_idx = rng.integers(-4, 5, size=(1, T, 8)).astype(np.float64)
    kb = oracle.compress(k_idx, 1)[0]
    for p in range(0, T, 7):
        q = rng.integers(-4, 5, size=8).astype(np.float64)
        s = k_idx[0, :p] @ q                      # token-level scores, computed directly
        sel = oracle.select_blocks(oracle.block_scores(q, kb, p), p, k)
        got = sorted(j for j in sel.tolist() if j >= 0)
        if p + 1 <= k:
            expect = list(range(p + 1))
        else:
            best = heapq.nlargest(k - 1, range(p), key=lambda j: (s[j], -j))
            expect = sorted(best + [p])
        assert got == expect


def test_selection_dense_when_budget_covers_context():
    rng = np.random.default_rng(5)
    T, B = 96, 8
    kb = oracle.compress(rng.integers(-4, 5, size=(1, T, 4)).astype(np.float64), B)[0]
    nb = oracle.num_blocks(T, B)
    for p in range(T):
        o = p // B
        s = oracle.block_scores(rng.integers(-4, 5, size=4), kb, o)
        sel = oracle.select_blocks(s, o, nb)
        assert [j for j in sel.tolist() if j >= 0] == list(range(o + 1))
        assert oracle.attended_tokens(sel, B, p, T).tolist() == list(range(p + 1))


def test_selection_nesting_and_shape():
    rng = np.random.default_rng(6)
    s = rng.integers(-3, 4, size=200).astype(np.float64)
    o = 200
    prev = set()
    for n_sel in range(1, 210):
        sel = oracle.select_blocks(s, o, n_sel)
        cur = {j for j in sel.tolist() if j >= 0}
        assert len(cur) == min(n_sel, o + 1)
        assert o in cur and max(cur) == o and min(cur) >= 0
        assert prev <= cur
        assert sorted(cur) == [j for j in sel.tolist() if j >= 0]
        prev = cur


def test_selection_scale_invariance_and_negative_zero():
    rng = np.random.default_rng(7)
    s = rng.integers(-3, 4, size=50).astype(np.float64)
    ref = oracle.select_blocks(s, 50, 11)
    np.testing.assert_array_equal(oracle.select_blocks(3.0 * s, 50, 11), ref)
    z = np.zeros(20)
    z[::2] = -0.0
    # -0.0 and +0.0 are equal scores: ties go to the lowest indices
    assert oracle.select_blocks(z, 20, 6).tolist() == [0, 1, 2, 3, 4, 20]


# ----------------------------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------------------------
def _sdpa_reference(inp, mask, scale):
    """torch SDPA in fp64 with an explicit boolean mask [T_q, T_kv], times sigmoid(gate)."""
    q = inp["q"].to(torch.float64)                      # [Bt, Tq, G, h, d]
    Bt, Tq, G, h, d = q.shape
    k = inp["k"].to(torch.float64).repeat_interleave(h, dim=1)   # [Bt, G*h, Tkv, d]
    v = inp["v"].to(torch.float64).repeat_interleave(h, dim=1)
    qh = q.reshape(Bt, Tq, G * h, d).transpose(1, 2)             # [Bt, G*h, Tq, d]
    o = torch.nn.functional.scaled_dot_product_attention(qh, k, v, attn_mask=mask, scale=scale)
    o = o.transpose(1, 2).reshape(Bt, Tq, G, h, d)
    return (o * torch.sigmoid(inp["gate"].to(torch.float64))).numpy()


@pytest.mark.parametrize("t_q,t_kv", [(40, 40), (13, 40), (1, 33)])
def test_attention_dense_equals_sdpa(t_q, t_kv):
    w, inp = generate_small(t_q=t_q, t_kv=t_kv, groups=2, heads=3, head_dim=8, index_dim=4,
                            block=8, topk=64, seed=3)
    sel, out, _ = oracle.forward(inp, w.block, w.topk, w.softmax_scale)
    pos = torch.arange(t_kv - t_q, t_kv)
    mask = torch.arange(t_kv)[None, :] <= pos[:, None]            # bottom-right causal
    ref = _sdpa_reference(inp, mask, w.softmax_scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_attention_sparse_equals_masked_sdpa():
    """A sparse selection equals dense SDPA under the selection's token mask (built from sel)."""
    w, inp = generate_small(t_q=48, t_kv=80, groups=2, heads=2, head_dim=8, index_dim=4,
                            block=4, topk=16, seed=9)
    sel, out, _ = oracle.forward(inp, w.block, w.topk, w.softmax_scale)
    pos = np.arange(w.t_kv - w.t_q, w.t_kv)
    for g in range(w.groups):
        mask = torch.zeros(w.t_q, w.t_kv, dtype=torch.bool)
        for i in range(w.t_q):
            chosen = set(sel[0, i, g].tolist()) - {-1}
            for t in range(w.t_kv):
                mask[i, t] = bool((t // w.block) in chosen and t <= int(pos[i]))
        sub = {n: inp[n][:, :, g:g + 1] for n in ("q", "gate")}
        sub.update({n: inp[n][:, g:g + 1] for n in ("k", "v")})
        ref = _sdpa_reference(sub, mask, w.softmax_scale)
        np.testing.assert_allclose(out[:, :, g:g + 1], ref, rtol=0, atol=1e-12)
        # the test is only meaningful if late queries really are sparse
        assert (sel[0, -1, g] >= 0).sum() == w.n_sel


def test_attention_constant_values_and_first_token():
    rng = np.random.default_rng(8)
    q = rng.normal(size=(4, 16))
    k = rng.normal(size=(30, 16))
    g = rng.normal(size=(4, 16))
    c = rng.normal(size=16)
    v = np.tile(c, (30, 1))
    toks = np.array([0, 3, 4, 9, 17])
    out = oracle.gated_attention(q, k, v, g, toks, 0.3)
    np.testing.assert_allclose(out, c[None, :] / (1 + np.exp(-g)), rtol=1e-14, atol=1e-15)
    v2 = rng.normal(size=(30, 16))
    out0 = oracle.gated_attention(q, k, v2, g, np.array([0]), 0.3)
    np.testing.assert_allclose(out0, v2[0][None, :] / (1 + np.exp(-g)), rtol=1e-14, atol=1e-15)


def test_attention_token_order_invariant():
    rng = np.random.default_rng(9)
    q, k, v, g = (rng.normal(size=s) for s in ((2, 8), (40, 8), (40, 8), (2, 8)))
    toks = np.array([1, 5, 6, 20, 33, 39])
    a = oracle.gated_attention(q, k, v, g, toks, 0.5)
    b = oracle.gated_attention(q, k, v, g, toks[::-1].copy(), 0.5)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------------------------
# inclusion rate (a measured property of the inputs): its definition's edge cases, and brute force
# on tiny inputs
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg_a,cfg_b", [((4, 16), (1, 8)), ((8, 16), (2, 12)), ((3, 9), (1, 5))])
def test_inclusion_rate_brute_force(cfg_a, cfg_b):
    """|A_a & A_b| / |A_b| per (query, group), with both selections taken by the O(n^2) rank count
    (no sort), the attended sets built token by token and the ratio as an exact fraction.  The two
    sets have different sizes, so swapping numerator and denominator roles, or the two configs,
    fails."""
    from fractions import Fraction
    T = 48
    w, inp = generate_small(t_q=20, t_kv=T, groups=2, index_dim=3, seed=31)
    rows = [(0, i) for i in range(20)]
    got = oracle.inclusion_rate(inp["q_idx"], inp["k_idx"], rows, T, cfg_a, cfg_b)
    k_idx = inp["k_idx"][0].double().numpy()
    q_idx = inp["q_idx"][0].double().numpy()

    def attended(q, p, B, k):
        nb = -(-T // B)
        kb = [[sum(k_idx[t, c] for t in range(j * B, min(j * B + B, T))) for c in range(3)]
              for j in range(nb)]
        o = p // B
        s = [sum(q[c] * kb[j][c] for c in range(3)) for j in range(o)]
        chosen = _brute_force_selection(s, o, k // B)
        return {t for t in range(p + 1) if t // B in chosen}

    n_strict = 0
    for r, (_, i) in enumerate(rows):
        p = T - 20 + i
        for g in range(2):
            a = attended(q_idx[i, g], p, *cfg_a)
            b = attended(q_idx[i, g], p, *cfg_b)
            want = Fraction(len(a & b), len(b))
            assert got[r, g] == float(want), (p, g)
            n_strict += want < 1
    assert n_strict > 0                      # the case exercises partial inclusion


def test_inclusion_rate_edge_cases():
    w, inp = generate_small(t_q=64, t_kv=64, groups=2, index_dim=4, seed=2)
    rows = [(0, i) for i in range(64)]
    same = oracle.inclusion_rate(inp["q_idx"], inp["k_idx"], rows, 64, (1, 16), (1, 16))
    assert np.all(same == 1.0)
    dense = oracle.inclusion_rate(inp["q_idx"], inp["k_idx"], rows, 64, (8, 64), (1, 16))
    assert np.all(dense == 1.0)          # a dense selection includes everything
    r = oracle.inclusion_rate(inp["q_idx"], inp["k_idx"], rows, 64, (8, 16), (1, 16))
    assert np.all((r >= 0) & (r <= 1)) and r.min() < 1.0


# ----------------------------------------------------------------------------------------------
# sequences of different lengths (decode over a cache)
# ----------------------------------------------------------------------------------------------
def test_sequence_rows_equal_lengths_is_forward():
    """With every sequence holding all t_kv tokens, the per-sequence reading is the forward's."""
    w, inp = generate_small(t_q=5, t_kv=90, groups=2, heads=2, head_dim=8, index_dim=4, block=8,
                            topk=32, seed=21, batch=3)
    rows = [(b, i) for b in range(3) for i in range(5)]
    s_ref, o_ref, _ = oracle.forward_rows(inp, w.block, w.topk, w.softmax_scale, rows)
    s, o, _ = oracle.sequence_rows(inp, [90, 90, 90], w.block, w.topk, w.softmax_scale, rows)
    assert np.array_equal(s, s_ref)
    np.testing.assert_array_equal(o, o_ref)


def test_sequence_rows_dense_equals_sdpa_on_prefix():
    """Budget covering the context: each sequence's queries are the last t_q of its own L tokens,
    so the result is dense SDPA over k[:, :L] with a bottom-right causal mask (torch, fp64)."""
    t_q, t_kv = 4, 70
    w, inp = generate_small(t_q=t_q, t_kv=t_kv, groups=2, heads=3, head_dim=8, index_dim=4,
                            block=8, topk=128, seed=5, batch=3)
    lens = [70, 41, 9]
    rows = [(b, i) for b in range(3) for i in range(t_q)]
    _, out, _ = oracle.sequence_rows(inp, lens, w.block, w.topk, w.softmax_scale, rows)
    for b, L in enumerate(lens):
        sub = {"q": inp["q"][b:b + 1], "gate": inp["gate"][b:b + 1],
               "k": inp["k"][b:b + 1, :, :L], "v": inp["v"][b:b + 1, :, :L]}
        pos = torch.arange(L - t_q, L)
        mask = torch.arange(L)[None, :] <= pos[:, None]
        ref = _sdpa_reference(sub, mask, w.softmax_scale)[0]
        np.testing.assert_allclose(out[b * t_q:(b + 1) * t_q], ref, rtol=0, atol=1e-12)


def test_sequence_rows_ignore_tokens_past_length():
    """Keys, values and index keys past a sequence's length do not change its rows."""
    w, inp = generate_small(t_q=3, t_kv=120, groups=2, heads=2, head_dim=8, index_dim=4, block=8,
                            topk=32, seed=8, batch=2)
    lens = [120, 77]
    rows = [(b, i) for b in range(2) for i in range(3)]
    s1, o1, k1 = oracle.sequence_rows(inp, lens, w.block, w.topk, w.softmax_scale, rows)
    other = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in inp.items()}
    other["k"][1, :, 77:] = 100.0
    other["v"][1, :, 77:] = -100.0
    other["k_idx"][1, 77:] = 4.0
    s2, o2, k2 = oracle.sequence_rows(other, lens, w.block, w.topk, w.softmax_scale, rows)
    assert np.array_equal(s1, s2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(k1[1], k2[1])
    assert k1[1].shape[0] == -(-77 // 8)


# ----------------------------------------------------------------------------------------------
# gated sliding-window attention
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("window", [1, 5, 16, 37])
def test_window_equals_band_masked_sdpa(window):
    """torch SDPA (fp64) with an explicit band mask t in [p - window + 1, p], times sigmoid(gate)."""
    t_q, t_kv = 30, 70
    w, inp = generate_small(t_q=t_q, t_kv=t_kv, groups=2, heads=3, head_dim=8, index_dim=4,
                            block=8, topk=64, seed=17)
    rows = [(0, i) for i in range(t_q)]
    out = oracle.window_rows(inp, window, w.softmax_scale, rows)
    pos = torch.arange(t_kv - t_q, t_kv)
    t = torch.arange(t_kv)[None, :]
    mask = (t <= pos[:, None]) & (t > pos[:, None] - window)
    ref = _sdpa_reference(inp, mask, w.softmax_scale)[0]
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_window_one_is_own_value_and_wide_window_is_dense():
    w, inp = generate_small(t_q=12, t_kv=40, groups=2, heads=2, head_dim=8, index_dim=4, block=8,
                            topk=64, seed=2)
    rows = [(0, i) for i in range(12)]
    one = oracle.window_rows(inp, 1, w.softmax_scale, rows)
    v = inp["v"].to(torch.float64).numpy()[0]               # [G, Tkv, d]
    gate = torch.sigmoid(inp["gate"].to(torch.float64)).numpy()[0]   # [Tq, G, h, d]
    for i in range(12):
        p = 40 - 12 + i
        np.testing.assert_allclose(one[i], gate[i] * v[:, p][:, None, :], rtol=0, atol=1e-15)
    wide = oracle.window_rows(inp, 1000, w.softmax_scale, rows)
    _, dense, _ = oracle.forward(inp, w.block, 4096, w.softmax_scale)
    np.testing.assert_allclose(wide, dense[0], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# fp8 e4m3 codes (the fp8-KV variant)
# ----------------------------------------------------------------------------------------------
def test_e4m3_decode_matches_torch_and_fixed_points():
    codes = np.arange(256)
    got = oracle.e4m3_decode(codes)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # hand-worked codes: 1.0, the largest finite value, the smallest subnormal, -2.0
    assert oracle.e4m3_decode([0x38, 0x7E, 0x01, 0xC0]).tolist() == [1.0, 448.0, 2.0 ** -9, -2.0]


# ----------------------------------------------------------------------------------------------
# backward of the gated attention step
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("topk", [16, 256])
def test_attention_backward_equals_autograd(topk):
    """torch autograd (fp64) through dense SDPA under the selection's token mask, times
    sigmoid(gate): the library routine's gradients equal the oracle's explicit chain rule."""
    w, inp = generate_small(t_q=24, t_kv=60, groups=2, heads=3, head_dim=8, index_dim=4, block=4,
                            topk=topk, seed=31)
    sel, _, _ = oracle.forward(inp, w.block, w.topk, w.softmax_scale)
    g = torch.Generator().manual_seed(5)
    dout = torch.randn(inp["q"].shape, generator=g, dtype=torch.float64)
    dq, dk, dv, dgate = oracle.attention_backward(inp, sel, dout, w.block, w.softmax_scale)

    pos = np.arange(w.t_kv - w.t_q, w.t_kv)
    leaves = {n: inp[n].to(torch.float64).clone().requires_grad_(True) for n in ("q", "k", "v", "gate")}
    outs = []
    for gg in range(w.groups):
        mask = torch.zeros(w.t_q, w.t_kv, dtype=torch.bool)
        for i in range(w.t_q):
            toks = oracle.attended_tokens(sel[0, i, gg], w.block, int(pos[i]), w.t_kv)
            mask[i, torch.from_numpy(toks)] = True
        qg = leaves["q"][0, :, gg].transpose(0, 1)                            # [h, Tq, d]
        kg = leaves["k"][0, gg].unsqueeze(0).expand(qg.shape[0], -1, -1)
        vg = leaves["v"][0, gg].unsqueeze(0).expand(qg.shape[0], -1, -1)
        o = torch.nn.functional.scaled_dot_product_attention(qg, kg, vg, attn_mask=mask,
                                                             scale=w.softmax_scale)
        outs.append(o.transpose(0, 1) * torch.sigmoid(leaves["gate"][0, :, gg]))
    out = torch.stack(outs, dim=1).unsqueeze(0)
    out.backward(dout)
    for name, mine in (("q", dq), ("k", dk), ("v", dv), ("gate", dgate)):
        np.testing.assert_allclose(mine, leaves[name].grad.numpy(), rtol=0, atol=1e-12, err_msg=name)


def test_attention_backward_single_token_closed_form():
    """One attended token (p = 0): out = sigmoid(g) v_0, so dq = 0, dk_0 = 0, dv_0 = sum over
    query heads of dout * sigmoid(g), dgate = dout * v_0 * sigmoid'(g)."""
    w, inp = generate_small(t_q=1, t_kv=1, groups=1, heads=2, head_dim=4, index_dim=4, block=4,
                            topk=8, seed=4)
    sel, _, _ = oracle.forward(inp, w.block, w.topk, w.softmax_scale)
    dout = torch.ones(inp["q"].shape, dtype=torch.float64) * 0.5
    dq, dk, dv, dgate = oracle.attention_backward(inp, sel, dout, w.block, w.softmax_scale)
    sg = torch.sigmoid(inp["gate"].to(torch.float64)).numpy()[0, 0, 0]        # [h, d]
    v0 = inp["v"].to(torch.float64).numpy()[0, 0, 0]
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
    np.testing.assert_allclose(dv[0, 0, 0], (0.5 * sg).sum(axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(dgate[0, 0, 0], 0.5 * v0[None, :] * sg * (1 - sg), rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------------------------
# softmax normaliser (log-sum-exp) a training forward keeps for the backward
# ----------------------------------------------------------------------------------------------
def test_lse_equals_masked_torch_logsumexp():
    """torch.logsumexp (fp64) of the scaled logits under the selection's token mask, -inf
    elsewhere, equals the oracle's per-row normaliser."""
    w, inp = generate_small(t_q=20, t_kv=52, groups=2, heads=3, head_dim=8, index_dim=4, block=4,
                            topk=16, seed=41)
    sel, _, _ = oracle.forward(inp, w.block, w.topk, w.softmax_scale)
    rows = list(range(w.t_q))
    lse = oracle.attention_lse(inp, sel, w.block, w.softmax_scale, rows)
    pos = np.arange(w.t_kv - w.t_q, w.t_kv)
    q64, k64 = inp["q"].to(torch.float64), inp["k"].to(torch.float64)
    for g in range(w.groups):
        mask = torch.zeros(w.t_q, w.t_kv, dtype=torch.bool)
        for i in range(w.t_q):
            toks = oracle.attended_tokens(sel[0, i, g], w.block, int(pos[i]), w.t_kv)
            mask[i, torch.from_numpy(toks)] = True
        s = w.softmax_scale * torch.einsum("ihd,td->iht", q64[0, :, g], k64[0, g])
        s = s.masked_fill(~mask[:, None, :], float("-inf"))
        ref = torch.logsumexp(s, dim=-1).numpy()
        np.testing.assert_allclose(lse[0, :, g], ref, rtol=0, atol=1e-12)


def test_lse_closed_forms():
    """q = 0: every logit is 0, so lse = ln(number of attended tokens); a query at position 0
    attends token 0 only, so lse = scale q.k_0."""
    w, inp = generate_small(t_q=12, t_kv=12, groups=1, heads=2, head_dim=8, index_dim=4, block=4,
                            topk=64, seed=42)                         # dense: every past token
    sel, _, _ = oracle.forward(inp, w.block, w.topk, w.softmax_scale)
    zero = dict(inp, q=torch.zeros_like(inp["q"]))
    lse0 = oracle.attention_lse(zero, sel, w.block, w.softmax_scale, list(range(w.t_q)))
    expect = np.log(np.arange(1, w.t_q + 1, dtype=np.float64))        # query i attends 0..i
    np.testing.assert_allclose(lse0[0, :, 0], np.repeat(expect[:, None], 2, axis=1), rtol=0,
                               atol=1e-14)
    lse = oracle.attention_lse(inp, sel, w.block, w.softmax_scale, [0])
    q0 = inp["q"].to(torch.float64).numpy()[0, 0, 0]                  # [h, d]
    k0 = inp["k"].to(torch.float64).numpy()[0, 0, 0]
    np.testing.assert_allclose(lse[0, 0, 0], w.softmax_scale * (q0 @ k0), rtol=0, atol=1e-14)


def test_lse_normalises_the_attention():
    """sum_t exp(s_t - lse) = 1, and sum_t exp(s_t - lse) v_t is the ungated attention output."""
    w, inp = generate_small(t_q=9, t_kv=40, groups=2, heads=2, head_dim=8, index_dim=4, block=4,
                            topk=12, seed=43)
    sel, out, _ = oracle.forward(inp, w.block, w.topk, w.softmax_scale)
    lse = oracle.attention_lse(inp, sel, w.block, w.softmax_scale, list(range(w.t_q)))
    pos = np.arange(w.t_kv - w.t_q, w.t_kv)
    q, k, v = (inp[n].to(torch.float64).numpy() for n in ("q", "k", "v"))
    sg = torch.sigmoid(inp["gate"].to(torch.float64)).numpy()
    for i in range(w.t_q):
        for g in range(w.groups):
            toks = oracle.attended_tokens(sel[0, i, g], w.block, int(pos[i]), w.t_kv)
            p = np.exp(w.softmax_scale * (q[0, i, g] @ k[0, g, toks].T) - lse[0, i, g][:, None])
            np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
            np.testing.assert_allclose(p @ v[0, g, toks] * sg[0, i, g], out[0, i, g], rtol=0,
                                       atol=1e-13)
