"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the same seeded inputs.

Selections and block scores must be bit-exact (integer-valued index data makes them exact);
outputs within max-abs 1e-5 (fp32) or 1e-2 (bf16).  Small cases are checked on every row; the
full-size workloads on stratified sampled rows plus structural checks of every row's selection.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_sgqa_amd as sg
import oracle
from gpu_helpers import (check_out, check_sel_rows, oracle_rows, run_forward, run_split,
                         sample_tokens, say, structural_check_sel, to_dev)
from sgqa_inputs import generate, generate_small, get_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()     # fails loudly if the HIP library is missing


# ----------------------------------------------------------------------------------------------
# tiny workload (fp32): every row, every step
# ----------------------------------------------------------------------------------------------
def test_tiny_every_step_every_row():
    w = get_workload("tiny")
    say("case: tiny", w)
    x = to_dev(generate(w, seed=0))
    prob = sg.Problem.from_workload(w)
    k_blk, scores, sel, out = run_split(prob, x)
    sel_ref, out_ref, kblk_ref = oracle.forward(x, w.block, w.topk, w.softmax_scale)
    np.testing.assert_array_equal(k_blk.cpu().double().numpy(), kblk_ref)
    # every defined score (j < p/B) equals the oracle's exactly
    sc = scores.cpu().double().numpy()
    kb = kblk_ref[0]
    qi = x["q_idx"].cpu().double().numpy()[0]
    for i in range(0, w.t_q, 97):
        o = i // w.block
        for g in range(w.groups):
            np.testing.assert_array_equal(sc[0, i, g, :o], oracle.block_scores(qi[i, g], kb, o))
    check_sel_rows(sel, sel_ref)
    check_out(out, out_ref, fp32=True, what="tiny split")
    out2, sel2 = run_forward(prob, x)
    assert torch.equal(sel2, sel)
    check_out(out2, out_ref, fp32=True, what="tiny forward")


# ----------------------------------------------------------------------------------------------
# small bf16 cases through the matrix-core path: ragged shapes, several block sizes, every row
# ----------------------------------------------------------------------------------------------
SMALL_CASES = [
    # t_q, t_kv, block, topk, groups, index_dim, sharp, head_dim, batch
    (300, 1001, 8, 256, 2, 128, False, 128, 1),
    (517, 517, 8, 128, 3, 64, False, 128, 1),
    (517, 517, 8, 128, 2, 128, True, 128, 1),
    (257, 700, 16, 256, 2, 32, False, 128, 1),
    (401, 601, 4, 128, 2, 128, False, 128, 1),
    (333, 333, 2, 64, 1, 128, True, 128, 1),
    (1, 333, 8, 64, 2, 128, False, 128, 1),
    (2, 2, 8, 64, 2, 128, False, 128, 1),
    (64, 64, 8, 4096, 2, 128, False, 128, 1),      # budget covers the whole context: dense
    (301, 999, 8, 256, 2, 128, True, 64, 1),       # head dim 64
    (203, 650, 16, 128, 2, 64, False, 64, 1),
    (150, 700, 8, 128, 2, 128, True, 128, 3),      # several sequences
    (7, 1300, 8, 256, 2, 128, False, 128, 2),      # a short query chunk at the end of the keys
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "tq%d-tk%d-B%d-k%d-G%d-di%d%s-d%d-b%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "-sharp" if c[6] else "", c[7], c[8]))
def test_small_bf16_every_row(case):
    t_q, t_kv, B, k, G, di, sharp, d, bt = case
    say("case:", case)
    w, x = generate_small(batch=bt, t_q=t_q, t_kv=t_kv, groups=G, heads=8, head_dim=d,
                          index_dim=di, block=B, topk=k, dtype="bf16", index_dtype="bf16",
                          scaled_qkv=True, needles=1 if (t_kv // B) >= 2 * G else 0, seed=11,
                          device="cuda", sharp=sharp)
    prob = sg.Problem.from_workload(w)
    k_blk, scores, sel, out = run_split(prob, x)
    sel_ref, out_ref, kblk_ref = oracle.forward(x, B, k, w.softmax_scale)
    np.testing.assert_array_equal(k_blk.cpu().double().numpy(), kblk_ref)
    check_sel_rows(sel, sel_ref)
    structural_check_sel(sel, prob)
    check_out(out, out_ref, fp32=False, what="split")
    out2, sel2 = run_forward(prob, x)
    assert torch.equal(sel2, sel)
    assert torch.equal(out2, out)


# ----------------------------------------------------------------------------------------------
# bf16 indexer scores, element by element, and the untouched tail of every score row
# ----------------------------------------------------------------------------------------------
# (t_q, t_kv, block, groups, index_dim, batch): the first three have at most 32 rows per sequence
# (index_rows32_kernel for index dims 128, 64 and 32); the others take the tiled index_bf16_kernel
INDEX_CASES = [
    (7, 1300, 8, 2, 128, 2),
    (5, 900, 8, 3, 64, 1),
    (16, 2000, 16, 2, 32, 1),
    (300, 1001, 8, 2, 128, 1),
    (517, 517, 8, 3, 64, 1),
    (257, 700, 16, 2, 32, 1),
    (401, 601, 4, 2, 128, 1),
    (150, 700, 8, 2, 128, 3),
]
SENTINEL = 0x7FC0BEEF          # a NaN payload no score can take


@pytest.mark.parametrize("case", INDEX_CASES, ids=lambda c: "tq%d-tk%d-B%d-G%d-di%d-b%d" % c)
def test_index_scores_every_row_bf16(case):
    """sgqa_index on bf16 index data: every defined score (j < p/B) equals the oracle's block score
    exactly, and every entry j >= p/B keeps the value the buffer held before the call."""
    t_q, t_kv, B, G, di, bt = case
    say("case: index scores", case)
    w, x = generate_small(batch=bt, t_q=t_q, t_kv=t_kv, groups=G, heads=8, head_dim=64,
                          index_dim=di, block=B, topk=64 * B, dtype="bf16", index_dtype="bf16",
                          scaled_qkv=True, needles=1 if (t_kv // B) >= 2 * G else 0, seed=21,
                          device="cuda")
    prob = sg.Problem.from_workload(w)
    scores = torch.empty((bt, t_q, G, prob.num_blocks), dtype=torch.float32, device="cuda")
    scores.view(torch.int32).fill_(SENTINEL)
    k_blk, scores = sg.index(prob, x["q_idx"], x["k_idx"], scores=scores)
    torch.cuda.synchronize()
    kblk_ref = oracle.compress(x["k_idx"].cpu().double().numpy(), B)
    np.testing.assert_array_equal(k_blk.cpu().double().numpy(), kblk_ref)
    sc = scores.cpu()
    bits = sc.view(torch.int32).numpy()
    sc = sc.double().numpy()
    qi = x["q_idx"].cpu().double().numpy()
    pos = oracle.query_positions(t_q, t_kv)
    for b in range(bt):
        for i in range(t_q):
            o = int(pos[i]) // B
            for g in range(G):
                np.testing.assert_array_equal(sc[b, i, g, :o], oracle.block_scores(qi[b, i, g], kblk_ref[b], o),
                                              err_msg=f"row b={b} i={i} g={g}")
                assert (bits[b, i, g, o:] == SENTINEL).all(), f"tail written at b={b} i={i} g={g}"


@pytest.mark.parametrize("sharp", [False, True])
def test_bf16_output_error_budget(sharp):
    """The bf16 forward's rounding budget, element by element.  The attention rounds each
    probability to bf16 for the P.V product (relative 2^-9 per weight, the same rounded values
    entering the row sum), rounds each unit range's partial O/l to bf16 before the merge (relative
    2^-9: the merged value is a convex combination of the partials, so this adds at most
    2^-9 max|v| over the attended tokens), and rounds the gated result once more (2^-9 |out|).
    Bound per element: sigmoid(gate) * 2 * 2^-9 * max|v| + 2^-9 |ref|, with max|v| taken over the
    whole (sequence, group) as an upper bound of the attended tokens' maximum, doubled for fp32
    accumulation and the exp2 approximation."""
    t_q, t_kv = 400, 2600
    w, x = generate_small(t_q=t_q, t_kv=t_kv, groups=2, heads=8, head_dim=128, index_dim=128,
                          block=8, topk=512, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          needles=2, seed=23, device="cuda", sharp=sharp)
    prob = sg.Problem.from_workload(w)
    out, sel = run_forward(prob, x)
    sel_ref, out_ref, _ = oracle.forward(x, w.block, w.topk, w.softmax_scale)
    check_sel_rows(sel, sel_ref)
    got = out.to("cpu", torch.float64).numpy()
    gate = x["gate"].to("cpu", torch.float64).numpy()
    vmax = x["v"].abs().amax(dim=(2, 3)).to("cpu", torch.float64).numpy()      # [Bt, G]
    sig = 1.0 / (1.0 + np.exp(-gate))
    bound = 2.0 * (sig * 2.0 * 2.0 ** -9 * vmax[:, None, :, None, None] + 2.0 ** -9 * np.abs(out_ref))
    err = np.abs(got - out_ref)
    ratio = float((err / bound).max())
    say(f"  error / budget: max {ratio:.3f}, max-abs err {float(err.max()):.3e}")
    assert ratio <= 1.0


# block sizes that neither divide 8 nor are multiples of 8 (the plain attention kernel), and
# one multiple of 8 above 16 (the range kernel), through both the split calls and the forward
OTHER_BLOCK_CASES = [
    # t_q, t_kv, block, topk, dtype
    (200, 700, 3, 96, "bf16"),
    (150, 601, 5, 100, "bf16"),
    (120, 900, 12, 144, "bf16"),
    (130, 1000, 24, 240, "bf16"),
    (90, 400, 3, 48, "f32"),
]


@pytest.mark.parametrize("case", OTHER_BLOCK_CASES, ids=lambda c: "tq%d-tk%d-B%d-k%d-%s" % c)
def test_other_block_sizes_every_row(case):
    t_q, t_kv, B, k, dt = case
    say("case: block size", case)
    w, x = generate_small(t_q=t_q, t_kv=t_kv, groups=2, heads=8, head_dim=64, index_dim=32,
                          block=B, topk=k, dtype=dt, index_dtype=dt, scaled_qkv=dt == "bf16",
                          needles=1, seed=29, device="cuda", sharp=True)
    prob = sg.Problem.from_workload(w)
    k_blk, scores, sel, out = run_split(prob, x)
    sel_ref, out_ref, kblk_ref = oracle.forward(x, B, k, w.softmax_scale)
    np.testing.assert_array_equal(k_blk.cpu().double().numpy(), kblk_ref)
    check_sel_rows(sel, sel_ref)
    structural_check_sel(sel, prob)
    check_out(out, out_ref, fp32=dt == "f32", what=f"split B={B}")
    out2, sel2 = run_forward(prob, x)
    assert torch.equal(sel2, sel)
    check_out(out2, out_ref, fp32=dt == "f32", what=f"forward B={B}")


def test_block_one_selection_is_token_level():
    """B = 1 (token-level, the pages' comparison setting) through index + top-k."""
    w, x = generate_small(t_q=700, t_kv=900, groups=2, heads=8, head_dim=128, index_dim=128,
                          block=1, topk=128, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          seed=5, device="cuda")
    prob = sg.Problem.from_workload(w)
    _, scores = sg.index(prob, x["q_idx"], x["k_idx"])
    sel = sg.topk(prob, scores)
    torch.cuda.synchronize()
    rows = [(0, i) for i in range(w.t_q)]
    sel_ref, _, _ = oracle_rows(prob, x, rows)
    check_sel_rows(sel[0], sel_ref)


def test_topk_long_rows_aligned_and_unaligned():
    """Split top-k on rows longer than its 2048-entry direct limit, with NB = 2501 blocks: score
    rows start at 16-byte aligned addresses only for every fourth row, so both the vector and the
    scalar streaming paths run; every row's selection must equal the oracle's."""
    w, x = generate_small(t_q=24, t_kv=20008, groups=2, heads=8, head_dim=64, index_dim=32,
                          block=8, topk=256, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          seed=9, device="cuda")
    say("case: top-k long rows, NB = 2501")
    prob = sg.Problem.from_workload(w)
    _, scores = sg.index(prob, x["q_idx"], x["k_idx"])
    sel = sg.topk(prob, scores)
    torch.cuda.synchronize()
    assert scores.shape[-1] == 2501
    rows = [(0, i) for i in range(w.t_q)]
    sel_ref, _, _ = oracle_rows(prob, x, rows)
    check_sel_rows(sel[0], sel_ref)


@pytest.mark.parametrize("t_kv,di", [(40000, 64), (40000, 128), (300000, 128)],
                         ids=["o5000-di64", "o5000-di128", "o37500-di128"])
def test_sampled_threshold_every_row(t_kv, di):
    """The fused selection's sampled thresholds on every row: about 5000 causal blocks (the
    384-sample path and 96-column tiles) and 37 500 (past 32 768: the two-pass histogram path)."""
    w, x = generate_small(t_q=24, t_kv=t_kv, groups=2, heads=8, head_dim=64, index_dim=di,
                          block=8, topk=4096, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          seed=12, device="cuda")
    say(f"case: sampled thresholds, t_kv={t_kv}, di={di}")
    prob = sg.Problem.from_workload(w)
    out, sel = run_forward(prob, x)
    rows = [(0, i) for i in range(w.t_q)]
    sel_ref, out_ref, _ = oracle_rows(prob, x, rows)
    check_sel_rows(sel[0], sel_ref)
    check_out(out[0], out_ref, fp32=False, what=f"sampled thresholds t_kv={t_kv}")


def test_more_failed_rows_than_wide_fallback():
    """Constant index keys on 320 rows (40 tokens x 8 groups) of about 2500 causal blocks: every
    block ties and passes its threshold, every candidate list overflows, and all 320 rows take the
    exact recomputation -- 256 through the wide score recompute, the rest through the per-row loop.
    Ties go to the lowest blocks."""
    w, x = generate_small(t_q=40, t_kv=20000, groups=8, heads=8, head_dim=64, index_dim=64,
                          block=8, topk=4096, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          seed=5, device="cuda")
    x["k_idx"].fill_(0.5)
    say("case: 320 failed rows (wide fallback + per-row loop)")
    prob = sg.Problem.from_workload(w)
    out, sel = run_forward(prob, x)
    rows = [(0, i) for i in range(w.t_q)]
    sel_ref, out_ref, _ = oracle_rows(prob, x, rows)
    check_sel_rows(sel[0], sel_ref)
    check_out(out[0], out_ref, fp32=False, what="320 failed rows")


def test_heavy_ties_and_negative_zero():
    """Constant index keys: every candidate ties, so the lowest block indices must win."""
    w, x = generate_small(t_q=600, t_kv=600, groups=2, heads=8, head_dim=128, index_dim=32,
                          block=8, topk=128, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          seed=3, device="cuda")
    x["k_idx"].fill_(1.0)
    x["q_idx"][:, :, 0].fill_(0.0)          # group 0: every score is +0.0
    x["q_idx"][:, :, 1].fill_(-1.0)         # group 1: every score is -32 (all equal)
    prob = sg.Problem.from_workload(w)
    k_blk, scores, sel, out = run_split(prob, x)
    sel_ref, out_ref, _ = oracle.forward(x, w.block, w.topk, w.softmax_scale)
    check_sel_rows(sel, sel_ref)
    check_out(out, out_ref, fp32=False, what="ties")


def test_forward_chunked_workspace_matches():
    """sgqa_forward with a workspace that forces many query-row chunks gives the same result."""
    w, x = generate_small(t_q=900, t_kv=1200, groups=2, heads=8, head_dim=128, index_dim=128,
                          block=8, topk=256, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          needles=2, seed=8, device="cuda")
    prob = sg.Problem.from_workload(w)
    out_a, sel_a = run_forward(prob, x)
    s = sg.sizes(prob)
    lo, hi = s["forward_workspace_min_bytes"], s["forward_workspace_bytes"]
    small = lo + (hi - lo) // 23                              # many query-token chunks
    ws = torch.empty(small, dtype=torch.uint8, device="cuda")
    out_b, sel_b = run_forward(prob, x, workspace=ws)
    assert torch.equal(sel_a, sel_b)
    assert torch.equal(out_a, out_b)


def test_run_to_run_bitwise():
    w, x = generate_small(t_q=512, t_kv=800, groups=2, heads=8, head_dim=128, index_dim=128,
                          block=8, topk=256, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          seed=4, device="cuda")
    prob = sg.Problem.from_workload(w)
    a = run_forward(prob, x)
    b = run_forward(prob, x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ----------------------------------------------------------------------------------------------
# full-size workloads: sampled rows against the oracle, structural checks on every row
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,n_random,sharp", [("32k", 24, False), ("128k", 12, False),
                                                ("1m", 6, False), ("32k", 24, True),
                                                ("128k", 12, True), ("1m", 6, True),
                                                ("128k-drift", 12, False)],
                         ids=["32k", "128k", "1m", "32k-sharp", "128k-sharp", "1m-sharp",
                              "128k-drift"])
def test_workload_sampled_rows(name, n_random, sharp):
    """Full-size workloads on stratified sampled rows.  The "sharp" variants leave q and k unscaled,
    so the softmax is far from uniform and a wrong weight or a dropped token shows in the output."""
    w = get_workload(name)
    say("case:", name, "sharp" if sharp else "")
    x = generate(w, device="cuda", seed=0, sharp=sharp)
    prob = sg.Problem.from_workload(w)
    out, sel = run_forward(prob, x)
    structural_check_sel(sel, prob)
    toks = sample_tokens(w.t_q, w.t_kv, w.block, w.n_sel, n_random)
    rows = [(0, i) for i in toks]
    say(f"  oracle on {len(rows)} tokens x {w.groups} groups")
    sel_ref, out_ref, _ = oracle_rows(prob, x, rows)
    check_sel_rows(sel[0, toks], sel_ref)
    check_out(out[0, toks], out_ref, fp32=False, what=name)
    # needles of a group are always among that group's picks for late queries
    last = sel[0, -1].cpu().numpy()
    for g in range(w.groups):
        assert set(x["needle_blocks"][g].tolist()) <= set(last[g].tolist())
    del x, out, sel
    torch.cuda.empty_cache()


@pytest.mark.parametrize("t_q", [64, 3])
def test_long_context_union_every_row(t_q):
    """Every row at 524 288 keys.  With t_q = 64 the group lists come from merging the tokens'
    selections (contexts past 128K tokens); with t_q = 3 there is one group of tokens, so the
    attention's waves take its unit ranges, the lists split at equal entry counts and they are
    built through bitmaps scanned four words at a time (2 048 words per token).

    q = 0 makes every logit 0, so each output is sigmoid(0) = 0.5 times the mean of v over the
    attended tokens; v is one-hot per token: dim (unit mod 64) and dim 64 + (unit // 64 mod 64).
    Each output is then a count of attended units per residue class divided by |A|, computed
    exactly on the device up to the bf16 rounding of the range partials and of the output
    (relative 2^-8 at most).  A residue class holds about 8 of a row's 512 units, so one dropped
    or extra 8-token unit moves some output by several percent of its value (or from 0 to about
    1e-3), far outside the 2^-7 relative bar below."""
    t_kv, G, B = 524288, 2, 8
    w, x = generate_small(t_q=t_q, t_kv=t_kv, groups=G, heads=8, head_dim=128, index_dim=128,
                          block=B, topk=4096, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          needles=2, seed=17, device="cuda")
    say(f"case: long-context unions, t_kv={t_kv}, t_q={t_q}")
    x["q"].zero_()
    x["gate"].zero_()
    unit = torch.arange(t_kv, device="cuda") // 8
    v = torch.zeros((t_kv, 128), dtype=torch.bfloat16, device="cuda")
    v[torch.arange(t_kv, device="cuda"), unit % 64] = 1.0
    v[torch.arange(t_kv, device="cuda"), 64 + (unit // 64) % 64] = 1.0
    x["v"] = v.expand(1, G, t_kv, 128).contiguous()
    prob = sg.Problem.from_workload(w)
    out, sel = run_forward(prob, x)
    structural_check_sel(sel, prob)
    rows = [(0, i) for i in range(t_q)]
    sel_ref, out_ref, _ = oracle_rows(prob, x, rows)
    check_sel_rows(sel[0], sel_ref)
    got = out[0].to("cpu", torch.float64).numpy()
    err = np.abs(got - out_ref)
    bar = 2.0 ** -7 * np.abs(out_ref) + 1e-7
    say(f"  max relative error {float((err / (np.abs(out_ref) + 1e-30)).max()):.3e}")
    assert (err <= bar).all(), f"{int((err > bar).sum())} outputs outside the bar"
    del x, out, sel
    torch.cuda.empty_cache()


@pytest.mark.parametrize("sharp", [False, True], ids=["plain", "sharp"])
def test_decode_sampled_sequences(sharp):
    w = get_workload("decode")
    say("case: decode", "sharp" if sharp else "")
    x = generate(w, device="cuda", seed=0, sharp=sharp)
    prob = sg.Problem.from_workload(w)
    out, sel = run_forward(prob, x)
    structural_check_sel(sel, prob)
    # a small grid (2 token pairs per sequence) leaves many loads in flight per wave: repeated runs
    # must agree bit for bit, or a pipelined kernel read an operand before it landed
    for _ in range(2):
        again, sel_again = run_forward(prob, x)
        assert torch.equal(again, out) and torch.equal(sel_again, sel), "decode run-to-run"
        del again, sel_again
    rows = [(b, i) for b in (0, 37) for i in range(w.t_q)]
    sel_ref, out_ref, _ = oracle_rows(prob, x, rows)
    check_sel_rows(torch.stack([sel[b, i] for b, i in rows]), sel_ref)
    check_out(torch.stack([out[b, i] for b, i in rows]), out_ref, fp32=False, what="decode")
    del x, out, sel
    torch.cuda.empty_cache()


def test_32k_split_equals_forward_and_coverage():
    """Split calls equal the one-call forward on the 32K workload; the B=1, k=2048 selection is
    run alongside and the token inclusion rate is reported (a measured property)."""
    w = get_workload("32k")
    x = generate(w, device="cuda", seed=0)
    prob = sg.Problem.from_workload(w)
    out_f, sel_f = run_forward(prob, x)
    _, scores = sg.index(prob, x["q_idx"], x["k_idx"])
    sel_s = sg.topk(prob, scores)
    del scores
    assert torch.equal(sel_s, sel_f)
    out_s = sg.attend(prob, x["q"], x["k"], x["v"], x["gate"], sel_s)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_f)
    # B = 1, k = 2048 on the same index data
    p1 = sg.Problem.from_workload(w, block=1, topk_tokens=2048)
    _, sc1 = sg.index(p1, x["q_idx"], x["k_idx"])
    sel1 = sg.topk(p1, sc1)
    del sc1
    torch.cuda.synchronize()
    toks = sample_tokens(w.t_q, w.t_kv, 1, 2048, 8, seed=1)
    sel1_ref, _, _ = oracle_rows(p1, x, [(0, i) for i in toks])
    check_sel_rows(sel1[0, toks], sel1_ref)
    rate_ref = oracle.inclusion_rate(x["q_idx"], x["k_idx"], [(0, i) for i in toks[-4:]], w.t_kv)
    say(f"  token inclusion (oracle, {len(toks[-4:])} late tokens): {rate_ref.mean():.4f}")


# ----------------------------------------------------------------------------------------------
# the fused selection's exact fallback (forced from the input data)
# ----------------------------------------------------------------------------------------------
def _fallback_case(kind):
    """64 late queries over 20000 keys (o ~ 2500 > the 2048-entry candidate list), B = 8."""
    w, x = generate_small(t_q=64, t_kv=20000, groups=2, heads=8, head_dim=128, index_dim=32,
                          block=8, topk=256, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          seed=6, device="cuda")
    if kind == "overflow":            # every score equal: all ~2500 candidates pass
        x["k_idx"].fill_(1.0)
        x["q_idx"].fill_(1.0)
    else:                             # only the sampled blocks (stride 5) score high: ~500 pass
        x["k_idx"].zero_()
        kv = x["k_idx"].view(1, -1, 8, 32)
        kv[:, 0::5] = 1.0
        x["q_idx"].fill_(1.0)
    return w, x


@pytest.mark.parametrize("kind", ["overflow", "underflow"])
def test_fused_selection_fallback(kind):
    w, x = _fallback_case(kind)
    prob = sg.Problem.from_workload(w)
    out, sel = run_forward(prob, x)
    sel_ref, out_ref, _ = oracle.forward(x, w.block, w.topk, w.softmax_scale)
    check_sel_rows(sel, sel_ref)
    check_out(out, out_ref, fp32=False, what=f"fallback {kind}")
    _, scores = sg.index(prob, x["q_idx"], x["k_idx"])
    assert torch.equal(sg.topk(prob, scores), sel)
