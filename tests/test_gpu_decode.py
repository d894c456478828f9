"""Decode over the paged cache, through the C ABI: appends, block keys and the decode step.

The oracle reads each sequence as the forward path on its own prefix (oracle.sequence_rows); the
cache holds the same tokens scattered over shuffled pages.  Checked: block keys bit for bit against
the oracle's block sums, the selection of every decoded row exactly, the outputs within the bf16
tolerance, run-to-run bit equality, and (small case) bit equality with the contiguous one-call
forward of each sequence, which runs the same attention arithmetic on packed copies.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_sgqa_amd as sg
import oracle
from gpu_helpers import check_out, check_sel_rows, say
from sgqa_inputs import generate, generate_small, get_workload

pytestmark = pytest.mark.gpu


def shuffled_table(lens, page_tokens, max_pages, spare, seed):
    """Block table giving every sequence distinct physical pages in random order."""
    need = [-(-L // page_tokens) for L in lens]
    num_pages = sum(need) + spare
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(seed)).tolist()
    table = torch.zeros(len(lens), max_pages, dtype=torch.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = torch.tensor(perm[at:at + n], dtype=torch.int32)
        at += n
    return table, num_pages


def gather_new(x, starts, n):
    """k, v [Bt, G, n, D] and k_idx [Bt, n, Di] of positions starts[b] .. starts[b] + n - 1."""
    k = torch.stack([x["k"][b, :, s:s + n] for b, s in enumerate(starts)]).contiguous()
    v = torch.stack([x["v"][b, :, s:s + n] for b, s in enumerate(starts)]).contiguous()
    ki = torch.stack([x["k_idx"][b, s:s + n] for b, s in enumerate(starts)]).contiguous()
    return k, v, ki


def append_each(prob_kw, cache, pools, table, x, b, L, dev):
    """Bulk append of tokens 0 .. L-1 of sequence b alone (a batch-1 call on row b)."""
    p1 = sg.Problem(batch=1, **prob_kw)
    one = {"k_cache": pools["k_cache"], "v_cache": pools["v_cache"],
           "kidx_cache": pools["kidx_cache"], "k_blk": pools["k_blk"][b:b + 1]}
    sg.cache_append(p1, cache, torch.tensor([L], dtype=torch.int32, device=dev),
                    table[b:b + 1].contiguous(), x["k"][b:b + 1, :, :L].contiguous(),
                    x["v"][b:b + 1, :, :L].contiguous(), x["k_idx"][b:b + 1, :L].contiguous(), one)


def check_decode_sel_structure(sel, lens, t_q, block, n_sel):
    for b, L in enumerate(lens):
        for i in range(t_q):
            o = (L - t_q + i) // block
            for row in sel[b, i].tolist():
                n = min(n_sel, o + 1)
                assert all(v >= 0 for v in row[:n]) and all(v == -1 for v in row[n:])
                assert row[:n] == sorted(set(row[:n])) and row[n - 1] == o and row[0] >= 0


@pytest.mark.parametrize("sharp", [False, True])
def test_paged_decode_small_varlen(sharp):
    dev = "cuda"
    lens = [700, 1300, 999]
    t_q, P, t_kv = 4, 64, 1300
    say(f"case: paged decode small varlen sharp={sharp}")
    w, x = generate_small(batch=3, t_q=t_q, t_kv=t_kv, groups=2, heads=8, head_dim=128,
                          index_dim=64, block=8, topk=256, dtype="bf16", index_dtype="bf16",
                          needles=4, scaled_qkv=True, seed=11, device=dev, sharp=sharp)
    prob_kw = dict(t_q=t_q, t_kv=t_kv, kv_groups=2, heads_per_group=8, head_dim=128, index_dim=64,
                   block=8, topk_tokens=256, softmax_scale=w.softmax_scale)
    max_pages = -(-t_kv // P) + 1
    table_cpu, num_pages = shuffled_table(lens, P, max_pages, spare=5, seed=3)
    table = table_cpu.to(dev)
    cache = sg.Cache(num_pages, P, max_pages)
    prob = sg.Problem(batch=3, **prob_kw)
    pools = sg.alloc_cache(prob, cache, dev)
    # prefill each sequence to L - 9 tokens, then 5 tokens to all, then the 4 decoded tokens
    for b, L in enumerate(lens):
        append_each(prob_kw, cache, pools, table, x, b, L - 9, dev)
    for n, back in ((5, 4), (4, 0)):
        starts = [L - back - n for L in lens]
        k_new, v_new, ki_new = gather_new(x, starts, n)
        seq = torch.tensor([L - back for L in lens], dtype=torch.int32, device=dev)
        sg.cache_append(prob, cache, seq, table, k_new, v_new, ki_new, pools)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    out, sel = sg.decode(prob, cache, seq_lens, table, x["q"], x["gate"], x["q_idx"], pools,
                         return_sel=True)
    again = sg.decode(prob, cache, seq_lens, table, x["q"], x["gate"], x["q_idx"], pools)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "decode run-to-run"

    xc = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}
    # block keys: the oracle's block sums of each sequence's prefix, bit for bit
    for b, L in enumerate(lens):
        ref = oracle.compress(xc["k_idx"][b:b + 1, :L].to(torch.float64).numpy(), 8)[0]
        got = pools["k_blk"][b, :ref.shape[0]].to(torch.float64).cpu().numpy()
        assert np.array_equal(got, ref), f"k_blk of sequence {b}"
    check_decode_sel_structure(sel.cpu(), lens, t_q, 8, 32)
    rows = [(b, i) for b in range(3) for i in range(t_q)]
    sel_ref, out_ref, _ = oracle.sequence_rows(xc, lens, 8, 256, w.softmax_scale, rows)
    check_sel_rows(torch.stack([sel[b, i] for b, i in rows]), sel_ref)
    check_out(torch.stack([out[b, i] for b, i in rows]), out_ref, fp32=False, what="paged decode")

    # the contiguous one-call forward of each sequence gives the same bits
    for b, L in enumerate(lens):
        pb = sg.Problem(batch=1, **dict(prob_kw, t_kv=L))
        o_fwd = sg.forward(pb, x["q"][b:b + 1].contiguous(), x["k"][b:b + 1, :, :L].contiguous(),
                           x["v"][b:b + 1, :, :L].contiguous(), x["gate"][b:b + 1].contiguous(),
                           x["q_idx"][b:b + 1].contiguous(), x["k_idx"][b:b + 1, :L].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o_fwd[0], out[b]), f"paged decode vs forward, sequence {b}"


@pytest.mark.parametrize("di,t_q,groups,ties", [(32, 4, 8, False), (64, 4, 8, False),
                                                (128, 4, 8, False), (128, 4, 8, True),
                                                (64, 5, 6, False), (128, 8, 8, False)],
                         ids=["di32", "di64", "di128", "di128-ties", "30rows-g6", "64rows-scores"])
def test_paged_decode_long_varlen(di, t_q, groups, ties):
    """Rows of three sequence lengths in one call: about 5000 causal blocks (past the candidate
    capacity: sampled thresholds), about 2000 (every block a candidate) and about 375 (dense).
    With ties, sequence 0's index keys are constant: every block passes its threshold, the list
    overflows and its rows take the exact recomputation (lowest blocks win the ties).  30 rows per
    sequence (5 tokens x 6 groups) leave the last group of 8 rows part-filled; 64 rows per sequence
    take the stored-score selection instead of candidate lists."""
    dev = "cuda"
    lens = [40000, 16000, 3000]
    P, t_kv = 64, 40000
    say(f"case: paged decode long varlen di={di} t_q={t_q} groups={groups} ties={ties}")
    w, x = generate_small(batch=3, t_q=t_q, t_kv=t_kv, groups=groups, heads=8, head_dim=64,
                          index_dim=di, block=8, topk=4096, dtype="bf16", index_dtype="bf16",
                          scaled_qkv=True, seed=21, device=dev)
    if ties:
        x["k_idx"][0].fill_(0.5)
    prob_kw = dict(t_q=t_q, t_kv=t_kv, kv_groups=groups, heads_per_group=8, head_dim=64,
                   index_dim=di, block=8, topk_tokens=4096, softmax_scale=w.softmax_scale)
    max_pages = -(-t_kv // P)
    table_cpu, num_pages = shuffled_table(lens, P, max_pages, spare=3, seed=5)
    table = table_cpu.to(dev)
    cache = sg.Cache(num_pages, P, max_pages)
    prob = sg.Problem(batch=3, **prob_kw)
    pools = sg.alloc_cache(prob, cache, dev)
    for b, L in enumerate(lens):
        append_each(prob_kw, cache, pools, table, x, b, L, dev)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    out, sel = sg.decode(prob, cache, seq_lens, table, x["q"], x["gate"], x["q_idx"], pools,
                         return_sel=True)
    again = sg.decode(prob, cache, seq_lens, table, x["q"], x["gate"], x["q_idx"], pools)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "decode run-to-run"
    check_decode_sel_structure(sel.cpu(), lens, t_q, 8, 512)
    xc = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}
    rows = [(b, i) for b in range(3) for i in range(t_q)]
    sel_ref, out_ref, _ = oracle.sequence_rows(xc, lens, 8, 4096, w.softmax_scale, rows)
    check_sel_rows(torch.stack([sel[b, i] for b, i in rows]), sel_ref)
    check_out(torch.stack([out[b, i] for b, i in rows]), out_ref, fp32=False,
              what=f"paged decode long varlen di={di}")


def test_paged_decode_workload():
    """The long-context decode workload: 64 sequences of 262 144 cached tokens + 4 new ones."""
    dev = "cuda"
    w = get_workload("decode")
    say("case: paged decode workload")
    x = generate(w, device=dev, seed=0)
    P = 64
    lens = [w.t_kv] * w.batch
    max_pages = -(-w.t_kv // P)
    table_cpu, num_pages = shuffled_table(lens, P, max_pages, spare=0, seed=1)
    table = table_cpu.to(dev)
    cache = sg.Cache(num_pages, P, max_pages)
    prob = sg.Problem.from_workload(w)
    pools = sg.alloc_cache(prob, cache, dev)
    # bulk prefill in chunks of 32768 tokens, then the 4 decoded tokens
    done, chunk = 0, 32768
    while done < w.t_kv:
        n = min(chunk, w.t_kv - w.t_q - done) if done < w.t_kv - w.t_q else w.t_q
        k_new, v_new, ki_new = gather_new(x, [done] * w.batch, n)
        seq = torch.full((w.batch,), done + n, dtype=torch.int32, device=dev)
        sg.cache_append(prob, cache, seq, table, k_new, v_new, ki_new, pools)
        del k_new, v_new, ki_new
        done += n
    say("  cache filled")
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    out, sel = sg.decode(prob, cache, seq_lens, table, x["q"], x["gate"], x["q_idx"], pools,
                         return_sel=True)
    again = sg.decode(prob, cache, seq_lens, table, x["q"], x["gate"], x["q_idx"], pools)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "decode run-to-run"
    rows = [(b, i) for b in (0, 37) for i in range(w.t_q)]
    for b in (0, 37):
        ref = oracle.compress(x["k_idx"][b:b + 1].to("cpu", torch.float64).numpy(), w.block)[0]
        got = pools["k_blk"][b, :ref.shape[0]].to("cpu", torch.float64).numpy()
        assert np.array_equal(got, ref), f"k_blk of sequence {b}"
    xs = {k: (v[[0, 37]].cpu() if torch.is_tensor(v) and k != "needle_blocks" else v)
          for k, v in x.items()}
    sel_ref, out_ref, _ = oracle.sequence_rows(xs, [w.t_kv] * 2, w.block, w.topk, w.softmax_scale,
                                               [(0, i) for i in range(w.t_q)] +
                                               [(1, i) for i in range(w.t_q)])
    check_sel_rows(torch.stack([sel[b, i] for b, i in rows]), sel_ref)
    check_out(torch.stack([out[b, i] for b, i in rows]), out_ref, fp32=False, what="paged decode")
    check_decode_sel_structure(sel[[0, 37]].cpu(), [w.t_kv] * 2, w.t_q, w.block, w.n_sel)
    del x, pools, out, sel, again
    torch.cuda.empty_cache()


def test_append_skips_out_of_range_page_entries():
    """A block_table entry outside [0, num_pages) makes the append store nothing for the tokens of
    that logical page: every pool page keeps its bytes, including the last page, which a clamped
    entry would have named.  The other sequence's append still lands."""
    dev = "cuda"
    P, t_kv = 64, 256
    w, x = generate_small(batch=2, t_q=4, t_kv=t_kv, groups=2, heads=8, head_dim=128,
                          index_dim=64, block=8, topk=64, dtype="bf16", index_dtype="bf16",
                          scaled_qkv=True, seed=13, device=dev)
    say("case: append with out-of-range block_table entries")
    prob = sg.Problem(batch=2, t_q=4, t_kv=t_kv, kv_groups=2, heads_per_group=8, head_dim=128,
                      index_dim=64, block=8, topk_tokens=64)
    max_pages, num_pages = 4, 8
    cache = sg.Cache(num_pages, P, max_pages)
    pools = sg.alloc_cache(prob, cache, dev)
    for name in ("k_cache", "v_cache", "kidx_cache"):
        pools[name].view(torch.int16).fill_(0x1234)
    table = torch.tensor([[0, 1, 2, 3], [num_pages, -1, num_pages + 5, 7]], dtype=torch.int32,
                         device=dev)
    before = {n: pools[n].clone() for n in ("k_cache", "v_cache", "kidx_cache")}
    n = 100                                     # positions 0..99: logical pages 0 and 1
    seq = torch.tensor([n, n], dtype=torch.int32, device=dev)
    sg.cache_append(prob, cache, seq, table, x["k"][:, :, :n].contiguous(),
                    x["v"][:, :, :n].contiguous(), x["k_idx"][:, :n].contiguous(), pools)
    torch.cuda.synchronize()
    for name in ("k_cache", "v_cache", "kidx_cache"):
        # sequence 0 owns pages 0 and 1; nothing else may change
        assert torch.equal(pools[name][2:], before[name][2:]), name
        assert not torch.equal(pools[name][:2], before[name][:2]), name
    # sequence 0's index keys landed where its table says
    ki = pools["kidx_cache"].view(num_pages * P, 64)
    assert torch.equal(ki[:n], x["k_idx"][0, :n])
