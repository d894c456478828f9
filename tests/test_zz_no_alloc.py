"""sgqa_decode_noalloc (no workspace argument; the library's fixed per-GPU scratch) against
sgqa_decode with a caller workspace, through the C ABI: two calls in a row, the second on a
smaller input, each bit-equal to the workspace entry point on the same input (selection and
output).  The first call also leaves the scratch holding its own data, which the second call must
not depend on."""
import pytest
import torch

import long_context_sparse_sgqa_amd as sg
from gpu_helpers import say
from sgqa_inputs import generate_small

pytestmark = pytest.mark.gpu


def _table(lens, page_tokens, max_pages, seed):
    need = [-(-L // page_tokens) for L in lens]
    num_pages = sum(need) + 3
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(seed)).tolist()
    table = torch.zeros(len(lens), max_pages, dtype=torch.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = torch.tensor(perm[at:at + n], dtype=torch.int32)
        at += n
    return table, num_pages


def _case(lens, t_kv, groups, seed):
    """A paged cache holding sequences of the given lengths; returns what decode needs."""
    dev = "cuda"
    t_q, P = 4, 64
    bt = len(lens)
    w, x = generate_small(batch=bt, t_q=t_q, t_kv=t_kv, groups=groups, heads=8, head_dim=128,
                          index_dim=128, block=8, topk=4096, dtype="bf16", index_dtype="bf16",
                          needles=4, scaled_qkv=True, seed=seed, device=dev)
    prob = sg.Problem(batch=bt, t_q=t_q, t_kv=t_kv, kv_groups=groups, heads_per_group=8,
                      head_dim=128, index_dim=128, block=8, topk_tokens=4096,
                      softmax_scale=w.softmax_scale)
    max_pages = -(-t_kv // P)
    table_cpu, num_pages = _table(lens, P, max_pages, seed)
    table = table_cpu.to(dev)
    cache = sg.Cache(num_pages, P, max_pages)
    pools = sg.alloc_cache(prob, cache, dev)
    for b, L in enumerate(lens):
        p1 = sg.Problem(batch=1, t_q=t_q, t_kv=t_kv, kv_groups=groups, heads_per_group=8,
                        head_dim=128, index_dim=128, block=8, topk_tokens=4096)
        one = {"k_cache": pools["k_cache"], "v_cache": pools["v_cache"],
               "kidx_cache": pools["kidx_cache"], "k_blk": pools["k_blk"][b:b + 1]}
        sg.cache_append(p1, cache, torch.tensor([L], dtype=torch.int32, device=dev),
                        table[b:b + 1].contiguous(), x["k"][b:b + 1, :, :L].contiguous(),
                        x["v"][b:b + 1, :, :L].contiguous(), x["k_idx"][b:b + 1, :L].contiguous(),
                        one)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    return prob, cache, pools, table, seq_lens, x


def _both(prob, cache, pools, table, seq_lens, x):
    ref_out, ref_sel = sg.decode(prob, cache, seq_lens, table, x["q"], x["gate"], x["q_idx"], pools,
                                 return_sel=True)
    out = torch.full_like(ref_out, float("nan"))
    sel = torch.full_like(ref_sel, -7)
    sg.decode_noalloc(prob, cache, seq_lens, table, x["q"], x["gate"], x["q_idx"], pools, out,
                      sel=sel)
    torch.cuda.synchronize()
    return ref_out, ref_sel, out, sel


def test_decode_noalloc_matches_decode_twice_shrinking():
    big = ([40000, 16000, 3000, 21000], 40000, 4, 5)
    small = ([9000, 700], 9000, 2, 6)
    for name, (lens, t_kv, groups, seed) in (("first, larger", big), ("second, smaller", small)):
        say(f"case: decode_noalloc {name}: lens={lens} groups={groups}")
        prob, cache, pools, table, seq_lens, x = _case(lens, t_kv, groups, seed)
        assert sg.decode_workspace_size(prob, cache) <= sg.DECODE_NOALLOC_SCRATCH_BYTES
        ref_out, ref_sel, out, sel = _both(prob, cache, pools, table, seq_lens, x)
        assert torch.equal(sel, ref_sel), f"{name}: selection differs from sgqa_decode"
        assert torch.equal(out, ref_out), f"{name}: output differs from sgqa_decode"
        del pools, x
    torch.cuda.empty_cache()
