"""Gated sliding-window attention through the C ABI against the oracle (oracle.window_rows)."""
import pytest
import torch

import long_context_sparse_sgqa_amd as sg
import oracle
from gpu_helpers import check_out, say
from sgqa_inputs import generate, generate_small, get_workload

pytestmark = pytest.mark.gpu

WINDOW_CASES = [
    # t_q, t_kv, window, groups, head_dim, sharp, batch
    (300, 1001, 256, 2, 128, False, 1),
    (517, 517, 5, 2, 128, True, 1),            # windows shorter than a unit
    (64, 64, 1, 2, 64, False, 1),              # only the own token
    (100, 333, 1000, 2, 128, True, 1),         # window past the context: dense causal
    (7, 1300, 64, 2, 128, False, 2),           # a short query chunk, two sequences
    (150, 700, 33, 1, 64, True, 3),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "tq%d-tk%d-W%d-G%d-d%d%s-b%d" % (
    c[0], c[1], c[2], c[3], c[4], "-sharp" if c[5] else "", c[6]))
def test_window_small_every_row(case):
    t_q, t_kv, window, G, d, sharp, bt = case
    say("case: window", case)
    w, x = generate_small(batch=bt, t_q=t_q, t_kv=t_kv, groups=G, heads=8, head_dim=d,
                          index_dim=32, block=8, topk=64, dtype="bf16", index_dtype="bf16",
                          scaled_qkv=True, seed=5, device="cuda", sharp=sharp)
    prob = sg.Problem.from_workload(w)
    out = sg.swa(prob, window, x["q"], x["k"], x["v"], x["gate"])
    again = sg.swa(prob, window, x["q"], x["k"], x["v"], x["gate"])
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    rows = [(b, i) for b in range(bt) for i in range(t_q)]
    ref = oracle.window_rows({k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()},
                             window, w.softmax_scale, rows)
    check_out(torch.stack([out[b, i] for b, i in rows]), ref, fp32=False, what=f"window {window}")


def test_window_32k_sampled_rows():
    w = get_workload("32k")
    say("case: window 4096 on the 32K workload")
    x = generate(w, device="cuda", seed=0)
    prob = sg.Problem.from_workload(w)
    out = sg.swa(prob, 4096, x["q"], x["k"], x["v"], x["gate"])
    torch.cuda.synchronize()
    toks = [0, 1, 7, 8, 4094, 4095, 4096, 4097, 5000, 12345, 32766, 32767]
    xc = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}
    ref = oracle.window_rows(xc, 4096, w.softmax_scale, [(0, i) for i in toks])
    check_out(out[0, toks], ref, fp32=False, what="window 4096, 32K")
    del x, out
    torch.cuda.empty_cache()
