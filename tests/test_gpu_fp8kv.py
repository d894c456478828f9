"""The fp8-KV forward (sgqa_forward_fp8kv) through the C ABI against the oracle on the dequantised
K and V (oracle.e4m3_decode(code) * scale): selection exact (the indexer does not read K or V),
outputs within the bf16 bar."""
import numpy as np
import pytest
import torch

import long_context_sparse_sgqa_amd as sg
import oracle
from gpu_helpers import check_out, check_sel_rows, say, structural_check_sel
from sgqa_inputs import generate, generate_small, get_workload, quantize_e4m3

pytestmark = pytest.mark.gpu

FP8_CASES = [
    # t_q, t_kv, block, topk, groups, index_dim, sharp, head_dim, batch
    (300, 1001, 8, 256, 2, 128, False, 128, 1),
    (517, 517, 8, 128, 2, 64, True, 128, 1),
    (301, 999, 8, 256, 2, 128, True, 64, 1),
    (150, 700, 8, 128, 2, 128, False, 128, 3),
    (7, 1300, 16, 256, 2, 32, True, 128, 2),
]


def dequantised(x, k8, ks, v8, vs):
    y = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}
    y["k"] = torch.from_numpy(oracle.e4m3_decode(k8.cpu().numpy()) * ks)
    y["v"] = torch.from_numpy(oracle.e4m3_decode(v8.cpu().numpy()) * vs)
    return y


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "tq%d-tk%d-B%d-k%d-G%d-di%d%s-d%d-b%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "-sharp" if c[6] else "", c[7], c[8]))
def test_fp8kv_small_every_row(case):
    t_q, t_kv, B, k, G, di, sharp, d, bt = case
    say("case: fp8 kv", case)
    w, x = generate_small(batch=bt, t_q=t_q, t_kv=t_kv, groups=G, heads=8, head_dim=d,
                          index_dim=di, block=B, topk=k, dtype="bf16", index_dtype="bf16",
                          scaled_qkv=True, needles=1 if (t_kv // B) >= 2 * G else 0, seed=13,
                          device="cuda", sharp=sharp)
    prob = sg.Problem.from_workload(w)
    k8, ks = quantize_e4m3(x["k"])
    v8, vs = quantize_e4m3(x["v"])
    out, sel = sg.forward_fp8kv(prob, x["q"], k8, v8, ks, vs, x["gate"], x["q_idx"], x["k_idx"],
                                return_sel=True)
    again = sg.forward_fp8kv(prob, x["q"], k8, v8, ks, vs, x["gate"], x["q_idx"], x["k_idx"])
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    sel_ref, out_ref, _ = oracle.forward(dequantised(x, k8, ks, v8, vs), B, k, w.softmax_scale)
    check_sel_rows(sel.reshape(-1, G, sel.shape[-1]), sel_ref.reshape(-1, G, sel_ref.shape[-1]))
    check_out(out, out_ref, fp32=False, what="fp8 kv")


@pytest.mark.parametrize("sharp", [False, True], ids=["plain", "sharp"])
def test_fp8kv_128k_sampled_rows(sharp):
    w = get_workload("128k")
    say("case: fp8 kv 128k", "sharp" if sharp else "")
    x = generate(w, device="cuda", seed=0, sharp=sharp)
    prob = sg.Problem.from_workload(w)
    k8, ks = quantize_e4m3(x["k"])
    v8, vs = quantize_e4m3(x["v"])
    out, sel = sg.forward_fp8kv(prob, x["q"], k8, v8, ks, vs, x["gate"], x["q_idx"], x["k_idx"],
                                return_sel=True)
    torch.cuda.synchronize()
    structural_check_sel(sel, prob)
    toks = [0, 8, 4095, 4096, 77777, 131071]
    xd = dequantised({n: x[n] for n in ("q", "gate", "q_idx", "k_idx")} | {"k": x["k"], "v": x["v"]},
                     k8, ks, v8, vs)
    sel_ref, out_ref, _ = oracle.forward_rows(xd, w.block, w.topk, w.softmax_scale,
                                              [(0, i) for i in toks])
    check_sel_rows(sel[0, toks], sel_ref)
    check_out(out[0, toks], out_ref, fp32=False, what="fp8 kv 128k")
    del x, out, sel, k8, v8
    torch.cuda.empty_cache()
