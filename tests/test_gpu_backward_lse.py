"""Training pair through the C ABI: sgqa_forward_with_lse (the forward plus each attention row's
softmax normaliser) and sgqa_attend_backward_with_lse (the gradients from the saved output and
normaliser, no forward recompute), against the oracle: oracle.attention_lse (pinned against
torch.logsumexp and closed forms) and oracle.attention_backward (pinned against torch autograd)."""
import numpy as np
import pytest
import torch

import long_context_sparse_sgqa_amd as sg
import oracle
from gpu_helpers import say
from sgqa_inputs import generate, generate_small, get_workload
from test_gpu_backward import BWD_CASES, check

pytestmark = pytest.mark.gpu

# The attention kernels sum each row's normaliser l from the probabilities rounded to bf16 (the
# same values the P.V product takes), each off by at most 2^-9 relative, so ln l is off by at most
# ln(1 + 2^-9) < 2^-9; the logits themselves are fp32 sums of exact bf16 products.  Bar: 2^-8.
LSE_ATOL = 2.0 ** -8


def check_lse(name, got, ref):
    got = got.detach().to("cpu", torch.float64).numpy()
    err = float(np.abs(got - ref).max())
    say(f"  {name}: max-abs err {err:.3e}, max |ref| {float(np.abs(ref).max()):.3e}")
    assert err <= LSE_ATOL, (name, err)


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "tq%d-tk%d-B%d-k%d-G%d%s-d%d-b%d" % (
    c[0], c[1], c[2], c[3], c[4], "-sharp" if c[6] else "", c[7], c[8]))
def test_forward_lse_and_saved_backward_every_element(case):
    t_q, t_kv, B, k, G, di, sharp, d, bt = case
    say("case: forward_with_lse + backward_with_lse", case)
    w, x = generate_small(batch=bt, t_q=t_q, t_kv=t_kv, groups=G, heads=8, head_dim=d,
                          index_dim=di, block=B, topk=k, dtype="bf16", index_dtype="bf16",
                          scaled_qkv=True, seed=23, device="cuda", sharp=sharp)
    prob = sg.Problem.from_workload(w)
    out, sel, lse = sg.forward_with_lse(prob, x["q"], x["k"], x["v"], x["gate"], x["q_idx"],
                                        x["k_idx"])
    out_plain, sel_plain = sg.forward(prob, x["q"], x["k"], x["v"], x["gate"], x["q_idx"],
                                      x["k_idx"], return_sel=True)
    torch.cuda.synchronize()
    # the normaliser is an extra output: the forward's own results are unchanged, bit for bit
    assert torch.equal(out, out_plain) and torch.equal(sel, sel_plain)
    xc = {n: (v.cpu() if torch.is_tensor(v) else v) for n, v in x.items()}
    sel_ref, _, _ = oracle.forward(xc, B, k, w.softmax_scale)
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_ref)
    check_lse("lse", lse, oracle.attention_lse(xc, sel_ref, B, w.softmax_scale, list(range(t_q))))

    g = torch.Generator(device="cuda").manual_seed(7)
    dout = torch.randn(x["q"].shape, generator=g, device="cuda").to(torch.bfloat16)
    dq, dk, dv, dgate = sg.attend_backward_with_lse(prob, x["q"], x["k"], x["v"], x["gate"], sel,
                                                    out, lse, dout)
    again = sg.attend_backward_with_lse(prob, x["q"], x["k"], x["v"], x["gate"], sel, out, lse,
                                        dout)
    torch.cuda.synchronize()
    for name, a1, a2 in zip(("dq", "dk", "dv", "dgate"), (dq, dk, dv, dgate), again):
        assert torch.equal(a1, a2), f"{name} differs between two runs"
    r_dq, r_dk, r_dv, r_dg = oracle.attention_backward(xc, sel_ref, dout.cpu(), B, w.softmax_scale)
    check("dq", dq, r_dq)
    check("dk", dk, r_dk)
    check("dv", dv, r_dv)
    check("dgate", dgate, r_dg)


def test_saved_backward_32k_sampled_rows_and_sums():
    """32K workload: lse, dq and dgate of sampled query rows against the oracle; dk and dv through
    the exact sums sum_t dv_t = sum over query rows of dO and sum_t dk_t = 0."""
    w = get_workload("32k")
    say("case: forward_with_lse + backward_with_lse 32K")
    x = generate(w, device="cuda", seed=0)
    prob = sg.Problem.from_workload(w)
    out, sel, lse = sg.forward_with_lse(prob, x["q"], x["k"], x["v"], x["gate"], x["q_idx"],
                                        x["k_idx"])
    g = torch.Generator(device="cuda").manual_seed(3)
    dout = torch.randn(x["q"].shape, generator=g, device="cuda").to(torch.bfloat16)
    dq, dk, dv, dgate = sg.attend_backward_with_lse(prob, x["q"], x["k"], x["v"], x["gate"], sel,
                                                    out, lse, dout)
    torch.cuda.synchronize()
    toks = [0, 5, 4095, 4096, 20000, 32767]
    xc = {n: x[n][:, toks].cpu() if n in ("q", "gate", "q_idx") else x[n].cpu()
          for n in ("q", "gate", "q_idx", "k", "v", "k_idx")}
    for j, i in enumerate(toks):
        # a one-row problem per sampled token keeps its position (t_kv - t_q + i)
        one = {n: (xc[n][:, j:j + 1] if n in ("q", "gate", "q_idx") else xc[n][:, :, :i + 1]
                   if n in ("k", "v") else xc[n][:, :i + 1]) for n in xc}
        sel_i = sel[:, i:i + 1].cpu().numpy()
        check_lse(f"lse row {i}", lse[:, i:i + 1],
                  oracle.attention_lse(one, sel_i, w.block, w.softmax_scale, [0]))
        r_dq, _, _, r_dg = oracle.attention_backward(one, sel_i, dout[:, i:i + 1].cpu(), w.block,
                                                      w.softmax_scale)
        check(f"dq row {i}", dq[:, i:i + 1], r_dq)
        check(f"dgate row {i}", dgate[:, i:i + 1], r_dg)
    sig = torch.sigmoid(x["gate"].float())
    want_v = (dout.float() * sig).sum(dim=(1, 3)).double()          # [Bt, G, D]
    err_v = float((dv.double().sum(dim=2) - want_v).abs().max())
    err_k = float(dk.double().sum(dim=2).abs().max())
    say(f"  sum dv err {err_v:.3e} (max {float(want_v.abs().max()):.3e}); sum dk {err_k:.3e}")
    assert err_v <= 2e-2 * float(want_v.abs().max())
    assert err_k <= 2e-2 * float(dk.double().abs().sum(dim=2).max())
    del x, out, sel, lse, dq, dk, dv, dgate
    torch.cuda.empty_cache()


def test_backward_long_context_every_row():
    """524 288 keys (the group lists' four-word bitmap scans, 65 536 units per group): both
    backward entry points against the oracle on every dq and dgate row and on every element of dk
    and dv (keys no query selected must come out exactly 0)."""
    t_q, t_kv, G, B, k = 64, 524288, 2, 8, 4096
    say(f"case: backward at t_kv={t_kv}, t_q={t_q}")
    w, x = generate_small(t_q=t_q, t_kv=t_kv, groups=G, heads=8, head_dim=128, index_dim=128,
                          block=B, topk=k, dtype="bf16", index_dtype="bf16", scaled_qkv=True,
                          needles=2, seed=29, device="cuda")
    prob = sg.Problem.from_workload(w)
    out, sel, lse = sg.forward_with_lse(prob, x["q"], x["k"], x["v"], x["gate"], x["q_idx"],
                                        x["k_idx"])
    g = torch.Generator(device="cuda").manual_seed(11)
    dout = torch.randn(x["q"].shape, generator=g, device="cuda").to(torch.bfloat16)
    grads = {
        "recompute": sg.attend_backward(prob, x["q"], x["k"], x["v"], x["gate"], sel, dout),
        "saved lse": sg.attend_backward_with_lse(prob, x["q"], x["k"], x["v"], x["gate"], sel, out,
                                                 lse, dout),
    }
    torch.cuda.synchronize()
    xc = {n: x[n].cpu() for n in ("q", "k", "v", "gate")}
    sel_c = sel.cpu().numpy()
    check_lse("lse", lse, oracle.attention_lse(xc, sel_c, B, w.softmax_scale, list(range(t_q))))
    r_dq, r_dk, r_dv, r_dg = oracle.attention_backward(xc, sel_c, dout.cpu(), B, w.softmax_scale)
    for name, (dq, dk, dv, dgate) in grads.items():
        say(f"  {name}:")
        check("dq", dq, r_dq)
        check("dk", dk, r_dk)
        check("dv", dv, r_dv)
        check("dgate", dgate, r_dg)
        untouched = torch.from_numpy((r_dv == 0).all(axis=-1))           # [Bt, G, Tk]
        assert bool((dv.cpu()[untouched] == 0).all()) and bool((dk.cpu()[untouched] == 0).all())
    del x, out, sel, lse, grads
    torch.cuda.empty_cache()
