"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, compare with the oracle."""
import sys

import numpy as np
import torch

import long_context_sparse_sgqa_amd as sg
import oracle

# bf16 tolerance: max-abs 1e-2 (the stated bar); also 5 % of the largest reference magnitude, which
# bf16 rounding of P (2^-9 relative per weight) and of the output (2^-9 relative) stays far inside.
BF16_ATOL = 1e-2
BF16_REL_OF_MAX = 5e-2
F32_ATOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inputs, dev="cuda"):
    return {k: (v.to(dev) if torch.is_tensor(v) and k != "needle_blocks" else v)
            for k, v in inputs.items()}


def run_split(prob, x):
    k_blk, scores = sg.index(prob, x["q_idx"], x["k_idx"])
    sel = sg.topk(prob, scores)
    out = sg.attend(prob, x["q"], x["k"], x["v"], x["gate"], sel)
    torch.cuda.synchronize()
    return k_blk, scores, sel, out


def run_forward(prob, x, workspace=None):
    out, sel = sg.forward(prob, x["q"], x["k"], x["v"], x["gate"], x["q_idx"], x["k_idx"],
                          return_sel=True, workspace=workspace)
    torch.cuda.synchronize()
    return out, sel


def check_out(out_gpu, ref, fp32: bool, what=""):
    got = out_gpu.detach().to("cpu", torch.float64).numpy()
    err = np.abs(got - ref)
    maxerr = float(err.max()) if err.size else 0.0
    refmax = float(np.abs(ref).max()) if ref.size else 0.0
    say(f"  {what} out: max-abs err {maxerr:.3e}, max |ref| {refmax:.3e}")
    if fp32:
        assert maxerr <= F32_ATOL, (what, maxerr)
    else:
        assert maxerr <= BF16_ATOL, (what, maxerr)
        assert maxerr <= BF16_REL_OF_MAX * refmax + 1e-6, (what, maxerr, refmax)
    return maxerr


def check_sel_rows(sel_gpu_rows, sel_ref):
    got = sel_gpu_rows.detach().to("cpu").numpy().astype(np.int64)
    bad = np.argwhere((got != sel_ref).any(axis=-1))
    assert bad.size == 0, f"selection mismatch at rows {bad[:5].tolist()}"


def structural_check_sel(sel, prob):
    """Every row of sel: valid prefix of length min(NS, o+1), ascending, inside [0, o], own block last
    of the prefix, -1 padding after it.  Runs on the device over all rows."""
    Tq, Tk, B, NS = prob.t_q, prob.t_kv, prob.block, prob.n_sel
    pos = torch.arange(Tk - Tq, Tk, device=sel.device, dtype=torch.int64)
    o = (pos // B).view(1, Tq, 1)
    nvalid = torch.clamp(o + 1, max=NS)                                  # [1, Tq, 1]
    ar = torch.arange(NS, device=sel.device).view(1, 1, 1, NS)
    s = sel.to(torch.int64)
    valid = (ar < nvalid.unsqueeze(-1)).expand(s.shape)
    assert bool(((s >= 0) == valid).all()), "valid prefix length"
    assert bool((s[~valid] == -1).all()), "padding"
    assert bool(((s <= o.unsqueeze(-1)) | ~valid).all()), "range"
    d = s[..., 1:] - s[..., :-1]
    assert bool(((d > 0) | ~valid[..., 1:]).all()), "ascending"
    last = torch.gather(s, -1, (nvalid.expand(s.shape[0], Tq, s.shape[2]) - 1).unsqueeze(-1))
    assert bool((last.squeeze(-1) == o).all()), "own block"


def sample_tokens(t_q, t_kv, block, n_sel, n_random, seed=0):
    """Query tokens stratified over the dense -> sparse boundary, block edges and the last token."""
    pos0 = t_kv - t_q
    dense_edge = n_sel * block                      # first position whose query is sparse
    want = {0, 7, 8, dense_edge - 9, dense_edge - 8, dense_edge - 1, dense_edge, dense_edge + 1,
            t_kv - 1, t_kv - 2, t_kv - 8, t_kv - 9}
    rng = np.random.default_rng(seed)
    toks = {p - pos0 for p in want if pos0 <= p < t_kv}
    toks |= set(rng.integers(0, t_q, size=n_random).tolist())
    return sorted(toks)


def oracle_rows(prob, x, rows):
    return oracle.forward_rows(x, prob.block, prob.topk_tokens, prob.softmax_scale, rows)
