"""The seeded input recipe: determinism, shapes, value ranges and the needle plan."""
import torch

from sgqa_inputs import WORKLOADS, generate, generate_small, get_workload


def test_deterministic_and_seeded():
    _, a = generate_small(seed=5, needles=2, t_kv=128, t_q=128)
    _, b = generate_small(seed=5, needles=2, t_kv=128, t_q=128)
    _, c = generate_small(seed=6, needles=2, t_kv=128, t_q=128)
    for n in ("q", "k", "v", "gate", "q_idx", "k_idx"):
        assert torch.equal(a[n], b[n])
    assert not torch.equal(a["q"], c["q"])


def test_shapes_and_index_values():
    w = get_workload("tiny")
    x = generate(w, seed=0)
    assert x["q"].shape == (1, 2048, 2, 4, 64) and x["q"].dtype == torch.float32
    assert x["k"].shape == (1, 2, 2048, 64)
    assert x["q_idx"].shape == (1, 2048, 2, 32) and x["k_idx"].shape == (1, 2048, 32)
    for n in ("q_idx", "k_idx"):
        t = x[n]
        assert torch.equal(t, t.round()) and t.min() >= -4 and t.max() <= 4
        assert set(torch.unique(t).tolist()) == set(range(-4, 5))


def test_needles_disjoint_and_biased():
    w, x = generate_small(t_q=256, t_kv=256, groups=2, index_dim=16, block=8, topk=32,
                          needles=3, seed=1, dtype="bf16", index_dtype="bf16", scaled_qkv=True)
    nb = x["needle_blocks"]
    assert nb.shape == (2, 3)
    assert len(set(nb.flatten().tolist())) == 6
    assert x["k_idx"].dtype == torch.bfloat16


def test_workloads_match_descriptions():
    assert WORKLOADS["128k"].num_blocks == 16384
    assert WORKLOADS["1m"].t_kv - WORKLOADS["1m"].t_q == 1040384
    assert WORKLOADS["decode"].t_kv == 262144 + 4 and WORKLOADS["decode"].t_q == 4


def test_drifting_index_queries():
    """q_idx_redraw < 1: along the tokens, a component keeps the previous token's value unless
    redrawn; the first token is the plain draw, and every other tensor is drawn as without drift."""
    w = get_workload("tiny").replace(q_idx_redraw=0.05)
    plain = generate(get_workload("tiny"), seed=3)
    x = generate(w, seed=3)
    for n in ("q", "k", "v", "gate", "k_idx"):
        assert torch.equal(x[n], plain[n]), n
    q = x["q_idx"]
    assert torch.equal(q[:, 0], plain["q_idx"][:, 0])
    same = (q[:, 1:] == q[:, :-1]).double().mean().item()
    assert 0.9 < same < 0.99                     # about 95 % of components carried over
    changed = q[:, 1:] != q[:, :-1]
    # a component that changed takes that token's own plain draw
    assert torch.equal(q[:, 1:][changed], plain["q_idx"][:, 1:][changed])
    assert torch.equal(x["q_idx"], generate(w, seed=3)["q_idx"])
