"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the algorithmic work counts
against per-query brute force, the union statistics against explicit sets, and the guard that
drops a stored counter reading once the kernel's sources change."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sgqa_inputs import get_workload  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]


@pytest.mark.parametrize("t_q,t_kv,block,topk", [(300, 300, 8, 64), (77, 1000, 16, 128), (64, 64, 8, 4096)])
def test_algorithmic_counts_brute_force(t_q, t_kv, block, topk):
    w = get_workload("tiny").replace(t_q=t_q, t_kv=t_kv, block=block, topk=topk, groups=3, batch=2)
    c = bench.algorithmic_counts(w)
    pairs = att = 0
    for i in range(t_q):
        p = t_kv - t_q + i
        own = p // block
        pairs += own                                  # strictly past blocks are scored
        # the own block plus the n_sel - 1 latest past blocks (any choice attends as many tokens)
        chosen = {own} | set(range(max(0, own - (w.n_sel - 1)), own))
        att += sum(1 for t in range(p + 1) if t // block in chosen)
    assert c["pairs"] == pairs * w.groups * w.batch
    assert c["attended"] == att * w.groups * w.batch
    assert c["index_flops"] == 2 * w.index_dim * c["pairs"]
    assert c["attention_flops"] == 4 * w.head_dim * w.heads * c["attended"]


def test_union_stats_brute_force():
    w = get_workload("tiny").replace(t_q=64, t_kv=200, groups=2, topk=96)   # 12 blocks per row
    rng = np.random.default_rng(5)
    sel = np.full((1, w.t_q, w.groups, w.n_sel), -1, dtype=np.int32)
    for i in range(w.t_q):
        o = (w.t_kv - w.t_q + i) // w.block
        for g in range(w.groups):
            k = min(o + 1, w.n_sel) - (i % 3)          # some rows leave -1 padding
            sel[0, i, g, :k] = np.sort(rng.choice(o + 1, size=k, replace=False))
    got = bench.union_stats(w, torch.from_numpy(sel))
    units, chunks = [], 0
    for q0 in range(0, w.t_q, 4):
        u_end = (w.t_kv - w.t_q + q0 + 3) // 8 + 1
        for g in range(w.groups):
            u = {int(b) for b in sel[0, q0:q0 + 4, g].ravel() if b >= 0}
            units.append(len(u))
            for r in range(4):
                lo, hi = (r * u_end) // 4, ((r + 1) * u_end) // 4
                n_r = sum(1 for x in u if lo <= x < hi) if r < 3 else sum(1 for x in u if x >= lo)
                chunks += -(-n_r // 4)
    assert got["union_units_per_4_tokens"] == pytest.approx(np.mean(units))
    assert got["union_over_one_selection"] == pytest.approx(np.mean(units) / w.n_sel)
    assert got["issued_chunks"] == chunks


def test_stale_traffic_record_is_ignored(tmp_path, monkeypatch):
    src = tmp_path / "long_context_sparse_sgqa_amd" / "csrc"
    src.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (src / "k.hip").write_text("kernel source v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"sources": ["k.hip"], "source_digest": bench.kernel_source_digest(["k.hip"]),
           "hbm_bytes_per_launch": 1.5e11}
    (tmp_path / "profiles" / "kern_wl_traffic.json").write_text(json.dumps(rec))
    assert bench.load_traffic("kern", "wl") == 1.5e11
    assert bench.load_traffic("kern", "other") is None              # no record
    (src / "k.hip").write_text("kernel source v2\n")
    assert bench.load_traffic("kern", "wl") is None                 # source changed since
