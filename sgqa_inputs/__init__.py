"""Seeded synthetic inputs for the Sparse GQA forward path.

This module is shared by the tests, the benchmark and the CPU oracle's callers.  It holds the
workload shapes and the recipe that draws the tensors, and none of the method's arithmetic: no
block compression, no scoring, no selection and no attention happen here.

The workloads follow the Sparse GQA description on the Step 5 Preview pages (page 1, section on model
structure and training stability; page 2, section on Sparse GQA and the 1M-token context): block size
B = 8, a budget of k = 4096 tokens (512 blocks), GQA with several query heads per KV group, contexts up
to 1,048,576 tokens.  The pages publish no dataset, so every tensor is synthetic:

* q, k, v ~ N(0, 1) (fp32 workloads) or N(0, 1)/sqrt(d) rounded to bf16 (bf16 workloads);
  the "sharp" variant keeps q and k unscaled so that the softmax is far from uniform.
* gate ~ N(0, 1).
* index queries and keys are integers drawn uniformly from [-4, 4], stored in the index dtype.
* "needles": per KV group a random sign vector u_g and 64 distinct blocks (disjoint across groups);
  every index key of a needle block gets +2 u_g and every index query of group g gets +2 u_g, both
  clamped to [-4, 4], so later queries of group g correlate with that group's needle blocks.

* "drift" (the 128k-drift workload only): adjacent tokens' index queries are correlated.  Along
  the tokens of each (sequence, group), every component of the index query keeps the previous
  token's value unless it is redrawn, with probability q_idx_redraw; a redrawn component takes the
  uniform draw above for that token (needle bias included).  The pages' premise for grouping
  adjacent query tokens is that their selections overlap; with independent queries (every other
  workload) two tokens share about 142 of their 512 blocks, with q_idx_redraw = 0.05 adjacent
  tokens share about 370.

Draw order (one generator, fixed seed): q, k, v, gate, k_idx, q_idx, u, needle blocks, then the
drift's redraw mask (only when q_idx_redraw < 1).
Large tensors are drawn in slices along their outermost axis so that fp32 temporaries stay small;
the slicing is part of the recipe, so a given (workload, device, seed) always yields the same bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "get_workload", "generate", "query_positions_host"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    t_q: int
    t_kv: int
    groups: int
    heads: int
    head_dim: int
    index_dim: int
    block: int
    topk: int
    dtype: str            # "f32" or "bf16" for q/k/v/gate/out
    index_dtype: str      # "f32" or "bf16" for q_idx/k_idx/k_blk
    needles: int          # planted needle blocks per KV group (0 = none)
    scaled_qkv: bool      # q, k, v drawn as N(0,1)/sqrt(d) when True
    description: str = ""
    q_idx_redraw: float = 1.0   # per token and component: probability of a fresh index query value

    @property
    def num_blocks(self) -> int:
        return -(-self.t_kv // self.block)

    @property
    def n_sel(self) -> int:
        return self.topk // self.block

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", batch=1, t_q=2048, t_kv=2048, groups=2, heads=4, head_dim=64, index_dim=32,
        block=8, topk=256, dtype="f32", index_dtype="f32", needles=0, scaled_qkv=False,
        description="tiny CPU-checkable prefill: T=2048, 2 KV groups x 4 heads, d=64, d_idx=32, "
                    "B=8, k=256 (32 blocks), fp32"),
    "32k": Workload(
        "32k", batch=1, t_q=32768, t_kv=32768, groups=8, heads=8, head_dim=128, index_dim=128,
        block=8, topk=4096, dtype="bf16", index_dtype="bf16", needles=64, scaled_qkv=True,
        description="32K prefill: 8 KV groups x 8 heads, d=128, d_idx=128, B=8, k=4096, bf16"),
    "128k": Workload(
        "128k", batch=1, t_q=131072, t_kv=131072, groups=8, heads=8, head_dim=128, index_dim=128,
        block=8, topk=4096, dtype="bf16", index_dtype="bf16", needles=64, scaled_qkv=True,
        description="128K prefill: 8 KV groups x 8 heads, d=128, d_idx=128, B=8, k=4096, bf16"),
    "decode": Workload(
        "decode", batch=64, t_q=4, t_kv=262148, groups=8, heads=8, head_dim=128, index_dim=128,
        block=8, topk=4096, dtype="bf16", index_dtype="bf16", needles=64, scaled_qkv=True,
        description="decode, 4 query tokens (MTP-3) per sequence after 262144 cached tokens, "
                    "64 sequences, 8 KV groups x 8 heads, d=128, bf16, B=8, k=4096"),
    "128k-drift": Workload(
        "128k-drift", batch=1, t_q=131072, t_kv=131072, groups=8, heads=8, head_dim=128,
        index_dim=128, block=8, topk=4096, dtype="bf16", index_dtype="bf16", needles=64,
        scaled_qkv=True, q_idx_redraw=0.05,
        description="128K prefill as 128k, with drifting index queries (each component redrawn "
                    "with probability 0.05 per token): adjacent tokens select overlapping blocks"),
    "1m": Workload(
        "1m", batch=1, t_q=8192, t_kv=1048576, groups=8, heads=8, head_dim=128, index_dim=128,
        block=8, topk=4096, dtype="bf16", index_dtype="bf16", needles=64, scaled_qkv=True,
        description="1M-context chunked prefill: 8192 queries at positions 1040384..1048575, "
                    "8 KV groups x 8 heads, d=128, bf16, B=8, k=4096"),
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w


def query_positions_host(t_q: int, t_kv: int):
    """Queries are the last t_q tokens of the key stream: absolute positions t_kv - t_q + i."""
    return list(range(t_kv - t_q, t_kv))


_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}

# Elements per drawing slice; bounds the fp32 temporaries (2^27 floats = 512 MiB).
_SLICE_ELEMS = 1 << 27


def _normal(shape, gen, device, dtype, scale):
    """Draw N(0,1)*scale in fp32, slice by slice along axis 0, then cast to `dtype`."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    per_row = flat.shape[1]
    rows = max(1, _SLICE_ELEMS // max(per_row, 1))
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        x = torch.randn((r1 - r0, per_row), generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[r0:r1].copy_(x)
    return out


def _randint(shape, gen, device, dtype, lo=-4, hi=4):
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    per_row = flat.shape[1]
    rows = max(1, _SLICE_ELEMS // max(per_row, 1))
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        x = torch.randint(lo, hi + 1, (r1 - r0, per_row), generator=gen, device=device,
                          dtype=torch.int32)
        flat[r0:r1].copy_(x)
    return out


def generate(w: Workload, device="cpu", seed: int = 0, sharp: bool = False) -> Dict[str, torch.Tensor]:
    """Draw one batch of the workload on `device`.

    Layouts (all contiguous):
      q, gate : [batch, t_q, groups, heads, head_dim]     (dtype)
      k, v    : [batch, groups, t_kv, head_dim]            (dtype)
      q_idx   : [batch, t_q, groups, index_dim]            (index dtype, integer valued)
      k_idx   : [batch, t_kv, index_dim]                   (index dtype, integer valued)
    `sharp=True` leaves q and k unscaled (N(0,1)) on the scaled workloads.
    Also returned: "needle_blocks" [groups, needles] int64 (empty when needles == 0).
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = _TORCH_DTYPES[w.dtype]
    idt = _TORCH_DTYPES[w.index_dtype]
    s = 1.0 / math.sqrt(w.head_dim) if w.scaled_qkv else 1.0
    qk_s = 1.0 if sharp else s
    B, Tq, Tk, G, H, D, Di = w.batch, w.t_q, w.t_kv, w.groups, w.heads, w.head_dim, w.index_dim

    q = _normal((B, Tq, G, H, D), gen, dev, dt, qk_s)
    k = _normal((B, G, Tk, D), gen, dev, dt, qk_s)
    v = _normal((B, G, Tk, D), gen, dev, dt, s)
    gate = _normal((B, Tq, G, H, D), gen, dev, dt, 1.0)
    k_idx = _randint((B, Tk, Di), gen, dev, idt)
    q_idx = _randint((B, Tq, G, Di), gen, dev, idt)

    needle_blocks = torch.empty((G, 0), dtype=torch.int64)
    if w.needles > 0:
        nb = w.num_blocks
        if w.needles * G > nb:
            raise ValueError("more needle blocks than blocks")
        u = torch.randint(0, 2, (G, Di), generator=gen, device=dev, dtype=torch.int32) * 2 - 1
        perm = torch.randperm(nb, generator=gen, device=dev)[: w.needles * G]
        needle_blocks = perm.view(G, w.needles).to("cpu", torch.int64)
        u = u.to(torch.float32)
        # index keys of needle blocks: +2 u_g, clamped
        for g in range(G):
            for blk in needle_blocks[g].tolist():
                t0, t1 = blk * w.block, min((blk + 1) * w.block, Tk)
                seg = k_idx[:, t0:t1, :].to(torch.float32) + 2.0 * u[g]
                k_idx[:, t0:t1, :] = seg.clamp_(-4, 4).to(idt)
            # every index query of group g: +2 u_g, clamped
            qs = q_idx[:, :, g, :].to(torch.float32) + 2.0 * u[g]
            q_idx[:, :, g, :] = qs.clamp_(-4, 4).to(idt)
    if w.q_idx_redraw < 1.0:
        # token i takes, per component, the value drawn at the last token <= i whose component was
        # redrawn (token 0 always is)
        redraw = torch.rand((B, Tq, G, Di), generator=gen, device=dev) < w.q_idx_redraw
        redraw[:, 0] = True
        tok = torch.arange(Tq, device=dev, dtype=torch.int64).view(1, Tq, 1, 1)
        src = torch.where(redraw, tok, torch.zeros((), dtype=torch.int64, device=dev))
        del redraw
        src = torch.cummax(src, dim=1).values
        q_idx = torch.gather(q_idx, 1, src)
        del src
    return {"q": q, "k": k, "v": v, "gate": gate, "q_idx": q_idx, "k_idx": k_idx,
            "needle_blocks": needle_blocks}


def generate_small(batch=1, t_q=64, t_kv=64, groups=2, heads=4, head_dim=64, index_dim=32,
                   block=8, topk=32, dtype="f32", index_dtype="f32", needles=0, scaled_qkv=False,
                   seed=0, device="cpu", sharp=False):
    """Convenience: a custom small workload (for tests), drawn with the same recipe."""
    w = Workload("custom", batch, t_q, t_kv, groups, heads, head_dim, index_dim, block, topk,
                 dtype, index_dtype, needles, scaled_qkv)
    return w, generate(w, device=device, seed=seed, sharp=sharp)


def quantize_e4m3(x: torch.Tensor):
    """Synthetic fp8 K / V for the fp8-KV variant: per-tensor amax scaling (scale = max|x| / 448)
    and torch's round-to-nearest-even conversion to OCP e4m3.  Returns (codes as uint8 of x's
    shape, scale as a Python float)."""
    amax = float(x.abs().max().item())
    scale = amax / 448.0 if amax > 0 else 1.0
    codes = (x.to(torch.float32) / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), scale
