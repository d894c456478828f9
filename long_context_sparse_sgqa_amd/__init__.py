"""Sparse GQA forward path on MI355X (gfx950): Python binding of the libsgqa.so C ABI.

Argument marshalling only.  Every step of the path (block compression, indexer, top-k selection,
gated attention) runs in the library's HIP kernels; torch supplies device memory and the current
stream.  There is no CPU fallback: if libsgqa.so is missing or cannot be loaded, importing the
binding's functions raises.

Layouts and semantics are those of include/sgqa.h:
  q, gate, out : [Bt, Tq, G, H, D]       k, v : [Bt, G, Tk, D]
  q_idx        : [Bt, Tq, G, Di]         k_idx: [Bt, Tk, Di]        k_blk: [Bt, NB, Di]
  scores       : [Bt, Tq, G, NB] fp32    sel  : [Bt, Tq, G, NS] int32
Decode over a paged cache (Cache: num_pages, page_tokens P, max_pages):
  k_cache [pages, G, P/8, 8 D]   v_cache [pages, G, P/8, D, 8]   kidx_cache [pages, P, Di]
  k_blk   [Bt, max_pages P / B, Di]   block_table [Bt, max_pages] int32   seq_lens [Bt] int32
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["Problem", "Cache", "load_library", "library_path", "abi_version", "sizes", "index",
           "topk", "attend", "forward", "alloc_cache", "cache_append", "decode_workspace_size",
           "decode", "decode_noalloc", "DECODE_NOALLOC_SCRATCH_BYTES", "swa_workspace_size", "swa",
           "forward_fp8kv", "attend_backward", "forward_with_lse", "attend_backward_with_lse",
           "SgqaError", "EXPORTED_SYMBOLS"]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libsgqa.so"

SGQA_F32, SGQA_BF16 = 0, 1
_DT = {torch.float32: SGQA_F32, torch.bfloat16: SGQA_BF16}

EXPORTED_SYMBOLS = ("sgqa_abi_version", "sgqa_status_string", "sgqa_last_error", "sgqa_sizes",
                    "sgqa_index", "sgqa_topk", "sgqa_attend", "sgqa_forward",
                    "sgqa_set_stage_events", "sgqa_cache_append", "sgqa_decode_workspace_size",
                    "sgqa_decode", "sgqa_decode_noalloc", "sgqa_swa_workspace_size", "sgqa_swa",
                    "sgqa_forward_fp8kv", "sgqa_attend_backward_workspace_size",
                    "sgqa_attend_backward", "sgqa_forward_with_lse",
                    "sgqa_attend_backward_with_lse")

# scratch sgqa_decode_noalloc holds per GPU (SGQA_DECODE_NOALLOC_SCRATCH_BYTES in include/sgqa.h)
DECODE_NOALLOC_SCRATCH_BYTES = 128 << 20


class SgqaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"sgqa status {status}: {detail}")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("t_q", ctypes.c_int64), ("t_kv", ctypes.c_int64),
                ("kv_groups", ctypes.c_int32), ("heads_per_group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("block", ctypes.c_int32), ("topk_tokens", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("index_dtype", ctypes.c_int32)]


class _Sizes(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("n_sel", ctypes.c_int64),
                ("k_blk_bytes", ctypes.c_size_t), ("scores_bytes", ctypes.c_size_t),
                ("sel_bytes", ctypes.c_size_t), ("attend_workspace_bytes", ctypes.c_size_t),
                ("forward_workspace_bytes", ctypes.c_size_t),
                ("forward_workspace_min_bytes", ctypes.c_size_t)]


class _Cache(ctypes.Structure):
    _fields_ = [("num_pages", ctypes.c_int64), ("page_tokens", ctypes.c_int32),
                ("max_pages", ctypes.c_int32)]


class Cache:
    """Paged cache descriptor (sgqa_cache)."""

    def __init__(self, num_pages, page_tokens, max_pages):
        self.num_pages, self.page_tokens, self.max_pages = int(num_pages), int(page_tokens), int(max_pages)

    def _c(self) -> _Cache:
        return _Cache(self.num_pages, self.page_tokens, self.max_pages)


class Problem:
    """Problem descriptor (sgqa_problem)."""

    def __init__(self, batch, t_q, t_kv, kv_groups, heads_per_group, head_dim, index_dim, block,
                 topk_tokens, softmax_scale=None, dtype=torch.bfloat16, index_dtype=torch.bfloat16):
        self.batch, self.t_q, self.t_kv = int(batch), int(t_q), int(t_kv)
        self.kv_groups, self.heads_per_group = int(kv_groups), int(heads_per_group)
        self.head_dim, self.index_dim = int(head_dim), int(index_dim)
        self.block, self.topk_tokens = int(block), int(topk_tokens)
        self.softmax_scale = float(softmax_scale if softmax_scale is not None
                                   else 1.0 / math.sqrt(head_dim))
        self.dtype, self.index_dtype = dtype, index_dtype

    @classmethod
    def from_workload(cls, w, **overrides):
        kw = dict(batch=w.batch, t_q=w.t_q, t_kv=w.t_kv, kv_groups=w.groups,
                  heads_per_group=w.heads, head_dim=w.head_dim, index_dim=w.index_dim,
                  block=w.block, topk_tokens=w.topk, softmax_scale=w.softmax_scale,
                  dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16,
                  index_dtype=torch.float32 if w.index_dtype == "f32" else torch.bfloat16)
        kw.update(overrides)
        return cls(**kw)

    @property
    def num_blocks(self):
        return -(-self.t_kv // self.block)

    @property
    def n_sel(self):
        return self.topk_tokens // self.block

    def _c(self) -> _Problem:
        return _Problem(self.batch, self.t_q, self.t_kv, self.kv_groups, self.heads_per_group,
                        self.head_dim, self.index_dim, self.block, self.topk_tokens,
                        self.softmax_scale, _DT.get(self.dtype, -1), _DT.get(self.index_dtype, -1))


_lib = None


def library_path() -> str:
    """The in-tree libsgqa.so, or the library SGQA_LIBRARY names (e.g. the host-sanitized build)."""
    return os.environ.get("SGQA_LIBRARY") or os.path.join(_PKG_DIR, _LIB_NAME)


def load_library():
    """Load libsgqa.so (built in-tree by long_context_sparse_sgqa_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m long_context_sparse_sgqa_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    P = ctypes.POINTER(_Problem)
    lib.sgqa_abi_version.restype = ctypes.c_int
    lib.sgqa_status_string.restype = ctypes.c_char_p
    lib.sgqa_status_string.argtypes = [ctypes.c_int]
    lib.sgqa_last_error.restype = ctypes.c_char_p
    lib.sgqa_sizes.argtypes = [P, ctypes.POINTER(_Sizes)]
    lib.sgqa_index.argtypes = [P, vp, vp, vp, vp, vp]
    lib.sgqa_topk.argtypes = [P, vp, vp, vp]
    lib.sgqa_attend.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sgqa_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sgqa_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    C = ctypes.POINTER(_Cache)
    lib.sgqa_cache_append.argtypes = [P, C, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sgqa_decode_workspace_size.argtypes = [P, C, ctypes.POINTER(ctypes.c_size_t)]
    lib.sgqa_decode.argtypes = [P, C, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sgqa_decode_noalloc.argtypes = [P, C, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sgqa_swa_workspace_size.argtypes = [P, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.sgqa_swa.argtypes = [P, i64, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    f32 = ctypes.c_float
    lib.sgqa_forward_fp8kv.argtypes = [P, vp, vp, vp, f32, f32, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
    lib.sgqa_attend_backward_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.sgqa_attend_backward.argtypes = [P] + [vp] * 11 + [ctypes.c_size_t, vp]
    lib.sgqa_forward_with_lse.argtypes = [P] + [vp] * 11 + [ctypes.c_size_t, vp]
    lib.sgqa_attend_backward_with_lse.argtypes = [P] + [vp] * 13 + [ctypes.c_size_t, vp]
    for name in ("sgqa_sizes", "sgqa_index", "sgqa_topk", "sgqa_attend", "sgqa_forward",
                 "sgqa_set_stage_events", "sgqa_cache_append", "sgqa_decode_workspace_size",
                 "sgqa_decode", "sgqa_decode_noalloc", "sgqa_swa_workspace_size", "sgqa_swa",
                 "sgqa_forward_fp8kv", "sgqa_attend_backward_workspace_size",
                 "sgqa_attend_backward", "sgqa_forward_with_lse", "sgqa_attend_backward_with_lse"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def abi_version() -> int:
    return load_library().sgqa_abi_version()


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise SgqaError(status, (lib.sgqa_last_error() or b"").decode())


def sizes(prob: Problem) -> dict:
    s = _Sizes()
    _check(load_library().sgqa_sizes(ctypes.byref(prob._c()), ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in _Sizes._fields_}


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor], name: str, shape, dtype):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shapes(p: Problem):
    Bt, Tq, Tk, G, H = p.batch, p.t_q, p.t_kv, p.kv_groups, p.heads_per_group
    D, Di, NB, NS = p.head_dim, p.index_dim, p.num_blocks, p.n_sel
    return dict(q=(Bt, Tq, G, H, D), k=(Bt, G, Tk, D), q_idx=(Bt, Tq, G, Di), k_idx=(Bt, Tk, Di),
                k_blk=(Bt, NB, Di), scores=(Bt, Tq, G, NB), sel=(Bt, Tq, G, NS))


def index(prob: Problem, q_idx, k_idx, k_blk=None, scores=None, stream=None):
    """Steps 1-2.  k_idx=None scores against the given k_blk.  Returns (k_blk, scores)."""
    lib = load_library()
    sh = _shapes(prob)
    dev = q_idx.device
    if k_blk is None:
        k_blk = torch.empty(sh["k_blk"], dtype=prob.index_dtype, device=dev)
    if scores is None:
        scores = torch.empty(sh["scores"], dtype=torch.float32, device=dev)
    _check(lib.sgqa_index(ctypes.byref(prob._c()), _ptr(q_idx, "q_idx", sh["q_idx"], prob.index_dtype),
                          _ptr(k_idx, "k_idx", sh["k_idx"], prob.index_dtype),
                          _ptr(k_blk, "k_blk", sh["k_blk"], prob.index_dtype),
                          _ptr(scores, "scores", sh["scores"], torch.float32), _stream(stream)))
    return k_blk, scores


def topk(prob: Problem, scores, sel=None, stream=None):
    """Step 3.  Returns sel [Bt, Tq, G, NS] int32."""
    lib = load_library()
    sh = _shapes(prob)
    if sel is None:
        sel = torch.empty(sh["sel"], dtype=torch.int32, device=scores.device)
    _check(lib.sgqa_topk(ctypes.byref(prob._c()), _ptr(scores, "scores", sh["scores"], torch.float32),
                         _ptr(sel, "sel", sh["sel"], torch.int32), _stream(stream)))
    return sel


def attend(prob: Problem, q, k, v, gate, sel, out=None, workspace=None, stream=None):
    """Step 4.  Returns out [Bt, Tq, G, H, D]."""
    lib = load_library()
    sh = _shapes(prob)
    if out is None:
        out = torch.empty(sh["q"], dtype=prob.dtype, device=q.device)
    need = sizes(prob)["attend_workspace_bytes"]
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.sgqa_attend(ctypes.byref(prob._c()), _ptr(q, "q", sh["q"], prob.dtype),
                           _ptr(k, "k", sh["k"], prob.dtype), _ptr(v, "v", sh["k"], prob.dtype),
                           _ptr(gate, "gate", sh["q"], prob.dtype),
                           _ptr(sel, "sel", sh["sel"], torch.int32),
                           _ptr(out, "out", sh["q"], prob.dtype),
                           workspace.data_ptr() if workspace is not None else None,
                           workspace.numel() if workspace is not None else 0, _stream(stream)))
    return out


def forward(prob: Problem, q, k, v, gate, q_idx, k_idx, k_blk=None, out=None, sel=None,
            return_sel=False, workspace=None, stream=None):
    """Steps 1-4.  k_idx=None reuses the block keys in k_blk.  Returns out (and sel)."""
    lib = load_library()
    sh = _shapes(prob)
    dev = q.device
    if k_blk is None:
        k_blk = torch.empty(sh["k_blk"], dtype=prob.index_dtype, device=dev)
    if out is None:
        out = torch.empty(sh["q"], dtype=prob.dtype, device=dev)
    if sel is None and return_sel:
        sel = torch.empty(sh["sel"], dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(sizes(prob)["forward_workspace_bytes"], dtype=torch.uint8, device=dev)
    _check(lib.sgqa_forward(ctypes.byref(prob._c()), _ptr(q, "q", sh["q"], prob.dtype),
                            _ptr(k, "k", sh["k"], prob.dtype), _ptr(v, "v", sh["k"], prob.dtype),
                            _ptr(gate, "gate", sh["q"], prob.dtype),
                            _ptr(q_idx, "q_idx", sh["q_idx"], prob.index_dtype),
                            _ptr(k_idx, "k_idx", sh["k_idx"], prob.index_dtype),
                            _ptr(k_blk, "k_blk", sh["k_blk"], prob.index_dtype),
                            _ptr(sel, "sel", sh["sel"], torch.int32),
                            _ptr(out, "out", sh["q"], prob.dtype), workspace.data_ptr(),
                            workspace.numel(), _stream(stream)))
    return (out, sel) if return_sel else out


def forward_with_lse(prob: Problem, q, k, v, gate, q_idx, k_idx, k_blk=None, out=None, sel=None,
                     lse=None, workspace=None, stream=None):
    """Steps 1-4 plus the per-row softmax normaliser ln sum_t exp(scale q.k_t), float32
    [Bt, Tq, G, H], for attend_backward_with_lse.  Returns out, sel, lse."""
    lib = load_library()
    sh = _shapes(prob)
    dev = q.device
    if k_blk is None:
        k_blk = torch.empty(sh["k_blk"], dtype=prob.index_dtype, device=dev)
    if out is None:
        out = torch.empty(sh["q"], dtype=prob.dtype, device=dev)
    if sel is None:
        sel = torch.empty(sh["sel"], dtype=torch.int32, device=dev)
    if lse is None:
        lse = torch.empty(sh["q"][:-1], dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(sizes(prob)["forward_workspace_bytes"], dtype=torch.uint8, device=dev)
    _check(lib.sgqa_forward_with_lse(
        ctypes.byref(prob._c()), _ptr(q, "q", sh["q"], prob.dtype),
        _ptr(k, "k", sh["k"], prob.dtype), _ptr(v, "v", sh["k"], prob.dtype),
        _ptr(gate, "gate", sh["q"], prob.dtype),
        _ptr(q_idx, "q_idx", sh["q_idx"], prob.index_dtype),
        _ptr(k_idx, "k_idx", sh["k_idx"], prob.index_dtype),
        _ptr(k_blk, "k_blk", sh["k_blk"], prob.index_dtype),
        _ptr(sel, "sel", sh["sel"], torch.int32), _ptr(out, "out", sh["q"], prob.dtype),
        _ptr(lse, "lse", sh["q"][:-1], torch.float32), workspace.data_ptr(), workspace.numel(),
        _stream(stream)))
    return out, sel, lse


# ----------------------------------------------------------------------------------------------
# decode over a paged cache
# ----------------------------------------------------------------------------------------------
def _cache_shapes(p: Problem, c: Cache):
    P = c.page_tokens
    return dict(k_cache=(c.num_pages, p.kv_groups, P // 8, 8 * p.head_dim),
                v_cache=(c.num_pages, p.kv_groups, P // 8, p.head_dim, 8),
                kidx_cache=(c.num_pages, P, p.index_dim),
                k_blk=(p.batch, c.max_pages * P // p.block, p.index_dim),
                block_table=(p.batch, c.max_pages), seq_lens=(p.batch,))


def alloc_cache(prob: Problem, cache: Cache, device) -> dict:
    """Zero-filled cache pools and block keys for `cache` (device memory from torch)."""
    sh = _cache_shapes(prob, cache)
    return {name: torch.zeros(sh[name], dtype=torch.bfloat16, device=device)
            for name in ("k_cache", "v_cache", "kidx_cache", "k_blk")}


def cache_append(prob: Problem, cache: Cache, seq_lens, block_table, k_new, v_new, kidx_new,
                 pools: dict, stream=None):
    """Append k_new, v_new [Bt, G, n, D] and kidx_new [Bt, n, Di] at positions seq_lens - n ..
    seq_lens - 1 and recompute the touched block keys.  `pools` as from alloc_cache."""
    lib = load_library()
    sh = _cache_shapes(prob, cache)
    n = int(k_new.shape[2])
    Bt, G, D, Di = prob.batch, prob.kv_groups, prob.head_dim, prob.index_dim
    _check(lib.sgqa_cache_append(
        ctypes.byref(prob._c()), ctypes.byref(cache._c()),
        _ptr(seq_lens, "seq_lens", sh["seq_lens"], torch.int32),
        _ptr(block_table, "block_table", sh["block_table"], torch.int32), n,
        _ptr(k_new, "k_new", (Bt, G, n, D), torch.bfloat16),
        _ptr(v_new, "v_new", (Bt, G, n, D), torch.bfloat16),
        _ptr(kidx_new, "kidx_new", (Bt, n, Di), torch.bfloat16),
        _ptr(pools["k_cache"], "k_cache", sh["k_cache"], torch.bfloat16),
        _ptr(pools["v_cache"], "v_cache", sh["v_cache"], torch.bfloat16),
        _ptr(pools["kidx_cache"], "kidx_cache", sh["kidx_cache"], torch.bfloat16),
        _ptr(pools["k_blk"], "k_blk", sh["k_blk"], torch.bfloat16), _stream(stream)))


def decode_workspace_size(prob: Problem, cache: Cache) -> int:
    n = ctypes.c_size_t()
    _check(load_library().sgqa_decode_workspace_size(ctypes.byref(prob._c()),
                                                     ctypes.byref(cache._c()), ctypes.byref(n)))
    return n.value


def decode(prob: Problem, cache: Cache, seq_lens, block_table, q, gate, q_idx, pools: dict,
           out=None, sel=None, return_sel=False, workspace=None, stream=None):
    """Steps 2-4 for the prob.t_q newest tokens of every sequence over the paged cache."""
    lib = load_library()
    sh = _shapes(prob)
    csh = _cache_shapes(prob, cache)
    dev = q.device
    if out is None:
        out = torch.empty(sh["q"], dtype=torch.bfloat16, device=dev)
    if sel is None and return_sel:
        sel = torch.empty(sh["sel"], dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(decode_workspace_size(prob, cache), dtype=torch.uint8, device=dev)
    _check(lib.sgqa_decode(
        ctypes.byref(prob._c()), ctypes.byref(cache._c()),
        _ptr(seq_lens, "seq_lens", csh["seq_lens"], torch.int32),
        _ptr(block_table, "block_table", csh["block_table"], torch.int32),
        _ptr(q, "q", sh["q"], torch.bfloat16), _ptr(gate, "gate", sh["q"], torch.bfloat16),
        _ptr(q_idx, "q_idx", sh["q_idx"], torch.bfloat16),
        _ptr(pools["k_cache"], "k_cache", csh["k_cache"], torch.bfloat16),
        _ptr(pools["v_cache"], "v_cache", csh["v_cache"], torch.bfloat16),
        _ptr(pools["k_blk"], "k_blk", csh["k_blk"], torch.bfloat16),
        _ptr(sel, "sel", sh["sel"], torch.int32), _ptr(out, "out", sh["q"], torch.bfloat16),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return (out, sel) if return_sel else out


def decode_noalloc(prob: Problem, cache: Cache, seq_lens, block_table, q, gate, q_idx, pools: dict,
                   out, sel=None, stream=None):
    """sgqa_decode without a workspace: the library's fixed per-GPU scratch serves instead, so the
    call allocates nothing (out and sel must be given).  Calls that overlap on one GPU race on
    that scratch."""
    lib = load_library()
    sh = _shapes(prob)
    csh = _cache_shapes(prob, cache)
    _check(lib.sgqa_decode_noalloc(
        ctypes.byref(prob._c()), ctypes.byref(cache._c()),
        _ptr(seq_lens, "seq_lens", csh["seq_lens"], torch.int32),
        _ptr(block_table, "block_table", csh["block_table"], torch.int32),
        _ptr(q, "q", sh["q"], torch.bfloat16), _ptr(gate, "gate", sh["q"], torch.bfloat16),
        _ptr(q_idx, "q_idx", sh["q_idx"], torch.bfloat16),
        _ptr(pools["k_cache"], "k_cache", csh["k_cache"], torch.bfloat16),
        _ptr(pools["v_cache"], "v_cache", csh["v_cache"], torch.bfloat16),
        _ptr(pools["k_blk"], "k_blk", csh["k_blk"], torch.bfloat16),
        _ptr(sel, "sel", sh["sel"], torch.int32), _ptr(out, "out", sh["q"], torch.bfloat16),
        _stream(stream)))
    return out


# ----------------------------------------------------------------------------------------------
# fp8 K/V
# ----------------------------------------------------------------------------------------------
def forward_fp8kv(prob: Problem, q, k8, v8, k_scale: float, v_scale: float, gate, q_idx, k_idx,
                  k_blk=None, out=None, sel=None, return_sel=False, workspace=None, stream=None):
    """Steps 1-4 with K and V given as e4m3 codes (torch.float8_e4m3fn or uint8 tensors of k's
    shape) dequantised by per-tensor scales."""
    lib = load_library()
    sh = _shapes(prob)
    dev = q.device
    k8 = k8.view(torch.uint8) if k8.dtype != torch.uint8 else k8
    v8 = v8.view(torch.uint8) if v8.dtype != torch.uint8 else v8
    if k_blk is None:
        k_blk = torch.empty(sh["k_blk"], dtype=prob.index_dtype, device=dev)
    if out is None:
        out = torch.empty(sh["q"], dtype=prob.dtype, device=dev)
    if sel is None and return_sel:
        sel = torch.empty(sh["sel"], dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(sizes(prob)["forward_workspace_bytes"], dtype=torch.uint8, device=dev)
    _check(lib.sgqa_forward_fp8kv(
        ctypes.byref(prob._c()), _ptr(q, "q", sh["q"], prob.dtype), _ptr(k8, "k8", sh["k"], torch.uint8),
        _ptr(v8, "v8", sh["k"], torch.uint8), float(k_scale), float(v_scale),
        _ptr(gate, "gate", sh["q"], prob.dtype), _ptr(q_idx, "q_idx", sh["q_idx"], prob.index_dtype),
        _ptr(k_idx, "k_idx", sh["k_idx"], prob.index_dtype),
        _ptr(k_blk, "k_blk", sh["k_blk"], prob.index_dtype), _ptr(sel, "sel", sh["sel"], torch.int32),
        _ptr(out, "out", sh["q"], prob.dtype), workspace.data_ptr(), workspace.numel(),
        _stream(stream)))
    return (out, sel) if return_sel else out


# ----------------------------------------------------------------------------------------------
# gated sliding-window attention
# ----------------------------------------------------------------------------------------------
def swa_workspace_size(prob: Problem, window: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().sgqa_swa_workspace_size(ctypes.byref(prob._c()), int(window),
                                                   ctypes.byref(n)))
    return n.value


def swa(prob: Problem, window: int, q, k, v, gate, out=None, workspace=None, stream=None):
    """Gated attention of every query over the last `window` tokens up to its position."""
    lib = load_library()
    sh = _shapes(prob)
    if out is None:
        out = torch.empty(sh["q"], dtype=prob.dtype, device=q.device)
    if workspace is None:
        workspace = torch.empty(swa_workspace_size(prob, window), dtype=torch.uint8, device=q.device)
    _check(lib.sgqa_swa(ctypes.byref(prob._c()), int(window), _ptr(q, "q", sh["q"], prob.dtype),
                        _ptr(k, "k", sh["k"], prob.dtype), _ptr(v, "v", sh["k"], prob.dtype),
                        _ptr(gate, "gate", sh["q"], prob.dtype), _ptr(out, "out", sh["q"], prob.dtype),
                        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out


# ----------------------------------------------------------------------------------------------
# backward of the attention step
# ----------------------------------------------------------------------------------------------
def attend_backward(prob: Problem, q, k, v, gate, sel, dout, workspace=None, stream=None):
    """Gradients of out = sigmoid(gate) * attention for a fixed selection.
    Returns dq, dk, dv, dgate (dq, dgate in q's dtype; dk, dv float32 [Bt, G, Tk, D])."""
    lib = load_library()
    sh = _shapes(prob)
    dev = q.device
    dq = torch.empty(sh["q"], dtype=prob.dtype, device=dev)
    dgate = torch.empty(sh["q"], dtype=prob.dtype, device=dev)
    dk = torch.empty(sh["k"], dtype=torch.float32, device=dev)
    dv = torch.empty(sh["k"], dtype=torch.float32, device=dev)
    if workspace is None:
        n = ctypes.c_size_t()
        _check(lib.sgqa_attend_backward_workspace_size(ctypes.byref(prob._c()), ctypes.byref(n)))
        workspace = torch.empty(n.value, dtype=torch.uint8, device=dev)
    _check(lib.sgqa_attend_backward(
        ctypes.byref(prob._c()), _ptr(q, "q", sh["q"], prob.dtype), _ptr(k, "k", sh["k"], prob.dtype),
        _ptr(v, "v", sh["k"], prob.dtype), _ptr(gate, "gate", sh["q"], prob.dtype),
        _ptr(sel, "sel", sh["sel"], torch.int32), _ptr(dout, "dout", sh["q"], prob.dtype),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dgate.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(stream)))
    return dq, dk, dv, dgate


def attend_backward_with_lse(prob: Problem, q, k, v, gate, sel, out, lse, dout, workspace=None,
                             stream=None):
    """attend_backward from the forward's saved output `out` and normaliser `lse` (as returned by
    forward_with_lse) instead of a forward recompute.  Returns dq, dk, dv, dgate."""
    lib = load_library()
    sh = _shapes(prob)
    dev = q.device
    dq = torch.empty(sh["q"], dtype=prob.dtype, device=dev)
    dgate = torch.empty(sh["q"], dtype=prob.dtype, device=dev)
    dk = torch.empty(sh["k"], dtype=torch.float32, device=dev)
    dv = torch.empty(sh["k"], dtype=torch.float32, device=dev)
    if workspace is None:
        n = ctypes.c_size_t()
        _check(lib.sgqa_attend_backward_workspace_size(ctypes.byref(prob._c()), ctypes.byref(n)))
        workspace = torch.empty(n.value, dtype=torch.uint8, device=dev)
    _check(lib.sgqa_attend_backward_with_lse(
        ctypes.byref(prob._c()), _ptr(q, "q", sh["q"], prob.dtype), _ptr(k, "k", sh["k"], prob.dtype),
        _ptr(v, "v", sh["k"], prob.dtype), _ptr(gate, "gate", sh["q"], prob.dtype),
        _ptr(sel, "sel", sh["sel"], torch.int32), _ptr(out, "out", sh["q"], prob.dtype),
        _ptr(lse, "lse", sh["q"][:-1], torch.float32), _ptr(dout, "dout", sh["q"], prob.dtype),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dgate.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(stream)))
    return dq, dk, dv, dgate
