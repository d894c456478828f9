"""The C-ABI library without a GPU: it loads, exports every symbol include/sgqa.h declares, and its
host-side validation rejects bad arguments with the documented status before touching a device.
No call here enqueues GPU work."""
import ctypes
import os
import re

import pytest
import torch

import long_context_sparse_sgqa_amd as sg
from sgqa_inputs import get_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(7)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sg.library_path()):
        pytest.fail("libsgqa.so is not built: run `python -m long_context_sparse_sgqa_amd.build`")
    return sg.load_library()


def _declared_functions():
    with open(os.path.join(ROOT, "include", "sgqa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgqa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(sg.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert sg.abi_version() == 2
    assert lib.sgqa_status_string(0) == b"ok"
    assert lib.sgqa_status_string(ERR_WORKSPACE) == b"workspace too small"


def _prob(**kw):
    return sg.Problem.from_workload(get_workload("128k"), **kw)


def test_sizes_headline_workload():
    s = sg.sizes(_prob())
    assert s["num_blocks"] == 16384 and s["n_sel"] == 512
    assert s["k_blk_bytes"] == 16384 * 128 * 2
    assert s["scores_bytes"] == 131072 * 8 * 16384 * 4
    assert s["sel_bytes"] == 131072 * 8 * 512 * 4
    assert s["attend_workspace_bytes"] >= 2 * 8 * 16384 * 8 * 128 * 2   # unit-packed K and V
    assert s["forward_workspace_bytes"] > s["forward_workspace_min_bytes"] > s["attend_workspace_bytes"]
    # the fused selection never stores full score rows: a 17 GiB chunk budget, not 68 GB
    assert s["forward_workspace_bytes"] < s["attend_workspace_bytes"] + s["sel_bytes"] + (18 << 30)


@pytest.mark.parametrize("kw,status", [
    (dict(block=0), ERR_SHAPE),
    (dict(topk_tokens=4100), ERR_SHAPE),             # not a multiple of B
    (dict(topk_tokens=4), ERR_SHAPE),                # k < B
    (dict(t_q=131073), ERR_SHAPE),                   # t_q > t_kv
    (dict(batch=0), ERR_SHAPE),
    (dict(softmax_scale=0.0), ERR_SHAPE),
    (dict(softmax_scale=float("nan")), ERR_SHAPE),
    (dict(head_dim=96), ERR_UNSUPPORTED),
    (dict(index_dim=48), ERR_UNSUPPORTED),
    (dict(dtype=torch.float16), ERR_UNSUPPORTED),
    (dict(topk_tokens=8 * 8192), ERR_UNSUPPORTED),   # more than 4096 selected blocks
    (dict(t_kv=1 << 27, t_q=1), ERR_UNSUPPORTED),
])
def test_sizes_rejects(kw, status):
    with pytest.raises(sg.SgqaError) as e:
        sg.sizes(_prob(**kw))
    assert e.value.status == status
    assert sg.load_library().sgqa_last_error()


def _call_forward(lib, prob, ptrs, ws_bytes):
    P = prob._c()
    return lib.sgqa_forward(ctypes.byref(P), *ptrs, ws_bytes, None)


def test_null_misaligned_and_workspace_errors(lib):
    """Bogus (never dereferenced) addresses: validation must fail before any device access."""
    prob = sg.Problem(1, 64, 64, 2, 8, 128, 128, 8, 32)
    good = 0x10000
    ptrs = [good] * 10      # q k v gate q_idx k_idx k_blk sel out workspace
    ptrs[0] = None
    assert _call_forward(lib, prob, ptrs, 1 << 20) == ERR_NULL
    ptrs[0] = good + 8
    assert _call_forward(lib, prob, ptrs, 1 << 20) == ERR_ALIGN
    ptrs[0] = good
    assert _call_forward(lib, prob, ptrs, 16) == ERR_WORKSPACE
    msg = lib.sgqa_last_error().decode()
    assert "workspace" in msg
    P = sg.Problem(1, 64, 64, 2, 8, 128, 128, 3, 24)._c()   # B=3: any block size is accepted
    assert lib.sgqa_attend(ctypes.byref(P), None, *([good] * 6), 1 << 20, None) == ERR_NULL
    assert lib.sgqa_topk(None, good, good, None) == ERR_NULL


def test_training_entry_points_reject_before_device_access(lib):
    """sgqa_forward_with_lse, sgqa_attend_backward and sgqa_attend_backward_with_lse: bogus (never
    dereferenced) addresses; every null argument, a misaligned lse and a short workspace are
    rejected on the host, and so are problems outside the backward's kernels."""
    good = 0x10000
    P = sg.Problem(1, 64, 64, 2, 8, 128, 128, 8, 32)._c()
    need = ctypes.c_size_t()
    assert lib.sgqa_attend_backward_workspace_size(ctypes.byref(P), ctypes.byref(need)) == OK
    assert need.value > 0
    # q k v gate sel dout dq dk dv dgate workspace
    for i in range(11):
        args = [good] * 11
        args[i] = None
        assert lib.sgqa_attend_backward(ctypes.byref(P), *args, need.value, None) == ERR_NULL, i
    assert lib.sgqa_attend_backward(ctypes.byref(P), *([good] * 11), need.value - 1, None) == ERR_WORKSPACE
    # q k v gate sel out lse dout dq dk dv dgate workspace
    for i in range(13):
        args = [good] * 13
        args[i] = None
        assert lib.sgqa_attend_backward_with_lse(ctypes.byref(P), *args, need.value, None) == ERR_NULL, i
    args = [good] * 13
    args[6] = good + 2                                   # lse: fp32, 4-byte aligned
    assert lib.sgqa_attend_backward_with_lse(ctypes.byref(P), *args, need.value, None) == ERR_ALIGN
    assert lib.sgqa_attend_backward_with_lse(ctypes.byref(P), *([good] * 13), need.value - 1,
                                             None) == ERR_WORKSPACE
    for kw in (dict(heads_per_group=4), dict(block=4), dict(head_dim=96)):
        base = dict(batch=1, t_q=64, t_kv=64, kv_groups=2, heads_per_group=8, head_dim=128,
                    index_dim=128, block=8, topk_tokens=32)
        base.update(kw)
        Pu = sg.Problem(**base)._c()
        assert lib.sgqa_attend_backward_workspace_size(ctypes.byref(Pu), ctypes.byref(need)) in (
            ERR_UNSUPPORTED, ERR_SHAPE), kw
    # forward with lse: q k v gate q_idx k_idx k_blk sel out lse workspace
    Pf = sg.Problem(1, 64, 64, 2, 8, 128, 128, 8, 32)
    ws = sg.sizes(Pf)["forward_workspace_bytes"]
    args = [good] * 11
    args[9] = None
    assert lib.sgqa_forward_with_lse(ctypes.byref(Pf._c()), *args, ws, None) == ERR_NULL
    args[9] = good + 2
    assert lib.sgqa_forward_with_lse(ctypes.byref(Pf._c()), *args, ws, None) == ERR_ALIGN
    args[9] = good
    assert lib.sgqa_forward_with_lse(ctypes.byref(Pf._c()), *args, 16, None) == ERR_WORKSPACE
    # the normaliser needs the range-split attention: B = 4 takes the pair kernel instead
    Pb = sg.Problem(1, 64, 64, 2, 8, 128, 128, 4, 32)
    wsb = sg.sizes(Pb)["forward_workspace_bytes"]
    assert lib.sgqa_forward_with_lse(ctypes.byref(Pb._c()), *([good] * 11), wsb, None) == ERR_UNSUPPORTED


# ----------------------------------------------------------------------------------------------
# decode over a paged cache: host-side validation and sizes
# ----------------------------------------------------------------------------------------------
def _dprob(**kw):
    base = dict(batch=64, t_q=4, t_kv=262148, kv_groups=8, heads_per_group=8, head_dim=128,
                index_dim=128, block=8, topk_tokens=4096)
    base.update(kw)
    return sg.Problem(**base)


def test_decode_workspace_size_decode_workload(lib):
    cache = sg.Cache(64 * 4097, 64, 4097)
    n = sg.decode_workspace_size(_dprob(), cache)
    rows = 64 * 4 * 8
    cand = rows * 2048 * 8                            # candidate lists (4 * 8 rows per sequence)
    scratch = 256 * 32769 * 4                         # fallback score rows
    sel = rows * 512 * 4
    assert cand + scratch + sel < n < cand + scratch + sel + (64 << 20)   # + row arrays, partials


@pytest.mark.parametrize("cache,kw,status", [
    ((40, 48, 6000), {}, ERR_SHAPE),                  # page not a power of two
    ((40, 4, 70000), {}, ERR_SHAPE),                  # page smaller than 8 tokens
    ((40, 64, 100), {}, ERR_SHAPE),                   # max_pages * page < t_kv
    ((0, 64, 4097), {}, ERR_SHAPE),
    ((64 * 4097, 64, 4097), dict(dtype=torch.float32), ERR_UNSUPPORTED),
    ((64 * 4097, 64, 4097), dict(heads_per_group=4), ERR_UNSUPPORTED),
    ((64 * 4097, 64, 4097), dict(block=4, topk_tokens=2048), ERR_UNSUPPORTED),
    ((1 << 30, 64, 4097), {}, ERR_UNSUPPORTED),       # pool units past 2^32
])
def test_decode_rejects(lib, cache, kw, status):
    with pytest.raises(sg.SgqaError) as e:
        sg.decode_workspace_size(_dprob(**kw), sg.Cache(*cache))
    assert e.value.status == status
    assert lib.sgqa_last_error()


def test_decode_and_append_null_and_workspace_errors(lib):
    """Bogus (never dereferenced) addresses: validation fails before any device access."""
    P = _dprob()._c()
    C = sg.Cache(64 * 4097, 64, 4097)._c()
    good = 0x10000
    # seq_lens block_table q gate q_idx k_cache v_cache k_blk sel out workspace
    ptrs = [good] * 11
    assert lib.sgqa_decode(ctypes.byref(P), ctypes.byref(C), *ptrs, 16, None) == ERR_WORKSPACE
    ptrs[0] = None
    assert lib.sgqa_decode(ctypes.byref(P), ctypes.byref(C), *ptrs, 1 << 40, None) == ERR_NULL
    ptrs[0] = good + 2
    assert lib.sgqa_decode(ctypes.byref(P), ctypes.byref(C), *ptrs, 1 << 40, None) == ERR_ALIGN
    ptrs[0] = good
    ptrs[2] = good + 4                                  # q needs 16 bytes
    assert lib.sgqa_decode(ctypes.byref(P), ctypes.byref(C), *ptrs, 1 << 40, None) == ERR_ALIGN
    assert lib.sgqa_decode(ctypes.byref(P), None, *([good] * 11), 1 << 40, None) == ERR_NULL
    # seq_lens block_table n_new k_new v_new kidx_new k_cache v_cache kidx_cache k_blk
    app = [good, good, 4] + [good] * 7
    app[2] = 0
    assert lib.sgqa_cache_append(ctypes.byref(P), ctypes.byref(C), *app, None) == ERR_SHAPE
    app[2] = 4
    app[3] = None
    assert lib.sgqa_cache_append(ctypes.byref(P), ctypes.byref(C), *app, None) == ERR_NULL


def test_decode_noalloc_rejects_before_device_access(lib):
    """sgqa_decode_noalloc: a problem whose decode workspace exceeds the fixed scratch is rejected
    with ERR_WORKSPACE, and a null argument with ERR_NULL, before the scratch is looked up (bogus,
    never dereferenced addresses; no device here)."""
    good = 0x10000
    big = _dprob(batch=256)
    Cb = sg.Cache(256 * 4097, 64, 4097)
    assert sg.decode_workspace_size(big, Cb) > sg.DECODE_NOALLOC_SCRATCH_BYTES
    assert sg.decode_workspace_size(_dprob(), sg.Cache(64 * 4097, 64, 4097)) <= \
        sg.DECODE_NOALLOC_SCRATCH_BYTES                 # the decode workload fits
    # seq_lens block_table q gate q_idx k_cache v_cache k_blk sel out
    ptrs = [good] * 10
    st = lib.sgqa_decode_noalloc(ctypes.byref(big._c()), ctypes.byref(Cb._c()), *ptrs, None)
    assert st == ERR_WORKSPACE
    assert b"scratch" in lib.sgqa_last_error()
    ptrs[9] = None
    P = _dprob()._c()
    C = sg.Cache(64 * 4097, 64, 4097)._c()
    assert lib.sgqa_decode_noalloc(ctypes.byref(P), ctypes.byref(C), *ptrs, None) == ERR_NULL
