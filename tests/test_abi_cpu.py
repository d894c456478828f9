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
    return sorted(set(re.findall(r"\b(sgqa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(sg.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert sg.abi_version() == 1
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
    # the fused selection never stores full score rows: a 2 GiB chunk budget, not 68 GB
    assert s["forward_workspace_bytes"] < s["attend_workspace_bytes"] + s["sel_bytes"] + (3 << 30)


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
    P = sg.Problem(1, 64, 64, 2, 8, 128, 128, 3, 24)._c()   # B=3: selection fine, attention not
    assert lib.sgqa_attend(ctypes.byref(P), *([good] * 7), 1 << 20, None) == ERR_UNSUPPORTED
    assert lib.sgqa_topk(None, good, good, None) == ERR_NULL
