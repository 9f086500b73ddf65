"""The allocation-free entry point (detk_topk_ragged_noalloc) against detk_topk_ragged.

Called through the C ABI (ctypes), two calls in a row on the library's per-GPU scratch
array -- the second with a smaller input, so it reuses what the first left behind -- each
compared byte for byte with the workspace entry point's output on the same input (and
with the oracle).  Also: a call whose workspace need exceeds the scratch array is refused
on the host before any launch, and a one-tile-per-row call needs no scratch at all.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import deterministic_exact_top_amd as detk
import workloads as W
from gpu_util import assert_same, log, run_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    detk.load_library()
    return torch.device("cuda:0")


def _both(dev, wl):
    """(noalloc outputs, workspace-entry outputs), each (idx, value bits) on the host."""
    import torch
    lib = detk.load_library()
    scores, rs, ln = to_dev(wl, dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    need = detk.workspace_size(wl.B, wl.k, wl.max_len)
    assert 0 < need <= detk.DETK_SCRATCH_BYTES, need
    ni = torch.full((wl.B, wl.k), -7, dtype=torch.int32, device=dev)
    nv = torch.full((wl.B, wl.k), 7.0, dtype=torch.float32, device=dev)
    st = lib.detk_topk_ragged_noalloc(p(scores), p(rs), p(ln), wl.B, wl.max_len, wl.k, p(ni), p(nv), stream)
    assert st == detk.DETK_OK, detk.status_string(st)
    ws = detk.new_workspace(wl.B, wl.k, wl.max_len, dev)
    wi = torch.full((wl.B, wl.k), -9, dtype=torch.int32, device=dev)
    wv = torch.full((wl.B, wl.k), 9.0, dtype=torch.float32, device=dev)
    st = lib.detk_topk_ragged(p(scores), p(rs), p(ln), wl.B, wl.max_len, wl.k, p(wi), p(wv), p(ws), ws.numel(),
                              stream)
    assert st == detk.DETK_OK, detk.status_string(st)
    torch.cuda.synchronize()
    return ((ni.cpu().numpy(), nv.cpu().numpy().view(np.uint32)), (wi.cpu().numpy(), wv.cpu().numpy().view(np.uint32)))


def test_noalloc_matches_workspace_entry_two_calls(dev):
    first = W.long_context(B=8, L=262144, k=2048, short_n=1500, name="noalloc_first")
    second = W.long_context(B=3, L=70000, k=2048, short_n=900, name="noalloc_second")
    for what, wl in (("first (8 x 262144)", first), ("second, smaller (3 x 70000)", second)):
        log("noalloc %s" % what)
        (ni, nv), (wi, wv) = _both(dev, wl)
        assert_same(ni, nv, wi, wv, "noalloc vs workspace entry, %s call" % what)
        oi, ov = run_oracle(wl)
        assert_same(ni, nv, oi, ov, "noalloc vs oracle, %s call" % what)


def test_noalloc_narrow_split_rows(dev):
    wl = W.narrow_range(B=24, L=65536, k=4096, name="noalloc_narrow")
    log("noalloc %s" % wl.name)
    (ni, nv), (wi, wv) = _both(dev, wl)
    assert_same(ni, nv, wi, wv, wl.name)


def test_noalloc_one_tile_rows(dev):
    """Rows that fit one workgroup need no scratch: the call runs the same kernels."""
    import torch
    wl = W.decode_ragged(B=40, n_lo=1, n_hi=30000, k=2048, name="noalloc_decode")
    log("noalloc %s" % wl.name)
    lib = detk.load_library()
    scores, rs, ln = to_dev(wl, dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    gi = torch.empty((wl.B, wl.k), dtype=torch.int32, device=dev)
    gv = torch.empty((wl.B, wl.k), dtype=torch.float32, device=dev)
    assert lib.detk_topk_ragged_noalloc(p(scores), p(rs), p(ln), wl.B, wl.max_len, wl.k, p(gi), p(gv),
                                        None) == detk.DETK_OK
    torch.cuda.synchronize()
    oi, ov = run_oracle(wl)
    assert_same(gi.cpu().numpy(), gv.cpu().numpy().view(np.uint32), oi, ov, wl.name)


def test_noalloc_refuses_more_than_the_scratch(dev):
    lib = detk.load_library()
    B, k, L = 4096, 4096, 65536  # about 280 MB of workspace
    assert detk.workspace_size(B, k, L) > detk.DETK_SCRATCH_BYTES
    dummy = ctypes.c_void_p(0x1000)  # never touched: the call is refused on the host
    assert lib.detk_topk_ragged_noalloc(dummy, None, None, B, L, k, dummy, None, None) == detk.DETK_ERR_WORKSPACE
