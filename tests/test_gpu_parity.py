"""GPU parity: the HIP path against the CPU oracle, bit for bit (indices and value bits).

Covers both launch shapes (one workgroup per row; several workgroups per row meeting
through the workspace), the LDS-staged and the rescan (staging overflow) refinement,
every named workload at full size (all 8192 rows of the prefill workload), edge rows, unaligned packed rows, the boundary's error codes.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import deterministic_exact_top_amd as detk
import workloads as W
from gpu_util import assert_same, debug_overrides, log, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    detk.load_library()
    return torch.device("cuda:0")


def _examples():
    import test_oracle_pins as pins
    return pins._examples()


def test_worked_examples(dev):
    import torch
    for row, k, idx, val in _examples():
        n = row.size
        buf = torch.from_numpy((row if n else np.zeros(1, np.uint32)).view(np.float32)).to(dev)
        rs = torch.zeros(1, dtype=torch.int32, device=dev)
        ln = torch.full((1,), n, dtype=torch.int32, device=dev)
        for path in (1, 2):
            with debug_overrides(path=path, multi_tile=4096):
                gi, gv = detk.topk_ragged(buf, rs, ln, k, max_len=max(n, 1))
                torch.cuda.synchronize()
            assert gi.cpu().numpy()[0].tolist() == idx, (row, k, path)
            assert gv.cpu().numpy().view(np.uint32)[0].tolist() == val, (row, k, path)


def _quantized(B=12, L=12000, k=2048, name="gpu_quantized"):
    """Few distinct values (multiples of 0.25 in [0, 4)): buckets full of equal keys."""
    buf = np.empty(B * L, np.float32)
    for b in range(B):
        rng = W.row_rng(W.seed_of(name), b)
        buf[b * L:(b + 1) * L] = (rng.integers(0, 16, L) * 0.25).astype(np.float32)
    return W.Workload(name, buf, (np.arange(B) * L).astype(np.int32), np.full(B, L, np.int32), L, k)


def _outliers(B=12, L=15000, k=2048, name="gpu_outliers"):
    """ReLU-sum rows with a few huge values, infinities and NaNs of both signs."""
    buf = np.empty(B * L, np.float32)
    specials = np.array([0x7FC00000, 0x7F800000, 0x7F7FFFFF, 0x7F800001, 0xFFC00000, 0xFF800000, 0x80000000,
                         0x00000001], np.uint32)
    for b in range(B):
        rng = W.row_rng(W.seed_of(name), b)
        row = W.relu_sum_mixture(rng, L, 0.5).view(np.uint32)
        pos = rng.choice(L, size=3 * b + 1, replace=False)
        row[pos] = specials[rng.integers(0, specials.size, pos.size)]
        buf[b * L:(b + 1) * L] = row.view(np.float32)
    return W.Workload(name, buf, (np.arange(B) * L).astype(np.int32), np.full(B, L, np.int32), L, k)


def _negative(B=8, L=9000, k=1500, name="gpu_negative"):
    """All-negative rows (pivot below every non-negative key) with -0.0 and -inf mixed in."""
    buf = np.empty(B * L, np.float32)
    for b in range(B):
        rng = W.row_rng(W.seed_of(name), b)
        row = -np.abs(rng.standard_normal(L)).astype(np.float32)
        row[rng.random(L) < 0.3] = -0.0
        row[rng.random(L) < 0.05] = -np.inf
        buf[b * L:(b + 1) * L] = row
    return W.Workload(name, buf, (np.arange(B) * L).astype(np.int32), np.full(B, L, np.int32), L, k)


def _tie_block(B=6, L=20000, k=2048, name="gpu_tie_block"):
    """Rows whose top k hold a block of 1500 bitwise-equal scores above the rest: the
    candidates above the pivot fall into one long bucket (exercises the long-bucket
    fallbacks: the exact path for one-workgroup rows, a full sort of the kept candidates
    for rows split over workgroups)."""
    buf = np.empty(B * L, np.float32)
    for b in range(B):
        rng = W.row_rng(W.seed_of(name), b)
        row = W.relu_sum_mixture(rng, L, 0.3)
        row = np.minimum(row, np.float32(4.0))
        pos = rng.choice(L, size=1500, replace=False)
        row[pos] = np.float32(5.0) if b % 2 == 0 else np.float32(-0.0)
        buf[b * L:(b + 1) * L] = row
    return W.Workload(name, buf, (np.arange(B) * L).astype(np.int32), np.full(B, L, np.int32), L, k)


SMALL = {
    "quantized": _quantized,
    "outliers": _outliers,
    "negative": _negative,
    "plateau": lambda: W.plateau_abs(B=6, L=4096, k=2048, name="gpu_plateau"),
    "decode_ragged": lambda: W.decode_ragged(B=24, n_lo=1, n_hi=20000, k=2048, name="gpu_decode"),
    "prefill_causal": lambda: W.prefill_causal(Q=160, ctx=9000, k=2048, name="gpu_prefill"),
    "narrow": lambda: W.narrow_range(B=6, L=30000, k=4096, name="gpu_narrow"),
    "long_context": lambda: W.long_context(B=5, L=40000, k=2048, short_n=1500, name="gpu_long"),
    "small_k": lambda: W.decode_ragged(B=16, n_lo=1, n_hi=6000, k=7, name="gpu_smallk"),
    "k_not_pow2": lambda: W.decode_ragged(B=16, n_lo=1, n_hi=12000, k=3000, name="gpu_k3000"),
    "tie_block": _tie_block,
}
_SMALL_CACHE = {}


def _small(name):
    if name not in _SMALL_CACHE:
        _SMALL_CACHE[name] = SMALL[name]()
    return _SMALL_CACHE[name]


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("shape", ["auto", "single", "single_exact", "single_pivot_miss", "wide", "wide_exact",
                                   "wide_pivot_miss", "wide_rescan", "multi4096", "multi8192", "multi16384",
                                   "multi32768", "multi_exact", "multi_pivot_miss", "multi_wave_select",
                                   "multi_block_select", "single_rescan", "multi_rescan", "multi_tinystage"])
def test_small_workloads(dev, name, shape):
    wl = _small(name)
    if (shape.startswith("single") or shape.startswith("wide")) and wl.max_len > 32768:
        pytest.skip("row longer than one workgroup tile")
    # single*: the many-row shapes (several rows per CU, one wave selects pivot digits);
    # wide*: the small-batch shapes (1024 threads per row, every wave selects)
    cfg = {
        "auto": {},
        "single": {"path": 1, "small": 1},
        "single_exact": {"path": 1, "fast": 0, "small": 1},
        "single_pivot_miss": {"path": 1, "fast": 2, "small": 1},
        "wide": {"path": 1, "small": 2},
        "wide_exact": {"path": 1, "fast": 0, "small": 2},
        "wide_pivot_miss": {"path": 1, "fast": 2, "small": 2},
        "wide_rescan": {"path": 1, "stage_cap": 0, "fast": 0, "small": 2},
        "multi_wave_select": {"path": 2, "multi_tile": 4096, "small": 2},
        "multi_block_select": {"path": 2, "multi_tile": 4096, "small": 1},
        "multi4096": {"path": 2, "multi_tile": 4096},
        "multi8192": {"path": 2, "multi_tile": 8192},
        "multi16384": {"path": 2, "multi_tile": 16384},
        "multi32768": {"path": 2, "multi_tile": 32768},
        "multi_exact": {"path": 2, "multi_tile": 4096, "fast": 0},
        "multi_pivot_miss": {"path": 2, "multi_tile": 4096, "fast": 2},
        "single_rescan": {"path": 1, "stage_cap": 0, "fast": 0, "small": 1},
        "multi_rescan": {"path": 2, "multi_tile": 4096, "stage_cap": 0, "fast": 0},
        "multi_tinystage": {"path": 2, "multi_tile": 4096, "stage_cap": 3, "fast": 0},
    }[shape]
    log("small workload %s shape %s B=%d max_len=%d k=%d" % (name, shape, wl.B, wl.max_len, wl.k))
    with debug_overrides(**cfg):
        gi, gv = run_gpu(wl, dev)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, "%s/%s" % (name, shape))


@pytest.mark.parametrize("name", ["plateau_4x4096", "decode_ragged_64", "narrow_128x65536", "long_context_8x262144"])
def test_full_workload_exact(dev, name):
    wl = W.full(name)
    log("full workload %s B=%d max_len=%d k=%d" % (name, wl.B, wl.max_len, wl.k))
    gi, gv = run_gpu(wl, dev)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, name)


@pytest.mark.parametrize("name", ["decode_ragged_64", "long_context_8x262144"])
def test_full_workload_forced_rescan(dev, name):
    wl = W.full(name)
    log("full workload %s, exact path with staging disabled (every refinement pass rescans)" % name)
    with debug_overrides(stage_cap=0, fast=0):
        gi, gv = run_gpu(wl, dev)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, name + "/rescan")


_PREFILL = {}


def _prefill():
    if "wl" not in _PREFILL:
        _PREFILL["wl"] = W.full("prefill_causal_8192x16384")
    return _PREFILL["wl"]


def test_full_prefill_every_row(dev):
    """The 8192 x 16384 causal prefill workload in the benchmark's launch shape: every
    one of its 8192 rows compared with the oracle element by element (indices and value
    bits), plus the canonical-order invariants checked on the whole batch at once."""
    wl = _prefill()
    log("full prefill workload: GPU run")
    gi, gv = run_gpu(wl, dev)
    log("full prefill workload: oracle on all %d rows" % wl.B)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, "prefill, every row")
    # Independent of the oracle: indices inside the window and unique, values are the
    # input bits, keys non-increasing along every row (every row is longer than k).
    n = wl.lengths.astype(np.int64)
    assert np.all(gi >= 0) and np.all(gi < n[:, None])
    srt = np.sort(gi, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])
    u = wl.scores.view(np.uint32)
    assert np.array_equal(u[wl.row_starts.astype(np.int64)[:, None] + gi], gv)
    key = np.where(gv >> 31 == 1, ~gv, gv | np.uint32(0x80000000)).astype(np.uint32)
    assert np.all(key[:, 1:] <= key[:, :-1])


def _edge_workload(L, k, lens, name):
    rng = np.random.default_rng(W.seed_of(name))
    B = len(lens)
    buf = np.empty(B * L, np.float32)
    for b in range(B):
        buf[b * L:(b + 1) * L] = W.relu_sum_mixture(rng, L, 0.7)
    return W.Workload(name, buf, (np.arange(B) * L).astype(np.int32), np.array(lens, np.int32), L, k)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_edge_lengths(dev, path):
    k = 2048
    L = 16384
    lens = [0, 1, 2, k - 1, k, k + 1, 4095, 4096, 4097, 8191, 8192, 8193, 16383, 16384, -3, 99999]
    wl = _edge_workload(L, k, lens, "edge")
    log("edge lengths path %d" % path)
    with debug_overrides(path=min(path, 2), multi_tile=4096, fast=0 if path == 3 else 1):
        gi, gv = run_gpu(wl, dev)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, "edge lengths path %d" % path)


@pytest.mark.parametrize("path", [1, 2])
def test_whole_rows_every_sort_size(dev, path):
    """Rows output whole (n <= k) through the exact path, whose final order comes from the
    bitonic sort of all n composites: every n from 1 to 130 and n around each power of two
    up to 4096, so the sort runs with every padded size, with stages inside one wave only
    and with stages that cross waves."""
    k = 4096
    L = 4096
    lens = list(range(1, 131))
    for e in range(8, 13):
        lens += [(1 << e) - 1, 1 << e, (1 << e) + 1]
    lens = [n for n in lens if n <= L]
    wl = _edge_workload(L, k, lens, "whole_rows_sort_sizes")
    log("whole rows, every sort size, path %d, B=%d" % (path, wl.B))
    with debug_overrides(path=path, multi_tile=4096, fast=0):
        gi, gv = run_gpu(wl, dev)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, "whole rows sort sizes path %d" % path)


@pytest.mark.parametrize("path", [1, 2])
def test_unaligned_packed_rows(dev, path):
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 9000, 40).astype(np.int32)
    starts = (np.cumsum(np.concatenate([[3], lens[:-1] + rng.integers(0, 5, 39)]))).astype(np.int32)
    total = int(starts[-1] + lens[-1] + 7)
    buf = np.full(total, W.QNAN, np.uint32).view(np.float32)
    for b in range(lens.size):
        buf[starts[b]:starts[b] + lens[b]] = W.relu_sum_mixture(rng, int(lens[b]), 0.5)
    wl = W.Workload("unaligned", buf, starts, lens, 9000, 1000)
    log("unaligned packed rows path %d" % path)
    with debug_overrides(path=path, multi_tile=4096):
        gi, gv = run_gpu(wl, dev)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, "unaligned path %d" % path)


def test_default_metadata_and_no_values(dev):
    import torch
    wl = W.plateau_abs(B=5, L=3000, k=1000, name="dense_default")
    m2 = torch.from_numpy(wl.scores.reshape(5, 3000)).to(dev)
    gi, _ = detk.topk_ragged(m2, None, None, 1000, with_values=False)
    gi2, gv2 = detk.topk_ragged(m2, None, None, 1000)
    torch.cuda.synchronize()
    oi, ov = run_oracle(wl)
    assert np.array_equal(gi.cpu().numpy(), oi)
    assert np.array_equal(gi2.cpu().numpy(), oi)
    assert np.array_equal(gv2.cpu().numpy().view(np.uint32), ov)


def test_many_rows_persistent_multi(dev):
    """More (row, tile) items than co-resident workgroups: the multi-workgroup grid
    loops over rounds of whole rows."""
    wl = W.decode_ragged(B=1500, n_lo=1, n_hi=9000, k=512, name="gpu_many_rows")
    log("many rows, multi path with 4096 tiles")
    with debug_overrides(path=2, multi_tile=4096):
        gi, gv = run_gpu(wl, dev)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, "many rows multi")


def test_error_codes(dev):
    import torch
    lib = detk.load_library()
    x = torch.zeros(4, 100, device=dev)
    idx = torch.empty(4, 10, dtype=torch.int32, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = ctypes.c_void_p
    call = lambda scores, B, max_len, k, out, ws=None, wsb=0: lib.detk_topk_ragged(
        scores, None, None, B, max_len, k, out, None, ws, wsb, s)
    assert call(p(x.data_ptr()), 4, 100, 0, p(idx.data_ptr())) == detk.DETK_ERR_INVALID_ARG
    assert call(p(x.data_ptr()), -1, 100, 10, p(idx.data_ptr())) == detk.DETK_ERR_INVALID_ARG
    assert call(p(x.data_ptr()), 4, -1, 10, p(idx.data_ptr())) == detk.DETK_ERR_INVALID_ARG
    assert call(None, 4, 100, 10, p(idx.data_ptr())) == detk.DETK_ERR_INVALID_ARG
    assert call(p(x.data_ptr()), 4, 100, 10, None) == detk.DETK_ERR_INVALID_ARG
    assert call(p(x.data_ptr()), 4, 100, 4097, p(idx.data_ptr())) == detk.DETK_ERR_UNSUPPORTED
    assert call(None, 0, 100, 10, None) == detk.DETK_OK
    # a split-row shape needs workspace
    big = torch.zeros(2, 300000, device=dev)
    out = torch.empty(2, 16, dtype=torch.int32, device=dev)
    need = detk.workspace_size(2, 16, 300000)
    assert need > 0
    assert lib.detk_topk_ragged(p(big.data_ptr()), None, None, 2, 300000, 16, p(out.data_ptr()), None, None, 0,
                                s) == detk.DETK_ERR_WORKSPACE
    ws = detk.new_workspace(2, 16, 300000, dev)
    assert lib.detk_topk_ragged(p(big.data_ptr()), None, None, 2, 300000, 16, p(out.data_ptr()), None,
                                p(ws.data_ptr()), need - 1, s) == detk.DETK_ERR_WORKSPACE
    assert lib.detk_topk_ragged(p(big.data_ptr()), None, None, 2, 300000, 16, p(out.data_ptr()), None,
                                p(ws.data_ptr()), need, s) == detk.DETK_OK
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), np.tile(np.arange(16, dtype=np.int32), (2, 1)))
    # every call leaves its workspace zero-filled again (ready for the next call)
    assert _ctl_words_zero(ws, 2)
    assert detk.can_implement(2048, 262144) == detk.DETK_OK
    assert detk.can_implement(4097, 10) == detk.DETK_ERR_UNSUPPORTED


def _ctl_words_zero(ws, B):
    """The per-row control words (16 bytes per row at the workspace's start) are zero
    after a call."""
    return int(ws[:B * 16].count_nonzero()) == 0


def test_envelope(dev):
    """The longest supported row is DETK_MAX_LEN = 2^30 elements; the pages' backend stops
    below 2^24 (SGLang PR #31115, hardening commit).  Checked at 2^24 - 1, 2^24, the bound
    and one past it, for both k regimes, with the workspace query agreeing."""
    lib = detk.load_library()
    size_max = (1 << 64) - 1
    for k in (2048, 4096):
        for L in ((1 << 24) - 1, 1 << 24, detk.DETK_MAX_LEN):
            assert detk.can_implement(k, L) == detk.DETK_OK, (k, L)
            assert 0 < lib.detk_workspace_size(0, 4, k, L) < size_max
        assert detk.can_implement(k, detk.DETK_MAX_LEN + 1) == detk.DETK_ERR_UNSUPPORTED
        assert lib.detk_workspace_size(0, 4, k, detk.DETK_MAX_LEN + 1) == size_max
    # the other refusals answer SIZE_MAX too, and "needs none" answers 0
    assert lib.detk_workspace_size(0, 4, 4097, 100) == size_max
    assert lib.detk_workspace_size(0, 4, 0, 100) == size_max
    assert lib.detk_workspace_size(0, 1 << 20, 4096, 100) == size_max  # B * k = 2^32
    assert lib.detk_workspace_size(0, 8, 2048, 32768) == 0
    assert lib.detk_workspace_size(0, 0, 2048, 1 << 20) == 0
    with pytest.raises(detk.DetkError):
        detk.workspace_size(4, 4097, 100)
