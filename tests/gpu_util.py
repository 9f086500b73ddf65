"""Helpers shared by the GPU tests: run the HIP path through the C ABI binding and
compare against the CPU oracle bit for bit."""
from __future__ import annotations

import contextlib
import sys

import numpy as np

import deterministic_exact_top_amd as detk
import oracle


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(wl, dev):
    import torch
    scores = torch.from_numpy(wl.scores).to(dev)
    rs = torch.from_numpy(wl.row_starts).to(dev)
    ln = torch.from_numpy(wl.lengths).to(dev)
    return scores, rs, ln


def run_gpu(wl, dev, scores=None, rs=None, ln=None, k=None):
    import torch
    if scores is None:
        scores, rs, ln = to_dev(wl, dev)
    idx, val = detk.topk_ragged(scores, rs, ln, k or wl.k, max_len=wl.max_len)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy().view(np.uint32)


def run_oracle(wl, rows=None, k=None):
    k = k or wl.k
    if rows is None:
        return oracle.topk_ragged(wl.scores, wl.row_starts, wl.lengths, k, wl.max_len)
    rows = np.asarray(rows)
    return oracle.topk_ragged(wl.scores, wl.row_starts[rows], wl.lengths[rows], k, wl.max_len)


def assert_same(gi, gv, oi, ov, what: str) -> None:
    if np.array_equal(gi, oi) and np.array_equal(gv, ov):
        return
    bad_rows = np.flatnonzero(~(np.all(gi == oi, axis=1) & np.all(gv == ov, axis=1)))
    b = int(bad_rows[0])
    pos = np.flatnonzero((gi[b] != oi[b]) | (gv[b] != ov[b]))
    p0 = int(pos[0])
    raise AssertionError(
        "%s: %d rows differ; first row %d, first slot %d: gpu (%d, %08X) vs oracle (%d, %08X); "
        "%d slots differ in that row" % (what, bad_rows.size, b, p0, gi[b, p0], gv[b, p0], oi[b, p0],
                                         ov[b, p0], pos.size))


@contextlib.contextmanager
def debug_overrides(path=None, stage_cap=None, multi_tile=None, fast=None, small=None, split_samples=None):
    try:
        if split_samples is not None:
            detk.debug_set(detk.DETK_DEBUG_SPLIT_SAMPLES, split_samples)
        if small is not None:
            detk.debug_set(detk.DETK_DEBUG_SMALL_BATCH, small)
        if fast is not None:
            detk.debug_set(detk.DETK_DEBUG_FAST, fast)
        if path is not None:
            detk.debug_set(detk.DETK_DEBUG_PATH, path)
        if stage_cap is not None:
            detk.debug_set(detk.DETK_DEBUG_STAGING_CAP, stage_cap)
        if multi_tile is not None:
            detk.debug_set(detk.DETK_DEBUG_MULTI_TILE, multi_tile)
        yield
    finally:
        detk.debug_set(detk.DETK_DEBUG_PATH, 0)
        detk.debug_set(detk.DETK_DEBUG_STAGING_CAP, -1)
        detk.debug_set(detk.DETK_DEBUG_MULTI_TILE, 0)
        detk.debug_set(detk.DETK_DEBUG_FAST, 1)
        detk.debug_set(detk.DETK_DEBUG_SMALL_BATCH, 0)
        detk.debug_set(detk.DETK_DEBUG_SPLIT_SAMPLES, 0)
