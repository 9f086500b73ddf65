"""GPU parity on edge cases and a seeded randomized sweep.

Every case is checked bit for bit against the CPU oracle (indices and value bits) and
against the invariants of the canonical order.  Cases: extreme k (1, 4096), rows made
entirely of one value (finite, +/-0.0, +inf, NaN payloads), overlapping windows, rows
whose length is a whole number of tiles on the split-row path, a tie block straddling
tile boundaries, empty and one-row batches, and ~40 random (shape, k, value family)
draws from a fixed seed.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from gpu_util import assert_same, debug_overrides, log, run_gpu, run_oracle
from topk_checks import check_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import deterministic_exact_top_amd as detk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    detk.load_library()
    return torch.device("cuda:0")


def _dense(rows, k, name, L=None):
    rows = [np.asarray(r, dtype=np.float32) for r in rows]
    L = L or max(1, max(r.size for r in rows))
    buf = np.full(len(rows) * L, W.QNAN, np.uint32).view(np.float32)
    for b, r in enumerate(rows):
        buf[b * L:b * L + r.size] = r
    starts = (np.arange(len(rows)) * L).astype(np.int32)
    lens = np.array([r.size for r in rows], np.int32)
    return W.Workload(name, buf, starts, lens, L, k)


def _check(dev, wl, what, **over):
    log("edge case %s: B=%d max_len=%d k=%d %s" % (what, wl.B, wl.max_len, wl.k, over))
    with debug_overrides(**over):
        gi, gv = run_gpu(wl, dev)
    oi, ov = run_oracle(wl)
    assert_same(gi, gv, oi, ov, what)
    check_batch(wl.scores.view(np.uint32), wl.row_starts, wl.lengths, wl.max_len, wl.k, gi, gv)


SHAPES = {"auto": {}, "single": {"path": 1, "small": 1}, "wide": {"path": 1, "small": 2},
          "multi": {"path": 2, "multi_tile": 4096}}


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("k", [1, 4096])
def test_extreme_k(dev, shape, k):
    rng = np.random.default_rng(11 + k)
    rows = [W.relu_sum_mixture(rng, n, 0.5) for n in (1, 5000, 9000, 16000)]
    _check(dev, _dense(rows, k, "extreme_k"), "k=%d/%s" % (k, shape), **SHAPES[shape])


CONSTANT = {
    "finite": np.float32(1.5),
    "pos_zero": np.float32(0.0),
    "neg_zero": np.float32(-0.0),
    "pos_inf": np.float32(np.inf),
    "neg_inf": np.float32(-np.inf),
    "qnan": np.uint32(0x7FC00000).view(np.float32),
    "neg_nan_payload": np.uint32(0xFFC00123).view(np.float32),
}


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("value", sorted(CONSTANT))
def test_constant_rows(dev, shape, value):
    v = CONSTANT[value]
    rows = [np.full(n, v, np.float32) for n in (3000, 12000, 20000)]
    _check(dev, _dense(rows, 2048, "constant"), "constant %s/%s" % (value, shape), **SHAPES[shape])


@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_two_values_half_and_half(dev, shape):
    rng = np.random.default_rng(5)
    rows = []
    for n in (4097, 10000, 18000):
        r = np.where(rng.random(n) < 0.5, np.float32(2.0), np.float32(1.0)).astype(np.float32)
        rows.append(r)
    _check(dev, _dense(rows, 2048, "two_values"), "two values/%s" % shape, **SHAPES[shape])


@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_overlapping_windows(dev, shape):
    rng = np.random.default_rng(9)
    buf = W.relu_sum_mixture(rng, 40000, 0.6)
    starts = np.array([0, 100, 5000, 5000, 20000, 39990], np.int32)
    lens = np.array([30000, 10000, 2000, 30000, 20000, 10], np.int32)
    wl = W.Workload("overlap", buf, starts, lens, 30000, 1000)
    _check(dev, wl, "overlapping windows/%s" % shape, **SHAPES[shape])


@pytest.mark.parametrize("n", [32768, 65536, 98304])
def test_split_rows_whole_tiles(dev, n):
    rng = np.random.default_rng(n)
    rows = [W.relu_sum_mixture(rng, n, 0.7), -np.abs(rng.standard_normal(n)).astype(np.float32)]
    _check(dev, _dense(rows, 2048, "whole_tiles"), "whole tiles n=%d" % n)


@pytest.mark.parametrize("tile", [4096, 32768])
def test_tie_block_across_tiles(dev, tile):
    """The boundary tie set (equal keys at the k-th place) spread over several tiles:
    the smallest indices must come first, tile order being index order."""
    rng = np.random.default_rng(3)
    n = 100000
    u = rng.random(n)
    r = np.full(n, np.float32(7.0), np.float32)            # the tie value: ~60% of the row
    hi = u < 0.01                                           # ~1000 keys above it (< k)
    r[hi] = np.abs(rng.standard_normal(int(hi.sum()))).astype(np.float32) + np.float32(10.0)
    r[u > 0.6] = np.float32(3.0)                            # keys below it
    rows = [r, r[::-1].copy()]
    _check(dev, _dense(rows, 4096, "tie_block"), "tie block across tiles %d" % tile, path=2, multi_tile=tile)


def test_one_row_and_tiny_rows(dev):
    rng = np.random.default_rng(4)
    _check(dev, _dense([W.relu_sum_mixture(rng, 7000, 0.3)], 300, "one_row"), "one row")
    _check(dev, _dense([rng.standard_normal(n).astype(np.float32) for n in (1, 2, 3)], 2, "tiny"), "tiny rows")


def test_empty_batch(dev):
    import torch
    import deterministic_exact_top_amd as detk
    s = torch.zeros(0, 100, device=dev)
    idx, val = detk.topk_ragged(s, None, None, 10)
    assert idx.shape == (0, 10) and val.shape == (0, 10)


FAMILIES = ["mixture", "normal", "quantized", "narrow", "mixed_signs"]


def _family(rng, fam, n):
    if fam == "mixture":
        return W.relu_sum_mixture(rng, n, float(rng.uniform(0.0, 0.95)))
    if fam == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if fam == "quantized":
        return (rng.integers(0, 16, n) / 4.0).astype(np.float32)
    if fam == "narrow":
        return W.narrow_bits(rng, n)
    r = rng.standard_normal(n).astype(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf], np.float32)
    pos = rng.random(n) < 0.05
    r[pos] = special[rng.integers(0, 4, int(pos.sum()))]
    return r


@pytest.mark.parametrize("case", range(40))
def test_random_sweep(dev, case):
    rng = np.random.default_rng(1000 + case)
    B = int(rng.integers(1, 24))
    max_len = int(rng.choice([100, 3000, 9000, 20000, 40000, 90000]))
    k = int(rng.choice([1, 7, 64, 500, 2048, 3000, 4096]))
    fam = FAMILIES[case % len(FAMILIES)]
    rows = [_family(rng, fam, int(rng.integers(0, max_len + 1))) for _ in range(B)]
    wl = _dense(rows, k, "sweep%d" % case, L=max_len)
    _check(dev, wl, "sweep %d (%s)" % (case, fam))


def _wave_positions(n, nt_threads=512, wave=0):
    """Window positions a 16K-element tile gives to one wave (slot (v, c) of lane t holds
    position (v * NT + t) * 4 + c)."""
    pos = []
    for v in range(n // (nt_threads * 4)):
        start = v * nt_threads * 4 + wave * 256
        pos.extend(range(start, start + 256))
    return np.array(pos, dtype=np.int64)


@pytest.mark.parametrize("shift", [0.25, 0.75, 1.5, 4.0])
def test_candidates_crowd_one_wave(dev, shift):
    """Keys above the pivot concentrated in one wave's share of the tile: its region fills
    and the rest go to the shared overflow pool (or, for the largest shifts, the pool runs
    out and the row takes the exact path).  Results must not depend on which."""
    rng = np.random.default_rng(int(shift * 100))
    n = 16384
    rows = []
    for wave in (0, 3, 7):
        r = np.abs(rng.standard_normal(n)).astype(np.float32)
        pw = _wave_positions(n, wave=wave)
        r[pw] += np.float32(shift)
        rows.append(r)
    _check(dev, _dense(rows, 2048, "crowd"), "candidates crowd one wave (shift %.2f)" % shift, path=1, small=1)


def test_only_one_wave_has_candidates(dev):
    """Every non-zero score sits in wave 0's share: the pivot lands on the 0.0 plateau, all
    2048 positives are candidates of one wave, and the pool cannot hold them."""
    rng = np.random.default_rng(21)
    n = 16384
    r = np.zeros(n, np.float32)
    pw = _wave_positions(n, wave=0)
    r[pw] = (np.abs(rng.standard_normal(pw.size)) + 0.01).astype(np.float32)
    _check(dev, _dense([r, r.copy()], 2048, "one_wave"), "only one wave has candidates", path=1, small=1)


def _bottom_family(rng, fam, n):
    """Rows whose least key takes a particular form (every row here is output whole)."""
    if fam == "zero_plateau":  # +0.0 on 80 % of the row, positive scores above it
        return W.relu_sum_mixture(rng, n, 0.8)
    if fam == "neg_inf_plateau":
        r = rng.standard_normal(n).astype(np.float32)
        r[rng.random(n) < 0.5] = np.float32(-np.inf)
        return r
    if fam == "neg_nan_bottom":  # negative NaNs order below -inf; two payloads
        r = rng.standard_normal(n).astype(np.float32)
        u = r.view(np.uint32)
        pick = rng.random(n)
        u[pick < 0.3] = np.uint32(0xFFC00123)
        u[pick > 0.9] = np.uint32(0xFF800001)
        return r
    if fam == "unique_min":
        return rng.standard_normal(n).astype(np.float32)
    if fam == "constant":
        return np.full(n, np.float32(-2.5), np.float32)
    # the least possible key (bits 0xFFFFFFFF) present: no pivot is taken then
    r = rng.standard_normal(n).astype(np.float32)
    r.view(np.uint32)[rng.random(n) < 0.2] = np.uint32(0xFFFFFFFF)
    return r


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("fam", ["zero_plateau", "neg_inf_plateau", "neg_nan_bottom", "unique_min", "constant",
                                 "least_key"])
def test_whole_row_outputs(dev, shape, fam):
    """Rows no longer than k (every element is output): the pivot is the row's least key,
    and the keys equal to it fill the tail in index order.  Row lengths from 1 to k, and
    one row longer than k for contrast."""
    rng = np.random.default_rng(len(fam) * 31 + len(shape))
    rows = [_bottom_family(rng, fam, n) for n in (1, 2, 7, 64, 1500, 2047, 2048, 2100)]
    _check(dev, _dense(rows, 2048, "whole_" + fam), "whole-row outputs %s/%s" % (fam, shape), **SHAPES[shape])


@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_whole_row_outputs_k4096(dev, shape):
    rng = np.random.default_rng(77)
    rows = [_bottom_family(rng, f, n) for f, n in (("zero_plateau", 4096), ("neg_inf_plateau", 3000),
                                                    ("neg_nan_bottom", 4095), ("unique_min", 1))]
    _check(dev, _dense(rows, 4096, "whole_k4096"), "whole-row outputs k=4096/%s" % shape, **SHAPES[shape])


def _plateau_family(rng, fam, n):
    """Rows where one key fills a long run of a kept bucket (the rest of the bucket: a few
    neighbouring keys)."""
    def with_neighbours(r, x, count):
        u = r.view(np.uint32)
        pos = rng.choice(n, size=count, replace=False)
        near = np.array([x], np.float32).view(np.uint32)[0] + rng.integers(-3, 4, count).astype(np.int64)
        u[pos] = near.astype(np.uint32)
        return r
    if fam == "zero_above_specials":  # whole row: +0.0 on 80 %, specials and negatives below it
        r = W.relu_sum_mixture(rng, n, 0.8)
        r[rng.random(n) < 0.05] = np.float32(-1.5)
        u = r.view(np.uint32)
        u[rng.choice(n, 6, replace=False)] = np.array([0x80000000, 0x00000001, 0xFFC00000, 0xFF800000,
                                                        0x80000001, 0x7FC00000], np.uint32)
        return r
    if fam == "one_above_gauss":  # whole row: 1.0 on 60 %, keys within 3 ulps of it on a few
        r = rng.standard_normal(n).astype(np.float32)
        r[rng.random(n) < 0.6] = np.float32(1.0)
        return with_neighbours(r, 1.0, 20)
    if fam == "minority_first":  # the first position holds a rare key of the long bucket
        r = W.relu_sum_mixture(rng, n, 0.8)
        r[rng.random(n) < 0.05] = np.float32(-1.0)
        r.view(np.uint32)[0] = np.uint32(0x00000001)
        return r
    if fam == "two_zeros":  # +0.0 and -0.0 share the bucket half and half
        r = W.relu_sum_mixture(rng, n, 0.8)
        z = np.flatnonzero(r == 0)
        r[z[rng.random(z.size) < 0.5]] = np.float32(-0.0)
        r[rng.random(n) < 0.05] = np.float32(-2.0)
        return r
    if fam in ("others_at_limit", "others_past_limit"):  # whole row: X = 1.0 with exactly 128
        # (or 129) keys within 3 ulps of it but not equal, the ranking limit of the others
        r = np.full(n, np.float32(1.0), np.float32)
        cnt = 128 if fam == "others_at_limit" else 129
        pos = 1 + rng.choice(n - 1, size=cnt + 2, replace=False)  # position 0 keeps X
        u = r.view(np.uint32)
        step = rng.integers(1, 4, cnt) * rng.choice(np.array([-1, 1]), cnt)
        u[pos[:cnt]] = (np.int64(0x3F800000) + step).astype(np.uint32)
        r[pos[cnt]] = np.float32(-100.0)
        r[pos[cnt + 1]] = np.float32(100.0)
        return r
    if fam == "kept_plateau":  # longer than k: a plateau of 1,500 at 3.0 inside the top k
        r = rng.standard_normal(n).astype(np.float32)
        r[rng.choice(n, 1500, replace=False)] = np.float32(3.0)
        return with_neighbours(r, 3.0, 12)
    # longer than k: the plateau straddles the k-th place (its key is the pivot)
    r = rng.standard_normal(n).astype(np.float32)
    r[rng.choice(n, 3000, replace=False)] = np.float32(3.0)
    return r


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("fam", ["zero_above_specials", "one_above_gauss", "minority_first", "two_zeros",
                                 "others_at_limit", "others_past_limit", "kept_plateau", "straddling_plateau"])
def test_plateau_buckets(dev, shape, fam):
    """One key repeated on a long run of a kept bucket: those elements are placed by position
    instead of ranked, the bucket's other keys ranked among themselves around them (or, when
    the bucket's first element has a rare key or two keys share it, the sort or the exact path
    takes the row).  Whole rows from 300 to k, and rows longer than k with the plateau inside
    or straddling the top k."""
    rng = np.random.default_rng(len(fam) * 17 + len(shape))
    whole = fam not in ("kept_plateau", "straddling_plateau")
    ns = (300, 1500, 2047, 2048) if whole else (4000, 9000, 16000)
    if fam.startswith("others_"):
        ns = (1500, 2048)
    rows = [_plateau_family(rng, fam, n) for n in ns]
    _check(dev, _dense(rows, 2048, "plateau_" + fam), "plateau bucket %s/%s" % (fam, shape), **SHAPES[shape])

@pytest.mark.parametrize("samples", [1, 2])
@pytest.mark.parametrize("fam", ["mixture", "plateau_top", "negative", "nan_heavy", "narrow"])
def test_split_row_sample_counts(dev, samples, fam):
    """Rows split over workgroups with 8192 (1) or 4096 (2) row samples forced, whatever the
    candidate list's room: the pivot only steers, so both give the oracle's output, also
    where the smaller sample overflows the list and the row falls back."""
    rng = np.random.default_rng(len(fam) * 7 + samples)
    def row(n):
        if fam == "mixture":
            return W.relu_sum_mixture(rng, n, 0.6)
        if fam == "plateau_top":  # a long run of the top key
            r = rng.standard_normal(n).astype(np.float32)
            r[rng.choice(n, 3000, replace=False)] = np.float32(5.0)
            return r
        if fam == "negative":
            return (-np.abs(rng.standard_normal(n)) - 1.0).astype(np.float32)
        if fam == "nan_heavy":
            r = rng.standard_normal(n).astype(np.float32)
            r.view(np.uint32)[rng.random(n) < 0.01] = np.uint32(0x7FC00001)
            return r
        u = (np.uint32(0x3F800000) | rng.integers(0, 8192, n).astype(np.uint32))
        return u.view(np.float32)
    rows = [row(n) for n in (40000, 70000, 150000)]
    _check(dev, _dense(rows, 2048, "split_samples_" + fam), "split-row samples %d/%s" % (samples, fam),
           split_samples=samples)
