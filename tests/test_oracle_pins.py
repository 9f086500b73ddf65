"""Pins for the CPU oracle: checked against things other than the oracle itself.

* the IEEE totalOrder table (tests/golden/total_order.txt) and hand-derived worked
  examples (tests/golden/worked_examples.txt);
* exhaustive / random brute force by rank counting (topk_checks.brute_force_row);
* an independent library routine (numpy.lexsort on a differently built key) and,
  for distinct finite rows, torch.topk's index set;
* closed forms that need no sort (0.0 plateau rows, all -inf rows, short rows, the
  8192-value narrow range via a counting sort);
* invariants on shrunken versions of every named workload;
* planted mistakes: mutated copies of the oracle source must fail these pins.
"""
from __future__ import annotations

import ctypes
import itertools
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W
from topk_checks import (NEG_INF_BITS, brute_force_row, check_batch, check_row, ieee_total_order_lt,
                         lexsort_reference, signed_key)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _table():
    out = []
    with open(os.path.join(GOLDEN, "total_order.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(int(line, 16))
    return out


def _examples():
    out = []
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fields = dict(tok.split("=", 1) for tok in line.split())
            row = [] if fields["row"] == "-" else [int(x, 16) for x in fields["row"].split(",")]
            k = int(fields["k"])
            idx = [int(x) for x in fields["idx"].split(",")]
            val = [int(x, 16) for x in fields["val"].split(",")]
            out.append((np.array(row, dtype=np.uint32), k, idx, val))
    return out


def _oracle_one(row_bits, k, lib_call=None):
    row_bits = np.ascontiguousarray(row_bits, dtype=np.uint32)
    n = row_bits.shape[0]
    call = lib_call or oracle.topk_ragged
    idx, val = call(row_bits if n else np.zeros(1, np.uint32), np.array([0], np.int32),
                    np.array([n], np.int32), k, max(n, 1))
    return idx[0], val[0]


# ------------------------------------------------------------------ total order

def test_total_order_table_matches_ieee_comparator():
    t = _table()
    for hi, lo in zip(t, t[1:]):
        assert ieee_total_order_lt(lo, hi), "%08X should be below %08X" % (lo, hi)
        assert not ieee_total_order_lt(hi, lo)
    for a in t:
        assert not ieee_total_order_lt(a, a)


def test_oracle_key_is_strictly_decreasing_over_table():
    keys = [oracle.key_of_bits(b) for b in _table()]
    assert all(a > b for a, b in zip(keys, keys[1:]))
    # Spot values of the mapping: +0.0 sits exactly above -0.0 at the middle.
    assert oracle.key_of_bits(0x00000000) == 0x80000000
    assert oracle.key_of_bits(0x80000000) == 0x7FFFFFFF
    assert oracle.key_of_bits(0xFFFFFFFF) == 0
    assert oracle.key_of_bits(0x7FFFFFFF) == 0xFFFFFFFF


def test_signed_key_agrees_with_ieee_comparator_on_random_pairs():
    rng = np.random.default_rng(11)
    bits = np.concatenate([rng.integers(0, 2**32, 4000, dtype=np.uint64).astype(np.uint32),
                           np.array(_table(), dtype=np.uint32)])
    sk = signed_key(bits)
    pairs = rng.integers(0, bits.size, size=(6000, 2))
    for i, j in pairs:
        a, b = int(bits[i]), int(bits[j])
        assert (sk[i] < sk[j]) == ieee_total_order_lt(a, b)


# ------------------------------------------------------------------ worked examples

@pytest.mark.parametrize("case", range(len(_examples())))
def test_worked_example(case):
    row, k, idx, val = _examples()[case]
    bi, bv = brute_force_row(row, k)
    assert bi == idx and bv == val, "brute force disagrees with the hand-derived example"
    oi, ov = _oracle_one(row, k)
    assert oi.tolist() == idx
    assert ov.tolist() == val


# ------------------------------------------------------------------ brute force

ALPHABETS = [
    [0x00000000, 0x80000000, 0x3F800000, 0x7FC00000],               # +0, -0, 1.0, +qNaN
    [0xFF800000, 0x00000001, 0x7F800001, 0xFFC00000],               # -inf, denorm, +sNaN, -qNaN
]


@pytest.mark.parametrize("alphabet", range(len(ALPHABETS)))
def test_exhaustive_small_rows_against_brute_force(alphabet):
    letters = ALPHABETS[alphabet]
    for k in range(1, 3):
        oi, ov = _oracle_one(np.zeros(0, np.uint32), k)
        assert oi.tolist() == [-1] * k and ov.tolist() == [NEG_INF_BITS] * k
    for n in range(1, 6):
        rows = np.array(list(itertools.product(letters, repeat=n)), dtype=np.uint32).reshape(-1, n)
        R = rows.shape[0]
        for k in range(1, n + 3):
            flat = np.ascontiguousarray(rows).reshape(-1)
            starts = (np.arange(R) * n).astype(np.int32)
            lens = np.full(R, n, np.int32)
            oi, ov = oracle.topk_ragged(flat, starts, lens, k, n)
            for r in range(R):
                bi, bv = brute_force_row(rows[r], k)
                assert oi[r].tolist() == bi and ov[r].tolist() == bv, (rows[r], k)


def test_random_rows_eleven_letter_alphabet_against_brute_force():
    letters = np.array([0x7FC00000, 0x7F800001, 0x7F800000, 0x40000000, 0x3F800000, 0x00000001,
                        0x00000000, 0x80000000, 0xBF800000, 0xFF800000, 0xFFC00000], dtype=np.uint32)
    rng = np.random.default_rng(2024)
    for _ in range(300):
        n = int(rng.integers(1, 13))
        row = letters[rng.integers(0, letters.size, n)]
        k = int(rng.integers(1, n + 3))
        bi, bv = brute_force_row(row, k)
        oi, ov = _oracle_one(row, k)
        assert oi.tolist() == bi and ov.tolist() == bv, (row, k)


# ------------------------------------------------------------------ independent library routine

def _random_bits_row(rng, n, mode):
    if mode == "bits":       # every float class, NaNs included
        return rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    if mode == "dups":       # heavy bitwise duplication
        pool = rng.integers(0, 2**32, max(1, n // 50), dtype=np.uint64).astype(np.uint32)
        return pool[rng.integers(0, pool.size, n)]
    if mode == "mixture":
        return W.relu_sum_mixture(rng, n, 0.7).view(np.uint32)
    raise ValueError(mode)


@pytest.mark.parametrize("mode", ["bits", "dups", "mixture"])
def test_oracle_equals_numpy_lexsort(mode):
    rng = np.random.default_rng(7 + len(mode))
    lens = np.array([1, 17, 1000, 4097, 30000, 100000], dtype=np.int32)
    rows = [_random_bits_row(rng, int(n), mode) for n in lens]
    flat = np.concatenate(rows)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    for k in (1, 7, 2048, 4096):
        oi, ov = oracle.topk_ragged(flat, starts, lens, k, int(lens.max()))
        for b, row in enumerate(rows):
            ri, rv = lexsort_reference(row, k)
            assert np.array_equal(oi[b], ri) and np.array_equal(ov[b], rv), (mode, b, k)


def test_index_set_equals_torch_topk_on_distinct_finite_rows():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    for n, k in ((4096, 2048), (10000, 512), (3000, 3000)):
        vals = rng.permutation(np.arange(n, dtype=np.float32) * 0.25 - 100.0)
        oi, _ = _oracle_one(vals.view(np.uint32), k)
        _, ti = torch.topk(torch.from_numpy(vals), min(k, n))
        assert set(oi[oi >= 0].tolist()) == set(ti.tolist())


# ------------------------------------------------------------------ closed forms

def test_plateau_rows_closed_form():
    """Rows of +0.0 and positive finite values: when fewer than k positives exist,
    the boundary is +0.0 and the selected zeros are the smallest zero positions."""
    wl = W.plateau_abs(B=6, L=4096, k=2048, p=0.6, name="pin_plateau")
    oi, ov = oracle.topk_ragged(wl.scores, wl.row_starts, wl.lengths, wl.k, wl.max_len)
    u = wl.scores.view(np.uint32)
    for b in range(wl.B):
        row = u[wl.row_starts[b]:wl.row_starts[b] + wl.lengths[b]]
        pos = np.flatnonzero(row != 0)
        zer = np.flatnonzero(row == 0)
        P = pos.size
        assert P < wl.k
        assert set(oi[b, :P].tolist()) == set(pos.tolist())
        assert np.array_equal(oi[b, P:], zer[:wl.k - P])
        assert np.all(ov[b, P:] == 0)


def test_all_neg_inf_and_short_rows_closed_form():
    L = 3000
    row_inf = np.full(L, 0xFF800000, np.uint32)
    rng = np.random.default_rng(3)
    row_short = rng.integers(0, 2**32, 700, dtype=np.uint64).astype(np.uint32)
    flat = np.concatenate([row_inf, row_short])
    oi, ov = oracle.topk_ragged(flat, np.array([0, L], np.int32), np.array([L, 700], np.int32), 2048, L)
    assert np.array_equal(oi[0], np.arange(2048))
    assert np.all(ov[0] == 0xFF800000)
    assert set(oi[1, :700].tolist()) == set(range(700))
    assert np.all(oi[1, 700:] == -1) and np.all(ov[1, 700:] == NEG_INF_BITS)


def test_narrow_range_counting_sort_closed_form():
    """Values 0x3F800000 | r, r < 8192: a counting sort over r that scans positions in
    ascending order gives the whole canonical order without any comparison sort."""
    wl = W.narrow_range(B=3, L=65536, k=4096, name="pin_narrow")
    oi, ov = oracle.topk_ragged(wl.scores, wl.row_starts, wl.lengths, wl.k, wl.max_len)
    u = wl.scores.view(np.uint32)
    for b in range(wl.B):
        r = u[wl.row_starts[b]:wl.row_starts[b] + wl.max_len] & 0x1FFF
        buckets = [[] for _ in range(8192)]
        for j, rv in enumerate(r.tolist()):
            buckets[rv].append(j)
        expect = []
        for rv in range(8191, -1, -1):
            expect.extend(buckets[rv])
            if len(expect) >= wl.k:
                break
        assert oi[b].tolist() == expect[:wl.k]


# ------------------------------------------------------------------ invariants at workload shapes

SMALL_WORKLOADS = {
    "plateau": lambda: W.plateau_abs(B=4, L=4096, k=2048),
    "decode_ragged": lambda: W.decode_ragged(B=12, n_lo=100, n_hi=9000, k=2048, name="small_decode"),
    "prefill_causal": lambda: W.prefill_causal(Q=96, ctx=4096, k=512, name="small_prefill"),
    "narrow": lambda: W.narrow_range(B=4, L=20000, k=4096, name="small_narrow"),
    "long_context": lambda: W.long_context(B=4, L=50000, k=2048, short_n=1500, name="small_long"),
}


@pytest.mark.parametrize("name", sorted(SMALL_WORKLOADS))
def test_invariants_on_shrunken_workloads(name):
    wl = SMALL_WORKLOADS[name]()
    oi, ov = oracle.topk_ragged(wl.scores, wl.row_starts, wl.lengths, wl.k, wl.max_len)
    check_batch(wl.scores, wl.row_starts, wl.lengths, wl.max_len, wl.k, oi, ov)


# ------------------------------------------------------------------ boundary semantics

def test_window_clamps_and_default_metadata():
    rng = np.random.default_rng(9)
    L = 50
    flat = rng.integers(0, 2**32, 4 * L, dtype=np.uint64).astype(np.uint32)
    # lengths are clamped to [0, max_len]; row_starts None means b * max_len
    lens = np.array([-5, 0, 80, 23], np.int32)
    oi, ov = oracle.topk_ragged(flat, None, lens, 30, L, B=4)
    assert np.all(oi[0] == -1) and np.all(oi[1] == -1)
    ri, rv = lexsort_reference(flat[2 * L:3 * L], 30)
    assert np.array_equal(oi[2], ri) and np.array_equal(ov[2], rv)
    ri, rv = lexsort_reference(flat[3 * L:3 * L + 23], 30)
    assert np.array_equal(oi[3], ri) and np.array_equal(ov[3], rv)
    # lengths None means max_len everywhere
    oi2, ov2 = oracle.topk_ragged(flat, None, None, 30, L, B=4)
    for b in range(4):
        ri, rv = lexsort_reference(flat[b * L:(b + 1) * L], 30)
        assert np.array_equal(oi2[b], ri) and np.array_equal(ov2[b], rv)


def test_thread_count_does_not_change_result():
    wl = W.decode_ragged(B=20, n_lo=10, n_hi=5000, k=300, name="thread_inv")
    a = oracle.topk_ragged(wl.scores, wl.row_starts, wl.lengths, wl.k, wl.max_len, threads=1)
    b = oracle.topk_ragged(wl.scores, wl.row_starts, wl.lengths, wl.k, wl.max_len, threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ planted mistakes

MUTATIONS = {
    "negatives_not_complemented": ("return ~bits;", "return bits;"),
    "positive_sign_not_set": ("return bits | 0x80000000u;", "return bits;"),
    "ties_by_descending_index": ("return a->pos < b->pos ? -1 : 1;", "return a->pos > b->pos ? -1 : 1;"),
    "ascending_scores": ("return a->key > b->key ? -1 : 1;", "return a->key < b->key ? -1 : 1;"),
    "index_off_by_one": ("oi[t] = items[t].pos;", "oi[t] = items[t].pos + 1;"),
    "value_from_wrong_slot": ("ov[t] = row[items[t].pos];", "ov[t] = row[t];"),
    "padding_value_zero": ("ov[t] = 0xFF800000u;", "ov[t] = 0u;"),
    "clamp_off_by_one": ("len = job->max_len;", "len = job->max_len - 1;"),
    "default_start_zero": ("(int64_t)b * job->max_len;", "0;"),
}


def _build_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "detk_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert old in src, "mutation anchor missing: %s" % name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new, 1))
    so = tmp_path / ("mut_%s.so" % name)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-pthread", str(path), "-o", str(so)])
    lib = ctypes.CDLL(str(so))
    lib.detk_oracle_topk_ragged.restype = ctypes.c_int
    lib.detk_oracle_topk_ragged.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int32, ctypes.c_int,
                                                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]

    def call(scores, row_starts, lengths, k, max_len, B=None):
        s = np.ascontiguousarray(scores, dtype=np.uint32)
        rs = None if row_starts is None else np.ascontiguousarray(row_starts, np.int32)
        ln = None if lengths is None else np.ascontiguousarray(lengths, np.int32)
        B = B if B is not None else (ln.shape[0] if ln is not None else rs.shape[0])
        oi = np.empty((B, k), np.int32)
        ov = np.empty((B, k), np.uint32)
        rc = lib.detk_oracle_topk_ragged(s.ctypes.data, None if rs is None else rs.ctypes.data,
                                         None if ln is None else ln.ctypes.data, B, max_len, k,
                                         oi.ctypes.data, ov.ctypes.data, 2)
        assert rc == 0
        return oi, ov
    return call


def _pins_pass(call) -> bool:
    try:
        for row, k, idx, val in _examples():
            if row.size == 0:
                continue
            oi, ov = _oracle_one(row, k, call)
            if oi.tolist() != idx or ov.tolist() != val:
                return False
        rng = np.random.default_rng(1)
        row = rng.integers(0, 2**32, 5000, dtype=np.uint64).astype(np.uint32)
        oi, ov = _oracle_one(row, 100, call)
        ri, rv = lexsort_reference(row, 100)
        if not (np.array_equal(oi, ri) and np.array_equal(ov, rv)):
            return False
        flat = rng.integers(0, 2**32, 200, dtype=np.uint64).astype(np.uint32)
        oi, ov = call(flat, None, np.array([80, 30], np.int32), 60, 50)
        for b, n in ((0, 50), (1, 30)):
            ri, rv = lexsort_reference(flat[b * 50:b * 50 + n], 60)
            if not (np.array_equal(oi[b], ri) and np.array_equal(ov[b], rv)):
                return False
        return True
    except AssertionError:
        return False


def test_pins_pass_on_unmutated_oracle(tmp_path):
    MUTATIONS_BACKUP = dict(MUTATIONS)
    MUTATIONS["identity"] = ("return ~bits;", "return ~bits;")
    try:
        assert _pins_pass(_build_mutant(tmp_path, "identity"))
    finally:
        MUTATIONS.clear()
        MUTATIONS.update(MUTATIONS_BACKUP)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    assert not _pins_pass(_build_mutant(tmp_path, name)), "pins missed planted mistake %s" % name
