"""Pins for the oracle's index transform (mode 1: offset + local index; mode 2: page table),
checked against things other than its own formula:

* hand-derived worked examples (tests/golden/index_transform.txt) and one end to end
  (top-k of a small row, then the page table);
* the meaning of a page table, built the other way round: a physical slot array is filled
  by scattering each logical token's tag (row, index) into its slot, page by page; every
  transformed index must point at the slot holding the selected token's tag;
* identity cases (zero offsets; a page table that maps page p to p) and -1 padding;
* planted mistakes: mutated copies of the oracle source must fail these pins.

Source of the operation: SGLang PR #31115, "Modifications" (the fused page-table transforms
that follow selection) and vLLM PR #55872, GB10 failure trace (top_k_ragged_transform).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "index_transform.txt")


def _golden():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fields = dict(tok.split("=", 1) for tok in line.split())
            local = [int(x) for x in fields["local"].split(",")]
            pt = None if fields["pt"] == "-" else [int(x) for x in fields["pt"].split(",")]
            out.append((local, int(fields["mode"]), int(fields["off"]), pt, int(fields["ps"]),
                        [int(x) for x in fields["out"].split(",")]))
    return out


def _run(fn, local, mode, off, pt, ps):
    li = np.array([local], np.int32)
    return fn(li, mode, offsets=np.array([off], np.int32),
              page_table=None if pt is None else np.array([pt], np.int32), page_size=ps)[0].tolist()


def _pins_pass(fn) -> bool:
    for local, mode, off, pt, ps, want in _golden():
        if _run(fn, local, mode, off, pt, ps) != want:
            return False
    if not _scatter_semantics_hold(fn):
        return False
    return True


def _scatter_semantics_hold(fn, seed=3) -> bool:
    """Fill a physical slot array by scattering tags of logical tokens through random page
    tables, then check that every transformed index lands on its token's tag."""
    rng = np.random.default_rng(seed)
    for ps in (1, 2, 3, 16, 64):
        B, n, k = 5, 300, 40
        pages = -(-n // ps)
        phys_pages = rng.permutation(B * pages + 7)[:B * pages].reshape(B, pages).astype(np.int32)
        slots = np.full((B * pages + 7) * ps, -1, np.int64)
        for b in range(B):
            for j in range(n):
                slots[phys_pages[b, j // ps] * ps + j % ps] = b * 100000 + j  # the token's tag
        local = np.full((B, k), -1, np.int32)
        for b in range(B):
            m = int(rng.integers(0, k + 1))
            local[b, :m] = rng.choice(n, m, replace=False)
        out = np.asarray(fn(local, 2, page_table=phys_pages, page_size=ps))
        for b in range(B):
            for t in range(k):
                j = int(local[b, t])
                if j < 0:
                    if out[b, t] != -1:
                        return False
                elif not (0 <= out[b, t] < slots.size) or slots[out[b, t]] != b * 100000 + j:
                    return False
        # offsets: an index into the packed buffer of all rows' tokens
        lens = rng.integers(1, n, B)
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
        packed_tags = np.concatenate([b * 100000 + np.arange(lens[b]) for b in range(B)])
        loc = np.where(local < lens[:, None], local, -1).astype(np.int32)
        out = np.asarray(fn(loc, 1, offsets=starts))
        for b in range(B):
            for t in range(k):
                j = int(loc[b, t])
                if j < 0:
                    if out[b, t] != -1:
                        return False
                elif packed_tags[out[b, t]] != b * 100000 + j:
                    return False
    return True


@pytest.mark.parametrize("case", range(len(_golden())))
def test_worked_example(case):
    local, mode, off, pt, ps, want = _golden()[case]
    assert _run(oracle.index_transform, local, mode, off, pt, ps) == want


def test_page_table_meaning_by_scatter():
    assert _scatter_semantics_hold(oracle.index_transform)


def test_identity_cases():
    rng = np.random.default_rng(9)
    local = rng.integers(-1, 5000, (7, 33)).astype(np.int32)
    assert np.array_equal(oracle.index_transform(local, 0), local)
    assert np.array_equal(oracle.index_transform(local, 1, offsets=np.zeros(7, np.int32)), local)
    for ps in (1, 4, 5, 128):
        ident = np.tile(np.arange(-(-5000 // ps), dtype=np.int32), (7, 1))
        assert np.array_equal(oracle.index_transform(local, 2, page_table=ident, page_size=ps), local)


def test_end_to_end_small_row():
    # scores [0, 3, 1, 3, 2], k = 3: canonical top-3 local indices 1, 3, 4 (3.0 tie by index);
    # pages of 2 tokens at physical pages 10, 20, 30: slots 21, 41, 60
    row = np.array([0.0, 3.0, 1.0, 3.0, 2.0], np.float32)
    li, _ = oracle.topk_ragged(row, np.array([0], np.int32), np.array([5], np.int32), 3, 5)
    assert li[0].tolist() == [1, 3, 4]
    out = oracle.index_transform(li, 2, page_table=np.array([[10, 20, 30]], np.int32), page_size=2)
    assert out[0].tolist() == [21, 41, 60]


# ------------------------------------------------------------------ planted mistakes

MUTATIONS = {
    "within_page_by_division": ("int32_t within = j % page_size;", "int32_t within = j / page_size;"),
    "page_by_modulo": ("int32_t page = j / page_size;", "int32_t page = j % page_size;"),
    "offset_off_by_one": ("v = offsets[b] + j;", "v = offsets[b] + j + 1;"),
    "row_stride_dropped": ("page_table[(int64_t)b * stride + page]", "page_table[page]"),
    "padding_transformed": ("if (j >= 0 && mode == 1)", "if (mode == 1)"),
    "page_not_scaled": ("* page_size + within;", "+ within;"),
}


def _mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "detk_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert old in src, "mutation anchor missing: %s" % name
    path = tmp_path / ("mutx_%s.c" % name)
    path.write_text(src.replace(old, new, 1))
    so = tmp_path / ("mutx_%s.so" % name)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-pthread", str(path), "-o", str(so)])
    lib = ctypes.CDLL(str(so))
    lib.detk_oracle_index_transform.restype = ctypes.c_int
    lib.detk_oracle_index_transform.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_void_p]

    def fn(local_idx, mode, offsets=None, page_table=None, page_size=1):
        li = np.ascontiguousarray(local_idx, np.int32)
        off = None if offsets is None else np.ascontiguousarray(offsets, np.int32)
        pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
        out = np.empty_like(li)
        rc = lib.detk_oracle_index_transform(li.ctypes.data, li.shape[0], li.shape[1], mode,
                                             None if off is None else off.ctypes.data,
                                             None if pt is None else pt.ctypes.data,
                                             0 if pt is None else pt.shape[1], page_size, out.ctypes.data)
        assert rc == 0
        return out
    return fn


def test_pins_pass_on_the_oracle():
    assert _pins_pass(oracle.index_transform)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_transform_mistake_is_caught(tmp_path, name):
    try:
        caught = not _pins_pass(_mutant(tmp_path, name))
    except (AssertionError, IndexError):
        caught = True
    assert caught, "pins missed planted mistake %s" % name
