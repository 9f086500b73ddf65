"""Pins for the oracle's 16-bit path (binary16 and bfloat16 rows), checked against things
other than the oracle itself:

* hand-derived worked examples (tests/golden/worked_examples16.txt);
* brute force by rank counting on tiny rows, through a value-preserving widening to
  float32 (bfloat16: the same bits in the top half; binary16: numpy's exact conversion),
  under which IEEE totalOrder and bitwise equality are unchanged;
* numpy.lexsort on a key built another way (sign-magnitude to a signed integer) on
  random rows of every value class;
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
from topk_checks import brute_force_row

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples16.txt")


def _golden():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fl = dict(tok.split("=", 1) for tok in line.split())
            out.append((fl["fmt"], np.array([int(x, 16) for x in fl["row"].split(",")], np.uint16), int(fl["k"]),
                        [int(x) for x in fl["idx"].split(",")], [int(x, 16) for x in fl["val"].split(",")]))
    return out


def widen(bits16: np.ndarray, fmt: str) -> np.ndarray:
    """Float32 bit patterns with the same values (and NaN classes) as the 16-bit patterns."""
    b = np.asarray(bits16, np.uint16)
    if fmt == "bf16":
        return b.astype(np.uint32) << 16
    return b.view(np.float16).astype(np.float32).view(np.uint32)


def signed16(bits16: np.ndarray) -> np.ndarray:
    u = np.asarray(bits16, np.uint16).astype(np.int64)
    mag = u & 0x7FFF
    return np.where(u >> 15 == 1, -mag - 1, mag)


def _one(call, row, k, fmt):
    n = row.size
    return call(row if n else np.zeros(1, np.uint16), np.array([0], np.int32), np.array([n], np.int32), k,
                max(n, 1), fmt)


def _pins_pass(call) -> bool:
    for fmt, row, k, idx, val in _golden():
        oi, ov = _one(call, row, k, fmt)
        if oi[0].tolist() != idx or ov[0].tolist() != val:
            return False
    rng = np.random.default_rng(4)
    for fmt in ("f16", "bf16"):
        pad = oracle.PAD16[fmt]
        for _ in range(60):
            n = int(rng.integers(1, 10))
            row = rng.integers(0, 2**16, n, dtype=np.uint32).astype(np.uint16)
            k = int(rng.integers(1, n + 3))
            bi, bv = brute_force_row(widen(row, fmt), k)
            oi, ov = _one(call, row, k, fmt)
            if oi[0].tolist() != bi:
                return False
            m = min(k, n)
            if ov[0][:m].tolist() != row[np.array(bi[:m], np.int64)].tolist() or any(v != pad for v in ov[0][m:]):
                return False
        row = rng.integers(0, 2**16, 6000, dtype=np.uint32).astype(np.uint16)
        oi, _ = _one(call, row, 700, fmt)
        order = np.lexsort((np.arange(row.size), -signed16(row)))[:700]
        if not np.array_equal(oi[0], order):
            return False
    return True


def _oracle16(row, rs, ln, k, max_len, fmt):
    return oracle.topk_ragged16(row, rs, ln, k, max_len, fmt=fmt)


@pytest.mark.parametrize("case", range(len(_golden())))
def test_worked_example16(case):
    fmt, row, k, idx, val = _golden()[case]
    bi, bv = brute_force_row(widen(row, fmt), k)
    assert bi == idx, "brute force disagrees with the hand-derived example"
    oi, ov = _one(_oracle16, row, k, fmt)
    assert oi[0].tolist() == idx and ov[0].tolist() == val


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_exhaustive_tiny_rows_against_brute_force(fmt):
    letters = [0x0000, 0x8000, 0x3C00 if fmt == "f16" else 0x3F80, 0x7E00 if fmt == "f16" else 0x7FC0,
               0xFC00 if fmt == "f16" else 0xFF80]
    for n in range(1, 5):
        rows = np.array(list(itertools.product(letters, repeat=n)), np.uint16).reshape(-1, n)
        flat = np.ascontiguousarray(rows).reshape(-1)
        R = rows.shape[0]
        for k in range(1, n + 2):
            oi, ov = oracle.topk_ragged16(flat, (np.arange(R) * n).astype(np.int32), np.full(R, n, np.int32), k, n,
                                          fmt=fmt)
            for r in range(R):
                bi, _ = brute_force_row(widen(rows[r], fmt), k)
                assert oi[r].tolist() == bi, (rows[r], k)


def test_key16_spot_values():
    assert oracle.key16_of_bits(0x0000) == 0x8000 and oracle.key16_of_bits(0x8000) == 0x7FFF
    assert oracle.key16_of_bits(0xFFFF) == 0 and oracle.key16_of_bits(0x7FFF) == 0xFFFF


def test_pins_pass_on_the_oracle():
    assert _pins_pass(_oracle16)


MUTATIONS = {
    "key16_negatives_not_complemented": ("return (uint16_t)~bits;", "return bits;"),
    "key16_sign_not_set": ("return bits | 0x8000u;", "return bits;"),
    "pad16_zero": ("ov[t] = t < m ? row16[items[t].pos] : job->pad16;", "ov[t] = t < m ? row16[items[t].pos] : 0;"),
    "value16_wrong_slot": ("ov[t] = t < m ? row16[items[t].pos] : job->pad16;",
                           "ov[t] = t < m ? row16[t] : job->pad16;"),
}


def _mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "detk_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert old in src, "mutation anchor missing: %s" % name
    path = tmp_path / ("mut16_%s.c" % name)
    path.write_text(src.replace(old, new, 1))
    so = tmp_path / ("mut16_%s.so" % name)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-pthread", str(path), "-o", str(so)])
    lib = ctypes.CDLL(str(so))
    lib.detk_oracle_topk_ragged16.restype = ctypes.c_int
    lib.detk_oracle_topk_ragged16.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int32, ctypes.c_int,
                                                                      ctypes.c_void_p, ctypes.c_void_p,
                                                                      ctypes.c_uint16, ctypes.c_int]

    def call(row, rs, ln, k, max_len, fmt):
        s = np.ascontiguousarray(row, np.uint16)
        B = ln.shape[0]
        oi = np.empty((B, k), np.int32)
        ov = np.empty((B, k), np.uint16)
        assert lib.detk_oracle_topk_ragged16(s.ctypes.data, rs.ctypes.data, ln.ctypes.data, B, max_len, k,
                                             oi.ctypes.data, ov.ctypes.data, oracle.PAD16[fmt], 2) == 0
        return oi, ov
    return call


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_16bit_mistake_is_caught(tmp_path, name):
    assert not _pins_pass(_mutant(tmp_path, name)), "pins missed planted mistake %s" % name
