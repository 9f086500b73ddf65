"""Test-side checks for exact ragged top-k that do not go through the oracle.

* ``ieee_total_order_lt`` -- IEEE 754-2019 section 5.10 totalOrder, written from the
  standard's case list (numeric order, -0 below +0, NaNs placed by sign, then quiet
  above signaling, then payload) with Python float comparisons for the numeric part.
  It never uses the "complement negatives / set the sign of positives" key trick.
* ``brute_force_row`` -- the canonical order by counting: an element's output slot is
  the number of elements strictly above it in totalOrder plus the number of
  bitwise-equal elements at smaller positions (O(n^2), no sort routine).
* ``signed_key`` -- a second construction of the total order (sign-magnitude to a
  two's-complement int64), used by the invariant checker.
* ``check_invariants`` -- what must hold for any correct output, at any size.

Sources: SGLang PR #31115 (canonical order and smallest-index tie subset, PR summary
and "Modifications"; bitwise total order rather than NaN-maximal, hardening commit)
and the docai.hu blog post ("The price of the fix": full sort, truncate, -1 pad).
"""
from __future__ import annotations

import struct

import numpy as np

NEG_INF_BITS = 0xFF800000


def _is_nan(bits: int) -> bool:
    return (bits & 0x7F800000) == 0x7F800000 and (bits & 0x007FFFFF) != 0


def _as_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def ieee_total_order_lt(a: int, b: int) -> bool:
    """True iff bit pattern ``a`` is strictly below ``b`` in IEEE totalOrder."""
    if a == b:
        return False
    sa, sb = a >> 31, b >> 31
    na, nb = _is_nan(a), _is_nan(b)
    if na or nb:
        if na and nb:
            if sa != sb:
                return sa == 1                      # -NaN below +NaN
            ta = ((a >> 22) & 1, a & 0x3FFFFF)      # (quiet bit, payload)
            tb = ((b >> 22) & 1, b & 0x3FFFFF)
            return ta < tb if sa == 0 else ta > tb  # reversed for negative NaNs
        if na:
            return sa == 1                          # -NaN below all, +NaN above all
        return sb == 0
    fa, fb = _as_float(a), _as_float(b)
    if fa != fb:
        return fa < fb
    return sa == 1                                  # equal numbers, different bits: -0 < +0


def brute_force_row(bits_row, k: int):
    """Canonical top-k of one row by rank counting.  Returns (idx list, val-bits list)."""
    bits = [int(x) for x in bits_row]
    n = len(bits)
    m = min(k, n)
    idx = [-1] * k
    val = [NEG_INF_BITS] * k
    for j in range(n):
        above = sum(1 for i in range(n) if ieee_total_order_lt(bits[j], bits[i]))
        earlier_equal = sum(1 for i in range(j) if bits[i] == bits[j])
        r = above + earlier_equal
        if r < m:
            assert idx[r] == -1, "two elements claimed one slot"
            idx[r] = j
            val[r] = bits[j]
    assert all(x >= 0 for x in idx[:m])
    return idx, val


def signed_key(bits: np.ndarray) -> np.ndarray:
    """Total order as int64: +x -> magnitude bits, -x -> -(magnitude bits) - 1."""
    u = np.asarray(bits, dtype=np.uint32).astype(np.int64)
    mag = u & 0x7FFFFFFF
    return np.where(u >> 31 == 1, -mag - 1, mag)


def window(scores_u32: np.ndarray, row_starts, lengths, max_len: int, b: int) -> np.ndarray:
    n = max_len if lengths is None else int(np.clip(lengths[b], 0, max_len))
    s = b * max_len if row_starts is None else int(row_starts[b])
    return scores_u32[s:s + n]


def lexsort_reference(row_bits: np.ndarray, k: int):
    """numpy.lexsort on (signed_key descending, position ascending), truncated."""
    n = row_bits.shape[0]
    m = min(k, n)
    order = np.lexsort((np.arange(n), -signed_key(row_bits)))[:m]
    idx = np.full(k, -1, dtype=np.int32)
    val = np.full(k, NEG_INF_BITS, dtype=np.uint32)
    idx[:m] = order
    val[:m] = row_bits[order]
    return idx, val


def check_row(row_bits: np.ndarray, k: int, idx: np.ndarray, val: np.ndarray, where: str = "") -> None:
    """Invariants of one output row (raises AssertionError with context)."""
    row_bits = np.asarray(row_bits, dtype=np.uint32)
    idx = np.asarray(idx)
    val = np.asarray(val).view(np.uint32) if np.asarray(val).dtype == np.float32 else np.asarray(val, np.uint32)
    n = row_bits.shape[0]
    m = min(k, n)
    assert idx.shape == (k,), where
    sel = idx[:m]
    assert np.all(idx[m:] == -1), "%s: slots after min(k, n) must be -1" % where
    assert np.all(val[m:] == NEG_INF_BITS), "%s: padded values must be -inf" % where
    assert np.all((sel >= 0) & (sel < n)), "%s: index outside the row window" % where
    assert np.unique(sel).size == m, "%s: duplicate index" % where
    assert np.array_equal(val[:m], row_bits[sel]), "%s: values are not the input bits" % where
    if m == 0:
        return
    key = signed_key(row_bits)
    ks = key[sel]
    assert np.all(ks[:-1] >= ks[1:]), "%s: keys not non-increasing" % where
    same = ks[:-1] == ks[1:]
    assert np.all(sel[:-1][same] < sel[1:][same]), "%s: equal keys not in index order" % where
    top = np.sort(key)[::-1][:m]
    assert np.array_equal(np.sort(ks)[::-1], top), "%s: selected key multiset != top-m" % where
    T = ks[-1]
    ties = np.flatnonzero(key == T)
    need = int(np.sum(ks == T))
    assert np.array_equal(np.sort(sel[ks == T]), ties[:need]), "%s: boundary ties not the smallest indices" % where


def check_batch(scores, row_starts, lengths, max_len, k, out_idx, out_val, rows=None) -> None:
    s = np.ascontiguousarray(scores).reshape(-1)
    s = s.view(np.uint32) if s.dtype == np.float32 else s
    B = out_idx.shape[0]
    for b in (range(B) if rows is None else rows):
        check_row(window(s, row_starts, lengths, max_len, b), k, out_idx[b], out_val[b], "row %d" % b)
