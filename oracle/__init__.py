"""CPU oracle for exact, bitwise-deterministic ragged top-k -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path
(``deterministic_exact_top_amd``) never imports it, and the two share no code.

The oracle is the plain definition (see ``detk_oracle.c``): for each row, sort the
window's positions by (total-order key descending, position ascending), keep the
first ``min(k, n)``, pad with -1 (indices) and -inf (values).  Sources: SGLang PR
#31115 (PR summary, "Modifications", hardening commit) and the docai.hu blog post,
section "The price of the fix".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "detk_oracle.c")
_LIB = os.path.join(_HERE, "libdetk_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, POSIX threads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.detk_oracle_topk_ragged.restype = ctypes.c_int
        lib.detk_oracle_topk_ragged.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.detk_oracle_key.restype = ctypes.c_uint32
        lib.detk_oracle_key.argtypes = [ctypes.c_uint32]
        lib.detk_oracle_key16.restype = ctypes.c_uint32
        lib.detk_oracle_key16.argtypes = [ctypes.c_uint16]
        lib.detk_oracle_topk_ragged16.restype = ctypes.c_int
        lib.detk_oracle_topk_ragged16.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint16, ctypes.c_int,
        ]
        lib.detk_oracle_index_transform.restype = ctypes.c_int
        lib.detk_oracle_index_transform.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
        ]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _as_u32(scores) -> np.ndarray:
    a = np.ascontiguousarray(scores)
    if a.dtype == np.float32:
        a = a.view(np.uint32)
    if a.dtype != np.uint32:
        raise TypeError("scores must be float32 or uint32 bit patterns, got %s" % a.dtype)
    return a.reshape(-1)


def topk_ragged(scores, row_starts, lengths, k: int, max_len: int | None = None, B: int | None = None,
                threads: int | None = None):
    """Run the oracle.  Returns ``(out_idx int32 (B, k), out_val uint32 bits (B, k))``.

    ``scores``: float32 (or uint32 bit patterns), any shape, read as a flat buffer.
    ``row_starts``: int32 absolute element offsets per row, or None for ``b * max_len``.
    ``lengths``: int32 per row, or None for ``max_len`` everywhere.
    """
    s = _as_u32(scores)
    rs = None if row_starts is None else np.ascontiguousarray(row_starts, dtype=np.int32)
    ln = None if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32)
    if B is None:
        if ln is not None:
            B = int(ln.shape[0])
        elif rs is not None:
            B = int(rs.shape[0])
        else:
            raise ValueError("B is required when neither row_starts nor lengths is given")
    if max_len is None:
        if ln is None:
            raise ValueError("max_len is required when lengths is None")
        max_len = int(ln.max()) if ln.size else 0
    out_idx = np.empty((B, k), dtype=np.int32)
    out_val = np.empty((B, k), dtype=np.uint32)
    lib = _load()
    rc = lib.detk_oracle_topk_ragged(
        s.ctypes.data if s.size else None,
        None if rs is None else rs.ctypes.data,
        None if ln is None else ln.ctypes.data,
        int(B), int(max_len), int(k), out_idx.ctypes.data, out_val.ctypes.data,
        int(threads or default_threads()),
    )
    if rc != 0:
        raise RuntimeError("oracle failed (status %d)" % rc)
    return out_idx, out_val


def key_of_bits(bits: int) -> int:
    """The oracle's total-order key of one float32 bit pattern."""
    return int(_load().detk_oracle_key(ctypes.c_uint32(bits & 0xFFFFFFFF)))


INDEX_LOCAL, INDEX_OFFSET, INDEX_PAGE_TABLE = 0, 1, 2


def index_transform(local_idx, mode: int, offsets=None, page_table=None, page_size: int = 1):
    """Transform a selection's local indices (``(B, k)`` int32, -1 padding), as the oracle
    writes it out (see ``detk_oracle_index_transform``): mode 1 adds ``offsets[b]``; mode 2
    maps through ``page_table`` (``(B, pages)`` int32, pages of ``page_size`` tokens).
    Returns a new ``(B, k)`` int32 array; -1 stays -1."""
    li = np.ascontiguousarray(local_idx, dtype=np.int32)
    B, k = li.shape
    off = None if offsets is None else np.ascontiguousarray(offsets, dtype=np.int32)
    pt = None if page_table is None else np.ascontiguousarray(page_table, dtype=np.int32)
    stride = 0 if pt is None else (int(pt.shape[1]) if pt.ndim == 2 else 0)
    out = np.empty_like(li)
    rc = _load().detk_oracle_index_transform(
        li.ctypes.data, int(B), int(k), int(mode), None if off is None else off.ctypes.data,
        None if pt is None else pt.ctypes.data, int(stride), int(page_size), out.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle index transform: bad arguments")
    return out


PAD16 = {"f16": 0xFC00, "bf16": 0xFF80}  # -inf of each 16-bit format


def topk_ragged16(scores, row_starts, lengths, k: int, max_len: int | None = None, fmt: str = "bf16",
                  B: int | None = None, threads: int | None = None):
    """The oracle on 16-bit floats (``fmt`` "f16" or "bf16"; ``scores`` float16 or uint16 bit
    patterns).  Returns ``(out_idx int32 (B, k), out_val uint16 bits (B, k))``; padded value
    slots hold the format's -inf."""
    a = np.ascontiguousarray(scores).reshape(-1)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("scores must be float16 or uint16 bit patterns, got %s" % a.dtype)
    rs = None if row_starts is None else np.ascontiguousarray(row_starts, dtype=np.int32)
    ln = None if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32)
    if B is None:
        B = int(ln.shape[0]) if ln is not None else int(rs.shape[0])
    if max_len is None:
        max_len = int(ln.max()) if ln is not None and ln.size else 0
    out_idx = np.empty((B, k), dtype=np.int32)
    out_val = np.empty((B, k), dtype=np.uint16)
    rc = _load().detk_oracle_topk_ragged16(
        a.ctypes.data if a.size else None, None if rs is None else rs.ctypes.data,
        None if ln is None else ln.ctypes.data, int(B), int(max_len), int(k), out_idx.ctypes.data,
        out_val.ctypes.data, PAD16[fmt], int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle failed (status %d)" % rc)
    return out_idx, out_val


def key16_of_bits(bits: int) -> int:
    """The oracle's total-order key of one 16-bit float pattern."""
    return int(_load().detk_oracle_key16(ctypes.c_uint16(bits & 0xFFFF)))
