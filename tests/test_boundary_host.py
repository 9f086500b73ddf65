"""Host-side checks of the C-ABI library that need no GPU: it loads, exports every
symbol include/detk.h declares, and rejects bad arguments before touching HIP."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import deterministic_exact_top_amd as detk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "detk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(detk_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(detk.library_path()):
        from deterministic_exact_top_amd.build import build_library
        build_library(force=True)
    return detk.load_library()


def test_header_declares_entry_points():
    names = _declared()
    for n in ("detk_topk_ragged", "detk_workspace_size", "detk_can_implement", "detk_status_string",
              "detk_debug_set", "detk_read_probe"):
        assert n in names


def test_read_probe_argument_errors(lib):
    # argument errors are found on the host, before any device call
    vp = ctypes.c_void_p
    assert lib.detk_read_probe(None, 0, None, None) == detk.DETK_OK          # nothing to read
    assert lib.detk_read_probe(None, 16, vp(256), None) == detk.DETK_ERR_INVALID_ARG
    assert lib.detk_read_probe(vp(256), 16, None, None) == detk.DETK_ERR_INVALID_ARG
    assert lib.detk_read_probe(vp(256), 20, vp(512), None) == detk.DETK_ERR_INVALID_ARG  # not a multiple of 16
    assert lib.detk_read_probe(vp(260), 16, vp(512), None) == detk.DETK_ERR_INVALID_ARG  # misaligned


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(detk.library_path())
    for name in _declared():
        assert hasattr(raw, name), "libdetk.so does not export %s" % name


def test_argument_errors_before_any_launch(lib):
    vp = ctypes.c_void_p
    dummy = vp(0x1000)  # never dereferenced: every case below fails (or returns) first
    call = lambda scores, B, max_len, k, out: lib.detk_topk_ragged(scores, None, None, B, max_len, k, out, None,
                                                                   None, 0, None)
    assert call(dummy, -1, 10, 5, dummy) == detk.DETK_ERR_INVALID_ARG
    assert call(dummy, 3, -1, 5, dummy) == detk.DETK_ERR_INVALID_ARG
    assert call(dummy, 3, 10, 0, dummy) == detk.DETK_ERR_INVALID_ARG
    assert call(None, 3, 10, 5, dummy) == detk.DETK_ERR_INVALID_ARG
    assert call(dummy, 3, 10, 5, None) == detk.DETK_ERR_INVALID_ARG
    assert call(dummy, 3, 10, 4097, dummy) == detk.DETK_ERR_UNSUPPORTED
    assert call(None, 0, 10, 5, None) == detk.DETK_OK  # empty batch: nothing to do


def test_status_strings_and_debug_overrides(lib):
    for st in range(5):
        assert detk.status_string(st).startswith("DETK_")
    assert "unknown" in detk.status_string(99)
    assert lib.detk_debug_set(1, 3) == detk.DETK_ERR_INVALID_ARG
    assert lib.detk_debug_set(2, -2) == detk.DETK_ERR_INVALID_ARG
    assert lib.detk_debug_set(3, 5000) == detk.DETK_ERR_INVALID_ARG
    assert lib.detk_debug_set(42, 0) == detk.DETK_ERR_INVALID_ARG
    for what, val in ((1, 2), (1, 0), (2, 0), (2, -1), (3, 4096), (3, 0)):
        assert lib.detk_debug_set(what, val) == detk.DETK_OK


def test_workspace_size_refusal_is_size_max(lib):
    # refused configurations answer SIZE_MAX, never 0 ("needs no workspace")
    size_max = (1 << 64) - 1
    assert lib.detk_workspace_size(0, 4, 0, 100) == size_max
    assert lib.detk_workspace_size(0, -1, 16, 100) == size_max
    assert lib.detk_workspace_size(0, 4, 16, -5) == size_max
    assert lib.detk_workspace_size(0, 4, 4097, 100) == size_max
    assert lib.detk_workspace_size(-1, 4, 16, 100) == size_max


def test_indexer_scores_argument_errors(lib):
    """The indexer producer's shape and window checks come before any device call."""
    vp = ctypes.c_void_p
    fake = vp(256)  # never dereferenced: every call below is refused (or empty) on the host
    f = lib.detk_indexer_scores
    assert f(fake, fake, fake, 100, None, 4, 8, 128, 100, fake, None) == detk.DETK_ERR_UNSUPPORTED   # 8 heads
    assert f(fake, fake, fake, 100, None, 4, 16, 64, 100, fake, None) == detk.DETK_ERR_UNSUPPORTED   # head dim 64
    assert f(fake, fake, fake, 100, None, 4, 16, 128, 101, fake, None) == detk.DETK_ERR_INVALID_ARG  # past the keys
    assert f(fake, fake, fake, 100, None, -1, 16, 128, 100, fake, None) == detk.DETK_ERR_INVALID_ARG
    assert f(None, None, None, 100, None, 0, 16, 128, 100, None, None) == detk.DETK_OK              # empty batch
    assert f(None, None, None, 100, None, 4, 16, 128, 0, None, None) == detk.DETK_OK                # empty windows
    assert f(None, fake, fake, 100, None, 4, 16, 128, 100, fake, None) == detk.DETK_ERR_INVALID_ARG  # q NULL
    assert f(vp(258), fake, fake, 100, None, 4, 16, 128, 100, fake, None) == detk.DETK_ERR_INVALID_ARG  # misaligned
    big = (2 ** 31) // 256  # 8,388,608 key rows: 2^31 bytes, one past the envelope
    assert f(fake, fake, fake, big, None, 4, 16, 128, 100, fake, None) == detk.DETK_ERR_UNSUPPORTED
