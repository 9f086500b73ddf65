"""Exact, bitwise-deterministic ragged top-k for AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/detk.h`` (``libdetk.so``, built from
``csrc/`` by :func:`deterministic_exact_top_amd.build.build_library`).  This module
only marshals arguments: every step of the computation runs in the HIP kernels.
PyTorch supplies device memory and the current stream.  There is no CPU fallback:
if the library is missing or fails, calls raise.

Operation: SGLang PR #31115 (PR summary, "Modifications", hardening commit) -- per
row, the k highest scores in canonical order (score descending under the bitwise
total order of the float bits, index ascending among bitwise-equal scores), local
indices front-packed and padded with -1.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "topk_ragged", "topk_ragged_noalloc", "workspace_size", "IndexTransform", "new_workspace", "can_implement", "status_string", "debug_set",
    "library_path", "load_library", "DETK_MAX_K", "DETK_MAX_LEN", "DetkError",
]

DETK_MAX_K = 4096
DETK_MAX_LEN = 1 << 30
DETK_WORKSPACE_UNSUPPORTED = (1 << 64) - 1  # SIZE_MAX: the configuration cannot run
DETK_SCRATCH_BYTES = 16 << 20  # the per-GPU scratch array behind topk_ragged_noalloc
DETK_OK, DETK_ERR_INVALID_ARG, DETK_ERR_UNSUPPORTED, DETK_ERR_WORKSPACE, DETK_ERR_HIP = range(5)
DETK_DEBUG_PATH, DETK_DEBUG_STAGING_CAP, DETK_DEBUG_MULTI_TILE, DETK_DEBUG_FAST, DETK_DEBUG_SMALL_BATCH = 1, 2, 3, 4, 5
DETK_DEBUG_SPLIT_SAMPLES = 6
DETK_INDEX_LOCAL, DETK_INDEX_OFFSET, DETK_INDEX_PAGE_TABLE = 0, 1, 2
DETK_DTYPE_F32, DETK_DTYPE_F16, DETK_DTYPE_BF16 = 0, 1, 2


class IndexTransform(ctypes.Structure):
    """detk_index_transform (include/detk.h): the index each selected local index j becomes."""
    _fields_ = [("mode", ctypes.c_int32), ("page_size", ctypes.c_int32), ("offsets", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("page_table_stride", ctypes.c_int64)]

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class DetkError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s" % (what, status_string(status)))
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libdetk.so")


def load_library():
    """Load libdetk.so (raises if it has not been built).

    torch is imported first: its wheel carries its own HIP runtime under the soname the
    library links against, so whichever is loaded first serves both.  Loaded after the
    library, torch would bring a second runtime, and calls given torch's streams would be
    lost in the library's runtime without an error."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (the HIP runtime the library must share)
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError("libdetk.so is missing at %s; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.detk_can_implement.argtypes = [ctypes.c_int, ctypes.c_int, i32]
    lib.detk_can_implement.restype = ctypes.c_int
    lib.detk_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i32]
    lib.detk_workspace_size.restype = sz
    lib.detk_topk_ragged.argtypes = [vp, vp, vp, ctypes.c_int, i32, ctypes.c_int, vp, vp, vp, sz, vp]
    lib.detk_topk_ragged.restype = ctypes.c_int
    lib.detk_topk_ragged_transform.argtypes = [vp, vp, vp, ctypes.c_int, i32, ctypes.c_int,
                                               ctypes.POINTER(IndexTransform), vp, vp, vp, sz, vp]
    lib.detk_topk_ragged_transform.restype = ctypes.c_int
    lib.detk_topk_ragged_16bit.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, i32, ctypes.c_int,
                                           ctypes.POINTER(IndexTransform), vp, vp, vp, sz, vp]
    lib.detk_topk_ragged_16bit.restype = ctypes.c_int
    lib.detk_topk_ragged_noalloc.argtypes = [vp, vp, vp, ctypes.c_int, i32, ctypes.c_int, vp, vp, vp]
    lib.detk_topk_ragged_noalloc.restype = ctypes.c_int
    lib.detk_status_string.argtypes = [ctypes.c_int]
    lib.detk_status_string.restype = ctypes.c_char_p
    lib.detk_indexer_scores.argtypes = [vp, vp, vp, i32, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32, vp, vp]
    lib.detk_indexer_scores.restype = ctypes.c_int
    lib.detk_debug_set.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.detk_read_probe.argtypes = [vp, sz, vp, vp]
    lib.detk_read_probe.restype = ctypes.c_int
    lib.detk_debug_set.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().detk_status_string(int(status)).decode()


def can_implement(k: int, max_len: int, device: int = 0) -> int:
    return int(load_library().detk_can_implement(int(device), int(k), int(max_len)))


def workspace_size(B: int, k: int, max_len: int, device: int = 0) -> int:
    """Bytes of workspace a call needs (0: none).  Raises DetkError when the configuration
    cannot run (the library answers SIZE_MAX then)."""
    need = int(load_library().detk_workspace_size(int(device), int(B), int(k), int(max_len)))
    if need == DETK_WORKSPACE_UNSUPPORTED:
        raise DetkError(can_implement(k, max_len, device) or DETK_ERR_UNSUPPORTED, "detk_workspace_size")
    return need


def new_workspace(B: int, k: int, max_len: int, device):
    """A zero-filled uint8 CUDA tensor of the size a call with these sizes needs (at least
    one byte).  The library requires a workspace to be zero-filled before its first use
    and leaves it zero-filled after every call, so one allocated here is reused as is,
    by calls of any shape that fits it."""
    import torch
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    return torch.zeros(max(workspace_size(B, k, max_len, idx), 1), dtype=torch.uint8, device=dev)


def debug_set(what: int, value: int) -> None:
    """Test-only overrides (see include/detk.h); they never change results."""
    st = load_library().detk_debug_set(int(what), int(value))
    if st != DETK_OK:
        raise DetkError(st, "detk_debug_set")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def read_probe(data, out, stream=None) -> None:
    """Measurement only: one plain streaming read of `data` (a contiguous CUDA tensor,
    16-byte aligned, size a multiple of 16 bytes), XOR-reduced into `out` (an int32 CUDA
    tensor of one element the caller zeroed).  Asynchronous on `stream`."""
    import torch
    lib = load_library()
    if not data.is_cuda or not data.is_contiguous() or out.dtype != torch.int32 or not out.is_cuda:
        raise ValueError("read_probe needs a contiguous CUDA tensor and an int32 CUDA word")
    s = stream if stream is not None else torch.cuda.current_stream(data.device)
    st = lib.detk_read_probe(_ptr(data), int(data.numel() * data.element_size()), _ptr(out),
                             ctypes.c_void_p(s.cuda_stream))
    if st != DETK_OK:
        raise DetkError(st, "detk_read_probe")


def topk_ragged(scores, row_starts=None, lengths=None, k: int = 2048, max_len: int | None = None,
                out_idx=None, out_val=None, workspace=None, with_values: bool = True, B: int | None = None,
                stream=None, index_offsets=None, page_table=None, page_size: int = 1):
    """Exact canonical top-k of each ragged row.

    scores      float32, float16 or bfloat16 CUDA tensor, contiguous (16-bit scores run
                detk_topk_ragged_16bit; their out_val has the scores' dtype).  2-D (B, L): rows are the matrix rows
                by default (row_starts None -> b * L, max_len defaults to L).  1-D:
                a packed buffer; pass row_starts and max_len.
    row_starts  int32 CUDA tensor (B,) of absolute element offsets, or None.
    lengths     int32 CUDA tensor (B,), or None (every row max_len long).
    k           1 <= k <= 4096.
    max_len     host-known bound on every row length (never read from the device).
    workspace   uint8 CUDA tensor from new_workspace() (zero-filled before its first use;
                every call leaves it zero-filled), or None to allocate one here.
    index_offsets  int32 CUDA tensor (B,): write index_offsets[b] + j for a selected local j
                (detk_topk_ragged_transform, DETK_INDEX_OFFSET).
    page_table  int32 CUDA tensor (B, pages), or (pages,) shared by every row: write the
                physical slot page_table[b, j // page_size] * page_size + j % page_size
                instead (DETK_INDEX_PAGE_TABLE).  At most one of the two.
    Returns (out_idx int32 (B, k), out_val float32 (B, k) or None).  All allocation
    happens here, before the call, so a captured graph can reuse preallocated
    out_idx / out_val / workspace passed in by the caller.
    """
    import torch
    lib = load_library()
    dtypes = {torch.float32: DETK_DTYPE_F32, torch.float16: DETK_DTYPE_F16, torch.bfloat16: DETK_DTYPE_BF16}
    if scores.dtype not in dtypes or not scores.is_cuda or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32, float16 or bfloat16 CUDA tensor")
    dtype = dtypes[scores.dtype]
    if max_len is None:
        if scores.dim() != 2:
            raise ValueError("max_len is required unless scores is 2-D")
        max_len = int(scores.shape[1])
    if B is None:
        if lengths is not None:
            B = int(lengths.shape[0])
        elif row_starts is not None:
            B = int(row_starts.shape[0])
        elif scores.dim() == 2:
            B = int(scores.shape[0])
        else:
            raise ValueError("B cannot be inferred")
    for name, t in (("row_starts", row_starts), ("lengths", lengths)):
        if t is not None:
            if t.dtype != torch.int32 or t.device != scores.device or not t.is_contiguous():
                raise ValueError("%s must be a contiguous int32 tensor on the scores' device" % name)
            if t.shape[0] < B:
                raise ValueError("%s has fewer than B entries" % name)
    dev = scores.device
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if with_values and out_val is None:
        out_val = torch.empty((B, k), dtype=scores.dtype, device=dev)
    need = workspace_size(B, k, max_len, dev.index if dev.index is not None else torch.cuda.current_device())
    if need and (workspace is None or workspace.numel() < need):
        # (zero-filled: the library needs a workspace zeroed before its first use)
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    args = (_ptr(out_idx), _ptr(out_val) if with_values else None, _ptr(workspace) if need else None,
            int(workspace.numel()) if need else 0, ctypes.c_void_p(s.cuda_stream))
    if index_offsets is None and page_table is None and dtype == DETK_DTYPE_F32:
        st = lib.detk_topk_ragged(_ptr(scores), _ptr(row_starts), _ptr(lengths), int(B), int(max_len), int(k), *args)
        what = "detk_topk_ragged"
    elif index_offsets is None and page_table is None:
        st = lib.detk_topk_ragged_16bit(_ptr(scores), dtype, _ptr(row_starts), _ptr(lengths), int(B), int(max_len),
                                        int(k), None, *args)
        what = "detk_topk_ragged_16bit"
    else:
        if index_offsets is not None and page_table is not None:
            raise ValueError("pass index_offsets or page_table, not both")
        xf = IndexTransform()
        for name, t in (("index_offsets", index_offsets), ("page_table", page_table)):
            if t is not None and (t.dtype != torch.int32 or t.device != dev or not t.is_contiguous()):
                raise ValueError("%s must be a contiguous int32 tensor on the scores' device" % name)
        if index_offsets is not None:
            xf.mode, xf.page_size, xf.offsets = DETK_INDEX_OFFSET, 1, index_offsets.data_ptr()
        else:
            xf.mode, xf.page_size, xf.page_table = DETK_INDEX_PAGE_TABLE, int(page_size), page_table.data_ptr()
            xf.page_table_stride = int(page_table.shape[1]) if page_table.dim() == 2 else 0
        if dtype == DETK_DTYPE_F32:
            st = lib.detk_topk_ragged_transform(_ptr(scores), _ptr(row_starts), _ptr(lengths), int(B), int(max_len),
                                                int(k), ctypes.byref(xf), *args)
            what = "detk_topk_ragged_transform"
        else:
            st = lib.detk_topk_ragged_16bit(_ptr(scores), dtype, _ptr(row_starts), _ptr(lengths), int(B),
                                            int(max_len), int(k), ctypes.byref(xf), *args)
            what = "detk_topk_ragged_16bit"
    if st != DETK_OK:
        raise DetkError(st, what)
    return out_idx, (out_val if with_values else None)


def topk_ragged_noalloc(scores, row_starts, lengths, k: int, max_len: int, out_idx, out_val=None, B: int | None = None,
                        stream=None):
    """detk_topk_ragged_noalloc: the same operation with no workspace argument (the library's
    per-GPU scratch array serves rows split over workgroups).  Nothing is allocated here
    either: the caller passes the outputs (out_idx int32 (B, k), out_val float32 (B, k) or
    None).  Calls overlapping on one GPU race."""
    import torch
    lib = load_library()
    if scores.dtype != torch.float32 or not scores.is_cuda or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 CUDA tensor")
    if B is None:
        B = int(out_idx.shape[0])
    s = stream if stream is not None else torch.cuda.current_stream(scores.device)
    st = lib.detk_topk_ragged_noalloc(_ptr(scores), _ptr(row_starts), _ptr(lengths), int(B), int(max_len), int(k),
                                      _ptr(out_idx), _ptr(out_val), ctypes.c_void_p(s.cuda_stream))
    if st != DETK_OK:
        raise DetkError(st, "detk_topk_ragged_noalloc")
    return out_idx, out_val


INDEXER_HEADS = 16
INDEXER_HEAD_DIM = 128


def indexer_scores(q, w, keys, lengths=None, max_len: int | None = None, out=None, stream=None):
    """detk_indexer_scores: out[b, t] = sum_h w[b, h] * max(0, q[b, h] . keys[t]) for t < n_b.

    q: bfloat16 (or its uint16/int16 bit patterns) CUDA tensor [B, 16, 128]; w: float32 [B, 16];
    keys: bfloat16 [n_keys, 128]; lengths: int32 [B] or None (every window max_len keys);
    max_len defaults to n_keys.  Returns out, float32 [B, max_len] (entries past a row's window
    are left as they were: zero when out is allocated here)."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("keys", keys)):
        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bfloat16 (or 16-bit pattern) CUDA tensor" % name)
    if w.dtype != torch.float32 or not w.is_cuda or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 CUDA tensor")
    if q.dim() != 3 or w.dim() != 2 or keys.dim() != 2:
        raise ValueError("q is [B, heads, head_dim], w [B, heads], keys [n_keys, head_dim]")
    B, H, D = (int(x) for x in q.shape)
    n_keys = int(keys.shape[0])
    if max_len is None:
        max_len = n_keys
    if lengths is not None and (lengths.dtype != torch.int32 or not lengths.is_cuda):
        raise ValueError("lengths must be an int32 CUDA tensor")
    if out is None:
        out = torch.zeros((B, max_len), dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lib.detk_indexer_scores(_ptr(q), _ptr(w), _ptr(keys), int(n_keys), _ptr(lengths), B, H, D, int(max_len),
                                 _ptr(out), ctypes.c_void_p(s.cuda_stream))
    if st != DETK_OK:
        raise DetkError(st, "detk_indexer_scores")
    return out
