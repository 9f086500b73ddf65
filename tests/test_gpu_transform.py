"""GPU parity of the fused index transform (detk_topk_ragged_transform) against the oracle:
the oracle's top-k, then the oracle's index transform (offset into a packed buffer, or
the row's page table), compared element by element; out_val must be the plain top-k's.
Covers both launch shapes (one workgroup per row, rows split over workgroups), the
exact and pivot-miss fallbacks, the tie tail, pages of a power-of-two size and of other
sizes, and the host-side refusals.  The operation: SGLang PR #31115, "Modifications"
(fused page-table transforms after selection); vLLM PR #55872, GB10 failure trace
(top_k_ragged_transform)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import deterministic_exact_top_amd as detk
import oracle
import workloads as W
from gpu_util import assert_same, debug_overrides, log, run_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    detk.load_library()
    return torch.device("cuda:0")


def _page_table(wl, ps, seed):
    """A page table whose rows own disjoint random physical pages (spare columns past the
    rows' pages hold -5, which no window reaches)."""
    rng = np.random.default_rng(seed)
    pages = -(-wl.max_len // ps)
    stride = pages + 3
    phys = rng.permutation(wl.B * pages + 11)[:wl.B * pages].reshape(wl.B, pages).astype(np.int32)
    pt = np.full((wl.B, stride), -5, np.int32)
    pt[:, :pages] = phys
    return pt


CASES = {
    "decode_offsets": (lambda: W.decode_ragged(B=40, n_lo=1, n_hi=30000, k=2048, name="xf_decode"), "offset", 1),
    "decode_pages64": (lambda: W.decode_ragged(B=40, n_lo=1, n_hi=30000, k=2048, name="xf_decode"), "pages", 64),
    "plateau_pages1": (lambda: W.plateau_abs(B=6, L=4096, k=2048, name="xf_plateau"), "pages", 1),
    "prefill_pages3": (lambda: W.prefill_causal(Q=96, ctx=9000, k=2048, name="xf_prefill"), "pages", 3),
    "long_pages64": (lambda: W.long_context(B=5, L=100000, k=2048, short_n=1500, name="xf_long"), "pages", 64),
    "long_offsets": (lambda: W.long_context(B=5, L=100000, k=2048, short_n=1500, name="xf_long"), "offset", 1),
    "narrow_pages7": (lambda: W.narrow_range(B=6, L=70000, k=4096, name="xf_narrow"), "pages", 7),
}
SHAPES = {"auto": {}, "exact": {"fast": 0}, "pivot_miss": {"fast": 2}, "split4096": {"path": 2, "multi_tile": 4096},
          "many_rows": {"small": 1}}


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("case", sorted(CASES))
def test_transform_matches_oracle(dev, case, shape):
    import torch
    make, kind, ps = CASES[case]
    wl = make()
    scores, rs, ln = to_dev(wl, dev)
    oi, ov = run_oracle(wl)
    if kind == "offset":
        offs = (wl.row_starts.astype(np.int64) + 1000).astype(np.int32)  # absolute index into the packed buffer
        want = oracle.index_transform(oi, oracle.INDEX_OFFSET, offsets=offs)
        kw = {"index_offsets": torch.from_numpy(offs).to(dev)}
    else:
        pt = _page_table(wl, ps, seed=len(case))
        want = oracle.index_transform(oi, oracle.INDEX_PAGE_TABLE, page_table=pt, page_size=ps)
        kw = {"page_table": torch.from_numpy(pt).to(dev), "page_size": ps}
    log("transform %s shape %s B=%d max_len=%d k=%d" % (case, shape, wl.B, wl.max_len, wl.k))
    with debug_overrides(**SHAPES[shape]):
        gi, gv = detk.topk_ragged(scores, rs, ln, wl.k, max_len=wl.max_len, **kw)
        torch.cuda.synchronize()
    assert_same(gi.cpu().numpy(), gv.cpu().numpy().view(np.uint32), want, ov, "%s/%s" % (case, shape))


def test_shared_page_table(dev):
    """Every query row of a prefill chunk reads one sequence's pages: a 1-D table (stride 0)."""
    import torch
    wl = W.prefill_causal(Q=64, ctx=20000, k=2048, name="xf_shared")
    ps = 64
    rng = np.random.default_rng(12)
    pt = rng.permutation(-(-wl.max_len // ps) + 40)[:-(-wl.max_len // ps)].astype(np.int32)
    scores, rs, ln = to_dev(wl, dev)
    oi, ov = run_oracle(wl)
    want = oracle.index_transform(oi, oracle.INDEX_PAGE_TABLE, page_table=pt, page_size=ps)
    for shape in ("auto", "split4096"):
        with debug_overrides(**SHAPES[shape]):
            gi, gv = detk.topk_ragged(scores, rs, ln, wl.k, max_len=wl.max_len, page_table=torch.from_numpy(pt).to(dev),
                                      page_size=ps)
            torch.cuda.synchronize()
        assert_same(gi.cpu().numpy(), gv.cpu().numpy().view(np.uint32), want, ov, "shared table/%s" % shape)


def test_transform_refusals(dev):
    import torch
    lib = detk.load_library()
    x = torch.zeros(4, 100, device=dev)
    out = torch.empty(4, 10, dtype=torch.int32, device=dev)
    pt = torch.zeros(4, 30, dtype=torch.int32, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())

    def call(**f):
        xf = detk.IndexTransform()
        for key, v in f.items():
            setattr(xf, key, v)
        return lib.detk_topk_ragged_transform(p(x), None, None, 4, 100, 10, ctypes.byref(xf), p(out), None, None, 0, s)
    assert call(mode=3) == detk.DETK_ERR_INVALID_ARG
    assert call(mode=-1) == detk.DETK_ERR_INVALID_ARG
    assert call(mode=1, offsets=None) == detk.DETK_ERR_INVALID_ARG
    assert call(mode=2, page_size=4, page_table=None, page_table_stride=30) == detk.DETK_ERR_INVALID_ARG
    assert call(mode=2, page_size=0, page_table=pt.data_ptr(), page_table_stride=30) == detk.DETK_ERR_INVALID_ARG
    assert call(mode=2, page_size=4, page_table=pt.data_ptr(), page_table_stride=24) == detk.DETK_ERR_INVALID_ARG
    assert call(mode=2, page_size=4, page_table=pt.data_ptr(), page_table_stride=-1) == detk.DETK_ERR_INVALID_ARG
    assert call(mode=2, page_size=4, page_table=pt.data_ptr(), page_table_stride=25) == detk.DETK_OK
    assert call(mode=2, page_size=4, page_table=pt.data_ptr(), page_table_stride=0) == detk.DETK_OK
    assert lib.detk_topk_ragged_transform(p(x), None, None, 4, 100, 10, None, p(out), None, None, 0, s) == detk.DETK_OK
    torch.cuda.synchronize()
