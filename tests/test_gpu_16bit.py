"""GPU parity on 16-bit float scores (detk_topk_ragged_16bit: binary16 and bfloat16)
against the oracle's 16-bit path, index and value bits element by element.  The 16-bit
workloads are the float32 ones rounded to each format (many more bitwise ties: bfloat16
keeps 8 significant bits), plus special values and unaligned packed rows (8-byte loads when
a tile is 8-byte aligned, 2-byte loads otherwise).  Both launch shapes, the exact and
pivot-miss fallbacks, the full prefill workload (every row) and the long-context workload
at full size, and a fused page table.  Source: SGLang PR #31115, "Speed Tests and
Profiling" (a 16-bit coarse first pass among the follow-up levers)."""
from __future__ import annotations

import numpy as np
import pytest

import deterministic_exact_top_amd as detk
import oracle
import workloads as W
from gpu_util import assert_same, debug_overrides, log

pytestmark = pytest.mark.gpu

TORCH_DTYPE = {"f16": "float16", "bf16": "bfloat16"}


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    detk.load_library()
    return torch.device("cuda:0")


def _run(dev, w16, **kw):
    import torch
    dt = getattr(torch, TORCH_DTYPE[w16.fmt])
    s = torch.from_numpy(w16.scores.view(np.int16)).to(dev).view(dt)
    rs = torch.from_numpy(w16.row_starts).to(dev)
    ln = torch.from_numpy(w16.lengths).to(dev)
    gi, gv = detk.topk_ragged(s, rs, ln, w16.k, max_len=w16.max_len, **kw)
    torch.cuda.synchronize()
    return gi.cpu().numpy(), gv.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle(w16):
    return oracle.topk_ragged16(w16.scores, w16.row_starts, w16.lengths, w16.k, w16.max_len, fmt=w16.fmt)


def _specials(B=6, L=12000, k=2048, name="sp16"):
    rng = np.random.default_rng(31)
    buf = np.empty(B * L, np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 65504.0, 1e-8], np.float32)
    for b in range(B):
        r = W.relu_sum_mixture(rng, L, 0.6)
        pos = rng.choice(L, 40 * (b + 1), replace=False)
        r[pos] = special[rng.integers(0, special.size, pos.size)]
        buf[b * L:(b + 1) * L] = r
    return W.Workload(name, buf, (np.arange(B) * L).astype(np.int32), np.full(B, L, np.int32), L, k)


def _unaligned(name="un16"):
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 9000, 30).astype(np.int32)
    starts = np.cumsum(np.concatenate([[1], lens[:-1] + rng.integers(0, 3, 29)])).astype(np.int32)
    buf = np.zeros(int(starts[-1] + lens[-1] + 5), np.float32)
    for b in range(lens.size):
        buf[starts[b]:starts[b] + lens[b]] = W.relu_sum_mixture(rng, int(lens[b]), 0.5)
    return W.Workload(name, buf, starts, lens, 9000, 1000)


SMALL = {
    "plateau": lambda: W.plateau_abs(B=6, L=4096, k=2048, name="p16"),
    "decode": lambda: W.decode_ragged(B=24, n_lo=1, n_hi=30000, k=2048, name="d16"),
    "prefill": lambda: W.prefill_causal(Q=96, ctx=9000, k=2048, name="q16"),
    "long": lambda: W.long_context(B=4, L=100000, k=2048, short_n=1500, name="l16"),
    "narrow": lambda: W.narrow_range(B=6, L=70000, k=4096, name="n16"),
    "specials": _specials,
    "unaligned": _unaligned,
}
SHAPES = {"auto": {}, "exact": {"fast": 0}, "pivot_miss": {"fast": 2}, "split4096": {"path": 2, "multi_tile": 4096},
          "many_rows": {"small": 1}}


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_16bit_matches_oracle(dev, name, fmt, shape):
    w16 = W.to16(SMALL[name](), fmt)
    log("16-bit %s %s shape %s B=%d max_len=%d k=%d" % (name, fmt, shape, w16.B, w16.max_len, w16.k))
    with debug_overrides(**SHAPES[shape]):
        gi, gv = _run(dev, w16)
    oi, ov = _oracle(w16)
    assert_same(gi, gv, oi, ov, "%s/%s/%s" % (name, fmt, shape))


@pytest.mark.parametrize("name", ["prefill_causal_8192x16384", "long_context_8x262144"])
def test_16bit_full_workloads(dev, name):
    w16 = W.to16(W.full(name), "bf16")
    log("16-bit full %s (bf16)" % name)
    gi, gv = _run(dev, w16)
    oi, ov = _oracle(w16)
    assert_same(gi, gv, oi, ov, name + "/bf16")


def test_16bit_with_page_table(dev):
    import torch
    w16 = W.to16(W.long_context(B=4, L=100000, k=2048, short_n=1500, name="l16pt"), "f16")
    ps = 16
    pages = -(-w16.max_len // ps)
    pt = np.random.default_rng(2).permutation(w16.B * pages).reshape(w16.B, pages).astype(np.int32)
    gi, gv = _run(dev, w16, page_table=torch.from_numpy(pt).to(dev), page_size=ps)
    oi, ov = _oracle(w16)
    want = oracle.index_transform(oi, oracle.INDEX_PAGE_TABLE, page_table=pt, page_size=ps)
    assert_same(gi, gv, want, ov, "f16 page table")
