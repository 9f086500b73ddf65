"""GPU parity of the lightning-indexer score producer (detk_indexer_scores) and of the
selection chained on its output.

Scores: float32 sums on the matrix cores in an order of their own, so each score is
compared with the oracle's float64 definition within the oracle's float32 forward error
bound, element by element.  The selection on top is integer work decided on the GPU's
float32 scores, so it is compared bit for bit with the oracle's selection over those same
scores.  Determinism: identical bits on repeated calls.
"""
from __future__ import annotations

import numpy as np
import pytest

import deterministic_exact_top_amd as detk
import oracle
from oracle import indexer as OI
import workloads as W
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    detk.load_library()
    return torch.device("cuda:0")


def _dev(inp, dev, lengths=True):
    import torch
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    k = torch.from_numpy(inp.keys.view(np.int16)).to(dev)
    ln = torch.from_numpy(inp.lengths).to(dev) if lengths else None
    return q, w, k, ln


def _sub(inp, rows):
    """The same inputs restricted to some query rows (for the oracle)."""
    rows = np.asarray(rows)
    return W.IndexerInputs(inp.name, inp.q[rows], inp.w[rows], inp.keys, inp.key_starts[rows],
                           inp.lengths[rows], inp.max_len, inp.k)


def _check_scores(inp, got, rows, what):
    sub = _sub(inp, rows)
    exact = OI.scores(sub.q, sub.w, sub.keys, sub.lengths, sub.max_len)
    bound = OI.error_bound(sub.q, sub.w, sub.keys, sub.lengths, sub.max_len)
    for i, b in enumerate(rows):
        n = int(min(max(int(inp.lengths[b]), 0), inp.max_len))
        g = got[b, :n].astype(np.float64)
        bad = np.flatnonzero(~(np.abs(g - exact[i, :n]) <= bound[i, :n]))
        assert bad.size == 0, "%s: row %d, %d of %d scores outside the bound; first t=%d gpu %r exact %r bound %r" % (
            what, b, bad.size, n, bad[0], g[bad[0]], exact[i, bad[0]], bound[i, bad[0]])


def _with_lengths(inp, lengths, name):
    return W.IndexerInputs(name, inp.q[:len(lengths)], inp.w[:len(lengths)], inp.keys,
                           np.zeros(len(lengths), np.int32), np.asarray(lengths, np.int32), inp.max_len, inp.k)


CASES = {
    # 40 rows (not a multiple of 16) over 3000 keys (at this batch size the launch takes
    # 1024-key chunks: three per row, a ragged last block)
    "causal_40x3000": lambda: W.indexer_causal(Q=40, ctx=3000, name="ix_a"),
    "causal_5x70": lambda: W.indexer_causal(Q=5, ctx=70, name="ix_b"),
    # one 16-row group over 20,000 keys: the launch takes 1024-key chunks, 20 per row
    "causal_8x20000": lambda: W.indexer_causal(Q=8, ctx=20000, name="ix_g"),
    # windows at and around block (64) and chunk (1024 here; 2048 and 4096 for larger batches)
    # edges, empty and clamped rows
    "edges": lambda: _with_lengths(W.indexer_causal(Q=20, ctx=4200, name="ix_c"),
                                   [0, -5, 1, 63, 64, 65, 2047, 2048, 2049, 4095, 4096, 4097, 4199, 4200, 9999,
                                    128, 130, 2, 3000, 4100], "ix_edges"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_scores_within_bound(dev, case):
    import torch
    inp = CASES[case]()
    log("indexer scores %s: B=%d H=%d D=%d max_len=%d" % (case, inp.B, inp.H, inp.D, inp.max_len))
    q, w, k, ln = _dev(inp, dev)
    out = torch.full((inp.B, inp.max_len), float("nan"), device=dev)
    detk.indexer_scores(q, w, k, ln, inp.max_len, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    _check_scores(inp, got, list(range(inp.B)), case)
    # entries past each window are left untouched
    for b in range(inp.B):
        n = int(min(max(int(inp.lengths[b]), 0), inp.max_len))
        assert np.all(np.isnan(got[b, n:])), (case, b)


# Batches whose launch takes the middle key-chunk sizes (the chunk halves from 16384 while
# fewer than 512 workgroups would fill the GPU's 256 CUs twice; a workgroup serves 16 query
# rows): 65, 129 and 257 row groups over 16,384 keys take 2048-, 4096- and 8192-key chunks,
# each with a partial last group.
CHUNK_CASES = {"chunk2048_1030": 1030, "chunk4096_2050": 2050, "chunk8192_4100": 4100}


@pytest.mark.parametrize("case", sorted(CHUNK_CASES))
def test_middle_chunk_sizes(dev, case):
    import torch
    B = CHUNK_CASES[case]
    inp = W.indexer_causal(Q=B, ctx=16384, name="ix_" + case)
    rows = sorted(set([0, 1, 15, 16, B // 2, (B // 16) * 16 - 1, (B // 16) * 16, B - 2, B - 1]
                      + list(np.linspace(0, B - 1, 6).astype(int))))
    log("indexer scores %s: B=%d max_len=%d, %d sampled rows" % (case, B, inp.max_len, len(rows)))
    q, w, k, ln = _dev(inp, dev)
    out = torch.full((inp.B, inp.max_len), float("nan"), device=dev)
    detk.indexer_scores(q, w, k, ln, inp.max_len, out=out)
    torch.cuda.synchronize()
    got = out[torch.tensor(rows, device=dev)].cpu().numpy()
    full = np.full((inp.B, inp.max_len), np.nan, np.float32)
    full[rows] = got
    _check_scores(inp, full, rows, case)
    for b in rows:
        n = int(min(max(int(inp.lengths[b]), 0), inp.max_len))
        assert np.all(np.isnan(full[b, n:])), (case, b)


def test_default_windows_and_repeat_bits(dev):
    import torch
    inp = W.indexer_causal(Q=33, ctx=2500, name="ix_d")
    q, w, k, _ = _dev(inp, dev, lengths=False)
    a = detk.indexer_scores(q, w, k).cpu().numpy()
    b = detk.indexer_scores(q, w, k).cpu().numpy()
    assert a.view(np.uint32).tobytes() == b.view(np.uint32).tobytes()
    full = _with_lengths(inp, [inp.max_len] * inp.B, "ix_d_full")
    _check_scores(full, a, list(range(inp.B)), "lengths NULL")


def _chain_check(inp, dev, k, rows_checked):
    """Scores on the GPU, selection on the GPU; the selection must equal the oracle's
    selection over the GPU's own scores, bit for bit, on every row."""
    import torch
    q, w, kk, ln = _dev(inp, dev)
    scores = detk.indexer_scores(q, w, kk, ln, inp.max_len)
    gi, gv = detk.topk_ragged(scores.view(-1), None, ln, k, max_len=inp.max_len)
    torch.cuda.synchronize()
    host = scores.cpu().numpy()
    oi, ov = oracle.topk_ragged(host.reshape(-1), None, inp.lengths, k, inp.max_len, B=inp.B)
    assert np.array_equal(gi.cpu().numpy(), oi)
    assert np.array_equal(gv.cpu().numpy().view(np.uint32), ov.view(np.uint32))
    _check_scores(inp, host, rows_checked, "chained")
    return host


def test_chain_topk_small(dev):
    inp = W.indexer_causal(Q=64, ctx=6000, k=2048, name="ix_e")
    host = _chain_check(inp, dev, 2048, [0, 17, 63])
    frac0 = float(np.mean(host[0, :inp.lengths[0]] == 0.0))
    assert frac0 > 0.3, frac0  # the structural 0.0 plateau is there for the selection to resolve


def test_full_prefill_indexer(dev):
    """The full chunked-prefill shape (8192 query rows over 16,384 keys, 16 heads of 128):
    scores on 24 sampled rows against the oracle within the bound, the selection of every row
    against the oracle's over the GPU's scores, bit for bit; two calls give the same bits."""
    import torch
    inp = W.indexer_causal(Q=8192, ctx=16384, name="indexer_causal")
    rows = sorted(set([0, 1, 15, 16, 8191, 8190, 4095, 4096] + list(np.linspace(0, 8191, 16).astype(int))))
    log("full prefill indexer: B=%d max_len=%d, %d sampled rows" % (inp.B, inp.max_len, len(rows)))
    host = _chain_check(inp, dev, 2048, rows)
    q, w, kk, ln = _dev(inp, dev)
    again = detk.indexer_scores(q, w, kk, ln, inp.max_len)
    torch.cuda.synchronize()
    a2 = again.cpu().numpy()
    for b in (0, 4096, 8191):
        n = int(inp.lengths[b])
        assert a2[b, :n].view(np.uint32).tobytes() == host[b, :n].view(np.uint32).tobytes()


def test_refusals(dev):
    import torch
    inp = W.indexer_causal(Q=4, ctx=100, name="ix_f")
    q, w, k, ln = _dev(inp, dev)
    with pytest.raises(detk.DetkError) as e:
        detk.indexer_scores(q, w, k, ln, max_len=101)  # windows past the keys
    assert e.value.status == detk.DETK_ERR_INVALID_ARG
    q8 = torch.zeros((4, 8, 128), dtype=torch.int16, device=dev)
    w8 = torch.zeros((4, 8), dtype=torch.float32, device=dev)
    with pytest.raises(detk.DetkError) as e:
        detk.indexer_scores(q8, w8, k, ln)
    assert e.value.status == detk.DETK_ERR_UNSUPPORTED
    qm = torch.zeros(4 * 16 * 128 + 1, dtype=torch.int16, device=dev)[1:].view(4, 16, 128)  # 2 bytes off
    with pytest.raises(detk.DetkError) as e:
        detk.indexer_scores(qm, w, k, ln)
    assert e.value.status == detk.DETK_ERR_INVALID_ARG


def test_graph_replay_of_producer_and_selection(dev):
    """Both calls captured in one HIP graph (torch.cuda.graph), replayed on new inputs copied
    into the captured buffers; every replay must equal an eager run on the same inputs."""
    import torch
    mk = lambda i: W.indexer_causal(Q=48, ctx=2600, k=512, name="ix_graph_%d" % i)
    inps = [mk(i) for i in range(3)]
    q, w, kk, ln = _dev(inps[0], dev)
    scores = torch.zeros((inps[0].B, inps[0].max_len), dtype=torch.float32, device=dev)
    oi = torch.empty((inps[0].B, 512), dtype=torch.int32, device=dev)
    ov = torch.empty((inps[0].B, 512), dtype=torch.float32, device=dev)
    ws = detk.new_workspace(inps[0].B, 512, inps[0].max_len, dev)
    def pair():
        detk.indexer_scores(q, w, kk, ln, inps[0].max_len, out=scores)
        detk.topk_ragged(scores.view(-1), None, ln, 512, max_len=inps[0].max_len, out_idx=oi, out_val=ov,
                         workspace=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pair()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pair()
    torch.cuda.synchronize()
    for inp in inps:
        q2, w2, k2, _ = _dev(inp, dev)
        q.copy_(q2); w.copy_(w2); kk.copy_(k2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (scores.cpu().numpy().copy(), oi.cpu().numpy().copy(), ov.cpu().numpy().copy())
        pair()  # eager, same buffers
        torch.cuda.synchronize()
        assert got[0].view(np.uint32).tobytes() == scores.cpu().numpy().view(np.uint32).tobytes()
        assert np.array_equal(got[1], oi.cpu().numpy())
        assert got[2].view(np.uint32).tobytes() == ov.cpu().numpy().view(np.uint32).tobytes()
