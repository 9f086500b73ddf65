"""GPU determinism: byte-identical output across repeated runs, batch compositions,
a busy sibling stream and HIP-graph replay.

The pages find races by replaying identical input many times while other work
perturbs scheduling (SGLang PR #31115, "Accuracy Tests": 30 repetitions with a busy
sibling stream; review-thread tie-safety harness) and require graph replay to equal
eager execution bitwise (PR "Modifications").  The selected set must be a pure
function of the input across batch compositions (review thread).
"""
from __future__ import annotations

import numpy as np
import pytest

import deterministic_exact_top_amd as detk
import workloads as W
from gpu_util import assert_same, debug_overrides, log, run_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    detk.load_library()
    return torch.device("cuda:0")


# Every named workload at full size, plus a 16-row narrow batch.
REPLAY = {
    "plateau": lambda: W.full("plateau_4x4096"),
    "decode_ragged": lambda: W.full("decode_ragged_64"),
    "prefill_causal": lambda: W.full("prefill_causal_8192x16384"),
    "narrow": lambda: W.full("narrow_128x65536"),
    "long_context": lambda: W.full("long_context_8x262144"),
    "narrow_small": lambda: W.narrow_range(B=16, L=65536, k=4096, name="replay_narrow"),
}


@pytest.mark.parametrize("name", sorted(REPLAY))
def test_twenty_runs_identical(dev, name):
    """20 calls on the same input into the same output buffers: every call's output is
    byte-identical to the oracle's (which also makes them identical to each other)."""
    import torch
    wl = REPLAY[name]()
    scores, rs, ln = to_dev(wl, dev)
    out_i = torch.empty((wl.B, wl.k), dtype=torch.int32, device=dev)
    out_v = torch.empty((wl.B, wl.k), dtype=torch.float32, device=dev)
    ws = detk.new_workspace(wl.B, wl.k, wl.max_len, dev)  # one workspace for every call
    log("replay x20: %s B=%d max_len=%d k=%d" % (name, wl.B, wl.max_len, wl.k))
    oi, ov = run_oracle(wl)
    for rep in range(20):
        out_i.fill_(-7)
        out_v.fill_(7.0)
        detk.topk_ragged(scores, rs, ln, wl.k, max_len=wl.max_len, out_idx=out_i, out_val=out_v, workspace=ws)
        torch.cuda.synchronize()
        assert_same(out_i.cpu().numpy(), out_v.cpu().numpy().view(np.uint32), oi, ov, "%s rep %d" % (name, rep))


def test_batch_composition_invariance(dev):
    """A row's output does not depend on which other rows share the call, their
    order, or the launch shape chosen for the batch."""
    import torch
    a = W.decode_ragged(B=24, n_lo=1, n_hi=30000, k=2048, name="comp_a")
    bwl = W.long_context(B=3, L=300000, k=2048, short_n=1700, name="comp_b")
    # One packed buffer holding both workloads' rows.
    buf = np.concatenate([a.scores, bwl.scores])
    starts = np.concatenate([a.row_starts.astype(np.int64), bwl.row_starts.astype(np.int64) + a.scores.size])
    lens = np.concatenate([a.lengths, bwl.lengths]).astype(np.int32)
    B = lens.size
    d_buf = torch.from_numpy(buf).to(dev)
    oi, ov = detk_oracle_rows(buf, starts, lens, 2048, 300000)

    def run(order):
        rs = torch.from_numpy(starts[order].astype(np.int32)).to(dev)
        ln = torch.from_numpy(lens[order]).to(dev)
        gi, gv = detk.topk_ragged(d_buf, rs, ln, 2048, max_len=300000)
        torch.cuda.synchronize()
        return gi.cpu().numpy(), gv.cpu().numpy().view(np.uint32)

    rng = np.random.default_rng(4)
    orders = [np.arange(B), np.arange(B)[::-1].copy(), rng.permutation(B)]
    for order in orders:
        log("composition order %s" % order[:6])
        gi, gv = run(order)
        assert_same(gi, gv, oi[order], ov[order], "composition")
    # each row alone, with the short-row launch shape where it fits one workgroup
    for b in (0, 5, B - 3, B - 2, B - 1):
        rs = torch.tensor([int(starts[b])], dtype=torch.int32, device=dev)
        ln = torch.tensor([int(lens[b])], dtype=torch.int32, device=dev)
        ml = int(max(lens[b], 1))
        gi, gv = detk.topk_ragged(d_buf, rs, ln, 2048, max_len=ml)
        torch.cuda.synchronize()
        assert np.array_equal(gi.cpu().numpy()[0], oi[b]) and np.array_equal(
            gv.cpu().numpy().view(np.uint32)[0], ov[b]), "row %d alone" % b


def detk_oracle_rows(buf, starts, lens, k, max_len):
    import oracle
    return oracle.topk_ragged(buf, starts.astype(np.int32), lens, k, max_len)


BUSY = {
    "plateau": "plateau_4x4096",          # boundary inside the 0.0 tie plateau
    "narrow": "narrow_128x65536",         # top digits collide, bitwise duplicates
    "long_context": "long_context_8x262144",
}


@pytest.mark.parametrize("name", sorted(BUSY))
def test_busy_sibling_stream(dev, name):
    """30 replays of one input while another stream runs large matmuls that compete for
    the CUs (SGLang PR #31115, "Accuracy Tests": 30 repetitions per input with a busy
    sibling stream); every replay must equal the oracle byte for byte."""
    import torch
    wl = W.full(BUSY[name])
    scores, rs, ln = to_dev(wl, dev)
    oi, ov = run_oracle(wl)
    side = torch.cuda.Stream()
    a = torch.randn(2048, 2048, device=dev)
    ws = detk.new_workspace(wl.B, wl.k, wl.max_len, dev)
    log("busy sibling stream replay x30: %s" % name)
    for rep in range(30):
        with torch.cuda.stream(side):
            for _ in range(4):
                a = (a @ a).clamp_(-1, 1)
        gi, gv = detk.topk_ragged(scores, rs, ln, wl.k, max_len=wl.max_len, workspace=ws)
        torch.cuda.synchronize()
        assert_same(gi.cpu().numpy(), gv.cpu().numpy().view(np.uint32), oi, ov, "busy rep %d" % rep)


def test_one_workspace_many_shapes(dev):
    """One workspace buffer, zero-filled once and sized for the largest call, serves a
    sequence of split-row calls of different shapes (rows, k, row length, tile count),
    in an order where a call with more rows follows calls with fewer: the per-row counters
    sit in a control area that no call's data ever overlaps, so each call still finds
    them at zero."""
    import torch
    wls = [W.long_context(B=3, L=70000, k=2048, short_n=900, name="ws_shapes_a"),
           W.narrow_range(B=24, L=65536, k=4096, name="ws_shapes_b"),
           W.long_context(B=8, L=262144, k=2048, short_n=1500, name="ws_shapes_c"),
           W.decode_ragged(B=64, n_lo=40000, n_hi=100000, k=1000, name="ws_shapes_d"),
           W.long_context(B=3, L=70000, k=2048, short_n=900, name="ws_shapes_a")]
    need = max(detk.workspace_size(w.B, w.k, w.max_len) for w in wls)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for rep in range(2):
        for w in wls:
            log("one workspace, rep %d: %s B=%d max_len=%d k=%d" % (rep, w.name, w.B, w.max_len, w.k))
            scores, rs, ln = to_dev(w, dev)
            gi, gv = detk.topk_ragged(scores, rs, ln, w.k, max_len=w.max_len, workspace=ws)
            torch.cuda.synchronize()
            oi, ov = run_oracle(w)
            assert_same(gi.cpu().numpy(), gv.cpu().numpy().view(np.uint32), oi, ov, "%s rep %d" % (w.name, rep))


def test_split_calls_on_two_streams(dev):
    """Split-row calls issued on two streams at once, each with a grid wider than the GPU
    holds, plus a one-workgroup-per-row call on a third: no workgroup of a split row waits
    for another, so the calls share the CUs in any proportion and all complete with the
    oracle's answer."""
    import torch
    wls = [W.long_context(B=24, L=300000, k=2048, short_n=1700, name="two_streams_a"),
           W.narrow_range(B=64, L=131072, k=4096, name="two_streams_b"),
           W.decode_ragged(B=200, n_lo=1, n_hi=32768, k=2048, name="two_streams_c")]
    refs = [run_oracle(w) for w in wls]
    bufs = [to_dev(w, dev) for w in wls]
    wss = [detk.new_workspace(w.B, w.k, w.max_len, dev) for w in wls]
    streams = [torch.cuda.Stream() for _ in wls]
    outs = [(torch.empty((w.B, w.k), dtype=torch.int32, device=dev),
             torch.empty((w.B, w.k), dtype=torch.float32, device=dev)) for w in wls]
    torch.cuda.synchronize()
    for rep in range(10):
        log("three streams, rep %d" % rep)
        for w, (sc, rs, ln), ws, st, (oi_, ov_) in zip(wls, bufs, wss, streams, outs):
            with torch.cuda.stream(st):
                detk.topk_ragged(sc, rs, ln, w.k, max_len=w.max_len, out_idx=oi_, out_val=ov_, workspace=ws,
                                 stream=st)
        torch.cuda.synchronize()
        for w, (oi, ov), (gi, gv) in zip(wls, refs, outs):
            assert_same(gi.cpu().numpy(), gv.cpu().numpy().view(np.uint32), oi, ov, "%s rep %d" % (w.name, rep))


@pytest.mark.parametrize("shape", ["single", "multi"])
def test_hip_graph_replay_matches_eager(dev, shape):
    """Capture one call into a HIP graph (through torch.cuda.graph), replay it on new
    inputs copied into the captured buffers, and check every replay against an eager
    call on the same input."""
    import torch
    if shape == "single":
        mk = lambda i: W.decode_ragged(B=32, n_lo=3000, n_hi=16000, k=2048, name="graph_%d" % i)
        max_len = 16000
    else:
        mk = lambda i: W.long_context(B=4, L=100000, k=2048, short_n=1234, name="graph_m%d" % i)
        max_len = 100000
    wls = [mk(i) for i in range(4)]
    size = max(w.scores.size for w in wls)
    B = wls[0].B
    s_buf = torch.zeros(size, device=dev)
    s_rs = torch.zeros(B, dtype=torch.int32, device=dev)
    s_ln = torch.zeros(B, dtype=torch.int32, device=dev)
    out_i = torch.empty(B, 2048, dtype=torch.int32, device=dev)
    out_v = torch.empty(B, 2048, device=dev)
    ws = detk.new_workspace(B, 2048, max_len, dev)

    def load(w):
        s_buf[:w.scores.size].copy_(torch.from_numpy(w.scores))
        s_rs.copy_(torch.from_numpy(w.row_starts))
        s_ln.copy_(torch.from_numpy(w.lengths))

    load(wls[0])
    # eager warmup on a side stream, then capture
    detk.topk_ragged(s_buf, s_rs, s_ln, 2048, max_len=max_len, out_idx=out_i, out_val=out_v, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        detk.topk_ragged(s_buf, s_rs, s_ln, 2048, max_len=max_len, out_idx=out_i, out_val=out_v, workspace=ws)
    torch.cuda.synchronize()
    for rep, w in enumerate(wls + wls[::-1]):
        load(w)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gi, gv = out_i.cpu().numpy().copy(), out_v.cpu().numpy().view(np.uint32).copy()
        ei, ev = detk.topk_ragged(s_buf, s_rs, s_ln, 2048, max_len=max_len)
        torch.cuda.synchronize()
        assert np.array_equal(gi, ei.cpu().numpy()), "replay %d idx" % rep
        assert np.array_equal(gv, ev.cpu().numpy().view(np.uint32)), "replay %d val" % rep
        oi, ov = run_oracle(w)
        assert_same(gi, gv, oi, ov, "graph replay %d" % rep)


def test_read_probe_reads_every_word(dev):
    """The streaming-read probe's XOR equals the XOR of every input word (so no load is
    skipped), for a size that leaves a ragged tail past the four-way unrolled loop."""
    import torch
    rng = np.random.default_rng(77)
    words = rng.integers(0, 2**32, size=(1 << 20) + 12, dtype=np.uint32)  # multiple of 4 words
    x = torch.from_numpy(words.view(np.int32)).to(dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    detk.read_probe(x, out)
    torch.cuda.synchronize()
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(words))
