#!/usr/bin/env python3
"""Benchmark: exact, bitwise-deterministic ragged top-k on one MI355X.

One step = one detk_topk_ragged call over the whole batch of the chosen synthetic
workload (default: the chunked-prefill causal indexer, 8192 query rows over a 16384
token context, row i window [0, 8192 + i], k = 2048, 0.0-plateau / ReLU-sum scores
with plateau fraction 0.7).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line with rows/s (value), score GB/s, the roofline object of the
dominant kernel (algorithmic bytes / event-timed launch duration, against the 8 TB/s
HBM peak) and the CPU oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "ragged top-k rows/s and score GB/s (% of HBM peak), k=2048, 1 GPU"
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


# Figures the pages report for other systems on other hardware.  They are carried beside
# the measurement as context only: none of them is this metric on this workload.
PAGES_CONTEXT = {
    "note": "other hardware and other systems; context, not a baseline for this metric",
    "qsa_prefill_tok_per_s_gb10": {
        "stock_racy_topk": 2360,
        "torch_topk_plus_canonical_sort": 1760,
        "hardware": "NVIDIA GB10 (DGX Spark)",
        "source": "docai.hu, Non-deterministic Qwen3.8-Flash-Next: summary; The price of the fix",
    },
    "flashinfer_filtered_topk_shared_mem_bytes": {
        "value": 131072, "k_max": 2048,
        "source": "vLLM PR #55872, GB10 failure trace and shared-memory comment",
    },
    "cutedsl_deterministic_topk_envelope": {
        "topk_max": 4096, "row_len_below": 2 ** 24,
        "source": "SGLang PR #31115, hardening commit",
    },
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


SELECTION_SOURCES = ("detk_api.hip", "topk_device.hpp", "kernels.hpp")
INDEXER_SOURCES = ("indexer.hip", "indexer.hpp")


def kernel_source_sha(names=SELECTION_SOURCES) -> str:
    """Hash of the kernel sources with comments and whitespace taken out, so that a
    comment edit does not mark counters taken on the same code as stale."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "deterministic_exact_top_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def cpu_threads() -> int:
    """Every core this process may run on."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, n)


ROUNDS = 7  # timed rounds of `steps` calls: the first is the headline, all give median and min


def scores_to_device(wl, dev):
    """The workload's scores as a CUDA tensor: float32, or float16 / bfloat16 for a 16-bit
    workload (its uint16 bit patterns reinterpreted)."""
    import torch
    fmt = getattr(wl, "fmt", None)
    if fmt is None:
        return torch.from_numpy(wl.scores).to(dev)
    t = torch.from_numpy(wl.scores.view(np.int16)).to(dev)
    return t.view(torch.float16 if fmt == "f16" else torch.bfloat16)


def time_gpu(wl, steps, warmup, rotate, rounds=ROUNDS, call_kw=None):
    """Warm up, then time `rounds` rounds of `steps` back-to-back calls.  Round 1 -- the
    `steps` calls right after the `warmup` calls -- is the headline figure; the later
    rounds give the median and the min per call.  Returns the timings and the outputs of
    the last call of round 1 (copied to the host) for the parity check."""
    import torch
    import deterministic_exact_top_amd as detk

    dev = torch.device("cuda:0")
    copies = []
    for _ in range(rotate):
        copies.append(scores_to_device(wl, dev))
    rs = torch.from_numpy(wl.row_starts).to(dev)
    ln = torch.from_numpy(wl.lengths).to(dev)
    out_i = torch.empty((wl.B, wl.k), dtype=torch.int32, device=dev)
    out_v = torch.empty((wl.B, wl.k), dtype=copies[0].dtype, device=dev)
    ws = detk.new_workspace(wl.B, wl.k, wl.max_len, dev)
    stream = torch.cuda.current_stream(dev)

    kw = {key: (torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else v) for key, v in (call_kw or {}).items()}

    def step(i):
        detk.topk_ragged(copies[i % rotate], rs, ln, wl.k, max_len=wl.max_len, out_idx=out_i, out_val=out_v,
                         workspace=ws, stream=stream, **kw)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    walls, avgs = [], []
    outputs = None
    for r in range(rounds):
        # The timed region: events on the stream the kernels run on, bracketing all
        # `steps` back-to-back calls (their average is the average launch duration, gaps
        # included), inside a host clock bracketed by device synchronisations.
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        avgs.append(e0.elapsed_time(e1) / steps)
        if r == 0:
            outputs = (out_i.cpu().numpy(), out_v.view(torch.int32 if out_v.element_size() == 4 else torch.int16)
                       .cpu().numpy().view(np.uint32 if out_v.element_size() == 4 else np.uint16))
    # Then each launch bracketed on its own (for the fastest launch; the event pair around
    # every call adds a little to each).
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return walls, avgs, launch_ms, ws.numel(), outputs


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rows(wl, rs, ln, threads):
    """The oracle (float32 or 16-bit, as the workload is) on the rows (rs, ln)."""
    import oracle
    if getattr(wl, "fmt", None) is None:
        return oracle.topk_ragged(wl.scores, rs, ln, wl.k, wl.max_len, threads=threads)
    return oracle.topk_ragged16(wl.scores, rs, ln, wl.k, wl.max_len, fmt=wl.fmt, threads=threads)


def cpu_baseline(wl, budget_s: float = 15.0):
    """The oracle as it stands, on the host cores, over rows of the same workload."""
    threads = cpu_threads()
    # Calibrate on a small slice, then size the sample to ~budget_s of CPU work.
    probe = min(wl.B, 64)
    t0 = time.perf_counter()
    oracle_rows(wl, wl.row_starts[:probe], wl.lengths[:probe], threads=1)
    per_row_cpu = (time.perf_counter() - t0) / probe
    rows = int(min(wl.B, max(probe, budget_s / max(per_row_cpu, 1e-9))))
    sel = np.linspace(0, wl.B - 1, rows).astype(np.int64) if rows < wl.B else np.arange(wl.B)
    rs, ln = wl.row_starts[sel], wl.lengths[sel]
    t0 = time.perf_counter()
    oracle_rows(wl, rs, ln, threads=threads)
    dt = time.perf_counter() - t0
    extra = {}
    if wl.B <= 64 and threads > 1:  # small batches: the single-thread figure as well
        t0 = time.perf_counter()
        oracle_rows(wl, rs, ln, threads=1)
        extra["value_1thread"] = rows / (time.perf_counter() - t0)
    return {
        "value": rows / dt,
        "unit": "rows/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d of %d rows (%s), qsort by (total-order key desc, index asc) + truncate, %d threads"
                  % (rows, wl.B, "all" if rows == wl.B else "evenly spaced", threads),
        "seconds": dt,
        "cpu_model": cpu_model(),
        **extra,
    }


def traffic_for(workload, algo_bytes, sources=SELECTION_SOURCES):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha") != kernel_source_sha(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def event_us(fn, reps: int, stream) -> list:
    """Per-call µs of fn() over `reps` back-to-back calls, 5 rounds (events on `stream`)."""
    import torch
    out = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / reps)
    return out


def attainable_bandwidth() -> dict:
    """What plain streaming kernels reach on this GPU, median of 5 rounds: the library's
    read probe (16-byte loads, every byte once) over 1 GiB, and a 512 MiB device copy."""
    import torch
    import deterministic_exact_top_amd as detk
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    x = torch.rand(1 << 28, device=dev)  # 1 GiB
    word = torch.zeros(1, dtype=torch.int32, device=dev)
    rd = event_us(lambda: detk.read_probe(x, word, stream), 10, stream)
    src = torch.rand(1 << 27, device=dev)  # 512 MiB
    dst = torch.empty_like(src)
    cp = event_us(lambda: dst.copy_(src), 10, stream)
    return {
        "stream_read_gbps": x.nbytes / (float(np.median(rd)) * 1e-6) / 1e9,
        "copy_gbps": 2 * src.nbytes / (float(np.median(cp)) * 1e-6) / 1e9,
        "kernels": "detk_read_probe over 1 GiB (read only); 512 MiB device copy (read + write)",
    }


def graph_timing(wl, calls: int = 20, outputs: bool = False) -> dict:
    """Per-call time with `calls` calls (over rotated input copies) captured in one HIP graph
    and replayed: no host work between the kernels (the launches are bound once, at
    capture).  outputs: also return the last replayed call's (out_idx, out_val)."""
    import torch
    import deterministic_exact_top_amd as detk
    dev = torch.device("cuda:0")
    rotate = max(1, min(calls, -(-2 * MALL_BYTES // max(wl.scores.nbytes, 1))))
    copies = [torch.from_numpy(wl.scores).to(dev) for _ in range(rotate)]
    rs = torch.from_numpy(wl.row_starts).to(dev)
    ln = torch.from_numpy(wl.lengths).to(dev)
    out_i = torch.empty((wl.B, wl.k), dtype=torch.int32, device=dev)
    out_v = torch.empty((wl.B, wl.k), dtype=torch.float32, device=dev)
    ws = detk.new_workspace(wl.B, wl.k, wl.max_len, dev)
    kw = dict(max_len=wl.max_len, out_idx=out_i, out_val=out_v, workspace=ws)
    detk.topk_ragged(copies[0], rs, ln, wl.k, **kw)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            detk.topk_ragged(copies[i % rotate], rs, ln, wl.k, **kw)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    per = [u / calls for u in event_us(g.replay, 1, torch.cuda.current_stream(dev))]
    res = {"graph_us_per_call": float(np.median(per)), "calls_per_graph": calls, "input_copies": rotate}
    if outputs:
        res["_outputs"] = (out_i.cpu().numpy(), out_v.cpu().numpy().view(np.uint32))
    return res


def empty_graph_floor(wl, calls: int = 20) -> float:
    """Per-call time of the same call with every row empty (padding only), replayed from a
    HIP graph: the launch and the smallest kernel, no host work."""
    import torch
    import deterministic_exact_top_amd as detk
    dev = torch.device("cuda:0")
    s = torch.zeros(16, device=dev)
    rs = torch.zeros(wl.B, dtype=torch.int32, device=dev)
    ln = torch.zeros(wl.B, dtype=torch.int32, device=dev)
    out_i = torch.empty((wl.B, wl.k), dtype=torch.int32, device=dev)
    out_v = torch.empty((wl.B, wl.k), dtype=torch.float32, device=dev)
    ws = detk.new_workspace(wl.B, wl.k, wl.max_len, dev)
    call = lambda: detk.topk_ragged(s, rs, ln, wl.k, max_len=wl.max_len, out_idx=out_i, out_val=out_v, workspace=ws)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            call()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    return float(np.median([u / calls for u in event_us(g.replay, 1, torch.cuda.current_stream(dev))]))


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bfloat16 matrix peak


def indexer_measure(steps: int, warmup: int) -> dict:
    """The score producer upstream of the selection (detk_indexer_scores) on the chunked-
    prefill shape: 8192 query rows over 16,384 keys, 16 heads of 128, causal windows.  Times
    `steps` producer calls after `warmup` (HIP events on the call's stream) and the same
    number of producer + selection pairs; checks 8 sampled rows' scores against the oracle
    within its float32 bound and the selection of every row against the oracle's selection
    over the GPU's scores, bit for bit."""
    import torch
    import oracle
    from oracle import indexer as OI
    import deterministic_exact_top_amd as detk
    import workloads as W
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    inp = W.indexer_causal(Q=8192, ctx=16384)
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    kk = torch.from_numpy(inp.keys.view(np.int16)).to(dev)
    ln = torch.from_numpy(inp.lengths).to(dev)
    out = torch.zeros((inp.B, inp.max_len), dtype=torch.float32, device=dev)
    oi = torch.empty((inp.B, inp.k), dtype=torch.int32, device=dev)
    ov = torch.empty((inp.B, inp.k), dtype=torch.float32, device=dev)
    ws = detk.new_workspace(inp.B, inp.k, inp.max_len, dev)
    prod = lambda: detk.indexer_scores(q, w, kk, ln, inp.max_len, out=out, stream=stream)
    pair = lambda: (prod(), detk.topk_ragged(out.view(-1), None, ln, inp.k, max_len=inp.max_len, out_idx=oi,
                                             out_val=ov, workspace=ws, stream=stream))
    for _ in range(warmup):
        pair()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record(stream)
    for _ in range(steps):
        prod()
    e[1].record(stream)
    for _ in range(steps):
        pair()
    e[2].record(stream)
    torch.cuda.synchronize()
    prod_us = e[0].elapsed_time(e[1]) * 1e3 / steps
    pair_us = e[1].elapsed_time(e[2]) * 1e3 / steps
    flops = 2.0 * inp.H * inp.D * inp.sum_n
    tflops = flops / (prod_us * 1e-6) / 1e12
    # parity
    host = out.cpu().numpy()
    rows = [0, 1, 1000, 4095, 4096, 6000, 8190, 8191]
    sub = W.IndexerInputs(inp.name, inp.q[rows], inp.w[rows], inp.keys, inp.key_starts[rows], inp.lengths[rows],
                          inp.max_len, inp.k)
    exact = OI.scores(sub.q, sub.w, sub.keys, sub.lengths, sub.max_len)
    bound = OI.error_bound(sub.q, sub.w, sub.keys, sub.lengths, sub.max_len)
    within = all(bool(np.all(np.abs(host[b, :inp.lengths[b]].astype(np.float64) - exact[i, :inp.lengths[b]])
                              <= bound[i, :inp.lengths[b]])) for i, b in enumerate(rows))
    ri, rv = oracle.topk_ragged(host.reshape(-1), None, inp.lengths, inp.k, inp.max_len, B=inp.B,
                                threads=cpu_threads())
    sel_ok = bool(np.array_equal(oi.cpu().numpy(), ri)) and bool(np.array_equal(ov.cpu().numpy().view(np.uint32), rv))
    bytes_ = inp.q.nbytes + inp.w.nbytes + inp.keys.nbytes + 4 * inp.sum_n
    return {
        "workload": "indexer_causal_8192x16384_h16_d128", "B": inp.B, "n_keys": inp.max_len, "heads": inp.H,
        "head_dim": inp.D, "k": inp.k, "sum_n": inp.sum_n, "steps": steps, "warmup": warmup,
        "producer_us": prod_us, "producer_plus_selection_us": pair_us,
        "zero_fraction": float(np.mean(host[0, :inp.lengths[0]] == 0.0)),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic_for("indexer_causal_8192x16384_h16_d128", bytes_, INDEXER_SOURCES),
                     "algorithmic_flops": flops, "algorithmic_bytes": bytes_,
                     "note": "2 H D sum(n) flops per call (the [H x D] x [D x n] products; the ReLU and head "
                             "sum are not counted), bfloat16 dense peak; traffic: HBM bytes per launch from "
                             "FETCH_SIZE and WRITE_SIZE"},
        "parity": {"ok": within and sel_ok, "scores_rows_checked": len(rows), "scores_within_bound": within,
                   "selection_rows_checked": inp.B, "selection_bit_exact": sel_ok},
    }


DECODE = ("plateau_4x4096", "decode_ragged_64")


def decode_latency() -> dict:
    """The decode-step figure: per-call latency of the small-batch workloads (rows fewer than
    CUs), calls replayed from a HIP graph, with the small-batch shapes the library picks for
    them (1024 threads per row, every wave selecting pivot digits) and, for comparison, with
    the many-row shapes forced (the library's test switch); beside it the same call with
    every row empty.  The replayed outputs are checked against the oracle."""
    import deterministic_exact_top_amd as detk
    import workloads as W
    out = {}
    for name in DECODE:
        wl = W.full(name)
        small = graph_timing(wl, outputs=True)
        par = parity_check(wl, small.pop("_outputs"))
        detk.debug_set(detk.DETK_DEBUG_SMALL_BATCH, 1)
        try:
            many = graph_timing(wl)
        finally:
            detk.debug_set(detk.DETK_DEBUG_SMALL_BATCH, 0)
        out[name] = {"B": wl.B, "max_len": wl.max_len, "k": wl.k, "sum_n": wl.sum_n,
                     "us_per_call": small["graph_us_per_call"],
                     "us_per_call_many_row_shapes": many["graph_us_per_call"],
                     "empty_call_us": empty_graph_floor(wl), "input_copies": small["input_copies"],
                     "parity": {"ok": par["ok"], "gpu_sha256_16": par["gpu_sha256_16"],
                                "oracle_sha256_16": par["oracle_sha256_16"]}}
    return out


def dispatch_floor(wl) -> dict:
    """Per-call time of the same call with every row empty (all padding): the host-side
    argument handling plus the launch, back to back."""
    import torch
    import deterministic_exact_top_amd as detk
    dev = torch.device("cuda:0")
    s = torch.zeros(16, device=dev)
    rs = torch.zeros(wl.B, dtype=torch.int32, device=dev)
    ln = torch.zeros(wl.B, dtype=torch.int32, device=dev)
    out_i = torch.empty((wl.B, wl.k), dtype=torch.int32, device=dev)
    out_v = torch.empty((wl.B, wl.k), dtype=torch.float32, device=dev)
    ws = detk.new_workspace(wl.B, wl.k, wl.max_len, dev)
    call = lambda: detk.topk_ragged(s, rs, ln, wl.k, max_len=wl.max_len, out_idx=out_i, out_val=out_v, workspace=ws)
    call()
    torch.cuda.synchronize()
    per = event_us(call, 200, torch.cuda.current_stream(dev))
    return {"empty_call_us": float(np.median(per)), "note": "same B, k and max_len, every length 0"}


def copy_probe(nbytes: int, reps: int) -> None:
    """A plain device-to-device copy of known size, to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


SECONDARY = "long_context_8x262144"


def parity_check(wl, outputs, transform=None) -> dict:
    """The timed calls' outputs (last call of the first round) against the oracle's, byte
    for byte, on every row (after the oracle's index transform when one is fused)."""
    import oracle
    gi, gv = outputs
    if getattr(wl, "fmt", None) is None:
        oi, ov = oracle.topk_ragged(wl.scores, wl.row_starts, wl.lengths, wl.k, wl.max_len, threads=cpu_threads())
    else:
        oi, ov = oracle.topk_ragged16(wl.scores, wl.row_starts, wl.lengths, wl.k, wl.max_len, fmt=wl.fmt,
                                      threads=cpu_threads())
    if transform is not None:
        oi = oracle.index_transform(oi, transform["mode"], offsets=transform.get("index_offsets"),
                                    page_table=transform.get("page_table"), page_size=transform.get("page_size", 1))
    same_i, same_v = bool(np.array_equal(gi, oi)), bool(np.array_equal(gv, ov))
    digest = lambda a, b: hashlib.sha256(np.ascontiguousarray(a).tobytes() + np.ascontiguousarray(b).tobytes()
                                         ).hexdigest()[:16]
    return {"ok": same_i and same_v, "rows_checked": int(wl.B), "gpu_sha256_16": digest(gi, gv),
            "oracle_sha256_16": digest(oi, ov), "what": "out_idx and out_val bits of the last call of round 1"}


def make_transform(wl, kind: str, page_size: int):
    """The fused index transform for a workload: offsets = the rows' starts in the packed
    buffer (absolute indices), or one shared page table of randomly placed pages (the query
    rows of one sequence).  Returns (keyword arguments for the call, oracle description)."""
    if kind == "none":
        return None, None
    rng = np.random.default_rng(17)
    if kind == "offset":
        offs = wl.row_starts.astype(np.int32)
        return {"index_offsets": offs}, {"mode": 1, "index_offsets": offs}
    pages = -(-wl.max_len // page_size)
    pt = rng.permutation(pages + 64)[:pages].astype(np.int32)
    return {"page_table": pt, "page_size": page_size}, {"mode": 2, "page_table": pt, "page_size": page_size}


def measure(wl, steps, warmup, rotate, transform_kind="none", page_size=64) -> dict:
    """Time one workload (rounds of `steps` calls after `warmup` calls) and check the timed
    outputs; the roofline object comes from round 1."""
    call_kw, xf = make_transform(wl, transform_kind, page_size)
    algo = wl.algorithmic_bytes()
    rotate = rotate or max(1, -(-2 * MALL_BYTES // max(wl.scores.nbytes, 1)))
    rotate = min(rotate, 200)
    log("timing %s: %d rounds of %d steps (+%d warmup), %d input copies" % (wl.name, ROUNDS, steps, warmup, rotate))
    walls, avgs, launch_ms, ws_bytes, outputs = time_gpu(wl, steps, warmup, rotate, call_kw=call_kw)
    log("checking the timed outputs against the oracle")
    parity = parity_check(wl, outputs, xf)
    per_round_us = [a * 1e3 for a in avgs]
    achieved = algo / (avgs[0] * 1e-3) / 1e9
    return {
        "rotate": rotate,
        "ms_per_step": 1e3 * walls[0] / steps,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            # (counters are stored for the plain call: none for a fused index transform)
            "traffic": traffic_for(wl.name, algo) if transform_kind == "none" else None,
            "algorithmic_bytes_per_launch": algo,
            "avg_launch_us": per_round_us[0],
            "min_launch_us": float(np.min(launch_ms)) * 1e3,
            "kernel": "topk_ragged_kernel",
            "workspace_bytes": ws_bytes,
        },
        "rounds": {
            "rounds": len(avgs), "steps_per_round": steps,
            "avg_launch_us_per_round": per_round_us,
            "median_us": float(np.median(per_round_us)), "min_us": float(np.min(per_round_us)),
            "frac_at_median": algo / (float(np.median(per_round_us)) * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "note": "round 1 (the headline) runs right after the warmup calls; the GPU clock may still "
                    "be ramping then, so later rounds can be faster",
        },
        "parity": parity,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 200 untimed calls (about 25 ms of GPU work on the prefill workload) bring the GPU to
    # its steady clocks; with 5, the timed calls ran about 15 % slower while it ramped.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="prefill_causal_8192x16384")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies cycled per step (0: enough to exceed the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--index-transform", choices=["none", "offset", "page_table"], default="none",
                    help="fuse the index transform into the call (offsets: the rows' starts; page table: one "
                         "shared table of randomly placed pages)")
    ap.add_argument("--page-size", type=int, default=64)
    ap.add_argument("--dtype", choices=["f32", "f16", "bf16"], default="f32",
                    help="score format: the workload's float32 scores, or rounded to binary16 / bfloat16")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the long-context workload measured beside the headline one")
    ap.add_argument("--copy-probe", type=int, default=0, help="run a plain copy of this many bytes and exit")
    ap.add_argument("--attainable", action="store_true",
                    help="add the bandwidth a plain streaming read and a plain copy reach on this GPU")
    ap.add_argument("--graph", action="store_true", help="add the per-call time with the calls replayed from a HIP graph")
    ap.add_argument("--floor", action="store_true", help="add the per-call time of the same call with every row empty")
    ap.add_argument("--force-exact", action="store_true",
                    help="time the exact radix path every row takes when the sampled pivot misses (the "
                         "library's test switch; the worst case of a call)")
    ap.add_argument("--no-indexer", action="store_true",
                    help="skip the indexer-score producer (matrix cores) measured upstream of the selection")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step latency of the small-batch workloads (graph replay)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the top-k rows are independent, so a multi-GPU "
              "run would only shard rows; the benchmark measures one GPU's share (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe, 5)
        return

    import workloads as W
    if args.force_exact:
        import deterministic_exact_top_amd as detk
        detk.debug_set(detk.DETK_DEBUG_FAST, 0)
    log("generating %s" % args.workload)
    wl = W.full(args.workload)
    if args.dtype != "f32":
        wl = W.to16(wl, args.dtype)
    m = measure(wl, args.steps, args.warmup, args.rotate, args.index_transform, args.page_size)
    ms_per_step = m["ms_per_step"]
    score_bytes = 4 if args.dtype == "f32" else 2
    score_gbps = score_bytes * wl.sum_n / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": wl.B / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32" if args.dtype == "f32" else "u16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "B": wl.B, "max_len": wl.max_len, "k": wl.k, "sum_n": wl.sum_n,
            "input_copies_rotated": m["rotate"], "parallelism": "none (1 GPU)",
            "path": "exact radix path forced on every row (worst case)" if args.force_exact else "default",
            "index_transform": args.index_transform if args.index_transform == "none" else
            "%s%s" % (args.index_transform, " (page size %d)" % args.page_size if args.index_transform == "page_table" else ""),
        },
        "score_gbps": score_gbps,
        "score_frac_of_hbm_peak": score_gbps / HBM_PEAK_GBPS,
        "roofline": m["roofline"],
        "rounds": m["rounds"],
        "parity": m["parity"],
    }
    if args.workload != SECONDARY and not args.no_secondary:
        log("generating %s (secondary)" % SECONDARY)
        wl2 = W.full(SECONDARY)
        if args.dtype != "f32":
            wl2 = W.to16(wl2, args.dtype)
        m2 = measure(wl2, max(args.steps, 200), args.warmup, 0, args.index_transform, args.page_size)
        result["secondary"] = {
            "workload": wl2.name, "B": wl2.B, "max_len": wl2.max_len, "k": wl2.k, "sum_n": wl2.sum_n,
            "steps": max(args.steps, 200), "warmup": args.warmup, "input_copies_rotated": m2["rotate"],
            "ms_per_step": m2["ms_per_step"], "rows_per_s": wl2.B / (m2["ms_per_step"] * 1e-3),
            "roofline": m2["roofline"], "rounds": m2["rounds"], "parity": m2["parity"],
        }
        if args.dtype == "f32" and args.index_transform == "none":
            # the same calls captured once in a HIP graph and replayed (no host work between
            # the kernels), beside the same call with every row empty
            log("timing %s from a graph" % SECONDARY)
            gr = graph_timing(wl2, outputs=True)
            par = parity_check(wl2, gr.pop("_outputs"))
            gr["parity_ok"] = bool(par["ok"])
            gr["empty_call_us"] = empty_graph_floor(wl2)
            result["secondary"]["graph_replay"] = gr
            m2["parity"]["ok"] = m2["parity"]["ok"] and gr["parity_ok"]
        ok_all = m["parity"]["ok"] and m2["parity"]["ok"]
    else:
        ok_all = m["parity"]["ok"]
    if not args.no_indexer and args.dtype == "f32" and args.index_transform == "none":
        log("timing the indexer-score producer")
        result["indexer"] = indexer_measure(max(args.steps, 20), max(args.warmup, 5))
        ok_all = ok_all and result["indexer"]["parity"]["ok"]
    if not args.no_decode and args.dtype == "f32" and args.index_transform == "none":
        log("timing decode-step latency")
        result["decode_latency"] = decode_latency()
        ok_all = ok_all and all(v["parity"]["ok"] for v in result["decode_latency"].values())
    if args.graph:
        log("timing graph replay")
        result["graph"] = graph_timing(wl)
    if args.floor:
        log("timing empty calls")
        result["floor"] = dispatch_floor(wl)
    if args.attainable:
        log("timing plain streaming kernels")
        result["attainable"] = attainable_bandwidth()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(wl)
    result["pages_context"] = PAGES_CONTEXT
    print(json.dumps(result))
    if not ok_all:
        log("PARITY FAILURE: the timed calls' outputs differ from the oracle's")
        sys.exit(1)


if __name__ == "__main__":
    main()
