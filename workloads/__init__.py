"""Seeded synthetic inputs for ragged top-k.

This module only draws inputs: it holds none of the top-k method's arithmetic.  Both
the GPU path's tests/benchmark and the CPU oracle consume the buffers it returns.

The pages measure on live model traffic and share no score captures (SGLang PR #31115,
review thread: synthetic, reproducible data only), so these generators stand in for
it.  They follow that thread's synthetic lightning-indexer recipe (a score is a sum
over heads of weight x ReLU(head logit), which puts many entries exactly on 0.0) and
its fixture families (0.0 plateau, narrow value range, ties, -inf rows).

Every row draws from its own stream ``PCG64(SeedSequence([seed, row]))`` with
``seed = crc32(b"detk:<workload>:v1")`` (stable across processes, unlike ``hash()``),
so any row can be regenerated alone and the result does not depend on thread count.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
import zlib

import numpy as np

QNAN = np.uint32(0x7FC00000)      # +quiet NaN: poison for cells outside every window
NEG_QNAN = np.uint32(0xFFC00000)
NAN_PAYLOAD1 = np.uint32(0x7F800001)
POS_INF = np.uint32(0x7F800000)
NEG_INF = np.uint32(0xFF800000)
POS_ZERO = np.uint32(0x00000000)
NEG_ZERO = np.uint32(0x80000000)
DENORM_MIN = np.uint32(0x00000001)

HEADS = 16


@dataclasses.dataclass
class Workload:
    name: str
    scores: np.ndarray          # float32, flat buffer
    row_starts: np.ndarray      # int32 absolute offsets (len B)
    lengths: np.ndarray         # int32 (len B)
    max_len: int
    k: int

    @property
    def B(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def sum_n(self) -> int:
        return int(np.clip(self.lengths.astype(np.int64), 0, self.max_len).sum())

    def algorithmic_bytes(self) -> int:
        """Scores read once + out_idx/out_val written + 8 B metadata per row."""
        return 4 * self.sum_n + 8 * self.B * self.k + 8 * self.B


def seed_of(name: str) -> int:
    return zlib.crc32(("detk:%s:v1" % name).encode())


def row_rng(seed: int, row: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, row])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def relu_sum_mixture(rng: np.random.Generator, n: int, p: float, heads: int = HEADS) -> np.ndarray:
    """One row of the plateau / ReLU-sum mixture as float32.

    Each entry is +0.0 with probability ``p``; otherwise it is
    ``float32(sum_h w_h * max(x_h, 0))`` with ``x_h ~ N(0, 1)`` per entry and head and
    ``w_h ~ U(0, 1)`` per row, accumulated in float64 in head order and rounded once.
    """
    w = rng.random(heads)
    plateau = rng.random(n) < p
    npos = int(n - plateau.sum())
    x = rng.standard_normal((heads, npos))
    acc = np.zeros(npos, dtype=np.float64)
    for h in range(heads):
        acc += w[h] * np.maximum(x[h], 0.0)
    out = np.zeros(n, dtype=np.float32)
    out[~plateau] = acc.astype(np.float32)
    return out


def abs_normal_plateau(rng: np.random.Generator, n: int, p: float) -> np.ndarray:
    """+0.0 with probability ``p``, else |z| with z ~ N(0, 1) drawn in float32."""
    plateau = rng.random(n) < p
    z = np.abs(rng.standard_normal(n, dtype=np.float32))
    z[plateau] = 0.0
    return z


def narrow_bits(rng: np.random.Generator, n: int, dup_frac: float = 0.01) -> np.ndarray:
    """Values in [1.0, 1.0 + 2^-10): 0x3F800000 | r with r ~ U{0..8191} (float32 has
    exactly 8192 values there), then floor(dup_frac * n) positions copy the bits of
    other positions of the same row."""
    bits = np.uint32(0x3F800000) | rng.integers(0, 8192, size=n, dtype=np.uint32)
    ndup = int(dup_frac * n)
    if ndup:
        dst = rng.choice(n, size=ndup, replace=False)
        src = rng.integers(0, n, size=ndup)
        bits[dst] = bits[src]
    return bits.view(np.float32)


def _fill_rows(buf: np.ndarray, starts, lens, make_row, parallel: bool = True) -> None:
    def one(b):
        buf[starts[b]:starts[b] + lens[b]] = make_row(b)
    rows = range(len(lens))
    if parallel and len(lens) > 8:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, rows))
    else:
        for b in rows:
            one(b)


# --------------------------------------------------------------------------------------
# Named workloads.  Defaults are the full sizes; tests shrink them through arguments.
# --------------------------------------------------------------------------------------

def plateau_abs(B: int = 4, L: int = 4096, k: int = 2048, p: float = 0.6,
                name: str = "plateau_4x4096") -> Workload:
    """Dense (B, L) rows: exact 0.0 with probability p else |N(0,1)|, so the k-th
    boundary falls inside the 0.0 tie plateau (the [4, 4096], k = 2048 call shape of
    vLLM PR #55872's FlashInfer call matrix)."""
    seed = seed_of(name)
    buf = np.empty(B * L, dtype=np.float32)
    starts = (np.arange(B, dtype=np.int64) * L).astype(np.int32)
    lens = np.full(B, L, dtype=np.int32)
    _fill_rows(buf, starts, lens, lambda b: abs_normal_plateau(row_rng(seed, b), L, p))
    return Workload(name, buf, starts, lens, L, k)


def decode_ragged(B: int = 64, n_lo: int = 2048, n_hi: int = 32768, k: int = 2048,
                  p_lo: float = 0.3, p_hi: float = 0.95, name: str = "decode_ragged_64") -> Workload:
    """Packed 1-D ragged batch: n_b ~ U{n_lo..n_hi}, plateau p_b ~ U(p_lo, p_hi),
    ReLU-sum positives; row_starts is the exclusive cumsum of the lengths."""
    seed = seed_of(name)
    meta = row_rng(seed, 0xFFFF)
    lens = meta.integers(n_lo, n_hi + 1, size=B).astype(np.int32)
    ps = meta.uniform(p_lo, p_hi, size=B)
    starts64 = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]])
    starts = starts64.astype(np.int32)
    buf = np.empty(int(lens.astype(np.int64).sum()), dtype=np.float32)
    _fill_rows(buf, starts, lens, lambda b: relu_sum_mixture(row_rng(seed, b), int(lens[b]), float(ps[b])))
    return Workload(name, buf, starts, lens, n_hi, k)


def prefill_causal(Q: int = 8192, ctx: int = 16384, k: int = 2048, p: float = 0.7,
                   name: str = "prefill_causal_8192x16384") -> Workload:
    """Chunked-prefill causal indexer: Q query rows over a ctx-token context laid out
    as a dense (Q, ctx) matrix; row i's window is [0, ctx - Q + i], i.e.
    n_i = ctx - Q + 1 + i, so the last row spans the whole context.  Cells outside
    the window hold +qNaN, so a stray read would change the answer."""
    seed = seed_of(name)
    buf = np.full(Q * ctx, QNAN, dtype=np.uint32).view(np.float32)
    starts = (np.arange(Q, dtype=np.int64) * ctx).astype(np.int32)
    lens = (ctx - Q + 1 + np.arange(Q)).astype(np.int32)
    _fill_rows(buf, starts, lens, lambda b: relu_sum_mixture(row_rng(seed, b), int(lens[b]), p))
    return Workload(name, buf, starts, lens, ctx, k)


def narrow_range(B: int = 128, L: int = 65536, k: int = 4096, name: str = "narrow_128x65536") -> Workload:
    """Dense (B, L) rows in [1.0, 1.0 + 2^-10) with 1 % bitwise duplicates: the top
    radix digits collide, so the threshold bin overflows any staging buffer."""
    seed = seed_of(name)
    buf = np.empty(B * L, dtype=np.float32)
    starts = (np.arange(B, dtype=np.int64) * L).astype(np.int32)
    lens = np.full(B, L, dtype=np.int32)
    _fill_rows(buf, starts, lens, lambda b: narrow_bits(row_rng(seed, b), L))
    return Workload(name, buf, starts, lens, L, k)


def long_context(B: int = 8, L: int = 262144, k: int = 2048, p: float = 0.8, short_n: int = 1500,
                 name: str = "long_context_8x262144") -> Workload:
    """Dense (B, L) long rows (B >= 3), plateau p, with edge rows:
    row 0 all -inf over the full window; row 1 only ``short_n`` < k long (the tail of
    its storage is +qNaN) holding one each of +0.0, -0.0, +inf, -inf, +qNaN, -qNaN,
    +NaN(payload 1) and the smallest denormal; row 2 full length with its zeros split
    between +0.0 and -0.0 and 64 each of +qNaN, +NaN(payload 1), -qNaN, +inf, -inf."""
    assert B >= 3
    seed = seed_of(name)
    buf = np.empty(B * L, dtype=np.float32)
    starts = (np.arange(B, dtype=np.int64) * L).astype(np.int32)
    lens = np.full(B, L, dtype=np.int32)
    lens[1] = short_n

    def make(b):
        rng = row_rng(seed, b)
        if b == 0:
            return np.full(L, NEG_INF, dtype=np.uint32).view(np.float32)
        if b == 1:
            row = relu_sum_mixture(rng, short_n, p).view(np.uint32)
            specials = np.array([POS_ZERO, NEG_ZERO, POS_INF, NEG_INF, QNAN, NEG_QNAN, NAN_PAYLOAD1,
                                 DENORM_MIN], dtype=np.uint32)
            pos = rng.choice(short_n, size=specials.size, replace=False)
            row[pos] = specials
            return row.view(np.float32)
        row = relu_sum_mixture(rng, L, p).view(np.uint32)
        if b == 2:
            zeros = np.flatnonzero(row == 0)
            row[zeros[rng.random(zeros.size) < 0.5]] = NEG_ZERO
            specials = np.repeat(np.array([QNAN, NAN_PAYLOAD1, NEG_QNAN, POS_INF, NEG_INF],
                                          dtype=np.uint32), 64)
            pos = rng.choice(L, size=specials.size, replace=False)
            row[pos] = specials
        return row.view(np.float32)

    for b in range(B):
        buf[starts[b]:starts[b] + L] = make(b) if b != 1 else np.concatenate(
            [make(b), np.full(L - short_n, QNAN, dtype=np.uint32).view(np.float32)])
    return Workload(name, buf, starts, lens, L, k)


def round_to_16bit(x32: np.ndarray, fmt: str) -> np.ndarray:
    """float32 values rounded to a 16-bit float format, as uint16 bit patterns: binary16
    ("f16", numpy's conversion, round to nearest even) or bfloat16 ("bf16": the top half of
    the float32 bits after round to nearest even; NaNs stay NaN with their sign, quieted)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if fmt == "f16":
        with np.errstate(over="ignore"):  # (beyond 65504 rounds to infinity, as intended)
            return x32.astype(np.float16).view(np.uint16)
    u = x32.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    rounded[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return rounded


@dataclasses.dataclass
class Workload16:
    """A workload's scores rounded to a 16-bit format (same windows, k and row layout)."""
    name: str
    fmt: str
    scores: np.ndarray          # uint16 bit patterns, flat buffer
    row_starts: np.ndarray
    lengths: np.ndarray
    max_len: int
    k: int

    @property
    def B(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def sum_n(self) -> int:
        return int(np.clip(self.lengths.astype(np.int64), 0, self.max_len).sum())

    def algorithmic_bytes(self) -> int:
        """Scores read once (2 bytes each) + out_idx (4) and out_val (2) written + 8 B metadata per row."""
        return 2 * self.sum_n + 6 * self.B * self.k + 8 * self.B


def to16(wl: Workload, fmt: str) -> Workload16:
    return Workload16(wl.name + "_" + fmt, fmt, round_to_16bit(wl.scores, fmt), wl.row_starts, wl.lengths,
                      wl.max_len, wl.k)


@dataclasses.dataclass
class IndexerInputs:
    """Inputs of the lightning-indexer score for a batch of query rows over one key sequence:
    q (bfloat16 bits, [B, H, D]), per-query head weights w (float32, [B, H]), keys
    (bfloat16 bits, [Lk, D]), and each row's key window (key_starts, lengths, max_len)."""
    name: str
    q: np.ndarray
    w: np.ndarray
    keys: np.ndarray
    key_starts: np.ndarray
    lengths: np.ndarray
    max_len: int
    k: int

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def D(self) -> int:
        return int(self.q.shape[2])

    @property
    def sum_n(self) -> int:
        return int(np.clip(self.lengths.astype(np.int64), 0, self.max_len).sum())


def indexer_causal(Q: int = 8192, ctx: int = 16384, H: int = HEADS, D: int = 128, rho: float = 0.9,
                   mu: float = -1.0, k: int = 2048, name: str = "indexer_causal") -> IndexerInputs:
    """Queries and keys whose per-head dot products follow the synthetic indexer model of the
    "score stats" script (SGLang PR #31115, review thread): the logit of head h against key t
    is mu + sqrt(rho) c_t + sqrt(1 - rho) z_ht, with c_t a shared relevance factor of the key.
    Here that model is carried by real vectors: key t = (1, c_t, r_t) with r_t ~ N(0, I / (D - 2)),
    query head h = (mu, sqrt(rho), sqrt(1 - rho) g_h) with g_h ~ N(0, I), so q.k = mu +
    sqrt(rho) c_t + sqrt(1 - rho) g_h.r_t (the last term ~ N(0, |r_t|^2), |r_t|^2 ~ 1); all
    rounded to bfloat16.  Head weights w ~ U(0, 1) / H per query row.  Windows as in the
    chunked-prefill causal workload: row i covers keys [0, ctx - Q + i] (n_i = ctx - Q + i + 1)."""
    seed = seed_of(name)
    kr = row_rng(seed, 0xFFFF)
    c = kr.standard_normal(ctx)
    keys = np.empty((ctx, D), np.float32)
    keys[:, 0] = 1.0
    keys[:, 1] = c
    keys[:, 2:] = kr.standard_normal((ctx, D - 2)) / np.sqrt(D - 2)
    q = np.empty((Q, H, D), np.float32)
    w = np.empty((Q, H), np.float32)
    def one(b):
        rng = row_rng(seed, b)
        q[b, :, 0] = mu
        q[b, :, 1] = np.sqrt(rho)
        q[b, :, 2:] = np.sqrt(1.0 - rho) * rng.standard_normal((H, D - 2))
        w[b] = (rng.random(H) / H).astype(np.float32)
    if Q > 8:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(Q)))
    else:
        for b in range(Q):
            one(b)
    lengths = (ctx - Q + 1 + np.arange(Q)).astype(np.int32)
    return IndexerInputs(name, round_to_16bit(q, "bf16").reshape(Q, H, D), w,
                         round_to_16bit(keys, "bf16").reshape(ctx, D), np.zeros(Q, np.int32), lengths, ctx, k)


FULL = {
    "plateau_4x4096": plateau_abs,
    "decode_ragged_64": decode_ragged,
    "prefill_causal_8192x16384": prefill_causal,
    "narrow_128x65536": narrow_range,
    "long_context_8x262144": long_context,
}


def full(name: str) -> Workload:
    return FULL[name]()
