"""Pins of the lightning-indexer score oracle (oracle/indexer.py) against what the pages
and the arithmetic fix, independent of the oracle's own code (CPU only).

Source of the definition: SGLang PR #31115, review thread -- the DSA lightning-indexer
score is a sum over heads of ReLU-ed per-head dot products, weighted per head, so keys
whose heads all score non-positive sit exactly on 0.0.  The synthetic workload follows the
"score stats" script's documented indexer model in the same thread.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import indexer as OI
import workloads as W


def _bf16(x) -> np.ndarray:
    """float32 values that are exact in bfloat16, as bit patterns (the top half)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "test values must be exact in bfloat16"
    return (u >> 16).astype(np.uint16)


def test_bf16_decoding():
    pats = np.array([0x3F80, 0xC040, 0x0000, 0x8000, 0x7F80, 0x3F81, 0x0001], np.uint16)
    got = OI.bf16_to_f64(pats)
    assert got[0] == 1.0 and got[1] == -3.0 and got[2] == 0.0
    assert got[3] == 0.0 and math.copysign(1.0, got[3]) == -1.0
    assert got[4] == math.inf
    assert got[5] == 1.0 + 2.0 ** -7
    assert got[6] == 2.0 ** -133  # smallest positive bfloat16 subnormal


def _brute(qf, wf, kf, lengths, max_len, key_starts):
    """The definition as explicit loops in Python floats (no numpy arithmetic)."""
    B, H, D = qf.shape
    out = [[None] * max_len for _ in range(B)]
    for b in range(B):
        n = min(max(int(lengths[b]), 0), max_len)
        s = int(key_starts[b])
        for t in range(n):
            acc = 0.0
            for h in range(H):
                dot = 0.0
                for d in range(D):
                    dot += float(qf[b, h, d]) * float(kf[s + t, d])
                acc += float(wf[b, h]) * max(0.0, dot)
            out[b][t] = acc
    return out


def test_brute_force_integer_valued():
    """Small integers and power-of-two weights: every product and sum is exact in float64,
    so the oracle must equal explicit loops bit for bit (catches a transposed operand, a
    wrong head/window index or a dropped ReLU)."""
    rng = np.random.default_rng(5)
    B, H, D, Lk = 4, 5, 6, 23
    qf = rng.integers(-4, 5, (B, H, D)).astype(np.float32)
    kf = rng.integers(-4, 5, (Lk, D)).astype(np.float32)
    wf = (2.0 ** rng.integers(-3, 2, (B, H))).astype(np.float32)
    lengths = np.array([7, 0, 12, 30], np.int32)  # 30 is clamped to max_len
    key_starts = np.array([3, 0, 9, 1], np.int32)
    max_len = 15
    got = OI.scores(_bf16(qf), wf, _bf16(kf), lengths, max_len, key_starts)
    ref = _brute(qf, wf, kf, lengths, max_len, key_starts)
    for b in range(B):
        n = min(max(int(lengths[b]), 0), max_len)
        assert [float(x) for x in got[b, :n]] == ref[b][:n]
        assert np.all(np.isnan(got[b, n:]))


def test_relu_plateau_closed_form():
    """q_h = c_h e0 and k_t = a_t e0: score = sum_h w_h max(0, c_h a_t) in closed form; keys
    with a_t < 0 against all-positive c_h score exactly 0.0 (the structural plateau)."""
    H, D = 4, 8
    c = np.array([1.0, 0.5, 2.0, 0.25], np.float32)
    a = np.array([-3.0, -0.5, 0.0, 1.0, 2.0], np.float32)
    w = np.array([[0.5, 1.0, 0.25, 2.0]], np.float32)
    q = np.zeros((1, H, D), np.float32)
    q[0, :, 0] = c
    k = np.zeros((a.size, D), np.float32)
    k[:, 0] = a
    got = OI.scores(_bf16(q), w, _bf16(k), np.array([a.size]), a.size)[0]
    want = [sum(float(w[0, h]) * max(0.0, float(c[h]) * float(x)) for h in range(H)) for x in a]
    assert got.tolist() == want
    assert got[0] == 0.0 and got[1] == 0.0 and got[2] == 0.0
    assert got[3] == 0.5 * 1.0 + 1.0 * 0.5 + 0.25 * 2.0 + 2.0 * 0.25


def test_head_permutation_and_weight_scaling():
    rng = np.random.default_rng(9)
    B, H, D, L = 3, 8, 16, 40
    q = W.round_to_16bit(rng.standard_normal((B, H, D)).astype(np.float32), "bf16")
    k = W.round_to_16bit(rng.standard_normal((L, D)).astype(np.float32), "bf16")
    w = rng.random((B, H)).astype(np.float32)
    ln = np.full(B, L, np.int32)
    base = OI.scores(q, w, k, ln, L)
    perm = rng.permutation(H)
    assert np.allclose(OI.scores(q[:, perm], w[:, perm], k, ln, L), base, rtol=1e-12, atol=0)
    assert np.array_equal(OI.scores(q, 2 * w, k, ln, L), 2 * base)  # scaling by 2 is exact
    assert np.all(base >= 0.0)


def test_error_bound_covers_float32_evaluations():
    """Two float32 evaluations in different orders (sequential over d and over heads; numpy's
    pairwise float32 sums) stay within the bound of the exact score, and the bound is tight
    enough to mean something (well under 1e-4 of the score's magnitude scale)."""
    rng = np.random.default_rng(11)
    B, H, D, L = 3, 16, 128, 64
    q = W.round_to_16bit(rng.standard_normal((B, H, D)).astype(np.float32), "bf16")
    k = W.round_to_16bit(rng.standard_normal((L, D)).astype(np.float32), "bf16")
    w = (rng.random((B, H)) / H).astype(np.float32)
    ln = np.full(B, L, np.int32)
    exact = OI.scores(q, w, k, ln, L)
    bound = OI.error_bound(q, w, k, ln, L)
    qf = OI.bf16_to_f64(q).astype(np.float32)
    kf = OI.bf16_to_f64(k).astype(np.float32)
    # order 1: sequential float32 accumulation
    seq = np.zeros((B, L), np.float32)
    for b in range(B):
        for t in range(L):
            acc = np.float32(0.0)
            for h in range(H):
                dot = np.float32(0.0)
                for d in range(D):
                    dot = np.float32(dot + qf[b, h, d] * kf[t, d])
                acc = np.float32(acc + w[b, h] * max(np.float32(0.0), dot))
            seq[b, t] = acc
    # order 2: numpy's float32 products and pairwise sums
    dots = np.einsum("bhd,td->bht", qf, kf).astype(np.float32)
    pw = (w[:, :, None] * np.maximum(dots, np.float32(0.0))).sum(axis=1, dtype=np.float32)
    for ev in (seq, pw):
        assert np.all(np.abs(ev.astype(np.float64) - exact) <= bound)
    mag = (np.abs(w[:, :, None]) * (np.abs(qf) @ np.abs(kf).T)).sum(axis=1)
    assert np.all(bound <= 1e-4 * mag + 1e-30)


def test_window_clamp_and_default_starts():
    rng = np.random.default_rng(3)
    B, H, D, Lk = 2, 2, 4, 10
    q = W.round_to_16bit(rng.standard_normal((B, H, D)).astype(np.float32), "bf16")
    k = W.round_to_16bit(rng.standard_normal((Lk, D)).astype(np.float32), "bf16")
    w = rng.random((B, H)).astype(np.float32)
    a = OI.scores(q, w, k, np.array([-2, 99]), 6)
    assert np.all(np.isnan(a[0])) and not np.any(np.isnan(a[1]))
    b = OI.scores(q, w, k, np.array([4, 4]), 6, key_starts=np.array([0, 3]))
    c = OI.scores(q, w, k[3:], np.array([4, 4]), 6)
    assert np.array_equal(b[1, :4], c[1, :4])


def _model_plateau_fraction(H, rho, mu):
    """P(all H head logits <= 0) under the synthetic indexer model, by quadrature over the
    shared factor c: E_c[Phi(-(mu + sqrt(rho) c) / sqrt(1 - rho))^H]."""
    from scipy import integrate, stats
    f = lambda c: stats.norm.pdf(c) * stats.norm.cdf(-(mu + math.sqrt(rho) * c) / math.sqrt(1 - rho)) ** H
    return integrate.quad(f, -12, 12)[0]


def test_synthetic_indexer_follows_the_model():
    """The generator's q.k realise the pages' model: the exact-0.0 fraction of the scores
    matches P(all heads <= 0) under it (|r_t|^2 ~ 1 only approximates unit variance of the
    noise term, and bfloat16 rounding perturbs the logits, hence the tolerance)."""
    inp = W.indexer_causal(Q=48, ctx=3000, H=16, D=128, name="pin_indexer")
    s = OI.scores(inp.q, inp.w, inp.keys, inp.lengths, inp.max_len, inp.key_starts)
    vals = s[~np.isnan(s)]
    frac0 = float(np.mean(vals == 0.0))
    want = _model_plateau_fraction(16, 0.9, -1.0)
    assert abs(frac0 - want) < 0.03, (frac0, want)
    assert np.all(vals >= 0.0)
    assert inp.lengths.tolist() == list(range(3000 - 48 + 1, 3000 + 1))
