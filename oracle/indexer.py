"""CPU oracle for the lightning-indexer score -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this module; the GPU product path never does, and shares no code with it.

What it computes (the plain definition, written out in float64).  SGLang PR #31115,
review thread: the DSA lightning-indexer score of a query against a key is a sum over
the indexer heads of ReLU-ed per-head dot products, weighted per head -- which is why
every key whose heads all score non-positive lands on exactly 0.0:

    score[b, t] = sum_h w[b, h] * max(0, sum_d q[b, h, d] * k[s_b + t, d])

for the positions t < n_b of query row b's key window (s_b = key_starts[b], 0 when
absent; n_b = clamp(lengths[b], 0, max_len)).  q and k are bfloat16 bit patterns, w is
float32; every value is widened exactly to float64 and the sums are taken in float64
(numpy's matrix product is one library step; nothing is blocked or reordered beyond it).

The GPU evaluates the same expression in float32 (exact bfloat16 products, float32
sums in an order of its own), so it is compared with this definition within
``error_bound``, a forward error bound for any float32 evaluation order.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24  # unit roundoff of float32


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64: the pattern is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _windows(B: int, lengths, max_len: int, key_starts):
    for b in range(B):
        n = int(min(max(int(lengths[b]) if lengths is not None else max_len, 0), max_len))
        s = int(key_starts[b]) if key_starts is not None else 0
        yield b, s, n


def scores(q_bits, w, k_bits, lengths, max_len: int, key_starts=None) -> np.ndarray:
    """score[b, t] for t < n_b (float64 [B, max_len]; NaN outside each window).

    q_bits: uint16 [B, H, D]; w: float32 [B, H]; k_bits: uint16 [Lk, D]."""
    Q = bf16_to_f64(q_bits)
    K = bf16_to_f64(k_bits)
    W = np.asarray(w, dtype=np.float32).astype(np.float64)
    B = Q.shape[0]
    out = np.full((B, max_len), np.nan)
    for b, s, n in _windows(B, lengths, max_len, key_starts):
        dots = Q[b] @ K[s:s + n].T          # [H, n]: per-head dot products
        out[b, :n] = W[b] @ np.maximum(dots, 0.0)
    return out


def error_bound(q_bits, w, k_bits, lengths, max_len: int, key_starts=None) -> np.ndarray:
    """Bound on |float32 evaluation - score| for every (b, t) of the windows (NaN outside).

    A float32 evaluation forms each product q*k exactly (bfloat16 has an 8-bit significand,
    so a product needs 16 bits), sums D of them in some order (at most D + 4 roundings,
    allowing a few partial sums to be added separately), applies the ReLU (which never
    increases an error), multiplies by w (one rounding) and sums H heads (at most H
    roundings) before the final result.  The standard bound for sums of n rounded terms,
    |fl(sum) - sum| <= n u sum|terms|, gives
        |err| <= (D + H + 8) u sum_h |w_h| sum_d |q_hd k_td|  (times 1.01 for second-order
    terms), u = 2^-24."""
    Q = bf16_to_f64(q_bits)
    K = bf16_to_f64(k_bits)
    W = np.abs(np.asarray(w, dtype=np.float32).astype(np.float64))
    B, H, D = Q.shape
    gamma = (D + H + 8) * U32 * 1.01
    out = np.full((B, max_len), np.nan)
    for b, s, n in _windows(B, lengths, max_len, key_starts):
        mags = np.abs(Q[b]) @ np.abs(K[s:s + n]).T  # [H, n]: sum_d |q k|
        out[b, :n] = gamma * (W[b] @ mags)
    return out
