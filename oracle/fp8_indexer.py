"""Plain CPU oracle for the fp8 reading of the lightning indexer: the indexer
tensors quantised to 8-bit floats (e4m3) with one scale per row, then the
same score.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path never
imports, calls or links it, and it imports nothing from the product path.

Why this exists: the pages keep the indexer's tensors out of quantisation
because top-k selection is sensitive to their precision [aiaulis para 5;
aiu "What happened"; devotd section 3]. This variant measures that
sensitivity: how much of the selection an 8-bit indexer keeps. The pages
print no fp8 format; the readings below are the plainest ones.

Readings:
  * Format: e4m3 without infinities (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; largest finite value 448, smallest subnormal 2^-9).
    Rounding to nearest, ties to even mantissa; magnitudes beyond 448 (only
    reachable through the float32 rounding of x / scale) become 448.
  * Scales: one per indexer-query head row and one per cached key row,
    scale = max_d |x_d| / 448 computed in float32 (1 for an all-zero row),
    so each row's largest entry maps to 448. The code of an entry is
    e4m3(float32(x / scale)): the division is rounded to float32 first, the
    precision the GPU quantises in (the codes are integers that floating
    point decides, so both sides decide in the same precision).
  * Score: with positive scales max(0, a b z) = a b max(0, z), so
        I8[i, s] = ks[s] * sum_h wq[i, h] * max(0, sum_d q8[i, h, d] k8[s, d])
    with wq = float32(w * qs) (the query scale folded into the head weight,
    rounded to float32 as stored), s <= p, -inf past p.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_round", "quantize_rows_fp8", "index_scores_fp8"]

E4M3_MAX = 448.0


def e4m3_round(x):
    """Nearest e4m3 value of each entry (ties to even mantissa), as float64;
    magnitudes past 448 saturate to 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # a = m * 2^ex with m in [0.5, 1): the leading bit has weight 2^(ex-1)
    _, ex = np.frexp(a)
    e = np.clip(ex - 1, -6, 8)          # normal exponents -6..8; below 2^-6 the subnormal step
    quantum = np.ldexp(1.0, e - 3)      # 3 mantissa bits
    r = np.round(a / quantum) * quantum  # np.round rounds half to even; a / quantum is exact
    r = np.minimum(r, E4M3_MAX)
    return np.where(x < 0, -r, r)


def quantize_rows_fp8(x):
    """(codes as float64 e4m3 values, float32 scale per row) of a [..., D]
    array: scale = float32(max |x| / 448) (1 for an all-zero row), code =
    e4m3(float32(x / scale))."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    ratio = (x32 / scale[..., None]).astype(np.float32)
    return e4m3_round(ratio), scale


def index_scores_fp8(qidx, w, kidx, q_pos0):
    """fp8 indexer scores of one sequence, in float64, from the unquantised
    inputs qidx [T, H_I, D_I], w [T, H_I], kidx [L, D_I]: quantise, then
        I8[i, s] = ks[s] * sum_h wq[i, h] * max(0, q8[i, h] . k8[s])
    for s <= p = q_pos0 + i, -inf past p. Returns (I8 [T, L], q8, wq, k8, ks)."""
    q8, qs = quantize_rows_fp8(qidx)
    k8, ks = quantize_rows_fp8(kidx)
    wq = (np.asarray(w, dtype=np.float32) * qs).astype(np.float32)
    T = q8.shape[0]
    L = k8.shape[0]
    out = np.full((T, L), -np.inf, dtype=np.float64)
    for i in range(T):
        n = min(q_pos0 + i + 1, L)
        z = q8[i] @ k8[:n].T                      # [H, n]
        out[i, :n] = ks[:n].astype(np.float64) * (wq[i].astype(np.float64) @ np.maximum(z, 0.0))
    return out + 0.0, q8, wq, k8, ks
