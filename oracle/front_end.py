"""Plain CPU oracle for the indexer front end: the three indexer tensors that
turn a token's activations into the indexer's inputs.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path never
imports, calls or links it, and it imports nothing from the product path.

Pages: the indexer of each DSA layer owns the tensors q_b, k and a
projection, which the release keeps out of quantisation because top-k
selection is sensitive to their precision [aiu "What happened"; devotd
section 3]; the indexer has 32 heads of dim 128 and no RoPE [aiu "What
happened"; devotd section 1 table].

Readings (the pages name the tensors but give no shapes or formula):
  * Each tensor is a plain linear map, applied in float64 here to the
    exactly widened bf16 inputs:
      q_b:        qidx[t, h, d] = sum_r q_lat[t, r] * w_qb[h * D_I + d, r]
                  (q_lat: the layer's compressed query, width q_rank)
      k:          kidx[t, d]    = sum_j x[t, j] * w_k[d, j]
      projection: w[t, h]       = sum_j x[t, j] * w_proj[h, j]
    (x: the layer's input activations, width hidden). Weight matrices are
    stored output-major ([out][in]), so each output is a dot product of two
    contiguous rows.
  * No RoPE (the pages rule it out), no scale, no bias, no norm: the table
    counts four indexer tensors per layer but the pages name only these
    three, and nothing they say fixes what a fourth would do.
  * kidx of the tokens at positions q_pos0 .. q_pos0 + T - 1 is appended to
    the layer's index-key cache at those positions [devotd section 2: the
    DSA layer keeps an index-key cache].
"""
from __future__ import annotations

import numpy as np

__all__ = ["indexer_front_end"]


def indexer_front_end(x, q_lat, w_qb, w_k, w_proj, idx_heads, idx_dim):
    """(qidx [T, H_I, D_I], kidx [T, D_I], w [T, H_I]) in float64 for one
    sequence's T tokens. x [T, hidden], q_lat [T, q_rank], w_qb
    [H_I * D_I, q_rank], w_k [D_I, hidden], w_proj [H_I, hidden]."""
    x = np.asarray(x, dtype=np.float64)
    q_lat = np.asarray(q_lat, dtype=np.float64)
    w_qb = np.asarray(w_qb, dtype=np.float64)
    w_k = np.asarray(w_k, dtype=np.float64)
    w_proj = np.asarray(w_proj, dtype=np.float64)
    T = x.shape[0]
    assert w_qb.shape == (idx_heads * idx_dim, q_lat.shape[1])
    assert w_k.shape == (idx_dim, x.shape[1]) and w_proj.shape == (idx_heads, x.shape[1])
    qidx = (q_lat @ w_qb.T).reshape(T, idx_heads, idx_dim)
    kidx = x @ w_k.T
    w = x @ w_proj.T
    return qidx, kidx, w
