"""Plain, slow CPU oracle for one DSA layer: lightning-indexer scores, top-k
selection applied as a mask over the cache, and attention over the kept keys.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path (the
HIP library and its Python binding) never imports, calls or links it, and this
module imports nothing from the product path.

Precision: every floating-point step runs in float64 (NumPy), with inputs
widened exactly from bf16 or fp32. The pages fix no precision. The one
decision that floating point turns into integers, which keys a query keeps, is
taken on scores rounded to float32, the precision the GPU kernels score in.

Pages cited (text of three news pages on llama.cpp build b12180):
  [aiaulis]  aiaulis.com, "llama.cpp kan nu köra Kimi-K3.1-Pro, men än så
             länge bara text" (Swedish), paragraphs 1-8.
  [aiu]      aiunderstanding.org, "llama.cpp adds support for Kimi-K3.1-Pro
             architecture with DSA indexer", sections "What happened",
             "Why it matters", "What to watch next".
  [devotd]   devotd.net, "llama.cpp b12180 Kimi-K3.1-Pro" (Korean),
             sections 1-4 and the indexer-configuration table of section 1.

Readings of points the pages leave open (each one is listed again with its
reason in the design notes):
  * Score: the pages say a light indexer scores earlier tokens and attention
    keeps the best-scored ones [aiaulis para 2], with 32 heads, key dim 128
    and no RoPE [aiu "What happened"; devotd section 1 table], but print no
    formula. Reading: I[t,s] = sum_h w[t,h] * max(0, q[t,h] . k[s]), one
    indexer key per cached token shared by all indexer heads, no scale.
  * Candidates of query t at absolute position p are s = 0..p (self
    included), so that top_k >= p+1 gives full causal attention
    [aiaulis para 7; devotd section 4].
  * Ties in score go to the lower token index. -0.0 equals +0.0.
  * One selection per query, shared by every attention head.
  * Rows with fewer than top_k candidates keep all of them.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "index_scores",
    "round_scores_fp32",
    "select_topk",
    "padded_indices",
    "pack_mask",
    "attend_selected",
    "full_causal_attention",
    "dsa_rows",
]


def index_scores(qidx, w, kidx, q_pos0):
    """Lightning-indexer scores of one sequence, in float64.

    qidx [T, H_I, D_I], w [T, H_I], kidx [L, D_I]. Query i sits at absolute
    position p = q_pos0 + i. Returns I [T, L] with
        I[i, s] = sum_h w[i, h] * max(0, sum_d qidx[i, h, d] * kidx[s, d])
    for s <= p and -inf for s > p (not a candidate).

    The indexer scores earlier tokens [aiaulis para 2]; 32 heads of key dim
    128 and no RoPE [aiu "What happened"; devotd section 1 table]; one key per
    cached token, the indexer-key cache [devotd section 2].
    """
    q = np.asarray(qidx, dtype=np.float64)
    wt = np.asarray(w, dtype=np.float64)
    k = np.asarray(kidx, dtype=np.float64)
    T, H, D = q.shape
    L = k.shape[0]
    assert wt.shape == (T, H) and k.shape[1] == D
    out = np.full((T, L), -np.inf, dtype=np.float64)
    for i in range(T):
        p = q_pos0 + i
        n = min(p + 1, L)
        # z[h, s] = q[i, h] . k[s] for the candidates s <= p
        z = q[i] @ k[:n].T
        out[i, :n] = wt[i] @ np.maximum(z, 0.0)
    # canonicalise -0.0 to +0.0 so equal values compare equal as bit patterns
    out = out + 0.0
    return out


def round_scores_fp32(scores):
    """Round float64 scores to float32 (round to nearest even), -0 -> +0.

    The selection is a decision that floating point turns into integers; it is
    taken in the precision the GPU kernels score in, float32.
    """
    s = np.asarray(scores, dtype=np.float64).astype(np.float32)
    return s + np.float32(0.0)


def select_topk(row, p, top_k):
    """Selected token indices of one query, ascending.

    row: scores of the query (any float dtype), p: its position. The
    candidates are s = 0..p. If top_k >= p+1 every candidate is kept.
    Otherwise the top_k highest scores are kept, ties going to the lower
    index: a full sort on (score descending, index ascending), first top_k.
    Each query keeps its top_k best-scored earlier tokens [aiaulis paras 2-3;
    aiu "What happened"; devotd section 1 table, 2048 keys].
    """
    n = p + 1
    if top_k >= n:
        return np.arange(n, dtype=np.int64)
    cand = np.asarray(row[:n])
    idx = np.arange(n, dtype=np.int64)
    # np.lexsort sorts by the last key first: score descending, then index
    order = np.lexsort((idx, -cand.astype(np.float64)))
    return np.sort(order[:top_k])


def padded_indices(sel, top_k):
    """The index list as the library writes it: ascending, -1 padded to top_k."""
    out = np.full(top_k, -1, dtype=np.int32)
    out[: len(sel)] = sel
    return out


def pack_mask(sel, n_kv):
    """Selection as a bitmask over the whole cache [aiaulis para 4; devotd
    section 2]: bit (s % 32) of 32-bit word s // 32 is set when token s is
    kept. The row has roundup(n_kv, 64) / 32 words; bits of tokens >= n_kv
    are zero."""
    lpad = (n_kv + 63) // 64 * 64
    words = np.zeros(lpad // 32, dtype=np.uint32)
    for s in np.asarray(sel, dtype=np.int64):
        assert 0 <= s < n_kv
        words[s >> 5] |= np.uint32(1) << np.uint32(s & 31)
    return words


def attend_selected(q_row, k_cache, v_cache, sel, scale):
    """Attention of one query over its kept keys only [aiaulis para 2;
    devotd section 1]: for each head h,
        x_j = scale * q[h] . K[s_j, g(h)],   s_j in sel
        O[h] = sum_j exp(x_j - m) V[s_j, g(h)] / sum_j exp(x_j - m)
    with m = max_j x_j and g(h) = h // (H / H_kv) the key/value head of h.
    Tokens outside the selection get exactly zero weight, which is what
    masking the whole cache does [aiaulis para 4; devotd section 2].
    Returns (O [H, D], lse [H]) in float64, lse = m + log(sum_j exp(x_j - m)).
    An empty selection gives O = 0 and lse = -inf.
    """
    q = np.asarray(q_row, dtype=np.float64)
    H, D = q.shape
    sel = np.asarray(sel, dtype=np.int64)
    Hkv = k_cache.shape[1]
    group = H // Hkv
    O = np.zeros((H, D), dtype=np.float64)
    lse = np.full(H, -np.inf, dtype=np.float64)
    if sel.size == 0:
        return O, lse
    Ks = np.asarray(k_cache[sel], dtype=np.float64)  # [n, Hkv, D]
    Vs = np.asarray(v_cache[sel], dtype=np.float64)
    for h in range(H):
        g = h // group
        x = scale * (Ks[:, g, :] @ q[h])
        m = x.max()
        e = np.exp(x - m)
        den = e.sum()
        O[h] = (e @ Vs[:, g, :]) / den
        lse[h] = m + np.log(den)
    return O, lse


def full_causal_attention(q, k_cache, v_cache, q_pos0, scale):
    """Full causal softmax attention, the computation the DSA layers replace
    and the reference the selection must reproduce when top_k covers the
    context [aiaulis para 7; devotd section 4]. q [T, H, D], caches [L, H_kv,
    D]; query i attends to tokens 0..q_pos0+i. Dense over the whole cache with
    a causal mask, written independently of attend_selected."""
    qq = np.asarray(q, dtype=np.float64)
    K = np.asarray(k_cache, dtype=np.float64)
    V = np.asarray(v_cache, dtype=np.float64)
    T, H, D = qq.shape
    L, Hkv, _ = K.shape
    group = H // Hkv
    pos = q_pos0 + np.arange(T)
    allowed = np.arange(L)[None, :] <= pos[:, None]  # [T, L]
    O = np.zeros((T, H, D), dtype=np.float64)
    for h in range(H):
        g = h // group
        x = scale * (qq[:, h, :] @ K[:, g, :].T)  # [T, L]
        x = np.where(allowed, x, -np.inf)
        m = x.max(axis=1, keepdims=True)
        e = np.exp(x - m)
        O[:, h, :] = (e @ V[:, g, :]) / e.sum(axis=1, keepdims=True)
    return O


def dsa_rows(qidx, w, kidx, q, k_cache, v_cache, q_pos0, top_k, scale, rows=None):
    """The whole layer for the chosen query rows of one sequence.

    Each row: scores (float64), rounded to float32 for the selection, top_k
    selection, attention over the kept keys. Returns a dict of per-row lists:
    scores64, scores32 (the candidate prefix s <= p only), sel, out [H, D],
    lse [H].
    """
    T = qidx.shape[0]
    rows = range(T) if rows is None else rows
    res = {"rows": [], "scores64": [], "scores32": [], "sel": [], "out": [], "lse": []}
    for i in rows:
        p = q_pos0 + i
        s64 = index_scores(qidx[i : i + 1], w[i : i + 1], kidx[: p + 1], p)[0]
        s32 = round_scores_fp32(s64)
        sel = select_topk(s32, p, top_k)
        O, lse = attend_selected(q[i], k_cache, v_cache, sel, scale)
        res["rows"].append(i)
        res["scores64"].append(s64)
        res["scores32"].append(s32)
        res["sel"].append(sel)
        res["out"].append(O)
        res["lse"].append(lse)
    return res
