"""Pins of the CPU oracle to facts other than its own code: hand-worked
fixtures, closed forms, library routines (torch's scaled_dot_product_attention
and scipy's logsumexp, both in float64 on the CPU), invariants, and brute force
on tiny inputs. Each test names the plausible oracle mistake it would catch."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import (
    attend_selected,
    dsa_rows,
    full_causal_attention,
    index_scores,
    pack_mask,
    padded_indices,
    round_scores_fp32,
    select_topk,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, str):
        return {"-inf": -np.inf, "-0.0": -0.0, "ln3": math.log(3.0), "ln4": math.log(4.0),
                "ln2": math.log(2.0)}[x]
    return float(x)


# ----------------------------------------------------------------------------- scores

def test_scores_hand_worked_example():
    """Hand-worked fixture: catches a dropped ReLU, a swapped w index, a
    transposed q (heads vs dims), an off-by-one in the causal range."""
    g = _load("indexer_tiny.json")
    q = np.array(g["qidx"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    k = np.array(g["kidx"], dtype=np.float64)
    want = np.array([[_num(x) for x in r] for r in g["scores"]])
    got = index_scores(q, w, k, g["q_pos0"])
    assert np.array_equal(got, want)
    for kk, sels in g["selections"].items():
        for t, sel in enumerate(sels):
            assert select_topk(round_scores_fp32(got[t]), t, int(kk)).tolist() == sel


def _rand_indexer(rng, T, H, D, L, ints=False):
    if ints:
        q = rng.integers(-4, 5, size=(T, H, D)).astype(np.float64)
        w = rng.integers(-2, 3, size=(T, H)).astype(np.float64)
        k = rng.integers(-4, 5, size=(L, D)).astype(np.float64)
    else:
        q = rng.standard_normal((T, H, D))
        w = rng.standard_normal((T, H))
        k = rng.standard_normal((L, D))
    return q, w, k


def test_scores_odd_part_closed_form():
    """ReLU(z) - ReLU(-z) = z, so I(q) - I(-q) = k . (sum_h w_h q_h) exactly in
    exact arithmetic: catches a dropped ReLU, a wrong sign, a wrong head weight
    and a transposed operand."""
    rng = np.random.default_rng(11)
    T, H, D, L = 7, 5, 6, 9
    q, w, k = _rand_indexer(rng, T, H, D, L)
    a = index_scores(q, w, k, q_pos0=2)
    b = index_scores(-q, w, k, q_pos0=2)
    lin = (np.einsum("th,thd->td", w, q)) @ k.T  # [T, L]
    for t in range(T):
        p = 2 + t
        n = min(p + 1, L)
        np.testing.assert_allclose(a[t, :n] - b[t, :n], lin[t, :n], rtol=1e-12, atol=1e-12)


def test_scores_even_part_closed_form():
    """ReLU(z) + ReLU(-z) = |z|: I(q) + I(-q) = sum_h w_h |q_h . k|."""
    rng = np.random.default_rng(12)
    T, H, D, L = 4, 3, 8, 4
    q, w, k = _rand_indexer(rng, T, H, D, L)
    a = index_scores(q, w, k, q_pos0=0)
    b = index_scores(-q, w, k, q_pos0=0)
    for t in range(T):
        for s in range(t + 1):
            want = sum(w[t, h] * abs(float(np.dot(q[t, h], k[s]))) for h in range(H))
            assert a[t, s] + b[t, s] == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_scores_one_hot_head_weight_is_relu_matmul():
    """w = e_h reduces the score to ReLU(q_h k^T), a NumPy matmul."""
    rng = np.random.default_rng(13)
    T, H, D, L = 6, 4, 5, 6
    q, _, k = _rand_indexer(rng, T, H, D, L)
    for h in range(H):
        w = np.zeros((T, H))
        w[:, h] = 1.0
        got = index_scores(q, w, k, q_pos0=0)
        want = np.maximum(q[:, h, :] @ k.T, 0.0)
        tri = np.tril(np.ones((T, L), dtype=bool))
        np.testing.assert_allclose(got[tri], want[tri], rtol=1e-13, atol=0)
        assert np.all(np.isneginf(got[~tri]))


def test_scores_head_permutation_invariant_and_integer_exact():
    """Permuting indexer heads jointly in (q, w) changes nothing (exact on
    integers); integer inputs give integer scores representable in float32."""
    rng = np.random.default_rng(14)
    T, H, D, L = 9, 32, 128, 9
    q, w, k = _rand_indexer(rng, T, H, D, L, ints=True)
    perm = rng.permutation(H)
    a = index_scores(q, w, k, 0)
    b = index_scores(q[:, perm], w[:, perm], k, 0)
    assert np.array_equal(a, b)
    fin = np.isfinite(a)
    assert np.array_equal(a[fin], np.round(a[fin]))
    assert np.abs(a[fin]).max() < 2**24
    assert np.array_equal(round_scores_fp32(a)[fin].astype(np.float64), a[fin])


def test_scores_causal_and_position_offset():
    """Scores past the query position are -inf and do not read those keys;
    a later q_pos0 equals the matching rows of a longer call."""
    rng = np.random.default_rng(15)
    T, H, D, L = 12, 3, 4, 12
    q, w, k = _rand_indexer(rng, T, H, D, L)
    full = index_scores(q, w, k, 0)
    part = index_scores(q[5:], w[5:], k, 5)
    assert np.array_equal(full[5:], part)
    k2 = k.copy()
    k2[8:] = 1e6
    alt = index_scores(q, w, k2, 0)
    assert np.array_equal(full[:8], alt[:8])
    assert np.all(np.isneginf(full[np.triu_indices(T, 1, L)]))


# ----------------------------------------------------------------------------- selection

def test_selection_hand_worked_ties():
    g = _load("selection_ties.json")
    for c in g["cases"]:
        row = np.array([_num(x) for x in c["row"]], dtype=np.float64)
        got = select_topk(round_scores_fp32(row), c["p"], c["top_k"]).tolist()
        assert got == c["sel"], c


def _threshold_prefix_select(row, p, k):
    """An independent selection: find the k-th largest value, keep everything
    strictly above it, then the lowest-index ties until k are kept."""
    vals = [float(v) + 0.0 for v in row[: p + 1]]
    if k >= len(vals):
        return list(range(len(vals)))
    kth = sorted(vals, reverse=True)[k - 1]
    above = [s for s, v in enumerate(vals) if v > kth]
    ties = [s for s, v in enumerate(vals) if v == kth]
    return sorted(above + ties[: k - len(above)])


def _is_valid_topk(row, p, k, sel):
    """Brute-force characterisation: |S| = min(k, p+1) and every kept token
    beats every dropped candidate (higher score, or equal score and lower
    index)."""
    vals = [float(v) + 0.0 for v in row[: p + 1]]
    S = set(int(s) for s in sel)
    if len(S) != min(k, p + 1) or any(s > p or s < 0 for s in S):
        return False
    for s in S:
        for r in range(p + 1):
            if r in S:
                continue
            if not (vals[s] > vals[r] or (vals[s] == vals[r] and s < r)):
                return False
    return True


@pytest.mark.parametrize("trial", range(60))
def test_selection_matches_independent_algorithm_and_brute_force(trial):
    rng = np.random.default_rng(100 + trial)
    n = int(rng.integers(1, 40))
    p = int(rng.integers(0, n))
    k = int(rng.integers(1, n + 3))
    if trial % 3 == 0:
        row = rng.integers(-3, 4, size=n).astype(np.float32)  # heavy ties
    elif trial % 3 == 1:
        row = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32), size=n)
    else:
        row = rng.standard_normal(n).astype(np.float32)
    sel = select_topk(row, p, k)
    assert sel.tolist() == _threshold_prefix_select(row, p, k)
    assert _is_valid_topk(row, p, k, sel)
    assert np.all(np.diff(sel) > 0)


def test_selection_invariant_under_power_of_two_scaling():
    rng = np.random.default_rng(7)
    row = rng.standard_normal(300).astype(np.float32)
    for j in (-3, 1, 5):
        assert np.array_equal(select_topk(row, 299, 50), select_topk(row * np.float32(2.0**j), 299, 50))


def test_selection_decided_on_float32_rounded_scores():
    # Scores 1 and 1 + 2^-30 differ in float64 but not in float32, whose
    # significand has 24 bits: decided in float32 the two tie and the lower
    # index is kept. Catches a selection taken on the float64 scores, and a
    # rounding that keeps the sign of a zero score.
    qidx = np.ones((2, 1, 1))
    w = np.ones((2, 1))
    kidx = np.array([[1.0], [1.0 + 2.0**-30]])
    zeros = np.zeros((2, 1, 1))
    r = dsa_rows(qidx, w, kidx, zeros, zeros, zeros, q_pos0=0, top_k=1, scale=1.0, rows=[1])
    assert r["scores64"][0][1] > r["scores64"][0][0]
    assert list(r["sel"][0]) == [0]
    s = round_scores_fp32(np.array([1.0 + 2.0**-30, -0.0]))
    assert s.dtype == np.float32
    assert s[0] == np.float32(1.0)
    assert s[1] == 0.0 and not np.signbit(s[1])


def test_padded_indices_and_mask_words():
    g = _load("mask_words.json")
    for c in g["cases"]:
        words = pack_mask(np.array(c["sel"], dtype=np.int64), c["n_kv"])
        assert [f"0x{int(x):08x}" for x in words] == c["words"]
    assert padded_indices(np.array([3, 9]), 5).tolist() == [3, 9, -1, -1, -1]


# ----------------------------------------------------------------------------- attention

def test_attention_hand_worked():
    g = _load("attention_tiny.json")
    for c in g["cases"]:
        O, lse = attend_selected(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                 np.array(c["sel"]), _num(c["scale"]))
        np.testing.assert_allclose(O, np.array(c["out"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, [_num(x) for x in c["lse"]], rtol=0, atol=1e-12)


def _sdpa(q, k, v, scale, mask=None, causal=False):
    # q [T,H,D], k/v [L,H,D] float64 -> torch [1,H,T,D]
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal,
                                                         scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("q_pos0", [0, 5])
@pytest.mark.parametrize("kv_heads", [4, 2])
def test_full_causal_attention_matches_torch_sdpa(q_pos0, kv_heads):
    """Library routine: torch's SDPA in float64 on the CPU. Catches a wrong
    scale, a wrong exponent base, a causal off-by-one and a wrong GQA head map."""
    rng = np.random.default_rng(21)
    T, H, D = 11, 4, 8
    L = q_pos0 + T
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((L, kv_heads, D))
    v = rng.standard_normal((L, kv_heads, D))
    scale = 0.37
    got = full_causal_attention(q, k, v, q_pos0, scale)
    rep = H // kv_heads
    kk = np.repeat(k, rep, axis=1)
    vv = np.repeat(v, rep, axis=1)
    mask = np.arange(L)[None, :] <= (q_pos0 + np.arange(T))[:, None]
    want = _sdpa(q, kk, vv, scale, mask=mask)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    if q_pos0 == 0:
        want2 = _sdpa(q, kk, vv, scale, causal=True)
        np.testing.assert_allclose(got, want2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv_heads", [6, 3, 1])
def test_attend_selected_matches_sdpa_on_gathered_rows_and_logsumexp(kv_heads):
    """Library routines on the gathered rows; kv_heads < heads pins the
    grouped-query head map (query head h reads key/value head h // group)."""
    rng = np.random.default_rng(22)
    H, D, L = 6, 16, 40
    q = rng.standard_normal((1, H, D))
    k = rng.standard_normal((L, kv_heads, D))
    v = rng.standard_normal((L, kv_heads, D))
    sel = np.array(sorted(rng.choice(L, size=13, replace=False)))
    O, lse = attend_selected(q[0], k, v, sel, 0.25)
    rep = H // kv_heads
    kk = np.repeat(k, rep, axis=1)
    vv = np.repeat(v, rep, axis=1)
    want = _sdpa(q, kk[sel], vv[sel], 0.25)[0]
    np.testing.assert_allclose(O, want, rtol=1e-12, atol=1e-12)
    for h in range(H):
        x = 0.25 * (kk[sel, h, :] @ q[0, h])
        assert lse[h] == pytest.approx(logsumexp(x), rel=1e-13)


def test_attention_closed_forms():
    rng = np.random.default_rng(23)
    H, D, L = 3, 8, 20
    q = rng.standard_normal((H, D))
    k = rng.standard_normal((L, H, D))
    v = rng.standard_normal((L, H, D))
    # one kept token: the output is that token's value row, exactly
    O, _ = attend_selected(q, k, v, np.array([7]), 0.5)
    assert np.array_equal(O, v[7])
    # constant value rows: the output is that constant
    vc = np.broadcast_to(np.arange(D, dtype=np.float64), (L, H, D)).copy()
    O, _ = attend_selected(q, k, vc, np.arange(0, L, 3), 0.5)
    np.testing.assert_allclose(O, vc[0], rtol=0, atol=1e-13)
    # empty selection: zero output, lse -inf
    O, lse = attend_selected(q, k, v, np.array([], dtype=np.int64), 0.5)
    assert np.all(O == 0) and np.all(np.isneginf(lse))


def test_layer_equals_full_attention_when_topk_covers_context():
    """The pages' one fixed invariant: with top_k at least the context, the
    layer's output is full causal attention [aiaulis para 7; devotd section 4];
    below the context it differs."""
    rng = np.random.default_rng(31)
    T, HI, DI, H, D = 48, 4, 8, 4, 16
    qidx = rng.standard_normal((T, HI, DI)).astype(np.float32)
    w = rng.standard_normal((T, HI)).astype(np.float32)
    kidx = rng.standard_normal((T, DI)).astype(np.float32)
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    scale = 1 / math.sqrt(D)
    full = full_causal_attention(q, k, v, 0, scale)
    for top_k in (T, T + 17):
        res = dsa_rows(qidx, w, kidx, q, k, v, 0, top_k, scale)
        np.testing.assert_allclose(np.stack(res["out"]), full, rtol=1e-12, atol=1e-12)
    res = dsa_rows(qidx, w, kidx, q, k, v, 0, 8, scale)
    diff = np.abs(np.stack(res["out"]) - full).max(axis=(1, 2))
    assert np.all(diff[:8] < 1e-12)      # rows with <= 8 candidates keep them all
    assert np.all(diff[8:] > 1e-6)       # later rows drop tokens and differ
