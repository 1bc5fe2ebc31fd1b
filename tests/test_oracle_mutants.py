"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a copy of an oracle function, on the CPU, swaps it in for the
original (in the pin module and in the oracle modules, so that the functions
that call it pick it up too) and runs every pin of that part of the oracle
(tests/test_oracle.py, test_oracle_fp8.py or test_oracle_front_end.py) with
all of its parameters. At least one pin must fail for every mistake.
"""
import itertools

import numpy as np
import pytest

import oracle
import oracle.dsa_oracle as od
import oracle.fp8_indexer as o8
import oracle.front_end as ofe
import test_oracle as pins
import test_oracle_fp8 as pins8
import test_oracle_front_end as pins_fe


def _pin_calls(pins):
    """(name, function, keyword arguments) for every pin and parameter set."""
    for name in sorted(dir(pins)):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        combos = [{}]
        for m in getattr(fn, "pytestmark", []):
            if m.name != "parametrize":
                continue
            names = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            new = []
            for c, v in itertools.product(combos, m.args[1]):
                v = v.values if hasattr(v, "values") else v
                v = (v,) if len(names) == 1 else tuple(v)
                new.append({**c, **dict(zip(names, v))})
            combos = new
        for kw in combos:
            yield name, fn, kw


PIN_CALLS = {m: list(_pin_calls(m)) for m in (pins, pins8, pins_fe)}


# ----------------------------------------------------------------------------- planted mistakes

def _scores(relu_after_sum=False, no_relu=False, diag_excluded=False, heads_reversed=False):
    def f(qidx, w, kidx, q_pos0):
        q = np.asarray(qidx, dtype=np.float64)
        wt = np.asarray(w, dtype=np.float64)
        k = np.asarray(kidx, dtype=np.float64)
        T = q.shape[0]
        L = k.shape[0]
        out = np.full((T, L), -np.inf)
        for i in range(T):
            p = q_pos0 + i
            n = min(p if diag_excluded else p + 1, L)
            z = q[i] @ k[:n].T
            wi = wt[i][::-1] if heads_reversed else wt[i]
            if no_relu:
                out[i, :n] = wi @ z
            elif relu_after_sum:
                out[i, :n] = np.maximum(wi @ z, 0.0)
            else:
                out[i, :n] = wi @ np.maximum(z, 0.0)
        return out + 0.0
    return f


def _select(ties_to_higher=False, unsorted=False):
    def f(row, p, top_k):
        n = p + 1
        if top_k >= n:
            return np.arange(n, dtype=np.int64)
        cand = np.asarray(row[:n]).astype(np.float64)
        idx = np.arange(n, dtype=np.int64)
        order = np.lexsort((-idx if ties_to_higher else idx, -cand))
        return order[:top_k] if unsorted else np.sort(order[:top_k])
    return f


def _round_identity(scores):
    return np.asarray(scores, dtype=np.float64) + 0.0


def _pack_mask_msb_first(sel, n_kv):
    lpad = (n_kv + 63) // 64 * 64
    words = np.zeros(lpad // 32, dtype=np.uint32)
    for s in np.asarray(sel, dtype=np.int64):
        words[s >> 5] |= np.uint32(1) << np.uint32(31 - (s & 31))
    return words


def _attend(no_scale=False, head_mod=False, lse_without_max=False, mean_not_sum=False):
    def f(q_row, k_cache, v_cache, sel, scale):
        q = np.asarray(q_row, dtype=np.float64)
        H, D = q.shape
        sel = np.asarray(sel, dtype=np.int64)
        Hkv = k_cache.shape[1]
        group = H // Hkv
        O = np.zeros((H, D))
        lse = np.full(H, -np.inf)
        if sel.size == 0:
            return O, lse
        Ks = np.asarray(k_cache[sel], dtype=np.float64)
        Vs = np.asarray(v_cache[sel], dtype=np.float64)
        for h in range(H):
            g = h % Hkv if head_mod else h // group
            x = (1.0 if no_scale else scale) * (Ks[:, g, :] @ q[h])
            m = x.max()
            e = np.exp(x - m)
            den = float(len(sel)) if mean_not_sum else e.sum()
            O[h] = (e @ Vs[:, g, :]) / den
            lse[h] = (np.log(e.sum()) if lse_without_max else m + np.log(e.sum()))
        return O, lse
    return f


def _full_causal_strict(q, k_cache, v_cache, q_pos0, scale):
    qq = np.asarray(q, dtype=np.float64)
    K = np.asarray(k_cache, dtype=np.float64)
    V = np.asarray(v_cache, dtype=np.float64)
    T, H, D = qq.shape
    L, Hkv, _ = K.shape
    group = H // Hkv
    pos = q_pos0 + np.arange(T)
    allowed = np.arange(L)[None, :] < pos[:, None] + (pos[:, None] == 0)  # the diagonal dropped (but row 0 keeps token 0)
    O = np.zeros((T, H, D))
    for h in range(H):
        g = h // group
        x = np.where(allowed, scale * (qq[:, h, :] @ K[:, g, :].T), -np.inf)
        e = np.exp(x - x.max(axis=1, keepdims=True))
        O[:, h, :] = (e @ V[:, g, :]) / e.sum(axis=1, keepdims=True)
    return O


def _front_end(dims_major=False, proj_heads_reversed=False):
    def f(x, q_lat, w_qb, w_k, w_proj, idx_heads, idx_dim):
        x = np.asarray(x, dtype=np.float64)
        q_lat = np.asarray(q_lat, dtype=np.float64)
        T = x.shape[0]
        q = q_lat @ np.asarray(w_qb, dtype=np.float64).T
        qidx = (q.reshape(T, idx_dim, idx_heads).transpose(0, 2, 1) if dims_major
                else q.reshape(T, idx_heads, idx_dim))
        wp = np.asarray(w_proj, dtype=np.float64)
        return qidx, x @ np.asarray(w_k, dtype=np.float64).T, x @ (wp[::-1] if proj_heads_reversed else wp).T
    return f


def _e4m3(ties_away=False, mant_bits=3, saturate=True):
    def f(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        _, ex = np.frexp(a)
        e = np.clip(ex - 1, -6, 8)
        quantum = np.ldexp(1.0, e - mant_bits)
        r = (np.floor(a / quantum + 0.5) if ties_away else np.round(a / quantum)) * quantum
        if saturate:
            r = np.minimum(r, 448.0)
        return np.where(x < 0, -r, r)
    return f


def _quantize_max(fmt_max):
    def f(x):
        x32 = np.asarray(x, dtype=np.float32)
        amax = np.max(np.abs(x32), axis=-1)
        scale = np.where(amax > 0, amax / np.float32(fmt_max), np.float32(1.0)).astype(np.float32)
        return o8.e4m3_round((x32 / scale[..., None]).astype(np.float32)), scale
    return f


def _scores_fp8(drop_key_scale=False, drop_query_scale=False):
    def f(qidx, w, kidx, q_pos0):
        q8, qs = o8.quantize_rows_fp8(qidx)
        k8, ks = o8.quantize_rows_fp8(kidx)
        wq = np.asarray(w, dtype=np.float32) * (np.float32(1.0) if drop_query_scale else qs)
        wq = wq.astype(np.float32)
        T, L = q8.shape[0], k8.shape[0]
        out = np.full((T, L), -np.inf)
        for i in range(T):
            n = min(q_pos0 + i + 1, L)
            z = q8[i] @ k8[:n].T
            sc = np.ones(n) if drop_key_scale else ks[:n].astype(np.float64)
            out[i, :n] = sc * (wq[i].astype(np.float64) @ np.maximum(z, 0.0))
        return out + 0.0, q8, wq, k8, ks
    return f


L, F8, FE = (pins, (od, oracle)), (pins8, (o8, oracle)), (pins_fe, (ofe, oracle))
MUTANTS = [
    ("scores: ReLU dropped", L, "index_scores", _scores(no_relu=True)),
    ("scores: ReLU after the head sum", L, "index_scores", _scores(relu_after_sum=True)),
    ("scores: the query's own position left out", L, "index_scores", _scores(diag_excluded=True)),
    ("scores: head weights applied in reverse head order", L, "index_scores", _scores(heads_reversed=True)),
    ("selection: ties to the higher index", L, "select_topk", _select(ties_to_higher=True)),
    ("selection: indices returned in score order", L, "select_topk", _select(unsorted=True)),
    ("selection: taken on float64 instead of float32 scores", L, "round_scores_fp32", _round_identity),
    ("mask: bit order reversed within a word", L, "pack_mask", _pack_mask_msb_first),
    ("attention: softmax scale dropped", L, "attend_selected", _attend(no_scale=True)),
    ("attention: query head h reads K/V head h mod H_kv", L, "attend_selected", _attend(head_mod=True)),
    ("attention: log-sum-exp without the maximum", L, "attend_selected", _attend(lse_without_max=True)),
    ("attention: divided by the kept count, not the weight sum", L, "attend_selected", _attend(mean_not_sum=True)),
    ("full attention: causal limit one short", L, "full_causal_attention", _full_causal_strict),
    ("front end: query heads split dims-major", FE, "indexer_front_end", _front_end(dims_major=True)),
    ("front end: projection rows in reverse head order", FE, "indexer_front_end", _front_end(proj_heads_reversed=True)),
    ("fp8: e4m3 ties rounded away from zero", F8, "e4m3_round", _e4m3(ties_away=True)),
    ("fp8: two mantissa bits (e5m2 step)", F8, "e4m3_round", _e4m3(mant_bits=2)),
    ("fp8: no saturation at 448", F8, "e4m3_round", _e4m3(saturate=False)),
    ("fp8: row maximum mapped to 240 (the fnuz format's maximum)", F8, "quantize_rows_fp8", _quantize_max(240.0)),
    ("fp8: key scales dropped from the score", F8, "index_scores_fp8", _scores_fp8(drop_key_scale=True)),
    ("fp8: query scales not folded into the head weights", F8, "index_scores_fp8", _scores_fp8(drop_query_scale=True)),
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("label,where,target,mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(label, where, target, mutant, monkeypatch):
    pin_module, oracle_modules = where
    for mod in (pin_module, *oracle_modules):
        if hasattr(mod, target):
            monkeypatch.setattr(mod, target, mutant)
    caught = []
    for name, fn, kw in PIN_CALLS[pin_module]:
        try:
            fn(**kw)
        except Exception:  # an assertion, or a shape the planted mistake breaks
            caught.append(name)
    assert caught, f"no pin fails when the oracle has the mistake: {label}"


@pytest.mark.parametrize("pin_module", [pins, pins8, pins_fe], ids=["layer", "fp8", "front_end"])
def test_pins_enumerated(pin_module):
    # every pin function is reached, each parameter set once
    names = {n for n, _, _ in PIN_CALLS[pin_module]}
    assert names == {n for n in dir(pin_module) if n.startswith("test_")}
    assert len(PIN_CALLS[pin_module]) >= len(names)
