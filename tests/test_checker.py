"""The comparator every GPU parity test goes through (tests/dsa_check.py)
accepts the oracle's own results and rejects planted errors just outside each
tolerance, while accepting errors inside it: a lenient comparator would let
the GPU parity tests pass whatever the kernels computed."""
import numpy as np
import pytest

from dsa_check import OUT_TOL, RowChecker, score_bound, selection_ok
from oracle import attend_selected, index_scores, round_scores_fp32, select_topk

T, L, HI, DI, H, D, K, Q0 = 6, 64, 4, 16, 4, 16, 10, 58


def _case(integer=False, seed=3):
    rng = np.random.default_rng(seed)
    if integer:
        qidx = rng.integers(-3, 4, (T, HI, DI)).astype(np.float64)
        w = rng.integers(0, 3, (T, HI)).astype(np.float64)
        kidx = rng.integers(-3, 4, (L, DI)).astype(np.float64)
    else:
        qidx = rng.standard_normal((T, HI, DI))
        w = rng.random((T, HI))
        kidx = rng.standard_normal((L, DI))
    q = rng.standard_normal((T, H, D))
    kc = rng.standard_normal((L, H, D))
    vc = rng.standard_normal((L, H, D))
    return qidx, w, kidx, q, kc, vc


def _oracle_row(c, i):
    qidx, w, kidx, q, kc, vc = c
    p = Q0 + i
    s64 = np.full(L, -np.inf)
    s64[: p + 1] = index_scores(qidx[i : i + 1], w[i : i + 1], kidx[: p + 1], p)[0]
    sel = select_topk(round_scores_fp32(s64[: p + 1]), p, K)
    out, lse = attend_selected(q[i], kc, vc, sel, 0.25)
    return s64.astype(np.float32), sel, out, lse


def _checker(c, dtype="fp32", integer=False):
    qidx, w, kidx, q, kc, vc = c
    return RowChecker(dtype, qidx, w, kidx, q, kc, vc, Q0, K, 0.25, integer=integer)


@pytest.mark.parametrize("integer", [False, True])
def test_accepts_the_oracle_itself(integer):
    c = _case(integer)
    rc = _checker(c, integer=integer)
    for i in range(T):
        s, sel, out, lse = _oracle_row(c, i)
        rc.check(i, gpu_scores_row=s, gpu_sel=sel, gpu_out=out, gpu_lse=lse)
    assert rc.stats["rows"] == T


def test_rejects_score_error_above_the_bound_and_accepts_below():
    c = _case()
    qidx, w, kidx = c[0], c[1], c[2]
    i = 2
    p = Q0 + i
    s, sel, _, _ = _oracle_row(c, i)
    bound = score_bound(qidx[i], w[i], kidx[: p + 1], DI, HI)
    s64 = index_scores(qidx[i : i + 1], w[i : i + 1], kidx[: p + 1], p)[0]
    j = 17
    bad = s.astype(np.float64).copy()
    bad[j] = s64[j] + 1.5 * bound[j]
    with pytest.raises(AssertionError, match="score error"):
        _checker(c).check(i, gpu_scores_row=bad)
    good = s64.copy()
    good[j] = s64[j] + 0.5 * bound[j]
    _checker(c).check(i, gpu_scores_row=np.concatenate([good, np.full(L - p - 1, -np.inf)]))


def test_rejects_one_ulp_on_integer_scores_and_a_finite_entry_past_the_position():
    c = _case(integer=True)
    i = 1
    s, _, _, _ = _oracle_row(c, i)
    bad = s.copy()
    bad[5] = np.nextafter(bad[5], np.float32(np.inf))
    with pytest.raises(AssertionError, match="bit-exact"):
        _checker(c, integer=True).check(i, gpu_scores_row=bad)
    bad = s.copy()
    bad[Q0 + i + 1] = 0.0
    with pytest.raises(AssertionError, match="past p"):
        _checker(c, integer=True).check(i, gpu_scores_row=bad)


def test_rejects_a_swapped_selection_and_accepts_a_near_tie():
    c = _case()
    i = 4
    p = Q0 + i
    s, sel, _, _ = _oracle_row(c, i)
    s64 = s.astype(np.float64)
    kept = set(sel.tolist())
    order = sorted(range(p + 1), key=lambda t: (-s64[t], t))
    best, worst_dropped = order[0], order[-1]
    swapped = sorted((kept - {best}) | {worst_dropped})
    with pytest.raises(AssertionError, match="beyond near-ties"):
        _checker(c).check(i, gpu_sel=np.array(swapped))
    with pytest.raises(AssertionError):
        _checker(c).check(i, gpu_sel=np.array(sorted(kept)[:-1]))  # one token short
    # the k-th and (k+1)-th scores made a near-tie: either choice is accepted
    kth, nxt = order[K - 1], order[K]
    s_tie = s64.copy()
    s_tie[nxt] = s_tie[kth] * (1 - 1e-4)
    ok, nd, _ = selection_ok(sorted((kept - {kth}) | {nxt}), sel, s_tie, p, K)
    assert ok and nd == 2
    ok, _, _ = selection_ok(sorted((kept - {kth}) | {order[K + 3]}), sel, s64, p, K)
    assert not ok


def test_integer_selection_must_be_bit_exact_even_on_ties():
    # the first seeded row with a dropped token tied with the k-th kept one
    for seed in range(100):
        c = _case(integer=True, seed=seed)
        for i in range(T):
            p = Q0 + i
            s, sel, _, _ = _oracle_row(c, i)
            s64 = s.astype(np.float64)
            kept = set(sel.tolist())
            kth = max(kept, key=lambda t: (-s64[t], t))
            tied = [t for t in range(p + 1) if t not in kept and s64[t] == s64[kth]]
            if tied:
                other = sorted((kept - {kth}) | {tied[0]})
                with pytest.raises(AssertionError, match="bit-exact"):
                    _checker(c, integer=True).check(i, gpu_sel=np.array(other))
                return
    pytest.fail("no seeded integer row has a tie at the threshold")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_output_and_lse_tolerances(dtype):
    c = _case()
    i = 3
    _, sel, out, lse = _oracle_row(c, i)
    tol = OUT_TOL[dtype]
    bad = out.copy()
    bad[1, 7] += 1.5 * tol
    with pytest.raises(AssertionError, match="output error"):
        _checker(c, dtype).check(i, gpu_sel=sel, gpu_out=bad)
    near = out.copy()
    near[1, 7] += 0.5 * tol
    _checker(c, dtype).check(i, gpu_sel=sel, gpu_out=near, gpu_lse=lse)
    with pytest.raises(AssertionError, match="lse"):
        _checker(c, dtype).check(i, gpu_sel=sel, gpu_out=out, gpu_lse=lse + 0.01)
