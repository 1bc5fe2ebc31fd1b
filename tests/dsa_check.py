"""Comparators between the HIP path and the CPU oracle (test helpers).

Tolerances:
  * Scores: float32 accumulation of exact products. For a sum of n terms the
    rounding error is at most gamma_n * sum|terms| with gamma_n = n u / (1 - n u),
    u = 2^-24. A score sums D_I products per head, then H_I weighted ReLUs, so
    |gpu - exact| <= 2 * gamma_{D_I + H_I + 2} * sum_h |w_h| sum_d |q_hd k_d|
    (factor 2 for margin). On integer inputs every partial sum is an integer
    below 2^24, so scores must be bit-exact.
  * Selection: identical sets, except that a token in the symmetric difference
    may differ when its float64 score is within 1e-3 relative of the oracle's
    k-th score (relative to max(|I_k|, 2^-7 * rms(row)), the floor covering
    thresholds near zero).
  * Attention output: max abs error 2e-2 for bf16 I/O, 1e-4 for fp32 I/O,
    against the oracle's attention over the GPU's own kept set (equal to the
    oracle's set wherever the sets agree).
  * Log-sum-exp: with bf16 I/O the kernels sum the probabilities as they
    enter P V, rounded to bf16 (relative error <= 2^-9 each), so the sum is
    within a factor (1 +- 2^-9) of the exact one and |lse error| <=
    -log(1 - 2^-9) < 1.96e-3; the tolerance is 2.5e-3 absolute. fp32 I/O
    keeps float32 probabilities: 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import attend_selected, index_scores, round_scores_fp32, select_topk

U32 = 2.0 ** -24
OUT_TOL = {"bf16": 2e-2, "fp32": 1e-4}
LSE_ATOL = {"bf16": 2.5e-3, "fp32": 1e-3}


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def score_bound(q_row64, w_row64, kidx64, di, hi):
    """Per-candidate error bound of a float32 score (see module doc)."""
    n = di + hi + 2
    gamma = n * U32 / (1 - n * U32)
    mag = np.abs(w_row64) @ (np.abs(q_row64) @ np.abs(kidx64).T)  # [L]
    return 2.0 * gamma * mag


def selection_ok(gpu_sel, ora_sel, s64, p, k, rel=1e-3):
    """Returns (ok, n_diff, n_floor_only)."""
    gs, os_ = set(int(x) for x in gpu_sel), set(int(x) for x in ora_sel)
    if len(gs) != min(k, p + 1) or any(x > p or x < 0 for x in gs):
        return False, -1, 0
    diff = gs ^ os_
    if not diff:
        return True, 0, 0
    ora_sorted = sorted(os_, key=lambda s: (-s64[s], s))
    ik = s64[ora_sorted[-1]]
    rms = float(np.sqrt(np.mean(s64[: p + 1] ** 2)))
    floor = 2.0 ** -7 * rms
    tol = rel * max(abs(ik), floor)
    floor_only = 0
    for s in diff:
        gap = abs(s64[s] - ik)
        if gap > tol:
            return False, len(diff), floor_only
        if gap > rel * abs(ik):
            floor_only += 1
    return True, len(diff), floor_only


class RowChecker:
    """Checks GPU results of chosen query rows of one sequence against the
    oracle, row by row."""

    def __init__(self, dtype, qidx, w, kidx, q, kc, vc, q_pos0, top_k, scale, integer=False):
        self.dtype = dtype
        self.qidx, self.w, self.kidx = qidx, w, kidx  # float64 numpy, one sequence
        self.q, self.kc, self.vc = q, kc, vc          # kc / vc may be callables: idx -> rows
        self.q_pos0, self.top_k, self.scale = q_pos0, top_k, scale
        self.integer = integer
        self.stats = {"rows": 0, "sel_diff_rows": 0, "sel_diff_tokens": 0, "floor_only": 0,
                      "max_out_err": 0.0, "max_score_err_over_bound": 0.0}

    def _rows(self, cache, sel):
        return cache(sel) if callable(cache) else cache[sel]

    def check(self, i, gpu_scores_row=None, gpu_sel=None, gpu_out=None, gpu_lse=None):
        p = self.q_pos0 + i
        di, hi = self.qidx.shape[2], self.qidx.shape[1]
        s64 = index_scores(self.qidx[i : i + 1], self.w[i : i + 1], self.kidx[: p + 1], p)[0]
        s32 = round_scores_fp32(s64)
        ora_sel = select_topk(s32, p, self.top_k)
        if gpu_scores_row is not None:
            g = gpu_scores_row[: p + 1].astype(np.float64)
            if self.integer:
                assert np.array_equal(g, s64[: p + 1]), f"row {i}: integer scores not bit-exact"
            else:
                bound = score_bound(self.qidx[i], self.w[i], self.kidx[: p + 1], di, hi)
                err = np.abs(g - s64[: p + 1])
                ratio = float(np.max(err / np.maximum(bound, 1e-300)))
                self.stats["max_score_err_over_bound"] = max(self.stats["max_score_err_over_bound"], ratio)
                assert np.all(err <= bound), f"row {i}: score error {err.max()} above bound"
            assert np.all(np.isneginf(gpu_scores_row[p + 1 :])), f"row {i}: entries past p not -inf"
        sel_for_out = ora_sel
        if gpu_sel is not None:
            gsel = np.array(sorted(int(x) for x in gpu_sel if x >= 0), dtype=np.int64)
            if self.integer:
                assert np.array_equal(gsel, ora_sel), f"row {i}: integer selection not bit-exact"
            else:
                ok, nd, fo = selection_ok(gsel, ora_sel, s64, p, self.top_k)
                assert ok, f"row {i}: selection differs beyond near-ties ({nd} tokens)"
                if nd:
                    self.stats["sel_diff_rows"] += 1
                    self.stats["sel_diff_tokens"] += nd
                    self.stats["floor_only"] += fo
            sel_for_out = gsel
        if gpu_out is not None:
            O, lse = attend_selected(self.q[i], self._rows(self.kc, sel_for_out),
                                     self._rows(self.vc, sel_for_out),
                                     np.arange(len(sel_for_out)), self.scale)
            err = float(np.max(np.abs(gpu_out.astype(np.float64) - O)))
            self.stats["max_out_err"] = max(self.stats["max_out_err"], err)
            assert err <= OUT_TOL[self.dtype], f"row {i}: output error {err}"
            if gpu_lse is not None:
                assert np.allclose(gpu_lse, lse, rtol=1e-4, atol=LSE_ATOL[self.dtype]), f"row {i}: lse mismatch"
        self.stats["rows"] += 1
        return ora_sel
