"""GPU parity of the indexer front end (dsa_indexer_project, through the C
ABI) against the CPU oracle on the same seeded inputs: every output element,
at the workload sizes and on ragged edge cases, plus the cache rows the call
must leave untouched.

Tolerance (derived from the arithmetic): the kernels sum the K exact bf16
products in float32 in some order, so |y32 - y| <= E = gamma_K * sum_k |a_k w_k|
with gamma_K = K u / (1 - K u), u = 2^-24. w is that float32 value. qidx and
kidx are then rounded to bf16 (unit roundoff 2^-8), so
|bf16(y32) - y| <= 2^-8 (|y| + E) + E."""
import math

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa
from dsa_workloads import FRONT_END_WORKLOADS, FrontEndWorkload, make_front_end_inputs
from oracle import indexer_front_end
from tests.dsa_check import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _gamma(K):
    u = 2.0 ** -24
    return K * u / (1 - K * u)


def _check_close(name, got, exact, absum, K, rounded_bf16):
    E = _gamma(K) * absum
    bound = (2.0 ** -8 * (np.abs(exact) + E) + E) if rounded_bf16 else E
    err = np.abs(got.astype(np.float64) - exact)
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements above the bound, worst err "
                           f"{err[bad].max()} at bound {bound[bad][np.argmax(err[bad])]}")
    return float(np.max(err / np.maximum(bound, 1e-300)))


def _run_and_check(wl, kv_capacity=None):
    cpu = make_front_end_inputs(wl, "cpu", kv_capacity)
    g = {k: v.to(DEV) for k, v in cpu.items()}
    before = g["kidx_cache"].clone()
    qidx, w = dsa.indexer_project(g["x"], g["q_lat"], g["w_qb"], g["w_k"], g["w_proj"], g["kidx_cache"],
                                  q_pos0=wl.q_pos0)
    torch.cuda.synchronize()
    qidx_np, w_np, cache_np = to_np(qidx), to_np(w), to_np(g["kidx_cache"])
    f64 = lambda t: to_np(t).astype(np.float64)
    wqb, wk, wp = f64(cpu["w_qb"]), f64(cpu["w_k"]), f64(cpu["w_proj"])
    HI, DI, T = wl.idx_heads, wl.idx_dim, wl.n_q
    worst = 0.0
    for b in range(wl.batch):
        x, ql = f64(cpu["x"][b]), f64(cpu["q_lat"][b])
        eq, ek, ew = indexer_front_end(x, ql, wqb, wk, wp, HI, DI)
        aq = (np.abs(ql) @ np.abs(wqb).T).reshape(T, HI, DI)
        ak, aw = np.abs(x) @ np.abs(wk).T, np.abs(x) @ np.abs(wp).T
        worst = max(worst, _check_close("qidx", qidx_np[b], eq, aq, wl.q_rank, True))
        worst = max(worst, _check_close("kidx", cache_np[b, wl.q_pos0 : wl.q_pos0 + T], ek, ak, wl.hidden, True))
        worst = max(worst, _check_close("w", w_np[b], ew, aw, wl.hidden, False))
    # rows outside q_pos0 .. q_pos0+T-1 are untouched
    keep = torch.ones(g["kidx_cache"].shape[1], dtype=torch.bool, device=DEV)
    keep[wl.q_pos0 : wl.q_pos0 + T] = False
    assert torch.equal(g["kidx_cache"][:, keep], before[:, keep])
    return qidx, w, g, worst


def test_front_end_prefill_T4096_all_elements():
    wl = FRONT_END_WORKLOADS["front_end_prefill_T4096"]
    qidx, w, g, worst = _run_and_check(wl)
    print(f"worst error / bound {worst:.3g}", flush=True)
    # deterministic: a second call gives identical bits
    q2, w2 = dsa.indexer_project(g["x"], g["q_lat"], g["w_qb"], g["w_k"], g["w_proj"], g["kidx_cache"])
    torch.cuda.synchronize()
    assert torch.equal(q2, qidx) and torch.equal(w2, w)


def test_front_end_decode_B64_all_elements():
    # the workload's 32768-row caches cut to 48 rows; the token goes to row 37
    wl = FRONT_END_WORKLOADS["front_end_decode_B64"]
    wl = FrontEndWorkload(**{**wl.__dict__, "q_pos0": 37, "kv_capacity": 48})
    _run_and_check(wl)


EDGE = [
    # name, B, T, q_pos0, cap, hidden, q_rank, HI, DI
    ("ragged_small_heads", 3, 45, 10, 60, 192, 128, 5, 32),
    ("wide_ragged_tokens", 1, 1100, 3, 1103, 256, 192, 32, 128),
    ("min_widths", 2, 7, 0, 7, 64, 64, 1, 32),
    ("idx_dim64_full_heads", 2, 130, 70, 200, 320, 256, 32, 64),
    ("wide_multi_batch", 2, 1024, 0, 1024, 128, 512, 16, 64),
    # few tokens over deep K: both products split K into float32 partials
    ("split_k_ragged", 2, 45, 5, 50, 2048, 1024, 7, 64),
]


@pytest.mark.parametrize("e", EDGE, ids=[e[0] for e in EDGE])
def test_front_end_edge_cases(e):
    name, B, T, p0, cap, hid, r, HI, DI = e
    wl = FrontEndWorkload(name, B, T, p0, cap, hid, r, HI, DI, seed=sum(map(ord, name)) % 997)
    _run_and_check(wl)


def _random_front_end(n, seed):
    """Seeded random shapes: decode-sized to 1200 tokens, ragged offsets and
    capacities, widths from 64 to 2560 (deep K takes the split path)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([int(rng.integers(1, 9)), int(rng.integers(9, 200)), int(rng.integers(200, 1200))]))
        p0 = int(rng.integers(0, 100))
        out.append((f"rand{i}", int(rng.integers(1, 4)), T, p0, p0 + T + int(rng.integers(0, 20)),
                    64 * int(rng.integers(1, 41)), 64 * int(rng.integers(1, 25)), int(rng.integers(1, 33)),
                    int(rng.choice([32, 64, 128]))))
    return out


RANDOM = _random_front_end(16, 2027)


@pytest.mark.parametrize("e", RANDOM, ids=[e[0] for e in RANDOM])
def test_front_end_random_shapes(e):
    name, B, T, p0, cap, hid, r, HI, DI = e
    wl = FrontEndWorkload(name, B, T, p0, cap, hid, r, HI, DI, seed=sum(map(ord, name)) % 997)
    _run_and_check(wl)
