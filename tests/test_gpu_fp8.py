"""GPU parity of the fp8 indexer reading (dsa_quantize_fp8 and
dsa_index_scores_fp8, through the C ABI) against the CPU oracle on the same
seeded inputs: e4m3 codes, scales and folded weights bit for bit, scores
within the float32 accumulation bound of the quantised operands, and the
top-k selection on those scores (exact up to near-ties)."""
import math
import zlib

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa
from dsa_workloads import Workload, make_inputs
from oracle import round_scores_fp32, select_topk
from oracle.fp8_indexer import index_scores_fp8, quantize_rows_fp8
from tests.dsa_check import score_bound, selection_ok, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _codes(t):
    """uint8 e4m3 codes -> float64 values."""
    return t.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


CASES = [
    # name, B, T, q_pos0, n_kv, cap, HI, top_k, integer
    ("prefill_T512", 1, 512, 0, 512, 512, 32, 100, False),
    ("ragged_batch", 2, 100, 37, 150, 160, 20, 40, False),
    ("multi_tile_chunk", 1, 200, 700, 900, 900, 32, 300, False),
    ("decode_single", 4, 1, 2999, 3000, 3000, 32, 333, False),
    ("decode_multi_query", 2, 5, 495, 500, 512, 16, 64, False),
    ("integer_inputs", 1, 300, 0, 300, 300, 32, 40, True),
]


def _random_cases(n, seed):
    """Seeded random calls: decode- and prefill-shaped, ragged offsets and
    capacities, 1 to 32 heads, top_k below and past the context, integer
    inputs now and then."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 9)) if i % 2 == 0 else int(rng.integers(9, 300))
        p0 = int(rng.integers(0, 1500))
        nkv = p0 + T + int(rng.integers(0, 40))
        k = int(rng.choice([int(rng.integers(1, 100)), int(rng.integers(100, 800)), nkv + 3]))
        out.append((f"rand{i}", int(rng.integers(1, 4)), T, p0, nkv, nkv + int(rng.integers(0, 20)),
                    int(rng.integers(1, 33)), k, bool(rng.random() < 0.25)))
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(12, 2028),
                         ids=[c[0] for c in CASES] + [c[0] for c in _random_cases(12, 2028)])
def test_fp8_indexer_parity(case):
    name, B, T, p0, nkv, cap, HI, k, integer = case
    full = Workload(name=name, dtype="bf16", batch=B, n_q=p0 + T, q_pos0=0, n_kv=nkv, idx_heads=HI, idx_dim=128,
                    top_k=k, heads=4, kv_heads=4, head_dim=64, seed=zlib.crc32(name.encode()) % 1000,
                    integer_indexer=integer, qidx_std=1 / math.sqrt(128), kidx_std=1.0, w_std=1 / math.sqrt(HI))
    cpu = make_inputs(full, "cpu", kv_capacity=cap)
    qidx, w, kidx = cpu["qidx"][:, p0:].contiguous(), cpu["w"][:, p0:].contiguous(), cpu["kidx"]
    g_q, g_w, g_k = qidx.to(DEV), w.to(DEV), kidx.to(DEV)
    q8, wq = dsa.quantize_fp8(g_q, g_w)
    k8, ks = dsa.quantize_keys_fp8(g_k, pos0=0, count=nkv)
    sc = dsa.index_scores_fp8(q8, wq, k8, ks, q_pos0=p0, n_kv=nkv)
    mask, idx = dsa.topk_mask(sc, q_pos0=p0, n_kv=nkv, top_k=k)
    torch.cuda.synchronize()
    sc_np, idx_np = to_np(sc), to_np(idx)
    q8_np, k8_np = _codes(q8), _codes(k8)
    for b in range(B):
        s64, oq8, owq, ok8, oks = index_scores_fp8(to_np(qidx[b]).astype(np.float64),
                                                   to_np(w[b]), to_np(kidx[b, :nkv]).astype(np.float64), p0)
        # quantisation: bit-exact codes, scales and folded weights
        assert np.array_equal(q8_np[b], oq8)
        assert np.array_equal(k8_np[b, :nkv], ok8)
        assert np.array_equal(to_np(ks[b, :nkv]), oks)
        assert np.array_equal(to_np(wq[b]), owq)
        s32 = round_scores_fp32(s64)
        for i in range(T):
            p = p0 + i
            bound = oks[: p + 1].astype(np.float64) * score_bound(oq8[i], owq[i].astype(np.float64),
                                                                  ok8[: p + 1], 128, HI)
            err = np.abs(sc_np[b, i, : p + 1].astype(np.float64) - s64[i, : p + 1])
            assert np.all(err <= bound), f"b{b} row {i}: fp8 score error {err.max()} above bound"
            assert np.all(np.isneginf(sc_np[b, i, p + 1 :]))
            gsel = np.array(sorted(int(x) for x in idx_np[b, i] if x >= 0))
            osel = select_topk(s32[i], p, k)
            ok, nd, _ = selection_ok(gsel, osel, s64[i], p, k)
            assert ok, f"b{b} row {i}: selection differs beyond near-ties ({nd})"


@pytest.mark.parametrize("case", [("decode_100000", 2, 1, 99999, 100000, 2048),
                                  ("prefill_chunk_70000", 1, 16, 69984, 70000, 2048)],
                         ids=["decode_100000", "prefill_chunk_70000"])
def test_fp8_indexer_past_65536_tokens(case):
    """The fp8 reading on caches past 65536 tokens (decode and prefill
    kernels, the streamed top-k): codes and scales bit-exact, scores within
    the quantised-operand bound, selections exact up to near-ties."""
    name, B, T, p0, nkv, k = case
    wl = Workload(name=name, dtype="bf16", batch=B, n_q=T, q_pos0=p0, n_kv=nkv, idx_heads=32, idx_dim=128,
                  top_k=k, heads=4, kv_heads=4, head_dim=64, seed=zlib.crc32(name.encode()) % 1000,
                  qidx_std=1 / math.sqrt(128), kidx_std=1.0, w_std=1 / math.sqrt(32))
    g = make_inputs(wl, DEV)
    q8, wq = dsa.quantize_fp8(g["qidx"], g["w"])
    k8, ks = dsa.quantize_keys_fp8(g["kidx"], pos0=0, count=nkv)
    sc = dsa.index_scores_fp8(q8, wq, k8, ks, q_pos0=p0, n_kv=nkv)
    mask, idx = dsa.topk_mask(sc, q_pos0=p0, n_kv=nkv, top_k=k)
    torch.cuda.synchronize()
    sc_np, idx_np = to_np(sc), to_np(idx)
    q8_np, k8_np = _codes(q8), _codes(k8)
    for b in range(B):
        qb, wb, kb = to_np(g["qidx"][b]).astype(np.float64), to_np(g["w"][b]), to_np(g["kidx"][b, :nkv]).astype(np.float64)
        s64, oq8, owq, ok8, oks = index_scores_fp8(qb, wb, kb, p0)
        assert np.array_equal(q8_np[b], oq8)
        assert np.array_equal(k8_np[b, :nkv], ok8)
        assert np.array_equal(to_np(ks[b, :nkv]), oks)
        assert np.array_equal(to_np(wq[b]), owq)
        s32 = round_scores_fp32(s64)
        for i in range(T):
            p = p0 + i
            bound = oks[: p + 1].astype(np.float64) * score_bound(oq8[i], owq[i].astype(np.float64),
                                                                  ok8[: p + 1], 128, 32)
            err = np.abs(sc_np[b, i, : p + 1].astype(np.float64) - s64[i, : p + 1])
            assert np.all(err <= bound), f"b{b} row {i}: fp8 score error {err.max()} above bound"
            assert np.all(np.isneginf(sc_np[b, i, p + 1 :]))
            gsel = np.array(sorted(int(x) for x in idx_np[b, i] if x >= 0))
            osel = select_topk(s32[i], p, k)
            ok, nd, _ = selection_ok(gsel, osel, s64[i], p, k)
            assert ok, f"b{b} row {i}: selection differs beyond near-ties ({nd})"


def test_fp8_indexer_prefill_L4096_sampled_rows():
    """Full-size prefill workload (the shape the bench's fp8 study runs): all
    rows scored and selected on the GPU, sampled rows checked against the
    oracle."""
    from dsa_workloads import WORKLOADS, sample_rows
    wl = WORKLOADS["prefill_bf16_L4096"]
    cpu = make_inputs(wl, "cpu")
    g_q, g_w, g_k = cpu["qidx"].to(DEV), cpu["w"].to(DEV), cpu["kidx"].to(DEV)
    q8, wq = dsa.quantize_fp8(g_q, g_w)
    k8, ks = dsa.quantize_keys_fp8(g_k)
    sc = dsa.index_scores_fp8(q8, wq, k8, ks, q_pos0=0, n_kv=wl.n_kv)
    _, idx = dsa.topk_mask(sc, q_pos0=0, n_kv=wl.n_kv, top_k=wl.top_k)
    torch.cuda.synchronize()
    sc_np, idx_np = to_np(sc[0]), to_np(idx[0])
    q64, w32, k64 = to_np(cpu["qidx"][0]).astype(np.float64), to_np(cpu["w"][0]), to_np(cpu["kidx"][0]).astype(np.float64)
    assert np.array_equal(_codes(k8[0]), quantize_rows_fp8(k64)[0])
    for i in sample_rows(wl, 48, seed=7):
        s64, oq8, owq, ok8, oks = index_scores_fp8(q64[i : i + 1], w32[i : i + 1], k64, i)
        bound = oks[: i + 1].astype(np.float64) * score_bound(oq8[0], owq[0].astype(np.float64), ok8[: i + 1],
                                                                128, wl.idx_heads)
        err = np.abs(sc_np[i, : i + 1].astype(np.float64) - s64[0, : i + 1])
        assert np.all(err <= bound), f"row {i}: fp8 score error {err.max()} above bound"
        gsel = np.array(sorted(int(x) for x in idx_np[i] if x >= 0))
        ok, nd, _ = selection_ok(gsel, select_topk(round_scores_fp32(s64)[0], i, wl.top_k), s64[0], i, wl.top_k)
        assert ok, f"row {i}: selection differs beyond near-ties ({nd})"
