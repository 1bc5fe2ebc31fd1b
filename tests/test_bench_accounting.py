"""The algorithmic work bench.py divides by (the numerator of every roofline
fraction it reports), checked against brute-force counts and closed forms.

Indexer: 2 * 32 * 128 flops for every (query, earlier token) pair, since every
earlier token is scored [aiaulis para 2]. Attention: 4 * 32 * 128 flops for
every (query, kept token) pair, with min(p + 1, top_k) kept tokens per query
[aiaulis paras 2-4; devotd section 1 table, 2048 tokens]. Decode is priced in
bytes: the index keys read once, the kept K/V rows gathered once.
"""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


bench = _bench()
from dsa_workloads import WORKLOADS  # noqa: E402


class _Wl:
    def __init__(self, top_k):
        self.top_k = top_k


@pytest.mark.parametrize("q_pos0,n_q,top_k", [(0, 1, 1), (0, 7, 3), (0, 300, 37), (5, 40, 2), (100, 50, 120),
                                              (100, 50, 160), (100, 50, 10_000), (1000, 1, 2048), (0, 4096, 2048),
                                              (4096, 4096, 2048), (2000, 100, 2048)])
def test_pair_counts_match_brute_force(q_pos0, n_q, top_k):
    causal = sum(p + 1 for p in range(q_pos0, q_pos0 + n_q))
    kept = sum(min(p + 1, top_k) for p in range(q_pos0, q_pos0 + n_q))
    assert bench.causal_pairs(_Wl(top_k), q_pos0, n_q) == causal
    assert bench.selected_pairs(_Wl(top_k), q_pos0, n_q) == kept


def _step_work(wl):
    tot = {}
    for q_pos0, n_q, n_kv in bench.chunk_calls(wl):
        res, _, _ = bench.op_work(wl, q_pos0, n_q, n_kv)
        for op, r in res.items():
            tot[op] = tot.get(op, 0) + r["work"]
    return tot


def test_prefill_4096_layer_work():
    w = _step_work(WORKLOADS["prefill_bf16_L4096"])
    # sum_{p<4096} (p + 1) pairs; rows p >= 2047 keep 2048 tokens, the others p + 1
    assert w["index_scores"] == 4096 * 4097 // 2 * (2 * 32 * 128) == 68_736_253_952
    kept = 2048 * 2049 // 2 + (4096 - 2048) * 2048
    assert w["sparse_attention"] == kept * (4 * 32 * 128) == 103_095_992_320


def test_chunked_65536_layer_work():
    for name in ("longctx_bf16_L65536_chunk4096", "longctx_mqa_bf16_L65536_chunk4096",
                 "longctx_kvshared_bf16_L65536_chunk4096"):
        wl = WORKLOADS[name]
        calls = bench.chunk_calls(wl)
        # the 16 calls cover positions 0 .. 65535 once, each seeing the cache up to its last query
        assert [c[0] for c in calls] == list(range(0, 65536, 4096))
        assert all(n_q == 4096 and n_kv == q_pos0 + n_q for q_pos0, n_q, n_kv in calls)
        w = _step_work(wl)
        assert w["index_scores"] == 65536 * 65537 // 2 * 8192 == 17_592_454_479_872
        kept = 2048 * 2049 // 2 + (65536 - 2048) * 2048
        assert w["sparse_attention"] == kept * 16384 == 2_164_680_294_400
        # matrix work of the whole layer, 19.76 TFLOP
        assert abs(w["index_scores"] + w["sparse_attention"] - 19.757e12) < 0.01e12


def test_decode_step_bytes():
    wl = WORKLOADS["decode_bf16_B64_L32768"]
    w = _step_work(wl)
    B, L = 64, 32768
    kidx = B * L * 128 * 2                          # every index key read once
    qw = B * (32 * 128 * 2 + 32 * 4)                # index queries and head weights
    scores_out = B * L * 4                          # one float score per cached token
    assert w["index_scores"] == kidx + qw + scores_out == 545_792_000
    gather = B * 2048 * 2 * 32 * 128 * 2            # K and V rows of the 2048 kept tokens, all heads
    q_and_out = 2 * B * 32 * 128 * 2
    mask_in = B * L // 8
    assert w["sparse_attention"] == gather + q_and_out + mask_in == 2_148_794_368
    # scores read once, mask and index list written
    assert w["topk_mask"] == B * L * 4 + B * L // 8 + B * 2048 * 4
    # the whole step: 2.70e9 bytes, 0.338 ms at 8 TB/s
    total = sum(w.values())
    assert abs(total - 2.7038e9) < 0.001e9


def test_every_op_names_its_bound_and_peak():
    for name, wl in WORKLOADS.items():
        for q_pos0, n_q, n_kv in bench.chunk_calls(wl):
            res, pc, ps = bench.op_work(wl, q_pos0, n_q, n_kv)
            assert set(res) == {"index_scores", "topk_mask", "sparse_attention"}, name
            assert 0 < ps <= pc, name
            for op, r in res.items():
                assert r["work"] > 0, (name, op)
                assert (r["bound"], r["unit"]) in {("mfma", "TFLOP/s"), ("hbm", "GB/s")}, (name, op)
                if r["bound"] == "hbm":
                    assert r["peak"] == 8000.0
                else:
                    assert r["peak"] == (2500.0 if wl.dtype == "bf16" else 157.3), (name, op)


def test_secondary_step_counts_stay_bounded():
    for name in bench.SECONDARY:
        wl = WORKLOADS[name]
        steps = bench.secondary_steps_for(wl)
        assert 3 <= steps <= 2000, name
        if wl.chunks > 1:
            assert steps <= 10, name  # tens of ms per step: a few steps fill ~100 ms
