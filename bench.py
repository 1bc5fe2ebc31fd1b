#!/usr/bin/env python3
"""Throughput of one DSA layer (lightning indexer -> top-k mask -> sparse
attention) on one MI355X, with the roofline fraction of its dominant kernel
and the CPU oracle timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole layer call (dsa_forward: indexer scores, top-k bitmask
plus index list, attention over the kept keys) over one batch of synthetic
input that is resident in HBM before the timed region starts. The headline
workload is single-layer prefill of one 4096-token sequence (32x128
indexer, top_k 2048, 32x128 attention); the batched decode step (64
sequences x 32768 cached tokens) and the chunked 65536-token prefill are
measured in the same run and reported under "secondary". Each query is one
token, so queries/s equals tokens/s. The indexer front end (the q_b, k and
projection products that produce the indexer's inputs) is timed on its own
prefill and decode shapes and reported under "front_end".

Per-kernel times come from HIP events recorded on the stream the kernels run
on, around the op-level entry points (dsa_index_scores, dsa_topk_mask,
dsa_sparse_attention), each of which launches the kernel it is named for.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA layer queries/sec (prefill & decode) + % of MFMA / HBM roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X fp32
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

HEADLINE = "prefill_bf16_L4096"
SECONDARY = ["decode_bf16_B64_L32768", "longctx_bf16_L65536_chunk4096", "longctx_mqa_bf16_L65536_chunk4096",
             "longctx_kvshared_bf16_L65536_chunk4096", "tiny_fp32_L256", "equiv_bf16_L1536_k2048",
             "ties_bf16_L1536_k512"]
# secondary workloads whose oracle is also timed on the host, and how many rows
CPU_BASELINE_ROWS = {"decode_bf16_B64_L32768": 64, "longctx_bf16_L65536_chunk4096": 512}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    # The GPU reaches its steady clocks only after tens of milliseconds of
    # back-to-back work: a 6 ms timed region after a 1.5 ms warmup measured
    # this step 17% slower than the steady state. The defaults time about
    # 50 ms of headline steps after about 25 ms of warmup.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--secondary", default=",".join(SECONDARY),
                    help="comma-separated workloads also measured ('' for none)")
    ap.add_argument("--secondary-steps", type=int, default=0,
                    help="steps timed per secondary workload (0 = enough for about 100 ms, "
                         "at least 3, after as many warmup steps)")
    ap.add_argument("--fp8-study", default=f"{HEADLINE},longctx_bf16_L65536_chunk4096",
                    help="workloads on which the fp8 indexer reading is timed and its selection "
                         "compared with bf16 ('' for none)")
    ap.add_argument("--stream-study", default="longctx_mqa_bf16_L65536_chunk4096",
                    help="workloads on which the streamed selection (dsa_forward_stream_select) is timed "
                         "beside the materialised one ('' for none)")
    ap.add_argument("--front-end-steps", type=int, default=20,
                    help="calls timed per indexer front-end workload (0 = skip)")
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="steps timed after a 512 MiB cache-evicting write each (median reported; 0 = skip)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="op-level calls of each workload run back to back for this long before its "
                         "timed reps and steps, so that they run at steady clocks")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle timing on the host (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB read + 1 GiB write kernel (reference for HBM counters)")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    return ap.parse_args()


# ----------------------------------------------------------------------------- work accounting

def causal_pairs(wl, q_pos0, n_q):
    """sum over queries of (p + 1), the indexer's candidate pairs."""
    p0 = q_pos0 + 1
    return n_q * p0 + n_q * (n_q - 1) // 2


def selected_pairs(wl, q_pos0, n_q):
    """sum over queries of min(p + 1, top_k): the (query, kept key) pairs."""
    tot = 0
    k = wl.top_k
    # rows with p + 1 <= k keep p + 1 keys, the rest keep k
    last_small = min(q_pos0 + n_q, k) - 1  # largest p with p + 1 <= k
    if last_small >= q_pos0:
        n_small = last_small - q_pos0 + 1
        tot += causal_pairs(wl, q_pos0, n_small)
        tot += (n_q - n_small) * k
    else:
        tot += n_q * k
    return tot


def chunk_calls(wl):
    """(q_pos0, n_q, n_kv) of each layer call of one step."""
    if wl.chunks == 1:
        return [(wl.q_pos0, wl.n_q, wl.n_kv)]
    C = wl.chunk_len
    return [(c * C, C, (c + 1) * C) for c in range(wl.chunks)]


def op_work(wl, q_pos0, n_q, n_kv):
    """Algorithmic work of each op for one call: the quantity its roofline
    counts (flops for matrix-core work, bytes for bandwidth-bound work)."""
    B, es = wl.batch, (2 if wl.dtype == "bf16" else 4)
    HI, DI, H, Hkv, D = wl.idx_heads, wl.idx_dim, wl.heads, wl.kv_heads, wl.head_dim
    lpad = (n_kv + 63) // 64 * 64
    pc = B * causal_pairs(wl, q_pos0, n_q)
    ps = B * selected_pairs(wl, q_pos0, n_q)
    decode = n_q <= 8
    peak_mfma = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    res = {}
    # indexer: 2*HI*DI flops per causal pair; decode reads each cached index key once
    idx_bytes = B * n_kv * DI * es + B * n_q * (HI * DI * es + HI * 4) + B * n_q * lpad * 4
    if decode:
        res["index_scores"] = dict(bound="hbm", work=idx_bytes, unit="GB/s", peak=PEAK_HBM_GBS)
    else:
        res["index_scores"] = dict(bound="mfma", work=2.0 * HI * DI * pc, unit="TFLOP/s", peak=peak_mfma)
    # top-k: reads every candidate score once, writes the mask and the index list
    topk_bytes = 4 * pc + B * n_q * (lpad // 8) + B * n_q * wl.top_k * 4
    res["topk_mask"] = dict(bound="hbm", work=topk_bytes, unit="GB/s", peak=PEAK_HBM_GBS)
    # attention: 4*H*D flops per selected pair; decode gathers the kept K/V rows
    if decode:
        attn_bytes = ps * 2 * Hkv * D * es + 2 * B * n_q * H * D * es + B * n_q * (lpad // 8)
        res["sparse_attention"] = dict(bound="hbm", work=attn_bytes, unit="GB/s", peak=PEAK_HBM_GBS)
    else:
        res["sparse_attention"] = dict(bound="mfma", work=4.0 * H * D * ps, unit="TFLOP/s", peak=peak_mfma)
    return res, pc, ps


# ----------------------------------------------------------------------------- GPU timing

def run_gpu(wl, steps, warmup, torch, dsa, make_inputs, cold_reps=5, settle_ms=200.0):
    dev = torch.device("cuda:0")
    log(f"[bench] {wl.name}: drawing inputs on the GPU")
    g = make_inputs(wl, dev)
    torch.cuda.synchronize()
    calls = chunk_calls(wl)
    B, H, D = wl.batch, wl.heads, wl.head_dim
    out = torch.empty_like(g["q"])
    idx = torch.empty((B, wl.n_q, wl.top_k), dtype=torch.int32, device=dev)
    # one workspace sized for the largest call
    big = calls[-1]
    dims = dsa.make_dims(batch=B, n_q=big[1], q_pos0=big[0], n_kv=big[2], kv_capacity=g["k"].shape[1],
                         idx_heads=wl.idx_heads, idx_dim=wl.idx_dim, top_k=wl.top_k, heads=H,
                         kv_heads=wl.kv_heads, head_dim=D, scale=wl.scale,
                         dtype=dsa.DSA_BF16 if wl.dtype == "bf16" else dsa.DSA_FP32)
    ws_bytes = max(dsa.workspace_size(dims, dsa.DSA_OP_FORWARD),
                   dsa.workspace_size(dims, dsa.DSA_OP_SPARSE_ATTENTION), 256)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def views(q0, nq):
        sl = slice(q0 - wl.q_pos0, q0 - wl.q_pos0 + nq)
        return (g["qidx"][:, sl], g["w"][:, sl], g["q"][:, sl], out[:, sl], idx[:, sl])

    call_views = [views(q0, nq) for (q0, nq, _) in calls]

    def step():
        for (q0, nq, nkv), (qi, wi, qq, oo, ii) in zip(calls, call_views):
            dsa.forward(qi, wi, g["kidx"], qq, g["k"], g["v"], top_k=wl.top_k, q_pos0=q0, n_kv=nkv,
                        scale=wl.scale, workspace=ws, out=oo, indices=ii)

    stream = torch.cuda.current_stream(dev)
    # Per-op times: the same calls through the op-level entry points, HIP
    # events on the stream they are launched on. Every rep is enqueued before
    # any event is read, so the GPU runs the ops back to back and the event
    # pairs measure device time, not host launch gaps.
    Lmax = (big[2] + 63) // 64 * 64
    scores = torch.empty((B, big[1], Lmax), dtype=torch.float32, device=dev)
    mask = torch.empty((B, big[1], Lmax // 32), dtype=torch.int32, device=dev)

    def op_level(q0, nq, nkv, qi, wi, qq, oo, ii, ev):
        lp = (nkv + 63) // 64 * 64
        sc = scores[:, :nq, :lp] if (nq, lp) != (big[1], Lmax) else scores
        mk = mask[:, :nq, : lp // 32] if (nq, lp) != (big[1], Lmax) else mask
        if not sc.is_contiguous():
            sc = torch.empty((B, nq, lp), dtype=torch.float32, device=dev)
            mk = torch.empty((B, nq, lp // 32), dtype=torch.int32, device=dev)
        if ev:
            ev[0].record(stream)
        dsa.index_scores(qi, wi, g["kidx"], q_pos0=q0, n_kv=nkv, out=sc)
        if ev:
            ev[1].record(stream)
        mk2, _ = dsa.topk_mask(sc, q_pos0=q0, n_kv=nkv, top_k=wl.top_k, indices=True, mask_out=mk, indices_out=ii)
        if ev:
            ev[2].record(stream)
        dsa.sparse_attention(qq, g["k"], g["v"], mk2, q_pos0=q0, n_kv=nkv, scale=wl.scale, workspace=ws, out=oo)
        if ev:
            ev[3].record(stream)
    op_ms = {"index_scores": 0.0, "topk_mask": 0.0, "sparse_attention": 0.0}
    op_work_tot = {}
    n_rep = max(1, min(steps, 10))
    pending = []
    # Before any timed rep, the op-level calls run back to back for
    # settle_ms: after an idle spell the GPU needs tens of milliseconds of
    # work to come back to its steady clocks (a 5-step warmup followed by
    # 20 timed steps, right after 0.5 s of idle, measured the 4096-token
    # layer 24% slower than the same steps at steady clocks).
    settle_reps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for (q0, nq, nkv), (qi, wi, qq, oo, ii) in zip(calls, call_views):
            op_level(q0, nq, nkv, qi, wi, qq, oo, ii, None)
        settle_reps += 1
        if settle_reps % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle_wall_ms = (time.perf_counter() - t_settle) * 1e3
    for rep in range(n_rep + 1):  # rep 0 warms up
        for (q0, nq, nkv), (qi, wi, qq, oo, ii) in zip(calls, call_views):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            op_level(q0, nq, nkv, qi, wi, qq, oo, ii, ev)
            if rep > 0:
                pending.append(ev)
                w_, _, _ = op_work(wl, q0, nq, nkv)
                for name, info in w_.items():
                    op_work_tot.setdefault(name, dict(info, work=0.0))
                    op_work_tot[name]["work"] += info["work"] / n_rep
    torch.cuda.synchronize()
    for ev in pending:
        for j, name in enumerate(("index_scores", "topk_mask", "sparse_attention")):
            op_ms[name] += ev[j].elapsed_time(ev[j + 1]) / n_rep

    # The timed steps: W warmup steps, then exactly K steps between two
    # synchronisations (wall clock).
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / steps

    # Cold steps: before each, a 512 MiB scratch write (twice the last-level
    # cache) on the same stream evicts the caches; HIP events bracket the step.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cold_reps > 0 else None
    cold_ms = []
    for r in range(cold_reps):
        scratch.fill_(r + 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold_ms.append(e0.elapsed_time(e1))
    del scratch
    cold = None
    if cold_ms:
        cold_ms.sort()
        med = cold_ms[len(cold_ms) // 2]
        cold = {"ms_per_step": round(med, 4), "value": wl.batch * wl.n_q / (med * 1e-3), "reps": len(cold_ms),
                "flush": "512 MiB scratch write before each step"}

    kernels = []
    for name, ms in op_ms.items():
        info = op_work_tot[name]
        scale = 1e-9 if info["unit"] == "GB/s" else 1e-12
        achieved = info["work"] * scale / (ms * 1e-3)
        kernels.append({"op": name, "ms_per_step": round(ms, 4), "bound": info["bound"],
                        "achieved": round(achieved, 2), "peak": info["peak"], "unit": info["unit"],
                        "frac": round(achieved / info["peak"], 4),
                        "work_per_step": info["work"],
                        "work_unit": "bytes" if info["unit"] == "GB/s" else "flop"})
    dominant = max(kernels, key=lambda k: k["ms_per_step"])
    queries = wl.batch * wl.n_q
    del g, out, idx, ws, scores, mask
    torch.cuda.empty_cache()
    return {
        "workload": wl.name,
        "queries_per_step": queries,
        "ms_per_step": ms_per_step,
        "value": queries / (ms_per_step * 1e-3),
        "kernels": kernels,
        "dominant": dominant,
        "calls_per_step": len(calls),
        "cold": cold,
        "settle_ms": round(settle_wall_ms, 1),
    }


def secondary_steps_for(wl):
    """Steps (and as many warmup steps) that fill about 100 ms for a
    secondary workload, from its algorithmic work at a nominal rate:
    chunked long-context steps take tens of ms, a decode step half of one,
    the small (<= 2048-token) configurations tens of microseconds."""
    est_ms = 25.0 if wl.chunks > 1 else (0.05 if wl.n_kv <= 2048 else 0.5)
    return int(min(2000, max(3, round(100.0 / est_ms))))


def front_end_work(fw):
    """Algorithmic flops and HBM bytes of one indexer front-end call: the
    three products, and every operand read once and every result written
    once (weights and activations bf16, w float32)."""
    M = fw.batch * fw.n_q
    HI, DI = fw.idx_heads, fw.idx_dim
    flops = 2.0 * M * (HI * DI * fw.q_rank + (DI + HI) * fw.hidden)
    weights = 2.0 * (HI * DI * fw.q_rank + (DI + HI) * fw.hidden)
    acts = 2.0 * M * (fw.hidden + fw.q_rank)
    outs = M * (2.0 * HI * DI + 2.0 * DI + 4.0 * HI)
    return flops, weights + acts + outs


def run_front_end(fw, steps, torch, dsa, make_front_end_inputs):
    """Times dsa_indexer_project on one front-end workload (HIP events on
    the stream it runs on; every rep enqueued before the events are read)."""
    dev = torch.device("cuda:0")
    g = make_front_end_inputs(fw, dev)
    d = dsa.make_proj_dims(batch=fw.batch, n_q=fw.n_q, q_pos0=fw.q_pos0, kv_capacity=fw.kv_capacity,
                           hidden=fw.hidden, q_rank=fw.q_rank, idx_heads=fw.idx_heads, idx_dim=fw.idx_dim)
    ws = torch.empty(max(dsa.proj_workspace_size(d), 256), dtype=torch.uint8, device=dev)
    qo = torch.empty((fw.batch, fw.n_q, fw.idx_heads, fw.idx_dim), dtype=torch.bfloat16, device=dev)
    wo = torch.empty((fw.batch, fw.n_q, fw.idx_heads), dtype=torch.float32, device=dev)

    def call():
        dsa.indexer_project(g["x"], g["q_lat"], g["w_qb"], g["w_k"], g["w_proj"], g["kidx_cache"],
                            q_pos0=fw.q_pos0, workspace=ws, qidx_out=qo, w_out=wo)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops, nbytes = front_end_work(fw)
    M = fw.batch * fw.n_q
    tflops, gbs = flops / (ms * 1e-3) / 1e12, nbytes / (ms * 1e-3) / 1e9
    # the bound is whichever roofline time is longer
    mfma_bound = flops / (PEAK_BF16_TFLOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9)
    roof = ({"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(tflops / PEAK_BF16_TFLOPS, 4)} if mfma_bound else
            {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(gbs / PEAK_HBM_GBS, 4)})
    del g, ws, qo, wo
    torch.cuda.empty_cache()
    return {"workload": fw.name, "ms_per_call": round(ms, 5), "tokens_per_s": M / (ms * 1e-3),
            "flop_per_call": flops, "bytes_per_call": nbytes, "roofline": roof,
            "kernel": "proj_gemm_kernel (+ proj_reduce_kernel for K-split products)"}


def _popcount32(x, torch):
    """Set bits per int32 word (as int64)."""
    v = x.to(torch.int64) & 0xFFFFFFFF
    v = v - ((v >> 1) & 0x55555555)
    v = (v & 0x33333333) + ((v >> 2) & 0x33333333)
    v = (v + (v >> 4)) & 0x0F0F0F0F
    return (v * 0x01010101 & 0xFFFFFFFF) >> 24


def fp8_indexer_study(wl, reps, torch, dsa, make_inputs):
    """The fp8 (e4m3, per-row scale) reading of the indexer on a workload:
    indexer time per step against the bf16 indexer (HIP events on the
    stream), and how much of the bf16 selection the fp8 selection keeps
    (per query row: kept tokens in both / kept tokens of bf16)."""
    dev = torch.device("cuda:0")
    g = make_inputs(wl, dev)
    calls = chunk_calls(wl)
    stream = torch.cuda.current_stream(dev)
    k8, ks = dsa.quantize_keys_fp8(g["kidx"], pos0=0, count=wl.n_kv)
    recall = []
    t_bf16 = t_fp8 = t_quant = 0.0
    for (q0, nq, nkv) in calls:
        sl = slice(q0 - wl.q_pos0, q0 - wl.q_pos0 + nq)
        qi, wi = g["qidx"][:, sl], g["w"][:, sl]
        sc = dsa.index_scores(qi, wi, g["kidx"], q_pos0=q0, n_kv=nkv)
        mb, _ = dsa.topk_mask(sc, q_pos0=q0, n_kv=nkv, top_k=wl.top_k, indices=False)
        q8, wq = dsa.quantize_fp8(qi.contiguous(), wi.contiguous())
        sc8 = dsa.index_scores_fp8(q8, wq, k8, ks, q_pos0=q0, n_kv=nkv, out=sc)
        m8, _ = dsa.topk_mask(sc8, q_pos0=q0, n_kv=nkv, top_k=wl.top_k, indices=False)
        both = _popcount32(mb & m8, torch).sum(-1)
        recall.append((both.double() / _popcount32(mb, torch).sum(-1).double()).flatten())
        del mb, m8
        qic, wic = qi.contiguous(), wi.contiguous()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        for _ in range(reps):
            dsa.index_scores(qi, wi, g["kidx"], q_pos0=q0, n_kv=nkv, out=sc)
        ev[1].record(stream)
        for _ in range(reps):
            dsa.quantize_fp8(qic, wic)
        ev[2].record(stream)
        for _ in range(reps):
            dsa.index_scores_fp8(q8, wq, k8, ks, q_pos0=q0, n_kv=nkv, out=sc)
        ev[3].record(stream)
        torch.cuda.synchronize()
        t_bf16 += ev[0].elapsed_time(ev[1]) / reps
        t_quant += ev[1].elapsed_time(ev[2]) / reps
        t_fp8 += ev[2].elapsed_time(ev[3]) / reps
        del sc, sc8
    r = torch.cat(recall)
    out = {"workload": wl.name, "bf16_index_ms_per_step": round(t_bf16, 4),
           "fp8_index_ms_per_step": round(t_fp8, 4), "fp8_query_quantize_ms_per_step": round(t_quant, 4),
           "indexer_speedup": round(t_bf16 / t_fp8, 3), "rows": int(r.numel()),
           "selection_recall_mean": round(r.mean().item(), 5), "selection_recall_min": round(r.min().item(), 5),
           "selection_recall_p01": round(torch.quantile(r.float().cpu(), 0.01).item(), 5)}
    del g, k8, ks
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- CPU oracle timing

def stream_select_study(wl, reps, torch, dsa, make_inputs):
    """Whole-layer steps with the selection streamed (sampled scores, survivor
    lists) against the default materialised one, on the same inputs: time per
    step of each and whether every index list came out identical."""
    dev = torch.device("cuda:0")
    g = make_inputs(wl, dev)
    calls = chunk_calls(wl)
    B = wl.batch
    big = calls[-1]
    dims = dsa.make_dims(batch=B, n_q=big[1], q_pos0=big[0], n_kv=big[2], kv_capacity=g["k"].shape[1],
                         idx_heads=wl.idx_heads, idx_dim=wl.idx_dim, top_k=wl.top_k, heads=wl.heads,
                         kv_heads=wl.kv_heads, head_dim=wl.head_dim, scale=wl.scale,
                         dtype=dsa.DSA_BF16 if wl.dtype == "bf16" else dsa.DSA_FP32)
    ws = torch.empty(max(dsa.workspace_size(dims, dsa.DSA_OP_FORWARD_STREAM), 256), dtype=torch.uint8,
                     device=dev)
    out = torch.empty_like(g["q"])
    idx = {m: torch.empty((B, wl.n_q, wl.top_k), dtype=torch.int32, device=dev) for m in (False, True)}

    def step(stream):
        for (q0, nq, nkv) in calls:
            sl = slice(q0 - wl.q_pos0, q0 - wl.q_pos0 + nq)
            dsa.forward(g["qidx"][:, sl], g["w"][:, sl], g["kidx"], g["q"][:, sl], g["k"], g["v"],
                        top_k=wl.top_k, q_pos0=q0, n_kv=nkv, scale=wl.scale, workspace=ws, out=out[:, sl],
                        indices=idx[stream][:, sl], stream_select=stream)

    ms = {}
    for stream in (False, True, False, True):
        step(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            step(stream)
        torch.cuda.synchronize()
        ms[stream] = 1e3 * (time.perf_counter() - t0) / reps
    same = bool(torch.equal(idx[False], idx[True]))
    del g, out, idx, ws
    torch.cuda.empty_cache()
    return {"workload": wl.name, "materialised_ms_per_step": round(ms[False], 4),
            "streamed_ms_per_step": round(ms[True], 4), "streamed_speedup": round(ms[False] / ms[True], 3),
            "indices_identical": same, "reps": reps}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s, torch, make_inputs, n_rows=None):
    """The oracle as it stands, on seeded rows of the same workload (the first
    and last row of every chunk first, then seeded random rows), until all
    `n_rows` rows are done or the time budget is spent. Inputs are drawn on
    the GPU with the bench's own recipe; the data a row needs (its query
    rows, the index keys up to its position, the K/V rows of the kept set)
    is copied to the host outside the timed oracle calls."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from dsa_workloads import sample_rows
    from oracle import attend_selected, index_scores, round_scores_fp32, select_topk

    log(f"[bench] oracle on the host: {wl.name}, up to {n_rows or 'all'} rows, ~{budget_s:.0f} s")
    g = make_inputs(wl, torch.device("cuda:0"))
    torch.cuda.synchronize()
    f64 = lambda t: t.double().cpu().numpy()  # bf16 / float32 widen exactly
    n_seq_rows = wl.n_q
    want = n_rows or wl.batch * n_seq_rows
    # (sequence, row) pairs: every sequence's rows interleaved for batches
    if wl.batch > 1:
        pairs = [(b, r) for r in range(n_seq_rows) for b in range(wl.batch)]
    else:
        rows = sample_rows(wl, min(want, n_seq_rows), seed=4321)
        must = sorted({r for c in range(wl.chunks) for r in (c * wl.chunk_len, c * wl.chunk_len + wl.chunk_len - 1)})
        rng = np.random.default_rng(4321)
        rest = [r for r in rng.permutation(np.asarray(rows)).tolist() if r not in set(must)]
        pairs = [(0, r) for r in must + rest]
    pairs = pairs[:want]
    kidx_host = {}
    done, spent = 0, 0.0
    for b, i in pairs:
        p = wl.q_pos0 + i
        if b not in kidx_host:
            kidx_host.clear()
            kidx_host[b] = f64(g["kidx"][b, : wl.q_pos0 + wl.n_q])
        qi, wi, qq = f64(g["qidx"][b, i : i + 1]), f64(g["w"][b, i : i + 1]), f64(g["q"][b, i])
        t0 = time.perf_counter()
        s64 = index_scores(qi, wi, kidx_host[b][: p + 1], p)[0]
        sel = select_topk(round_scores_fp32(s64), p, wl.top_k)
        spent += time.perf_counter() - t0
        idx_t = torch.as_tensor(sel, device="cuda:0")
        ks, vs = f64(g["k"][b].index_select(0, idx_t)), f64(g["v"][b].index_select(0, idx_t))
        t0 = time.perf_counter()
        attend_selected(qq, ks, vs, np.arange(len(sel)), wl.scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s and done >= 8:
            break
    del g
    torch.cuda.empty_cache()
    threads = 1
    for pool in threadpool_info():
        if pool.get("user_api") == "blas":
            threads = max(threads, int(pool.get("num_threads", 1)))
    return {
        "value": done / spent,
        "unit": "queries/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {len(pairs)} seeded query rows of {wl.name} (whole layer per row: float64 "
                  f"scores, float32-rounded top-k selection, attention over the kept keys), "
                  f"{spent:.1f} s of oracle time",
        "blas_threads": threads,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
    }


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(this DSA layer build runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch

    import dsa_lightning_indexer_03_amd as dsa
    from dsa_workloads import FRONT_END_WORKLOADS, WORKLOADS, make_front_end_inputs, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dsa.lib()  # fails loudly if libdsa.so is missing

    wl = WORKLOADS[args.workload]
    # The headline is measured last, right after the other GPU work, so that
    # its warmup and timed steps run at the steady clocks that tens of
    # milliseconds of back-to-back work bring the GPU to.
    secondary = []
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        steps2 = args.secondary_steps or secondary_steps_for(WORKLOADS[name])
        r = run_gpu(WORKLOADS[name], steps2, steps2, torch, dsa, make_inputs, args.cold_reps, args.settle_ms)
        log(f"[bench] {name}: {r['ms_per_step']:.3f} ms/step, {r['value']:.4g} queries/s")
        secondary.append({
            "workload": name, "value": r["value"], "unit": "queries/s",
            "ms_per_step": round(r["ms_per_step"], 4), "steps": steps2, "warmup": steps2, "cold": r["cold"],
            "roofline": _roofline(r["dominant"], name), "kernels": r["kernels"],
        })
    front_end = []
    if args.front_end_steps > 0:
        for fw in FRONT_END_WORKLOADS.values():
            r = run_front_end(fw, args.front_end_steps, torch, dsa, make_front_end_inputs)
            log(f"[bench] {fw.name}: {1e3 * r['ms_per_call']:.1f} us/call, "
                f"{r['roofline']['achieved']} {r['roofline']['unit']}")
            front_end.append(r)
    fp8_study = []
    for name in [s_ for s_ in args.fp8_study.split(",") if s_]:
        r = fp8_indexer_study(WORKLOADS[name], 3, torch, dsa, make_inputs)
        log(f"[bench] fp8 indexer on {name}: {r['fp8_index_ms_per_step']} ms vs bf16 "
            f"{r['bf16_index_ms_per_step']} ms, recall mean {r['selection_recall_mean']}")
        fp8_study.append(r)
    stream_study = []
    for name in [s_ for s_ in args.stream_study.split(",") if s_]:
        r = stream_select_study(WORKLOADS[name], 3, torch, dsa, make_inputs)
        log(f"[bench] streamed selection on {name}: {r['streamed_ms_per_step']} ms vs materialised "
            f"{r['materialised_ms_per_step']} ms, indices identical {r['indices_identical']}")
        stream_study.append(r)
    head = run_gpu(wl, args.steps, args.warmup, torch, dsa, make_inputs, args.cold_reps, args.settle_ms)
    log(f"[bench] {wl.name}: {head['ms_per_step']:.3f} ms/step, {head['value']:.4g} queries/s")
    if args.copy_calibration:
        # one plain streaming kernel of known size (2^28 float32: 1 GiB read,
        # 1 GiB written) as the reference reading for the HBM byte counters
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("[bench] copy calibration: torch.neg over 2^28 float32 (1 GiB read + 1 GiB written)")
        del src, dst
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, args.cpu_seconds, torch, make_inputs)
        # the oracle on the decode batch (all 64 rows) and on 512 seeded rows
        # of the 65536-token prefill, as the secondary lines
        for ent in secondary:
            n_rows = CPU_BASELINE_ROWS.get(ent["workload"])
            if n_rows:
                ent["cpu_baseline"] = cpu_baseline(WORKLOADS[ent["workload"]], args.cpu_seconds, torch,
                                                   make_inputs, n_rows=n_rows)
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.batch, "n_q": wl.n_q, "q_pos0": wl.q_pos0,
            "n_kv": wl.n_kv, "chunks": wl.chunks, "indexer": f"{wl.idx_heads}x{wl.idx_dim}",
            "top_k": wl.top_k, "attention": f"{wl.heads}x{wl.head_dim}", "kv_heads": wl.kv_heads,
            "tokens_per_s": head["value"],
        },
        "roofline": _roofline(head["dominant"], wl.name),
        "settle_ms": head["settle_ms"],
        "cold": head["cold"],
        "cpu_baseline": cpu,
        "kernels": head["kernels"],
        "secondary": secondary,
        "front_end": front_end,
        "fp8_indexer": fp8_study,
        "stream_select": stream_study,
        "device": torch.cuda.get_device_name(0),
    }
    text = json.dumps(line)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(text + "\n")
    print(text, flush=True)


def kernel_sources_digest():
    """sha256 over the library's kernel and host sources: traffic figures
    taken from counters are reported only while the kernels are unchanged."""
    import hashlib
    d = os.path.join(ROOT, "dsa_lightning_indexer_03_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, op):
    """HBM bytes per launch of `op` on `workload` from profiles/traffic.json
    (rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by the calibration
    kernel's readings), or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    ent = table.get("entries", {}).get(workload, {}).get(op)
    if not ent or table.get("sources_sha256") != kernel_sources_digest():
        return None
    return 1024.0 * (ent["fetch_kib"] * table["fetch_scale"] + ent["write_kib"] * table["write_scale"])


def _roofline(k, workload=None):
    return {"bound": k["bound"], "achieved": k["achieved"], "peak": k["peak"], "unit": k["unit"],
            "frac": k["frac"], "traffic": measured_traffic(workload, k["op"]), "kernel": k["op"]}


if __name__ == "__main__":
    main()
