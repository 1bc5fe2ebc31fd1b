"""Seeded synthetic inputs for the DSA-layer workloads.

This module only draws random tensors of the right shapes and distributions.
It holds none of the layer's arithmetic, and both the GPU path's tests and the
oracle receive the very same tensors from it (the oracle as host copies).

Shapes follow the indexer configuration of the pages (32 indexer heads, key
dim 128, 2048 kept tokens, no RoPE) [aiu "What happened"; devotd section 1
table]. The pages measure nothing on a dataset; these draws stand in for real
activations.

Layouts (row-major, batch outermost):
  qidx [B, T, H_I, D_I]   indexer queries         (bf16 or fp32)
  w    [B, T, H_I]        indexer head weights    (fp32)
  kidx [B, L, D_I]        indexer-key cache       (bf16 or fp32)
  q    [B, T, H, D]       attention queries
  k, v [B, L, H_kv, D]    attention key / value caches
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "fp32" or "bf16": dtype of qidx, kidx, q, k, v and out
    batch: int
    n_q: int              # queries per sequence in one layer call
    q_pos0: int           # absolute position of query 0
    n_kv: int             # cached tokens visible to the call
    idx_heads: int
    idx_dim: int
    top_k: int
    heads: int
    kv_heads: int
    head_dim: int
    seed: int
    chunks: int = 1       # >1: n_q queries are processed in `chunks` equal calls
    integer_indexer: bool = False   # qidx, kidx ~ U{-4..4}, w ~ U{-2..2}
    qidx_std: float = 1.0
    kidx_std: float = 1.0
    w_std: float = 1.0
    qkv_std: float = 1.0
    shared_kv: bool = False  # one buffer serves as K and V (kv_heads == 1: a key-only cache)
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def chunk_len(self) -> int:
        return self.n_q // self.chunks


def _ws(h):
    return 1.0 / math.sqrt(h)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="tiny_fp32_L256",
            dtype="fp32", batch=1, n_q=256, q_pos0=0, n_kv=256,
            idx_heads=4, idx_dim=32, top_k=64, heads=4, kv_heads=4, head_dim=64,
            seed=0, w_std=_ws(4),
            description="one sequence, L=256 causal, indexer 4x32, top_k 64, "
                        "attention 4x64, fp32",
        ),
        Workload(
            name="equiv_bf16_L1536_k2048",
            dtype="bf16", batch=1, n_q=1536, q_pos0=0, n_kv=1536,
            idx_heads=32, idx_dim=128, top_k=2048, heads=32, kv_heads=32, head_dim=128,
            seed=1, qidx_std=_ws(128), kidx_std=_ws(128), w_std=_ws(32),
            description="one sequence, L=1536, top_k 2048 >= L: must equal full "
                        "causal attention",
        ),
        Workload(
            name="ties_bf16_L1536_k512",
            dtype="bf16", batch=1, n_q=1536, q_pos0=0, n_kv=1536,
            idx_heads=32, idx_dim=128, top_k=512, heads=32, kv_heads=32, head_dim=128,
            seed=5, integer_indexer=True,
            description="one sequence, L=1536, integer indexer inputs (exact "
                        "fp32 scores, many ties), top_k 512",
        ),
        Workload(
            name="prefill_bf16_L4096",
            dtype="bf16", batch=1, n_q=4096, q_pos0=0, n_kv=4096,
            idx_heads=32, idx_dim=128, top_k=2048, heads=32, kv_heads=32, head_dim=128,
            seed=2, qidx_std=_ws(128), kidx_std=_ws(128), w_std=_ws(32),
            description="single-layer prefill, one sequence, L=4096 causal",
        ),
        Workload(
            name="decode_bf16_B64_L32768",
            dtype="bf16", batch=64, n_q=1, q_pos0=32767, n_kv=32768,
            idx_heads=32, idx_dim=128, top_k=2048, heads=32, kv_heads=32, head_dim=128,
            seed=3, w_std=_ws(32),
            description="batched decode: 64 sequences, one new query each "
                        "against a 32768-token cache",
        ),
        Workload(
            name="longctx_bf16_L65536_chunk4096",
            dtype="bf16", batch=1, n_q=65536, q_pos0=0, n_kv=65536,
            idx_heads=32, idx_dim=128, top_k=2048, heads=32, kv_heads=32, head_dim=128,
            seed=4, chunks=16, qidx_std=_ws(128), kidx_std=_ws(128), w_std=_ws(32),
            description="long-context prefill, L=65536 in 16 chunks of 4096 "
                        "queries against the growing cache",
        ),
        Workload(
            name="longctx_mqa_bf16_L65536_chunk4096",
            dtype="bf16", batch=1, n_q=65536, q_pos0=0, n_kv=65536,
            idx_heads=32, idx_dim=128, top_k=2048, heads=32, kv_heads=1, head_dim=128,
            seed=6, chunks=16, qidx_std=_ws(128), kidx_std=_ws(128), w_std=_ws(32),
            description="long-context prefill as above with one K/V row per token "
                        "shared by all 32 heads (separate K and V rows)",
        ),
        Workload(
            name="longctx_kvshared_bf16_L65536_chunk4096",
            dtype="bf16", batch=1, n_q=65536, q_pos0=0, n_kv=65536,
            idx_heads=32, idx_dim=128, top_k=2048, heads=32, kv_heads=1, head_dim=128,
            seed=7, chunks=16, qidx_std=_ws(128), kidx_std=_ws(128), w_std=_ws(32), shared_kv=True,
            description="long-context prefill with the key-only cache: one row per token "
                        "serves as K and V for all 32 heads",
        ),
    ]
}


def _normal(shape, std, dtype, gen, device):
    x = torch.randn(shape, dtype=torch.float32, generator=gen, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def _ints(shape, lo, hi, dtype, gen, device):
    return torch.randint(lo, hi + 1, shape, generator=gen, device=device).to(dtype)


def make_inputs(wl: Workload, device="cpu", kv_capacity=None):
    """Draw every input tensor of a workload with torch's seeded generator on
    `device`. Draw order: qidx, w, kidx, q, k, v. The big caches are drawn one
    sequence at a time (no full-size float32 temporaries)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    dt = wl.torch_dtype
    B, T, L = wl.batch, wl.n_q, wl.n_kv
    cap = L if kv_capacity is None else kv_capacity
    HI, DI, H, HKV, D = wl.idx_heads, wl.idx_dim, wl.heads, wl.kv_heads, wl.head_dim
    if wl.integer_indexer:
        qidx = _ints((B, T, HI, DI), -4, 4, dt, gen, dev)
        w = _ints((B, T, HI), -2, 2, torch.float32, gen, dev)
    else:
        qidx = _normal((B, T, HI, DI), wl.qidx_std, dt, gen, dev)
        w = _normal((B, T, HI), wl.w_std, torch.float32, gen, dev)
    kidx = torch.zeros((B, cap, DI), dtype=dt, device=dev)
    for b in range(B):
        if wl.integer_indexer:
            kidx[b, :L] = _ints((L, DI), -4, 4, dt, gen, dev)
        else:
            kidx[b, :L] = _normal((L, DI), wl.kidx_std, dt, gen, dev)
    q = _normal((B, T, H, D), wl.qkv_std, dt, gen, dev)
    k = torch.zeros((B, cap, HKV, D), dtype=dt, device=dev)
    v = torch.zeros((B, cap, HKV, D), dtype=dt, device=dev)
    if wl.shared_kv:  # one buffer, drawn once
        v = k
    for cache in (k,) if wl.shared_kv else (k, v):
        for b in range(B):
            cache[b, :L] = _normal((L, HKV, D), wl.qkv_std, dt, gen, dev)
    return {"qidx": qidx, "w": w, "kidx": kidx, "q": q, "k": k, "v": v}


def sample_rows(wl: Workload, n_rows: int, seed: int = 1234):
    """Seeded query rows to check at full size: the first and last row of
    every chunk plus distinct random rows, sorted, `n_rows` in total."""
    T, C = wl.n_q, wl.chunk_len
    must = sorted({r for c in range(wl.chunks) for r in (c * C, c * C + C - 1)})
    g = torch.Generator().manual_seed(seed)
    must_set = set(must)
    rest = [int(r) for r in torch.randperm(T, generator=g).tolist() if r not in must_set]
    rows = must + rest[: max(0, n_rows - len(must))]
    return sorted(rows)


@dataclasses.dataclass(frozen=True)
class FrontEndWorkload:
    """Shapes of one indexer front-end call. The pages give no model widths;
    hidden 7168 and q_rank 1536 are synthetic stand-ins of the size of
    public MLA models of this family."""
    name: str
    batch: int
    n_q: int
    q_pos0: int
    kv_capacity: int
    hidden: int
    q_rank: int
    idx_heads: int
    idx_dim: int
    seed: int
    description: str = ""


FRONT_END_WORKLOADS = {
    w.name: w
    for w in [
        FrontEndWorkload("front_end_prefill_T4096", 1, 4096, 0, 4096, 7168, 1536, 32, 128, 11,
                         "indexer front end of the 4096-token prefill"),
        FrontEndWorkload("front_end_decode_B64", 64, 1, 32767, 32768, 7168, 1536, 32, 128, 12,
                         "indexer front end of one decode step of 64 sequences"),
    ]
}


def make_front_end_inputs(wl: FrontEndWorkload, device="cpu", kv_capacity=None):
    """x, q_lat ~ N(0, 1) and weights ~ N(0, 1/in) (so outputs are O(1)),
    all rounded to bf16, drawn in that order with torch's seeded generator.
    The index-key cache is drawn too (rows the call must leave untouched)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    bf = torch.bfloat16
    B, T, hid, r, HI, DI = wl.batch, wl.n_q, wl.hidden, wl.q_rank, wl.idx_heads, wl.idx_dim
    cap = wl.kv_capacity if kv_capacity is None else kv_capacity
    return {
        "x": _normal((B, T, hid), 1.0, bf, gen, dev),
        "q_lat": _normal((B, T, r), 1.0, bf, gen, dev),
        "w_qb": _normal((HI * DI, r), 1.0 / math.sqrt(r), bf, gen, dev),
        "w_k": _normal((DI, hid), 1.0 / math.sqrt(hid), bf, gen, dev),
        "w_proj": _normal((HI, hid), 1.0 / math.sqrt(hid), bf, gen, dev),
        "kidx_cache": _normal((B, cap, DI), 1.0, bf, gen, dev),
    }
