"""dsa_forward_noalloc, the whole-layer call for callers that cannot allocate
(its workspace is the library's fixed device array), against dsa_forward on
the same inputs: identical indices, mask, out and lse, on calls in a row of
decreasing size (the later calls run over what the earlier ones left in the
array), and no allocation during the call."""
import math
import sys

import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa
from dsa_workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _wl(name, B, T, q_pos0, n_kv, top_k, H, Hkv, D, seed):
    return Workload(name=name, dtype="bf16", batch=B, n_q=T, q_pos0=q_pos0, n_kv=n_kv, idx_heads=32, idx_dim=128,
                    top_k=top_k, heads=H, kv_heads=Hkv, head_dim=D, seed=seed, qidx_std=1.0, kidx_std=1.0,
                    w_std=1 / math.sqrt(32))


# a decode batch past 65536 cached tokens (the streamed top-k), a decode
# batch (split partials in the array), a smaller decode batch, then a small
# prefill-shaped call (score rows and mask in the array)
CALLS = [
    _wl("noalloc_decode_B2_L100000", 2, 1, 99999, 100000, 2048, 16, 4, 128, 20),
    _wl("noalloc_decode_B8_L8192", 8, 1, 8191, 8192, 2048, 32, 32, 128, 21),
    _wl("noalloc_decode_B3_L1500", 3, 1, 1499, 1500, 300, 16, 16, 128, 22),
    _wl("noalloc_prefill_B2_T300", 2, 300, 100, 400, 64, 8, 8, 128, 23),
]


def _outputs(wl):
    B, T = wl.batch, wl.n_q
    return {"out": torch.empty((B, T, wl.heads, wl.head_dim), dtype=torch.bfloat16, device=DEV),
            "indices": torch.empty((B, T, wl.top_k), dtype=torch.int32, device=DEV),
            "mask": torch.empty((B, T, dsa.lpad(wl.n_kv) // 32), dtype=torch.int32, device=DEV),
            "lse": torch.empty((B, T, wl.heads), dtype=torch.float32, device=DEV)}


def _call(wl, g, outs, noalloc):
    return dsa.forward(g["qidx"], g["w"], g["kidx"], g["q"], g["k"], g["v"], top_k=wl.top_k, q_pos0=wl.q_pos0,
                       n_kv=wl.n_kv, scale=wl.scale, noalloc=noalloc, **outs)


def test_noalloc_forward_equals_forward_on_calls_in_a_row():
    for wl in CALLS:
        print(f"[noalloc] {wl.name}", flush=True)
        sys.stdout.flush()
        g = make_inputs(wl, DEV)
        ref = _call(wl, g, _outputs(wl), noalloc=False)
        outs = _outputs(wl)
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats(DEV)["allocation.all.allocated"]  # allocations so far
        got = _call(wl, g, outs, noalloc=True)
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats(DEV)["allocation.all.allocated"] == before, "the call allocated"
        for key in ("indices", "mask", "out", "lse"):
            assert got[key] is outs[key]
            assert torch.equal(got[key], ref[key]), f"{wl.name}: {key} differs from dsa_forward"
