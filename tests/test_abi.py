"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every entry point include/dsa.h declares, and rejects invalid arguments on the
host before anything is enqueued. Every call here fails validation, so no
kernel is ever launched. Pointers passed are fake, aligned addresses that the
library never dereferences on these paths."""
import ctypes
import os
import re

import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_WORKSPACE, ERR_HIP = range(7)
FAKE = 0x10000  # aligned, never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = dsa.lib()
    names = _declared_functions()
    assert {"dsa_index_scores", "dsa_topk_mask", "dsa_sparse_attention", "dsa_forward"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dsa_abi_version() == 1
    assert lib.dsa_status_string(ERR_WORKSPACE) == b"workspace too small"


def _dims(**kw):
    base = dict(batch=1, n_q=16, q_pos0=0, n_kv=64, kv_capacity=64, idx_heads=32, idx_dim=128,
                top_k=8, heads=32, kv_heads=32, head_dim=128, scale=None, dtype=dsa.DSA_BF16)
    base.update(kw)
    return dsa.make_dims(**base)


def _scores(d, qidx=FAKE, w=FAKE, kidx=FAKE, scores=FAKE):
    return dsa.lib().dsa_index_scores(ctypes.byref(d) if d is not None else None, qidx, w, kidx, scores, None)


def _forward(d, ws=FAKE, ws_bytes=1 << 40, out=FAKE, idx=None, mask=None):
    return dsa.lib().dsa_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, out, None, idx, mask,
                                 ws, ws_bytes, None)


def _err():
    return dsa.lib().dsa_last_error().decode()


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(n_q=0), ERR_SHAPE),
        (dict(batch=0), ERR_SHAPE),
        (dict(q_pos0=-1), ERR_SHAPE),
        (dict(q_pos0=60, n_q=16), ERR_SHAPE),          # q_pos0 + n_q > n_kv
        (dict(kv_capacity=32), ERR_SHAPE),              # capacity < n_kv
        (dict(idx_heads=0), ERR_SHAPE),
        (dict(idx_heads=33), ERR_UNSUPPORTED),
        (dict(idx_dim=96), ERR_UNSUPPORTED),
        (dict(idx_dim=128, dtype=dsa.DSA_FP32), ERR_UNSUPPORTED),
        (dict(dtype=7), ERR_UNSUPPORTED),
        (dict(n_kv=262145, kv_capacity=262145), ERR_UNSUPPORTED),
    ],
)
def test_index_scores_rejects_bad_dims(kw, status):
    assert _scores(_dims(**kw)) == status
    assert _err() != ""


def test_null_and_misaligned_pointers_are_rejected():
    assert _scores(None) == ERR_NULL
    assert _scores(_dims(), qidx=None) == ERR_NULL
    assert _scores(_dims(), scores=None) == ERR_NULL
    assert _scores(_dims(), w=FAKE + 4) == ERR_MISALIGNED
    assert "w" in _err()


def test_attention_and_forward_validation():
    lib = dsa.lib()
    d = _dims(head_dim=96)
    assert lib.dsa_sparse_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ERR_UNSUPPORTED
    d = _dims(heads=30, kv_heads=4)
    assert lib.dsa_sparse_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ERR_SHAPE
    d = _dims(scale=-1.0)
    assert _forward(d) == ERR_SHAPE
    d = _dims(top_k=0)
    assert _forward(d) == ERR_SHAPE
    d = _dims()
    assert _forward(d, out=None) == ERR_NULL
    need = dsa.workspace_size(d, dsa.DSA_OP_FORWARD)
    assert need > 0
    assert _forward(d, ws=None) == ERR_NULL
    assert _forward(d, ws_bytes=need - 1) == ERR_WORKSPACE
    assert "need" in _err()


def test_forward_noalloc_validation():
    """The allocation-free forward validates like dsa_forward and refuses
    calls whose workspace exceeds its fixed device array, all on the host
    before it looks the array up or enqueues anything."""
    lib = dsa.lib()

    def call(d, out=FAKE):
        return lib.dsa_forward_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, out, None, None, None,
                                       None)

    assert call(_dims(top_k=0)) == ERR_SHAPE
    assert call(_dims(), out=None) == ERR_NULL
    # 256 decode sequences of 32768 tokens: about 100 MiB of workspace
    big = _dims(batch=256, n_q=1, q_pos0=32767, n_kv=32768, kv_capacity=32768, top_k=2048)
    assert dsa.workspace_size(big, dsa.DSA_OP_FORWARD) > 32 << 20
    assert call(big) == ERR_WORKSPACE
    assert "scratch" in _err()
    # the decode batch of 64 sequences x 32768 tokens fits
    dec = _dims(batch=64, n_q=1, q_pos0=32767, n_kv=32768, kv_capacity=32768, top_k=2048)
    assert dsa.workspace_size(dec, dsa.DSA_OP_FORWARD) <= 32 << 20


def test_topk_validation():
    lib = dsa.lib()
    d = _dims(top_k=0)
    assert lib.dsa_topk_mask(ctypes.byref(d), FAKE, FAKE, None, None, 0, None) == ERR_SHAPE
    d = _dims()
    assert lib.dsa_topk_mask(ctypes.byref(d), FAKE, None, None, None, 0, None) == ERR_NULL
    assert lib.dsa_topk_mask(ctypes.byref(d), FAKE, FAKE, FAKE + 8, None, 0, None) == ERR_MISALIGNED


def test_workspace_sizes():
    # prefill-shaped forward: scores [B, T, Lpad] + mask, each 256-B aligned
    d = _dims(n_q=64, n_kv=100, kv_capacity=128)
    lp = 128
    want = (64 * lp * 4 + 255) // 256 * 256 + (64 * lp // 8 + 255) // 256 * 256
    assert dsa.workspace_size(d, dsa.DSA_OP_FORWARD) == want
    assert dsa.workspace_size(d, dsa.DSA_OP_SPARSE_ATTENTION) == 0
    assert dsa.workspace_size(d, dsa.DSA_OP_INDEX_SCORES) == 0
    # decode-shaped calls gather kept rows and need split partials
    d = _dims(batch=4, n_q=1, q_pos0=999, n_kv=1000, kv_capacity=1000, top_k=300)
    assert dsa.workspace_size(d, dsa.DSA_OP_SPARSE_ATTENTION) > 0
    assert dsa.workspace_size(_dims(n_q=0), dsa.DSA_OP_FORWARD) == 0


def test_stream_select_workspace():
    """The streamed selection needs room only for calls it applies to (>= 512
    rows, longest row past 16384 candidates, top_k <= 2048): sampled scores
    (every 16th 64-key tile), guesses, 8192-entry survivor lists, counters and
    flags on top of the materialised layout."""
    small = _dims(n_q=64, n_kv=100, kv_capacity=128)
    assert dsa.workspace_size(small, dsa.DSA_OP_FORWARD_STREAM) == dsa.workspace_size(small, dsa.DSA_OP_FORWARD)
    B, T, p0, L = 1, 1024, 20000, 21024
    d = _dims(batch=B, n_q=T, q_pos0=p0, n_kv=L, kv_capacity=L, top_k=2048)
    rows, sample_ld, nqt = B * T, (L + 1023) // 1024 * 64, (T + 31) // 32
    al = lambda x: (x + 255) // 256 * 256
    extra = al(rows * sample_ld * 4) + al(rows * 4) + al(rows * 8192 * 8) + al((2 * rows + B * nqt) * 4)
    assert dsa.workspace_size(d, dsa.DSA_OP_FORWARD_STREAM) == dsa.workspace_size(d, dsa.DSA_OP_FORWARD) + extra
    big_k = _dims(batch=B, n_q=T, q_pos0=p0, n_kv=L, kv_capacity=L, top_k=4096)
    assert dsa.workspace_size(big_k, dsa.DSA_OP_FORWARD_STREAM) == dsa.workspace_size(big_k, dsa.DSA_OP_FORWARD)


def test_binding_refuses_host_tensors():
    """No CPU fallback: the binding raises instead of computing on the host."""
    q = torch.zeros(1, 4, 32, 128, dtype=torch.bfloat16)
    w = torch.zeros(1, 4, 32)
    k = torch.zeros(1, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dsa.index_scores(q, w, k)


def _varlen(d, seq=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return dsa.lib().dsa_forward_varlen(ctypes.byref(d), seq, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                        None, None, ws, ws_bytes, None)


def test_forward_varlen_validation():
    # decode-shaped: q_pos0 must be n_kv - n_q (the longest sequence's layout)
    d = _dims(batch=4, n_q=1, q_pos0=10, n_kv=1000, kv_capacity=1000, top_k=300)
    assert _varlen(d) == ERR_SHAPE
    assert "q_pos0" in _err()
    # prefill-shaped calls have no varlen kernel
    d = _dims(batch=2, n_q=16, q_pos0=48, n_kv=64, kv_capacity=64)
    assert _varlen(d) == ERR_UNSUPPORTED
    d = _dims(batch=4, n_q=2, q_pos0=998, n_kv=1000, kv_capacity=1000, top_k=300)
    assert _varlen(d, seq=None) == ERR_NULL
    assert _varlen(d, seq=FAKE + 4) == ERR_MISALIGNED
    need = dsa.workspace_size(d, dsa.DSA_OP_FORWARD)
    assert need > 0
    assert _varlen(d, ws_bytes=need - 1) == ERR_WORKSPACE


def _proj(d, ws=FAKE, ws_bytes=1 << 40, x=FAKE):
    return dsa.lib().dsa_indexer_project(ctypes.byref(d), x, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                                         ws_bytes, None)


def _pdims(**kw):
    base = dict(batch=1, n_q=64, q_pos0=0, kv_capacity=64, hidden=256, q_rank=128, idx_heads=32, idx_dim=128)
    base.update(kw)
    return dsa.make_proj_dims(**base)


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(n_q=0), ERR_SHAPE),
        (dict(q_pos0=1), ERR_SHAPE),               # q_pos0 + n_q > kv_capacity
        (dict(hidden=100), ERR_UNSUPPORTED),
        (dict(q_rank=0), ERR_UNSUPPORTED),
        (dict(idx_heads=33), ERR_UNSUPPORTED),
        (dict(idx_dim=96), ERR_UNSUPPORTED),
        (dict(batch=65536, n_q=128, kv_capacity=128), ERR_SHAPE),
    ],
)
def test_indexer_project_rejects_bad_dims(kw, status):
    assert _proj(_pdims(**kw)) == status
    assert _err() != ""
    assert dsa.proj_workspace_size(_pdims(**kw)) == 0


def test_indexer_project_pointers_and_workspace():
    d = _pdims(hidden=1024)
    assert _proj(d, x=None) == ERR_NULL
    assert _proj(d, x=FAKE + 2) == ERR_MISALIGNED
    # 64 tokens x 160 outputs over K=1024 is split over K: partials needed
    need = dsa.proj_workspace_size(d)
    assert need > 0
    assert _proj(d, ws=None) == ERR_NULL
    assert _proj(d, ws_bytes=need - 1) == ERR_WORKSPACE
    # a 4096-token prefill needs partials only for the thin k / projection product
    big = _pdims(n_q=4096, kv_capacity=4096, hidden=7168, q_rank=1536)
    assert dsa.proj_workspace_size(big) == 8 * 4096 * 160 * 4


def test_fp8_entry_points_validation():
    lib = dsa.lib()
    q = lambda d, *p: lib.dsa_quantize_fp8(ctypes.byref(d), *p, None)
    s = lambda d, *p: lib.dsa_index_scores_fp8(ctypes.byref(d), *p, None)
    # fp8 needs bf16 inputs with idx_dim 128
    assert q(_dims(idx_dim=64), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == ERR_UNSUPPORTED
    assert q(_dims(dtype=dsa.DSA_FP32, idx_dim=64), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == ERR_UNSUPPORTED
    assert s(_dims(idx_dim=32), FAKE, FAKE, FAKE, FAKE, FAKE) == ERR_UNSUPPORTED
    # nothing to quantise, or half a group given
    assert q(_dims(), None, None, None, None, None, None, None) == ERR_NULL
    assert q(_dims(), FAKE, FAKE, None, None, FAKE, None, None) == ERR_NULL       # qidx8 missing
    assert q(_dims(), None, None, FAKE, None, None, FAKE, None) == ERR_NULL       # kscale missing
    assert q(_dims(), FAKE, FAKE + 4, None, FAKE, FAKE, None, None) == ERR_MISALIGNED
    assert s(_dims(), FAKE, FAKE, FAKE, None, FAKE) == ERR_NULL                   # kscale missing
    assert s(_dims(q_pos0=60), FAKE, FAKE, FAKE, FAKE, FAKE) == ERR_SHAPE
