"""MI355X-native DSA (DeepSeek-style sparse attention) layer.

A thin ctypes binding of libdsa.so (the gfx950 HIP kernels behind the C ABI
declared in include/dsa.h). This module only marshals arguments: it reads
shapes from torch tensors, allocates outputs and workspace with torch, and
passes raw device pointers and the current HIP stream to the library. Every
step of the layer runs in the library's kernels. There is no fallback: if the
library is missing or a tensor is not on the GPU, calls raise.

Entry points (same names as the C ABI, without the prefix):
  index_scores, topk_mask, sparse_attention, forward (with stream_select /
  noalloc: dsa_forward_stream_select / dsa_forward_noalloc), forward_varlen,
  indexer_project, quantize_fp8, quantize_keys_fp8, index_scores_fp8,
  workspace_size
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # imported before libdsa.so so both resolve to one HIP runtime

__all__ = [
    "DsaError", "DSA_OP_INDEX_SCORES", "DSA_OP_TOPK_MASK", "DSA_OP_SPARSE_ATTENTION",
    "DSA_OP_FORWARD", "DSA_OP_FORWARD_STREAM", "library_path", "lib", "make_dims", "index_scores", "topk_mask",
    "sparse_attention", "forward", "forward_varlen", "indexer_project", "ProjDims",
    "make_proj_dims", "proj_workspace_size", "quantize_fp8", "quantize_keys_fp8", "index_scores_fp8",
    "workspace_size", "lpad",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libdsa.so")

DSA_FP32, DSA_BF16 = 0, 1
DSA_OP_INDEX_SCORES, DSA_OP_TOPK_MASK, DSA_OP_SPARSE_ATTENTION, DSA_OP_FORWARD = 0, 1, 2, 3
DSA_OP_FORWARD_STREAM = 4


class DsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"dsa status {status}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("q_pos0", ctypes.c_int32),
        ("n_kv", ctypes.c_int32), ("kv_capacity", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32), ("top_k", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class ProjDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("q_pos0", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32), ("hidden", ctypes.c_int32), ("q_rank", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_SIGS = {
    "dsa_index_scores": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P]),
    "dsa_topk_mask": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "dsa_sparse_attention": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P,
                                            ctypes.c_size_t, _P]),
    "dsa_forward": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, ctypes.c_size_t, _P]),
    "dsa_forward_stream_select": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                 _P, _P, ctypes.c_size_t, _P]),
    "dsa_forward_varlen": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _P, _P, ctypes.c_size_t, _P]),
    "dsa_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P]),
    "dsa_quantize_fp8": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P]),
    "dsa_index_scores_fp8": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P]),
    "dsa_indexer_project": (ctypes.c_int, [ctypes.POINTER(ProjDims), _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, ctypes.c_size_t, _P]),
    "dsa_indexer_project_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(ProjDims)]),
    "dsa_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Dims), ctypes.c_int32]),
    "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_abi_version": (ctypes.c_int32, []),
}

_lib = None


def lib():
    """The loaded libdsa.so (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is not built; run __graft_entry__.build()")
        handle = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int):
    if status != 0:
        detail = lib().dsa_last_error().decode()
        raise DsaError(status, detail or lib().dsa_status_string(status).decode())


def lpad(n_kv: int) -> int:
    return (n_kv + 63) // 64 * 64


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_gpu(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("DSA tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("DSA tensors must be contiguous")


def _expect(name, t, shape, dtype=None):
    """Shape (and dtype) check before any pointer reaches the library: the C
    ABI sees raw pointers only, so a wrong extent here would become an
    out-of-bounds access on the device."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def make_dims(*, batch, n_q, q_pos0, n_kv, kv_capacity, idx_heads=1, idx_dim=32, top_k=1,
              heads=1, kv_heads=1, head_dim=64, scale=None, dtype=DSA_BF16) -> Dims:
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Dims(batch, n_q, q_pos0, n_kv, kv_capacity, idx_heads, idx_dim, top_k, heads,
                kv_heads, head_dim, scale, dtype)


def workspace_size(dims: Dims, op: int) -> int:
    return int(lib().dsa_workspace_size(ctypes.byref(dims), op))


def _workspace(dims: Dims, op: int, device, ws=None):
    need = workspace_size(dims, op)
    if need == 0:
        return None, 0
    if ws is not None:
        if ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes, need {need}")
        return ws, ws.numel() * ws.element_size()
    return torch.empty(need, dtype=torch.uint8, device=device), need


def index_scores(qidx, w, kidx, *, q_pos0=0, n_kv=None, out=None):
    """scores [B, T, Lpad] float32 of the lightning indexer; -inf for s > p."""
    _need_gpu(qidx, w, kidx, out)
    B, T, HI, DI = qidx.shape
    cap = kidx.shape[1]
    n_kv = cap if n_kv is None else n_kv
    _expect("w", w, (B, T, HI), torch.float32)
    _expect("kidx", kidx, (B, cap, DI), qidx.dtype)
    _expect("out", out, (B, T, lpad(n_kv)), torch.float32)
    d = make_dims(batch=B, n_q=T, q_pos0=q_pos0, n_kv=n_kv, kv_capacity=cap, idx_heads=HI,
                  idx_dim=DI, dtype=_dtype_code(qidx))
    if out is None:
        out = torch.empty((B, T, lpad(n_kv)), dtype=torch.float32, device=qidx.device)
    _check(lib().dsa_index_scores(ctypes.byref(d), _ptr(qidx), _ptr(w), _ptr(kidx), _ptr(out),
                                  _stream(qidx)))
    return out


def topk_mask(scores, *, q_pos0=0, n_kv, top_k, indices=True, mask_out=None, indices_out=None):
    """(mask [B, T, Lpad/32] int32 bit patterns, indices [B, T, top_k] int32 or None).
    `mask_out` / `indices_out` are written instead of allocating when given."""
    _need_gpu(scores, mask_out, indices_out)
    B, T, L = scores.shape
    d = make_dims(batch=B, n_q=T, q_pos0=q_pos0, n_kv=n_kv, kv_capacity=n_kv, top_k=top_k)
    if L != lpad(n_kv):
        raise ValueError(f"scores rows must have {lpad(n_kv)} entries")
    _expect("mask_out", mask_out, (B, T, L // 32), torch.int32)
    _expect("indices_out", indices_out, (B, T, top_k), torch.int32)
    mask = mask_out if mask_out is not None else torch.empty((B, T, L // 32), dtype=torch.int32,
                                                              device=scores.device)
    idx = indices_out
    if idx is None and indices:
        idx = torch.empty((B, T, top_k), dtype=torch.int32, device=scores.device)
    _check(lib().dsa_topk_mask(ctypes.byref(d), _ptr(scores), _ptr(mask), _ptr(idx), None, 0,
                               _stream(scores)))
    return mask, idx


def sparse_attention(q, k, v, mask, *, q_pos0=0, n_kv=None, scale=None, lse=False, workspace=None,
                     out=None):
    """out [B, T, H, D] (and lse [B, T, H] float32) over the masked-in keys.
    `out` is written instead of allocating when given."""
    _need_gpu(q, k, v, mask, workspace, out)
    B, T, H, D = q.shape
    cap, Hkv = k.shape[1], k.shape[2]
    n_kv = cap if n_kv is None else n_kv
    _expect("k", k, (B, cap, Hkv, D), q.dtype)
    _expect("v", v, (B, cap, Hkv, D), q.dtype)
    _expect("mask", mask, (B, T, lpad(n_kv) // 32), torch.int32)
    d = make_dims(batch=B, n_q=T, q_pos0=q_pos0, n_kv=n_kv, kv_capacity=cap, heads=H,
                  kv_heads=Hkv, head_dim=D, scale=scale, dtype=_dtype_code(q))
    _expect("out", out, (B, T, H, D), q.dtype)
    out = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, T, H), dtype=torch.float32, device=q.device) if lse else None
    ws, nbytes = _workspace(d, DSA_OP_SPARSE_ATTENTION, q.device, workspace)
    _check(lib().dsa_sparse_attention(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(mask),
                                      _ptr(out), _ptr(lse_t), _ptr(ws), nbytes, _stream(q)))
    return (out, lse_t) if lse else out


def forward(qidx, w, kidx, q, k, v, *, top_k, q_pos0=0, n_kv=None, scale=None,
            return_indices=True, return_mask=False, return_lse=False, workspace=None, out=None,
            indices=None, mask=None, lse=None, seq_lens=None, stream_select=False, noalloc=False):
    """The whole DSA layer. Returns a dict with 'out' and the requested extras
    ('indices' [B, T, top_k] int32, 'mask' [B, T, Lpad/32] int32, 'lse').
    Passing `out`, `indices`, `mask`, `lse` or `workspace` tensors makes the
    call write into them instead of allocating (each passed extra is also
    returned). With `seq_lens` (int32 [B] on the GPU) the call goes to
    dsa_forward_varlen: sequence b has seq_lens[b] cached tokens and its
    queries are its last T positions; `n_kv` (default: the caches' capacity)
    is the longest sequence and `q_pos0` is ignored. With `stream_select` the
    call goes to dsa_forward_stream_select (the same results; long rows take
    their selection from survivor lists instead of stored scores). With
    `noalloc` the call goes to dsa_forward_noalloc (the same results; the
    workspace is the library's fixed device array, so no workspace tensor is
    allocated; pass `out` and the wanted extras to allocate nothing here
    either)."""
    _need_gpu(qidx, w, kidx, q, k, v, workspace, out, indices, mask, lse, seq_lens)
    B, T, HI, DI = qidx.shape
    H, D = q.shape[2], q.shape[3]
    cap, Hkv = k.shape[1], k.shape[2]
    n_kv = cap if n_kv is None else n_kv
    if seq_lens is not None:
        _expect("seq_lens", seq_lens, (B,), torch.int32)
        q_pos0 = n_kv - T
    _expect("w", w, (B, T, HI), torch.float32)
    _expect("kidx", kidx, (B, cap, DI), qidx.dtype)
    _expect("q", q, (B, T, H, D), qidx.dtype)
    _expect("k", k, (B, cap, Hkv, D), q.dtype)
    _expect("v", v, (B, cap, Hkv, D), q.dtype)
    _expect("out", out, (B, T, H, D), q.dtype)
    d = make_dims(batch=B, n_q=T, q_pos0=q_pos0, n_kv=n_kv, kv_capacity=cap, idx_heads=HI,
                  idx_dim=DI, top_k=top_k, heads=H, kv_heads=Hkv, head_dim=D, scale=scale,
                  dtype=_dtype_code(q))
    dev = q.device
    res = {"out": torch.empty_like(q) if out is None else out}
    extras = (("indices", indices, return_indices, (B, T, top_k), torch.int32),
              ("mask", mask, return_mask, (B, T, lpad(n_kv) // 32), torch.int32),
              ("lse", lse, return_lse, (B, T, H), torch.float32))
    for name, given, wanted, shape, dt in extras:
        if given is not None:
            if tuple(given.shape) != shape or given.dtype != dt:
                raise ValueError(f"{name} must be {dt} of shape {shape}")
            res[name] = given
        elif wanted:
            res[name] = torch.empty(shape, dtype=dt, device=dev)
    if stream_select and seq_lens is not None:
        raise ValueError("stream_select applies to prefill-shaped calls, not varlen decode batches")
    if noalloc:
        if stream_select or seq_lens is not None or workspace is not None:
            raise ValueError("noalloc takes no workspace and applies to dsa_forward calls only")
        _check(lib().dsa_forward_noalloc(ctypes.byref(d), _ptr(qidx), _ptr(w), _ptr(kidx), _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(res["out"]), _ptr(res.get("lse")),
                                         _ptr(res.get("indices")), _ptr(res.get("mask")), _stream(q)))
        return res
    ws, nbytes = _workspace(d, DSA_OP_FORWARD_STREAM if stream_select else DSA_OP_FORWARD, dev, workspace)
    tail = (_ptr(qidx), _ptr(w), _ptr(kidx), _ptr(q), _ptr(k), _ptr(v), _ptr(res["out"]),
            _ptr(res.get("lse")), _ptr(res.get("indices")), _ptr(res.get("mask")), _ptr(ws), nbytes,
            _stream(q))
    if stream_select:
        _check(lib().dsa_forward_stream_select(ctypes.byref(d), *tail))
    elif seq_lens is None:
        _check(lib().dsa_forward(ctypes.byref(d), *tail))
    else:
        _check(lib().dsa_forward_varlen(ctypes.byref(d), _ptr(seq_lens), *tail))
    return res


def forward_varlen(qidx, w, kidx, q, k, v, seq_lens, *, top_k, **kw):
    """forward() for a decode batch of different sequence lengths (see there)."""
    return forward(qidx, w, kidx, q, k, v, top_k=top_k, seq_lens=seq_lens, **kw)


def make_proj_dims(*, batch, n_q, q_pos0, kv_capacity, hidden, q_rank, idx_heads, idx_dim) -> ProjDims:
    return ProjDims(batch, n_q, q_pos0, kv_capacity, hidden, q_rank, idx_heads, idx_dim)


def proj_workspace_size(dims: ProjDims) -> int:
    return int(lib().dsa_indexer_project_workspace_size(ctypes.byref(dims)))


def indexer_project(x, q_lat, w_qb, w_k, w_proj, kidx_cache, *, q_pos0=0, workspace=None,
                    qidx_out=None, w_out=None):
    """Indexer front end (bf16): returns (qidx [B, T, H_I, D_I] bf16, w [B, T, H_I]
    float32) and writes kidx of the T tokens into rows q_pos0 .. q_pos0+T-1 of
    `kidx_cache` [B, L, D_I] in place. Weights are [out][in]: w_qb
    [H_I*D_I, q_rank], w_k [D_I, hidden], w_proj [H_I, hidden]."""
    _need_gpu(x, q_lat, w_qb, w_k, w_proj, kidx_cache, workspace, qidx_out, w_out)
    B, T, hidden = x.shape
    q_rank = q_lat.shape[2]
    HI = w_proj.shape[0]
    DI = w_k.shape[0]
    cap = kidx_cache.shape[1]
    bf = torch.bfloat16
    _expect("x", x, (B, T, hidden), bf)
    _expect("q_lat", q_lat, (B, T, q_rank), bf)
    _expect("w_qb", w_qb, (HI * DI, q_rank), bf)
    _expect("w_k", w_k, (DI, hidden), bf)
    _expect("w_proj", w_proj, (HI, hidden), bf)
    _expect("kidx_cache", kidx_cache, (B, cap, DI), bf)
    _expect("qidx_out", qidx_out, (B, T, HI, DI), bf)
    _expect("w_out", w_out, (B, T, HI), torch.float32)
    d = make_proj_dims(batch=B, n_q=T, q_pos0=q_pos0, kv_capacity=cap, hidden=hidden, q_rank=q_rank,
                       idx_heads=HI, idx_dim=DI)
    qidx = qidx_out if qidx_out is not None else torch.empty((B, T, HI, DI), dtype=bf, device=x.device)
    w = w_out if w_out is not None else torch.empty((B, T, HI), dtype=torch.float32, device=x.device)
    need = proj_workspace_size(d)
    ws, nbytes = None, 0
    if need > 0:
        if workspace is not None:
            nbytes = workspace.numel() * workspace.element_size()
            if nbytes < need:
                raise ValueError(f"workspace of {nbytes} bytes, need {need}")
            ws = workspace
        else:
            ws, nbytes = torch.empty(need, dtype=torch.uint8, device=x.device), need
    _check(lib().dsa_indexer_project(ctypes.byref(d), _ptr(x), _ptr(q_lat), _ptr(w_qb), _ptr(w_k),
                                     _ptr(w_proj), _ptr(qidx), _ptr(w), _ptr(kidx_cache), _ptr(ws),
                                     nbytes, _stream(x)))
    return qidx, w


def quantize_fp8(qidx, w, kidx=None, *, q_pos0=0, kidx8=None, kscale=None):
    """e4m3 quantisation of the indexer's queries (qidx [B, T, H_I, 128] bf16,
    w [B, T, H_I] float32) -> (qidx8 uint8 [B, T, H_I, 128], wq [B, T, H_I]),
    one scale per head row folded into wq. With `kidx` [B, L, 128] also
    quantises its rows q_pos0 .. q_pos0+T-1 (the call's tokens) into `kidx8`
    [B, L, 128] uint8 and `kscale` [B, L] float32 (allocated zero-filled when
    not given) and returns (qidx8, wq, kidx8, kscale)."""
    _need_gpu(qidx, w, kidx, kidx8, kscale)
    B, T, HI, DI = qidx.shape
    _expect("w", w, (B, T, HI), torch.float32)
    qidx8 = torch.empty((B, T, HI, DI), dtype=torch.uint8, device=qidx.device)
    wq = torch.empty((B, T, HI), dtype=torch.float32, device=qidx.device)
    cap = T + q_pos0
    if kidx is not None:
        cap = kidx.shape[1]
        _expect("kidx", kidx, (B, cap, DI), qidx.dtype)
        if kidx8 is None:
            kidx8 = torch.zeros((B, cap, DI), dtype=torch.uint8, device=qidx.device)
        if kscale is None:
            kscale = torch.zeros((B, cap), dtype=torch.float32, device=qidx.device)
        _expect("kidx8", kidx8, (B, cap, DI), torch.uint8)
        _expect("kscale", kscale, (B, cap), torch.float32)
    d = make_dims(batch=B, n_q=T, q_pos0=q_pos0, n_kv=cap, kv_capacity=cap, idx_heads=HI, idx_dim=DI,
                  dtype=_dtype_code(qidx))
    _check(lib().dsa_quantize_fp8(ctypes.byref(d), _ptr(qidx), _ptr(w), _ptr(kidx), _ptr(qidx8), _ptr(wq),
                                  _ptr(kidx8 if kidx is not None else None),
                                  _ptr(kscale if kidx is not None else None), _stream(qidx)))
    return (qidx8, wq) if kidx is None else (qidx8, wq, kidx8, kscale)


def quantize_keys_fp8(kidx, *, pos0=0, count=None, kidx8=None, kscale=None):
    """e4m3 quantisation of key rows pos0 .. pos0+count-1 (default: all) of
    kidx [B, L, 128] bf16 into kidx8 [B, L, 128] uint8 and kscale [B, L]."""
    _need_gpu(kidx, kidx8, kscale)
    B, cap, DI = kidx.shape
    count = cap - pos0 if count is None else count
    if kidx8 is None:
        kidx8 = torch.zeros((B, cap, DI), dtype=torch.uint8, device=kidx.device)
    if kscale is None:
        kscale = torch.zeros((B, cap), dtype=torch.float32, device=kidx.device)
    _expect("kidx8", kidx8, (B, cap, DI), torch.uint8)
    _expect("kscale", kscale, (B, cap), torch.float32)
    d = make_dims(batch=B, n_q=count, q_pos0=pos0, n_kv=cap, kv_capacity=cap, idx_heads=1, idx_dim=DI,
                  dtype=_dtype_code(kidx))
    _check(lib().dsa_quantize_fp8(ctypes.byref(d), None, None, _ptr(kidx), None, None, _ptr(kidx8),
                                  _ptr(kscale), _stream(kidx)))
    return kidx8, kscale


def index_scores_fp8(qidx8, wq, kidx8, kscale, *, q_pos0=0, n_kv=None, out=None):
    """fp8 indexer scores [B, T, Lpad] float32 (-inf for s > p) from the
    quantised tensors of quantize_fp8 / quantize_keys_fp8."""
    _need_gpu(qidx8, wq, kidx8, kscale, out)
    B, T, HI, DI = qidx8.shape
    cap = kidx8.shape[1]
    n_kv = cap if n_kv is None else n_kv
    _expect("qidx8", qidx8, (B, T, HI, DI), torch.uint8)
    _expect("wq", wq, (B, T, HI), torch.float32)
    _expect("kidx8", kidx8, (B, cap, DI), torch.uint8)
    _expect("kscale", kscale, (B, cap), torch.float32)
    _expect("out", out, (B, T, lpad(n_kv)), torch.float32)
    d = make_dims(batch=B, n_q=T, q_pos0=q_pos0, n_kv=n_kv, kv_capacity=cap, idx_heads=HI, idx_dim=DI,
                  dtype=DSA_BF16)
    if out is None:
        out = torch.empty((B, T, lpad(n_kv)), dtype=torch.float32, device=qidx8.device)
    _check(lib().dsa_index_scores_fp8(ctypes.byref(d), _ptr(qidx8), _ptr(wq), _ptr(kidx8), _ptr(kscale),
                                      _ptr(out), _stream(qidx8)))
    return out
