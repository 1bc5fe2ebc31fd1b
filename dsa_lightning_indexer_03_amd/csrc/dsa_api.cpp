// C ABI of libdsa.so: argument validation (host only, before anything is
// enqueued), workspace carving and kernel dispatch. See include/dsa.h.
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "dsa_internal.hpp"
#include "dsa_kernels.hpp"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status ok() {
  g_last_error.clear();
  return DSA_OK;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("DSA_DEBUG_SYNC");
    return e && e[0] == '1';
  }();
  return on;
}

dsa_status hip_status(hipError_t e, const char* what, hipStream_t st) {
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DSA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t lpad_of(const dsa_dims& d) { return ((int64_t)d.n_kv + 63) / 64 * 64; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape rules shared by every op. `need_idx` / `need_attn` select which
// dimension groups are checked.
dsa_status check_dims(const dsa_dims* d, bool need_idx, bool need_attn, bool need_topk) {
  if (!d) return fail(DSA_ERR_NULL, "dims is NULL");
  if (d->batch < 1 || d->n_q < 1) return fail(DSA_ERR_SHAPE, "batch (%d) and n_q (%d) must be >= 1", d->batch, d->n_q);
  if (d->q_pos0 < 0) return fail(DSA_ERR_SHAPE, "q_pos0 (%d) must be >= 0", d->q_pos0);
  if (d->n_kv < 1 || (int64_t)d->q_pos0 + d->n_q > d->n_kv)
    return fail(DSA_ERR_SHAPE, "need q_pos0 + n_q (%lld) <= n_kv (%d)", (long long)d->q_pos0 + d->n_q, d->n_kv);
  if (d->kv_capacity < d->n_kv) return fail(DSA_ERR_SHAPE, "kv_capacity (%d) < n_kv (%d)", d->kv_capacity, d->n_kv);
  if (d->dtype != DSA_FP32 && d->dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "dtype %d not supported", d->dtype);
  if (d->n_kv > dsa::kTopkMaxRowBig)
    return fail(DSA_ERR_UNSUPPORTED, "n_kv %d above the supported maximum %d", d->n_kv, dsa::kTopkMaxRowBig);
  if ((int64_t)d->batch * d->n_q > (1ll << 30)) return fail(DSA_ERR_SHAPE, "batch * n_q too large");
  if (need_idx) {
    if (d->idx_heads < 1 || d->idx_heads > 32)
      return fail(d->idx_heads < 1 ? DSA_ERR_SHAPE : DSA_ERR_UNSUPPORTED, "idx_heads %d not in [1, 32]", d->idx_heads);
    if (d->idx_dim != 32 && d->idx_dim != 64 && d->idx_dim != 128)
      return fail(DSA_ERR_UNSUPPORTED, "idx_dim %d not in {32, 64, 128}", d->idx_dim);
    if (d->dtype == DSA_FP32 && d->idx_dim == 128)
      return fail(DSA_ERR_UNSUPPORTED, "idx_dim 128 needs bf16 (fp32 supports 32 and 64)");
  }
  if (need_topk && d->top_k < 1) return fail(DSA_ERR_SHAPE, "top_k (%d) must be >= 1", d->top_k);
  if (need_attn) {
    if (d->heads < 1 || d->kv_heads < 1 || d->heads % d->kv_heads != 0)
      return fail(DSA_ERR_SHAPE, "heads (%d) must be a positive multiple of kv_heads (%d)", d->heads, d->kv_heads);
    if (d->head_dim != 64 && d->head_dim != 128)
      return fail(DSA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", d->head_dim);
    if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return fail(DSA_ERR_SHAPE, "scale must be finite and > 0");
  }
  return DSA_OK;
}

dsa_status check_ptr(const void* p, const char* name, bool required = true) {
  if (!p) return required ? fail(DSA_ERR_NULL, "%s is NULL", name) : DSA_OK;
  if (!aligned16(p)) return fail(DSA_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return DSA_OK;
}

#define DSA_TRY(x)                     \
  do {                                 \
    dsa_status s_ = (x);               \
    if (s_ != DSA_OK) return s_;       \
  } while (0)

// The gather (decode) attention path runs for few queries per sequence.
bool use_gather(const dsa_dims& d) { return d.n_q <= 8 && dsa::gather_supported(d.heads, d.head_dim); }

// Prefill-shaped forward calls with one K/V row per token (kv_heads == 1)
// attend over the top-k index list directly (gather + MFMA with the heads as
// M) instead of the masked-dense tile loop.
bool use_mqa_list(const dsa_dims& d) {
  return !use_gather(d) && d.dtype == DSA_BF16 && dsa::attn_mqa_bf16_supported(d.heads, d.kv_heads, d.head_dim);
}

int gather_splits(int64_t max_kept) { return (int)((max_kept + dsa::kGatherSplit - 1) / dsa::kGatherSplit); }

// Workspace layouts. Every region starts 256-B aligned.
struct AttnWs {
  size_t list = 0, counts = 0, part_o = 0, part_ml = 0, total = 0;
  int list_stride = 0, n_splits = 0;
};
AttnWs attn_ws(const dsa_dims& d, bool have_list) {
  AttnWs w;
  const bool mqa = use_mqa_list(d);
  if (!use_gather(d) && !mqa) return w;
  const int64_t rows = (int64_t)d.batch * d.n_q;
  const int64_t max_p1 = (int64_t)d.q_pos0 + d.n_q;
  int64_t max_kept = max_p1;
  size_t off = 0;
  if (mqa) {  // a kept-token list per row (compacted from the mask when none is given)
    if (!have_list) {
      w.list_stride = (int)max_p1;
      w.list = off;
      off += align_up((size_t)rows * w.list_stride * 4);
      w.counts = off;
      off += align_up((size_t)rows * 4);
    }
    w.total = off;
    return w;
  }
  if (!have_list) {
    w.list_stride = (int)max_p1;
    w.list = off;
    off += align_up((size_t)rows * w.list_stride * 4);
    w.counts = off;
    off += align_up((size_t)rows * 4);
  } else {
    max_kept = std::min<int64_t>(max_p1, d.top_k);
  }
  w.n_splits = gather_splits(max_kept);
  w.part_o = off;
  off += align_up((size_t)rows * w.n_splits * d.heads * d.head_dim * 4);
  w.part_ml = off;
  off += align_up((size_t)rows * w.n_splits * d.heads * 2 * 4);
  w.total = off;
  return w;
}

// Streaming selection: prefill-shaped calls with many long rows score a
// sample of each row first (every kStreamStride-th 64-key tile), guess each
// row's survivor threshold from it, and have the indexer keep only the
// (key, token) pairs reaching the guess (at most kStreamCap per row) instead
// of storing every score; rows the lists cannot decide take the
// materialised scores and top-k (their query tiles only).
constexpr int kStreamStride = 16;
constexpr int kStreamCap = 8192;
bool use_stream_select(const dsa_dims& d) {
  const int64_t rows = (int64_t)d.batch * d.n_q;
  return d.n_q > 8 && (int64_t)d.q_pos0 + d.n_q > 16384 && d.n_kv <= dsa::kTopkMaxRow && d.top_k <= 2048 &&
         rows >= 512;
}
int stream_sample_ld(const dsa_dims& d) { return (d.n_kv + 64 * kStreamStride - 1) / (64 * kStreamStride) * 64; }
int stream_nqt(const dsa_dims& d) { return (d.n_q + dsa::kIdxQueryTile - 1) / dsa::kIdxQueryTile; }

struct FwdWs {
  size_t scores = 0, mask = 0, indices = 0, attn = 0, total = 0;
  // streaming selection: sampled scores, guesses, survivor lists, and the
  // counters and flags (one contiguous block, zeroed per call)
  size_t sample = 0, guess = 0, cand = 0, counters = 0, n_counters = 0;
  AttnWs aw;
};
FwdWs fwd_ws(const dsa_dims& d, bool user_mask, bool user_indices, bool stream = false) {
  FwdWs w;
  const int64_t rows = (int64_t)d.batch * d.n_q;
  const int64_t lp = lpad_of(d);
  size_t off = 0;
  w.scores = off;
  off += align_up((size_t)rows * lp * 4);
  if (stream && use_stream_select(d)) {
    w.sample = off;
    off += align_up((size_t)rows * stream_sample_ld(d) * 4);
    w.guess = off;
    off += align_up((size_t)rows * 4);
    w.cand = off;
    off += align_up((size_t)rows * kStreamCap * 8);
    w.counters = off;
    w.n_counters = (size_t)rows * 2 + (size_t)d.batch * stream_nqt(d);  // counts, row flags, tile flags
    off += align_up(w.n_counters * 4);
  }
  if (!user_mask) {
    w.mask = off;
    off += align_up((size_t)rows * (lp / 32) * 4);
  }
  const bool gather = use_gather(d) || use_mqa_list(d);
  if (gather && !user_indices) {
    w.indices = off;
    off += align_up((size_t)rows * d.top_k * 4);
  }
  w.aw = attn_ws(d, /*have_list=*/true);
  w.attn = off;
  off += w.aw.total;
  w.total = off;
  return w;
}

dsa::IndexerParams indexer_params(const dsa_dims& d, const void* qidx, const float* w, const void* kidx,
                                  float* scores, bool write_upper, const int32_t* seq_len) {
  dsa::IndexerParams p{};
  p.qidx = qidx;
  p.w = w;
  p.kidx = kidx;
  p.scores = scores;
  p.B = d.batch;
  p.T = d.n_q;
  p.q_pos0 = d.q_pos0;
  p.n_kv = d.n_kv;
  p.kv_cap = d.kv_capacity;
  p.HI = d.idx_heads;
  p.Lpad = (int)lpad_of(d);
  p.write_upper = write_upper ? 1 : 0;
  p.seq_len = seq_len;
  return p;
}

dsa_status run_scores(const dsa_dims& d, const void* qidx, const float* w, const void* kidx, float* scores,
                      bool write_upper, hipStream_t st, const int32_t* seq_len = nullptr, int row0 = 0,
                      int T_ld = 0) {
  dsa::IndexerParams p = indexer_params(d, qidx, w, kidx, scores, write_upper, seq_len);
  p.row0 = row0;
  p.T_ld = T_ld;
  return hip_status(dsa::launch_indexer(p, d.dtype, d.idx_dim, st), "indexer launch", st);
}

dsa_status run_topk(const dsa_dims& d, const float* scores, uint32_t* mask, int32_t* indices, hipStream_t st,
                    const int32_t* seq_len = nullptr, const uint32_t* row_flag = nullptr) {
  dsa::TopkParams p{};
  p.scores = scores;
  p.mask = mask;
  p.indices = indices;
  p.B = d.batch;
  p.T = d.n_q;
  p.q_pos0 = d.q_pos0;
  p.n_kv = d.n_kv;
  p.Lpad = (int)lpad_of(d);
  p.top_k = d.top_k;
  p.seq_len = seq_len;
  p.row_flag = row_flag;
  return hip_status(dsa::launch_topk(p, st), "top-k launch", st);
}

// Scores and selection of a forward call whose rows are long: sampled
// scores -> guesses -> survivor lists -> selection, then the materialised
// path for the query tiles with undecided rows (both launches return at once
// when there are none).
dsa_status run_stream_select(const dsa_dims& d, const void* qidx, const float* w, const void* kidx, unsigned char* wsb,
                             const FwdWs& fw, uint32_t* mask, int32_t* indices, hipStream_t st) {
  const int64_t rows = (int64_t)d.batch * d.n_q;
  uint32_t* counters = reinterpret_cast<uint32_t*>(wsb + fw.counters);
  uint32_t* cand_count = counters;
  uint32_t* row_flag = counters + rows;
  uint32_t* tile_flag = counters + 2 * rows;
  float* scores = reinterpret_cast<float*>(wsb + fw.scores);
  dsa::StreamSelParams sp{};
  sp.sample = reinterpret_cast<const float*>(wsb + fw.sample);
  sp.sample_ld = stream_sample_ld(d);
  sp.kt_stride = kStreamStride;
  sp.guess = reinterpret_cast<uint32_t*>(wsb + fw.guess);
  sp.cand = reinterpret_cast<const uint2*>(wsb + fw.cand);
  sp.cand_count = cand_count;
  sp.cand_cap = kStreamCap;
  sp.row_flag = row_flag;
  sp.tile_flag = tile_flag;
  sp.nqt = stream_nqt(d);
  sp.mask = mask;
  sp.indices = indices;
  sp.B = d.batch;
  sp.T = d.n_q;
  sp.q_pos0 = d.q_pos0;
  sp.n_kv = d.n_kv;
  sp.Lpad = (int)lpad_of(d);
  sp.top_k = d.top_k;

  dsa::IndexerParams ps = indexer_params(d, qidx, w, kidx, reinterpret_cast<float*>(wsb + fw.sample), false, nullptr);
  ps.Lpad = sp.sample_ld;
  ps.kt_stride = kStreamStride;
  DSA_TRY(hip_status(dsa::launch_indexer(ps, d.dtype, d.idx_dim, st), "sampled indexer launch", st));
  DSA_TRY(hip_status(dsa::launch_zero_u32(counters, fw.n_counters, st), "counter reset launch", st));
  DSA_TRY(hip_status(dsa::launch_stream_guess(sp, st), "threshold guess launch", st));
  dsa::IndexerParams pf = indexer_params(d, qidx, w, kidx, nullptr, false, nullptr);
  pf.guess = sp.guess;
  pf.cand = reinterpret_cast<uint2*>(wsb + fw.cand);
  pf.cand_count = cand_count;
  pf.cand_cap = kStreamCap;
  DSA_TRY(hip_status(dsa::launch_indexer(pf, d.dtype, d.idx_dim, st), "filtering indexer launch", st));
  DSA_TRY(hip_status(dsa::launch_stream_select(sp, st), "survivor selection launch", st));
  dsa::IndexerParams pm = indexer_params(d, qidx, w, kidx, scores, false, nullptr);
  pm.tile_flag = tile_flag;
  DSA_TRY(hip_status(dsa::launch_indexer(pm, d.dtype, d.idx_dim, st), "indexer launch", st));
  DSA_TRY(run_topk(d, scores, mask, indices, st, nullptr, row_flag));
  return ok();
}

dsa_status run_attention(const dsa_dims& d, const void* q, const void* k, const void* v, const uint32_t* mask,
                         const int32_t* list, void* out, float* lse, unsigned char* ws, const AttnWs& aw,
                         hipStream_t st, const int32_t* seq_len = nullptr) {
  const float scale_log2 = d.scale * 1.4426950408889634f;
  const bool mqa = use_mqa_list(d);
  if (!use_gather(d) && !mqa) {
    dsa::AttnParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.mask = mask;
    p.out = out;
    p.lse = lse;
    p.B = d.batch;
    p.T = d.n_q;
    p.q_pos0 = d.q_pos0;
    p.n_kv = d.n_kv;
    p.kv_cap = d.kv_capacity;
    p.H = d.heads;
    p.Hkv = d.kv_heads;
    p.Lpad = (int)lpad_of(d);
    p.scale_log2 = scale_log2;
    return hip_status(dsa::launch_attn_prefill(p, d.dtype, d.head_dim, st), "attention launch", st);
  }
  dsa::GatherParams g{};
  g.q = q;
  g.k = k;
  g.v = v;
  if (list) {
    g.list = list;
    g.counts = nullptr;
    g.list_stride = d.top_k;
  } else {
    dsa::CompactParams cp{};
    cp.mask = mask;
    cp.list = reinterpret_cast<int32_t*>(ws + aw.list);
    cp.counts = reinterpret_cast<int32_t*>(ws + aw.counts);
    cp.B = d.batch;
    cp.T = d.n_q;
    cp.q_pos0 = d.q_pos0;
    cp.n_kv = d.n_kv;
    cp.Lpad = (int)lpad_of(d);
    cp.list_stride = aw.list_stride;
    DSA_TRY(hip_status(dsa::launch_mask_compact(cp, st), "mask compaction launch", st));
    g.list = cp.list;
    g.counts = cp.counts;
    g.list_stride = aw.list_stride;
  }
  g.top_k = d.top_k;
  if (mqa) {
    g.out = out;
    g.lse = lse;
    g.B = d.batch;
    g.T = d.n_q;
    g.q_pos0 = d.q_pos0;
    g.n_kv = d.n_kv;
    g.kv_cap = d.kv_capacity;
    g.H = d.heads;
    g.Hkv = d.kv_heads;
    g.scale_log2 = scale_log2;
    return hip_status(dsa::launch_attn_mqa_bf16(g, st), "kept-list attention launch", st);
  }
  g.part_o = reinterpret_cast<float*>(ws + aw.part_o);
  g.part_ml = reinterpret_cast<float*>(ws + aw.part_ml);
  g.out = out;
  g.lse = lse;
  g.B = d.batch;
  g.T = d.n_q;
  g.q_pos0 = d.q_pos0;
  g.n_kv = d.n_kv;
  g.kv_cap = d.kv_capacity;
  g.H = d.heads;
  g.Hkv = d.kv_heads;
  g.n_splits = aw.n_splits;
  g.scale_log2 = scale_log2;
  g.seq_len = seq_len;
  return hip_status(dsa::launch_attn_gather(g, d.dtype, d.head_dim, st), "gather attention launch", st);
}

dsa_status check_proj_dims(const dsa_proj_dims* d) {
  if (!d) return fail(DSA_ERR_NULL, "dims is NULL");
  if (d->batch < 1 || d->n_q < 1) return fail(DSA_ERR_SHAPE, "batch (%d) and n_q (%d) must be >= 1", d->batch, d->n_q);
  if (d->q_pos0 < 0 || (int64_t)d->q_pos0 + d->n_q > d->kv_capacity)
    return fail(DSA_ERR_SHAPE, "need 0 <= q_pos0 and q_pos0 + n_q (%lld) <= kv_capacity (%d)",
                (long long)d->q_pos0 + d->n_q, d->kv_capacity);
  if ((int64_t)d->batch * d->n_q > 65535ll * 128)
    return fail(DSA_ERR_SHAPE, "batch * n_q (%lld) above %d", (long long)d->batch * d->n_q, 65535 * 128);
  if (d->hidden < 64 || d->hidden % 64 != 0 || d->q_rank < 64 || d->q_rank % 64 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "hidden (%d) and q_rank (%d) must be positive multiples of 64", d->hidden,
                d->q_rank);
  if (d->hidden > (1 << 20) || d->q_rank > (1 << 20)) return fail(DSA_ERR_SHAPE, "hidden / q_rank too large");
  if (d->idx_heads < 1 || d->idx_heads > 32)
    return fail(d->idx_heads < 1 ? DSA_ERR_SHAPE : DSA_ERR_UNSUPPORTED, "idx_heads %d not in [1, 32]", d->idx_heads);
  if (d->idx_dim != 32 && d->idx_dim != 64 && d->idx_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "idx_dim %d not in {32, 64, 128}", d->idx_dim);
  return DSA_OK;
}

size_t proj_ws(const dsa_proj_dims& d) {
  const int M = d.batch * d.n_q;
  return dsa::proj_pair_partial_bytes(M, d.idx_heads * d.idx_dim, d.q_rank, d.idx_dim + d.idx_heads, d.hidden);
}

}  // namespace

static dsa_status forward_impl(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx, const void* q,
                        const void* k_cache, const void* v_cache, void* out, float* lse, int32_t* indices,
                        uint32_t* mask, void* ws, size_t ws_bytes, void* stream, bool stream_select,
                        dsa::WorkspaceProvider provider = nullptr) {
  DSA_TRY(check_dims(dims, true, true, true));
  DSA_TRY(check_ptr(qidx, "qidx"));
  DSA_TRY(check_ptr(w, "w"));
  DSA_TRY(check_ptr(kidx, "kidx"));
  DSA_TRY(check_ptr(q, "q"));
  DSA_TRY(check_ptr(k_cache, "k_cache"));
  DSA_TRY(check_ptr(v_cache, "v_cache"));
  DSA_TRY(check_ptr(out, "out"));
  DSA_TRY(check_ptr(lse, "lse", false));
  DSA_TRY(check_ptr(indices, "indices", false));
  DSA_TRY(check_ptr(mask, "mask", false));
  const dsa_dims& d = *dims;
  const FwdWs fw = fwd_ws(d, mask != nullptr, indices != nullptr, stream_select);
  if (provider) DSA_TRY(provider(fw.total, &ws, &ws_bytes));
  DSA_TRY(check_ptr(ws, "workspace"));
  if (ws_bytes < fw.total) return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, fw.total);
  hipStream_t st = (hipStream_t)stream;
  unsigned char* wsb = (unsigned char*)ws;
  float* scores = reinterpret_cast<float*>(wsb + fw.scores);
  uint32_t* m = mask ? mask : reinterpret_cast<uint32_t*>(wsb + fw.mask);
  const bool gather = use_gather(d);
  const bool mqa = use_mqa_list(d);
  int32_t* idx = indices ? indices : (gather || mqa ? reinterpret_cast<int32_t*>(wsb + fw.indices) : nullptr);
  if (stream_select && use_stream_select(d)) {
    DSA_TRY(run_stream_select(d, qidx, w, kidx, wsb, fw, m, idx, st));
  } else {
    // A query at position p with p + 1 <= top_k keeps every earlier token
    // whatever the scores say, and the top-k writes its selection without
    // reading a score, so its row is not scored. These are the first `skip`
    // rows of every sequence: the indexer runs over the remaining rows of
    // every sequence in one launch (row offset `skip` into each sequence's
    // qidx, w and scores rows), and not at all when no row is left.
    const int skip = std::min(std::max(d.top_k - d.q_pos0, 0), d.n_q);
    if (skip == 0) {
      DSA_TRY(run_scores(d, qidx, w, kidx, scores, false, st));
    } else if (skip < d.n_q) {
      dsa_dims ds = d;
      ds.n_q = d.n_q - skip;
      ds.q_pos0 = d.q_pos0 + skip;
      DSA_TRY(run_scores(ds, qidx, w, kidx, scores, false, st, nullptr, skip, d.n_q));
    }
    DSA_TRY(run_topk(d, scores, m, idx, st));
  }
  DSA_TRY(run_attention(d, q, k_cache, v_cache, m, gather || mqa ? idx : nullptr, out, lse, wsb + fw.attn, fw.aw,
                        st));
  return ok();
}

namespace dsa {

dsa_status forward_with_provider(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx,
                                 const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                 int32_t* indices, uint32_t* mask, WorkspaceProvider provider, void* stream) {
  return forward_impl(dims, qidx, w, kidx, q, k_cache, v_cache, out, lse, indices, mask, nullptr, 0, stream, false,
                      provider);
}

dsa_status set_error(dsa_status st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace dsa

extern "C" {

dsa_status dsa_indexer_project(const dsa_proj_dims* dims, const void* x, const void* q_lat, const void* w_qb,
                               const void* w_k, const void* w_proj, void* qidx, float* w, void* kidx_cache,
                               void* ws, size_t ws_bytes, void* stream) {
  DSA_TRY(check_proj_dims(dims));
  DSA_TRY(check_ptr(x, "x"));
  DSA_TRY(check_ptr(q_lat, "q_lat"));
  DSA_TRY(check_ptr(w_qb, "w_qb"));
  DSA_TRY(check_ptr(w_k, "w_k"));
  DSA_TRY(check_ptr(w_proj, "w_proj"));
  DSA_TRY(check_ptr(qidx, "qidx"));
  DSA_TRY(check_ptr(w, "w"));
  DSA_TRY(check_ptr(kidx_cache, "kidx_cache"));
  const dsa_proj_dims& d = *dims;
  const size_t need = proj_ws(d);
  if (need > 0) {
    DSA_TRY(check_ptr(ws, "workspace"));
    if (ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  }
  hipStream_t st = (hipStream_t)stream;
  dsa::ProjParams q{};
  q.x = q_lat;
  q.w0 = w_qb;
  q.w1 = nullptr;
  q.M = d.batch * d.n_q;
  q.N0 = d.idx_heads * d.idx_dim;
  q.N1 = 0;
  q.K = d.q_rank;
  q.mode = 0;
  q.out_bf16 = qidx;
  q.partial = need > 0 ? static_cast<float*>(ws) : nullptr;
  dsa::ProjParams k{};
  k.x = x;
  k.w0 = w_k;
  k.w1 = w_proj;
  k.M = d.batch * d.n_q;
  k.N0 = d.idx_dim;
  k.N1 = d.idx_heads;
  k.K = d.hidden;
  k.mode = 1;
  k.out_bf16 = kidx_cache;
  k.out_f32 = w;
  k.T = d.n_q;
  k.q_pos0 = d.q_pos0;
  k.kv_cap = d.kv_capacity;
  k.partial = need > 0 ? static_cast<float*>(ws) : nullptr;
  DSA_TRY(hip_status(dsa::launch_proj_pair(q, k, ws_bytes, st), "front-end projection launch", st));
  return ok();
}

dsa_status dsa_quantize_fp8(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx,
                            uint8_t* qidx8, float* wq, uint8_t* kidx8, float* kscale, void* stream) {
  DSA_TRY(check_dims(dims, true, false, false));
  const dsa_dims& d = *dims;
  if (d.dtype != DSA_BF16 || d.idx_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "fp8 indexer needs bf16 inputs with idx_dim 128 (dtype %d, idx_dim %d)", d.dtype,
                d.idx_dim);
  const bool do_q = qidx || w || qidx8 || wq, do_k = kidx || kidx8 || kscale;
  if (!do_q && !do_k) return fail(DSA_ERR_NULL, "nothing to quantise (queries and keys both NULL)");
  if (do_q) {
    DSA_TRY(check_ptr(qidx, "qidx"));
    DSA_TRY(check_ptr(w, "w"));
    DSA_TRY(check_ptr(qidx8, "qidx8"));
    DSA_TRY(check_ptr(wq, "wq"));
  }
  if (do_k) {
    DSA_TRY(check_ptr(kidx, "kidx"));
    DSA_TRY(check_ptr(kidx8, "kidx8"));
    DSA_TRY(check_ptr(kscale, "kscale"));
  }
  hipStream_t st = (hipStream_t)stream;
  dsa::QuantParams p{};
  p.qidx = do_q ? qidx : nullptr;
  p.w = w;
  p.kidx = do_k ? kidx : nullptr;
  p.qidx8 = qidx8;
  p.wq = wq;
  p.kidx8 = kidx8;
  p.kscale = kscale;
  p.B = d.batch;
  p.T = d.n_q;
  p.q_pos0 = d.q_pos0;
  p.kv_cap = d.kv_capacity;
  p.HI = d.idx_heads;
  DSA_TRY(hip_status(dsa::launch_quantize_fp8(p, st), "fp8 quantisation launch", st));
  return ok();
}

dsa_status dsa_index_scores_fp8(const dsa_dims* dims, const uint8_t* qidx8, const float* wq, const uint8_t* kidx8,
                                const float* kscale, float* scores, void* stream) {
  DSA_TRY(check_dims(dims, true, false, false));
  const dsa_dims& d = *dims;
  if (d.dtype != DSA_BF16 || d.idx_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "fp8 indexer needs bf16 inputs with idx_dim 128 (dtype %d, idx_dim %d)", d.dtype,
                d.idx_dim);
  DSA_TRY(check_ptr(qidx8, "qidx8"));
  DSA_TRY(check_ptr(wq, "wq"));
  DSA_TRY(check_ptr(kidx8, "kidx8"));
  DSA_TRY(check_ptr(kscale, "kscale"));
  DSA_TRY(check_ptr(scores, "scores"));
  hipStream_t st = (hipStream_t)stream;
  dsa::IndexerParams p{};
  p.qidx = qidx8;
  p.w = wq;
  p.kidx = kidx8;
  p.kscale = kscale;
  p.scores = scores;
  p.B = d.batch;
  p.T = d.n_q;
  p.q_pos0 = d.q_pos0;
  p.n_kv = d.n_kv;
  p.kv_cap = d.kv_capacity;
  p.HI = d.idx_heads;
  p.Lpad = (int)lpad_of(d);
  p.write_upper = 1;
  DSA_TRY(hip_status(dsa::launch_indexer(p, dsa::kIndexerFp8, 128, st), "fp8 indexer launch", st));
  return ok();
}

size_t dsa_indexer_project_workspace_size(const dsa_proj_dims* dims) {
  if (check_proj_dims(dims) != DSA_OK) return 0;
  return proj_ws(*dims);
}


dsa_status dsa_index_scores(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx,
                            float* scores, void* stream) {
  DSA_TRY(check_dims(dims, true, false, false));
  DSA_TRY(check_ptr(qidx, "qidx"));
  DSA_TRY(check_ptr(w, "w"));
  DSA_TRY(check_ptr(kidx, "kidx"));
  DSA_TRY(check_ptr(scores, "scores"));
  DSA_TRY(run_scores(*dims, qidx, w, kidx, scores, true, (hipStream_t)stream));
  return ok();
}

dsa_status dsa_topk_mask(const dsa_dims* dims, const float* scores, uint32_t* mask, int32_t* indices, void* ws,
                         size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  DSA_TRY(check_dims(dims, false, false, true));
  DSA_TRY(check_ptr(scores, "scores"));
  DSA_TRY(check_ptr(mask, "mask"));
  DSA_TRY(check_ptr(indices, "indices", false));
  DSA_TRY(run_topk(*dims, scores, mask, indices, (hipStream_t)stream));
  return ok();
}

dsa_status dsa_sparse_attention(const dsa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                                const uint32_t* mask, void* out, float* lse, void* ws, size_t ws_bytes,
                                void* stream) {
  DSA_TRY(check_dims(dims, false, true, false));
  DSA_TRY(check_ptr(q, "q"));
  DSA_TRY(check_ptr(k_cache, "k_cache"));
  DSA_TRY(check_ptr(v_cache, "v_cache"));
  DSA_TRY(check_ptr(mask, "mask"));
  DSA_TRY(check_ptr(out, "out"));
  DSA_TRY(check_ptr(lse, "lse", false));
  const AttnWs aw = attn_ws(*dims, false);
  if (aw.total > 0) {
    DSA_TRY(check_ptr(ws, "workspace"));
    if (ws_bytes < aw.total)
      return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, aw.total);
  }
  DSA_TRY(run_attention(*dims, q, k_cache, v_cache, mask, nullptr, out, lse, (unsigned char*)ws, aw,
                        (hipStream_t)stream));
  return ok();
}

dsa_status dsa_forward(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx, const void* q,
                       const void* k_cache, const void* v_cache, void* out, float* lse, int32_t* indices,
                       uint32_t* mask, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(dims, qidx, w, kidx, q, k_cache, v_cache, out, lse, indices, mask, ws, ws_bytes, stream,
                      false);
}

dsa_status dsa_forward_stream_select(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx,
                                     const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                     int32_t* indices, uint32_t* mask, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(dims, qidx, w, kidx, q, k_cache, v_cache, out, lse, indices, mask, ws, ws_bytes, stream,
                      true);
}

dsa_status dsa_forward_varlen(const dsa_dims* dims, const int32_t* seq_lens, const void* qidx, const float* w,
                              const void* kidx, const void* q, const void* k_cache, const void* v_cache, void* out,
                              float* lse, int32_t* indices, uint32_t* mask, void* ws, size_t ws_bytes,
                              void* stream) {
  DSA_TRY(check_dims(dims, true, true, true));
  const dsa_dims& d = *dims;
  if (d.q_pos0 != d.n_kv - d.n_q)
    return fail(DSA_ERR_SHAPE, "varlen calls need q_pos0 == n_kv - n_q (got q_pos0 %d, n_kv %d, n_q %d)", d.q_pos0,
                d.n_kv, d.n_q);
  if (!use_gather(d))
    return fail(DSA_ERR_UNSUPPORTED, "varlen calls support n_q <= 8 with the gather attention (n_q %d, heads %d, head_dim %d)",
                d.n_q, d.heads, d.head_dim);
  DSA_TRY(check_ptr(seq_lens, "seq_lens"));
  DSA_TRY(check_ptr(qidx, "qidx"));
  DSA_TRY(check_ptr(w, "w"));
  DSA_TRY(check_ptr(kidx, "kidx"));
  DSA_TRY(check_ptr(q, "q"));
  DSA_TRY(check_ptr(k_cache, "k_cache"));
  DSA_TRY(check_ptr(v_cache, "v_cache"));
  DSA_TRY(check_ptr(out, "out"));
  DSA_TRY(check_ptr(lse, "lse", false));
  DSA_TRY(check_ptr(indices, "indices", false));
  DSA_TRY(check_ptr(mask, "mask", false));
  const FwdWs fw = fwd_ws(d, mask != nullptr, indices != nullptr);
  DSA_TRY(check_ptr(ws, "workspace"));
  if (ws_bytes < fw.total) return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, fw.total);
  hipStream_t st = (hipStream_t)stream;
  unsigned char* wsb = (unsigned char*)ws;
  float* scores = reinterpret_cast<float*>(wsb + fw.scores);
  uint32_t* m = mask ? mask : reinterpret_cast<uint32_t*>(wsb + fw.mask);
  int32_t* idx = indices ? indices : reinterpret_cast<int32_t*>(wsb + fw.indices);
  DSA_TRY(run_scores(d, qidx, w, kidx, scores, false, st, seq_lens));
  DSA_TRY(run_topk(d, scores, m, idx, st, seq_lens));
  DSA_TRY(run_attention(d, q, k_cache, v_cache, m, idx, out, lse, wsb + fw.attn, fw.aw, st, seq_lens));
  return ok();
}

size_t dsa_workspace_size(const dsa_dims* dims, int32_t op) {
  if (!dims) return 0;
  const dsa_dims& d = *dims;
  switch (op) {
    case DSA_OP_INDEX_SCORES:
    case DSA_OP_TOPK_MASK:
      return 0;
    case DSA_OP_SPARSE_ATTENTION:
      if (check_dims(dims, false, true, false) != DSA_OK) return 0;
      return attn_ws(d, false).total;
    case DSA_OP_FORWARD:
      if (check_dims(dims, true, true, true) != DSA_OK) return 0;
      return fwd_ws(d, false, false).total;
    case DSA_OP_FORWARD_STREAM:
      if (check_dims(dims, true, true, true) != DSA_OK) return 0;
      return fwd_ws(d, false, false, true).total;
    default:
      return 0;
  }
}

const char* dsa_status_string(int32_t status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "null pointer";
    case DSA_ERR_SHAPE: return "invalid shape";
    case DSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSA_ERR_MISALIGNED: return "misaligned pointer";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

}  // extern "C"
