/*
 * dsa.h - C ABI of the MI355X (gfx950) DSA layer library, libdsa.so.
 *
 * One DSA (DeepSeek-style sparse attention) layer: a lightning indexer scores
 * every earlier cached token for each query, each query keeps its top_k
 * best-scored tokens, the selection is applied as a bitmask over the whole
 * cache, and attention runs only over the kept keys.
 *
 * Pages this interface follows (text of three news pages on llama.cpp build
 * b12180 and the Kimi-K3.1-Pro model):
 *   [aiaulis] aiaulis.com, "llama.cpp kan nu köra Kimi-K3.1-Pro, men än så
 *             länge bara text", paragraphs 2-4 and 7.
 *   [aiu]     aiunderstanding.org, "llama.cpp adds support for Kimi-K3.1-Pro
 *             architecture with DSA indexer", section "What happened".
 *   [devotd]  devotd.net, "llama.cpp b12180 Kimi-K3.1-Pro", sections 1, 2, 4
 *             and the indexer-configuration table of section 1.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE memory allocated and owned by the caller.
 *    The library allocates nothing and keeps no state between calls besides a
 *    thread-local error string. Calls are reentrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *    call only enqueues kernels on it and returns; results are ready once the
 *    caller synchronises the stream.
 *  - Validation is done on the host before anything is enqueued. A call that
 *    returns an error status has enqueued nothing and written no output.
 *    DSA_ERR_HIP means a launch failed; a fault during execution surfaces at
 *    the caller's next synchronisation.
 *  - All pointers must be 16-byte aligned (DSA_ERR_MISALIGNED otherwise).
 *  - Inputs must be finite. Non-finite inputs are not detected.
 *  - Query i of a sequence sits at absolute position p = q_pos0 + i. Its
 *    candidates are the cached tokens s = 0..p (causal, itself included).
 *  - Lpad = roundup(n_kv, 64): the row length of score rows, and 32 times the
 *    number of 32-bit words in a mask row.
 *
 * Tensor layouts (row-major, batch outermost, T = n_q, L = kv_capacity):
 *   qidx    [B][T][idx_heads][idx_dim]   indexer queries, dtype
 *   w       [B][T][idx_heads]            indexer head weights, float32
 *   kidx    [B][L][idx_dim]              indexer-key cache, dtype
 *   scores  [B][T][Lpad]                 float32
 *   mask    [B][T][Lpad/32]              uint32; token s is kept when bit
 *                                        (s & 31) of word (s >> 5) is set
 *   indices [B][T][top_k]                int32, ascending, -1 padded
 *   q, out  [B][T][heads][head_dim]      dtype
 *   k, v    [B][L][kv_heads][head_dim]   attention key/value caches, dtype
 *   lse     [B][T][heads]                float32, natural-log sum-exp
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer (or dims) is NULL          */
  DSA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range            */
  DSA_ERR_UNSUPPORTED = 3, /* valid request the library has no kernel for   */
  DSA_ERR_MISALIGNED = 4,  /* a pointer is not 16-byte aligned              */
  DSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required       */
  DSA_ERR_HIP = 6          /* the HIP runtime rejected a launch             */
} dsa_status;

typedef enum { DSA_FP32 = 0, DSA_BF16 = 1 } dsa_dtype;

typedef enum {
  DSA_OP_INDEX_SCORES = 0,
  DSA_OP_TOPK_MASK = 1,
  DSA_OP_SPARSE_ATTENTION = 2,
  DSA_OP_FORWARD = 3,
  DSA_OP_FORWARD_STREAM = 4
} dsa_op;

/* Problem sizes of one call.
 * Supported: dtype in {DSA_FP32, DSA_BF16}; idx_dim in {32, 64, 128} for bf16
 * and {32, 64} for fp32;
 * head_dim in {64, 128}; 1 <= idx_heads <= 32; heads % kv_heads == 0;
 * n_kv <= 262144 and q_pos0 + n_q <= n_kv <= kv_capacity; top_k >= 1.
 * The configuration of the pages is idx_heads 32, idx_dim 128, top_k 2048
 * [aiu "What happened"; devotd section 1 table]. */
typedef struct {
  int32_t batch;       /* B: independent sequences                          */
  int32_t n_q;         /* T: queries per sequence in this call              */
  int32_t q_pos0;      /* absolute position of query 0                      */
  int32_t n_kv;        /* cached tokens 0..n_kv-1 that may be read          */
  int32_t kv_capacity; /* L: token capacity of the caches (batch stride)    */
  int32_t idx_heads;   /* H_I: indexer heads                                */
  int32_t idx_dim;     /* D_I: indexer query/key dim                        */
  int32_t top_k;       /* tokens kept per query                             */
  int32_t heads;       /* H: attention query heads                          */
  int32_t kv_heads;    /* H_kv: key/value heads (heads % kv_heads == 0)     */
  int32_t head_dim;    /* D: attention head dim                             */
  float scale;         /* softmax scale, > 0 (usually 1/sqrt(head_dim))     */
  int32_t dtype;       /* dsa_dtype of qidx, kidx, q, k, v, out             */
} dsa_dims;

/* Lightning-indexer scores [aiaulis para 2; aiu "What happened"; devotd
 * sections 1-2]. The pages give no formula; the reading implemented is
 *   scores[b][i][s] = sum_h w[b][i][h] * max(0, sum_d qidx[b][i][h][d] * kidx[b][s][d])
 * for s <= p, accumulated in float32 (bf16 products are exact in float32);
 * no RoPE, no scale. Entries s > p (and s >= n_kv) are written as -inf.
 * Reads qidx, w, kidx[b][0..n_kv-1]; writes scores. No workspace. */
dsa_status dsa_index_scores(const dsa_dims* dims, const void* qidx, const float* w,
                            const void* kidx, float* scores, void* stream);

/* Top-k selection applied as a mask over the whole cache [aiaulis paras 3-4;
 * devotd sections 1-2]. Per query row: if top_k >= p+1 every candidate
 * 0..p is kept; otherwise the top_k largest scores among s = 0..p, ties going
 * to the lower index (-0.0 equals +0.0). Writes mask (bits of tokens not kept,
 * s > p and s >= n_kv are zero) and, when `indices` is not NULL, the kept
 * indices ascending, padded with -1 to top_k. Reads scores[b][i][0..p] only.
 * `ws` may be NULL when dsa_workspace_size(dims, DSA_OP_TOPK_MASK) is 0. */
dsa_status dsa_topk_mask(const dsa_dims* dims, const float* scores, uint32_t* mask,
                         int32_t* indices, void* ws, size_t ws_bytes, void* stream);

/* Attention over the kept keys only [aiaulis paras 2 and 4; devotd section
 * 2]: for each query i and head h, over the keys S_i = {s <= p, s < n_kv,
 * mask bit s set},
 *   out[b][i][h] = sum_{s in S_i} softmax_s(scale * q[b][i][h] . k[b][s][g]) v[b][s][g],
 * g = h / (heads / kv_heads). Keys outside S_i get exactly zero weight. An
 * empty S_i gives out = 0 and lse = -inf. lse (optional, may be NULL) is the
 * natural-log sum-exp of the scaled scores over S_i.
 * Prefill-shaped calls run a masked flash attention over 64-key tiles; calls
 * with few queries per sequence gather the kept rows instead, and so do
 * prefill-shaped bf16 calls with kv_heads == 1, head_dim 128 and 16 or 32
 * heads (one K/V row per token serves every head; a key-only cache passes
 * the same buffer as k_cache and v_cache). All compute the same function.
 * Needs dsa_workspace_size(dims, DSA_OP_SPARSE_ATTENTION) bytes of
 * workspace (for the kv_heads == 1 prefill case: an int32 kept-token list of
 * q_pos0 + n_q entries per query row, compacted from the mask). */
dsa_status dsa_sparse_attention(const dsa_dims* dims, const void* q, const void* k_cache,
                                const void* v_cache, const uint32_t* mask, void* out,
                                float* lse, void* ws, size_t ws_bytes, void* stream);

/* The whole layer: dsa_index_scores -> dsa_topk_mask -> dsa_sparse_attention
 * with the scores kept in the workspace [aiaulis paras 2-4; devotd sections
 * 1-2]. `indices`, `mask` and `lse` are optional outputs (NULL = not
 * written; the mask then lives in the workspace). Attention paths that
 * gather kept rows read top-k's index list directly. Queries at positions
 * below top_k keep every earlier token and are not scored (the workspace
 * holds no scores for them; no output depends on them). Needs
 * dsa_workspace_size(dims, DSA_OP_FORWARD) bytes of workspace. */
dsa_status dsa_forward(const dsa_dims* dims, const void* qidx, const float* w,
                       const void* kidx, const void* q, const void* k_cache,
                       const void* v_cache, void* out, float* lse, int32_t* indices,
                       uint32_t* mask, void* ws, size_t ws_bytes, void* stream);

/* The whole layer, as dsa_forward, for a decode batch whose sequences have
 * different lengths [aiaulis paras 2-4; devotd sections 1-2]. The pages
 * describe one causal sequence; a batch is read as B independent layers that
 * share one launch, so the result for sequence b is exactly dsa_forward's on
 * that sequence alone. Sequence b holds
 * len_b = clamp(seq_lens[b], n_q, n_kv) cached tokens, and its n_q queries sit
 * at positions len_b - n_q .. len_b - 1: every candidate, score, kept index
 * and attended key of sequence b lies below len_b; mask bits and scores past
 * it are as for a row whose query sits at len_b - 1 (zero bits, never read).
 *  - seq_lens: DEVICE int32 [batch], read by the kernels (values outside
 *    [n_q, n_kv] are clamped to it; they are not checked on the host).
 *  - dims->n_kv is the longest sequence (the row length of scores and mask,
 *    Lpad = roundup(n_kv, 64)), and dims->q_pos0 must equal n_kv - n_q
 *    (DSA_ERR_SHAPE otherwise), so that dsa_workspace_size(dims,
 *    DSA_OP_FORWARD) sizes the workspace.
 *  - Decode-shaped calls only: n_q <= 8 and a head configuration the
 *    gather attention supports (DSA_ERR_UNSUPPORTED otherwise).
 * Every other argument, layout and error behaviour is dsa_forward's. */
dsa_status dsa_forward_varlen(const dsa_dims* dims, const int32_t* seq_lens, const void* qidx,
                              const float* w, const void* kidx, const void* q,
                              const void* k_cache, const void* v_cache, void* out, float* lse,
                              int32_t* indices, uint32_t* mask, void* ws, size_t ws_bytes,
                              void* stream);

/* The whole layer, as dsa_forward, with the selection streamed instead of
 * materialised for calls with long rows: matching every cached key against
 * the queries is the cost the layer keeps [aiu "Why it matters"; devotd
 * section 4], and storing every score only to keep top_k of them per row is
 * traffic on top of it. Calls with n_q > 8, more than 16384 candidates in the
 * longest row, n_kv <= 65536, top_k <= 2048 and at least 512 query rows
 * (others run exactly as dsa_forward): the indexer scores every 16th 64-key
 * tile of each row first; a threshold guessed from that sample lets the
 * indexer keep only the (score, token) pairs reaching it (at most 8192 per
 * row) instead of storing every score; the selection is taken from those
 * lists, and rows they cannot decide (fewer than top_k or more than 8192
 * survivors) are scored and selected the materialised way, their query tiles
 * only. The kept sets are exactly dsa_forward's (both select from the same
 * float32 scores with the same tie rule), so every output is identical.
 * Needs dsa_workspace_size(dims, DSA_OP_FORWARD_STREAM) bytes of workspace;
 * every other argument, layout and error behaviour is dsa_forward's. */
dsa_status dsa_forward_stream_select(const dsa_dims* dims, const void* qidx, const float* w,
                                     const void* kidx, const void* q, const void* k_cache,
                                     const void* v_cache, void* out, float* lse, int32_t* indices,
                                     uint32_t* mask, void* ws, size_t ws_bytes, void* stream);

/* dsa_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The workspace is a
 * fixed device array of DSA_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU, held until the process ends; its device address is looked up once
 * per device (on the first call with that device current) and nothing is
 * allocated or freed, by the library or any routine it calls.
 *  - Runs on the calling thread's current device; `stream` must belong to it.
 *  - Calls whose dsa_forward workspace (dsa_workspace_size(dims,
 *    DSA_OP_FORWARD), less the mask and index-list regions when `mask` /
 *    `indices` are given) exceeds DSA_NOALLOC_SCRATCH_BYTES return
 *    DSA_ERR_WORKSPACE and enqueue nothing. The decode batch of 64 sequences
 *    x 32768 cached tokens (32 x 128 indexer and attention heads, top_k 2048)
 *    needs about 25 MiB.
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one
 *    GPU (concurrent streams, or threads) race and give undefined results;
 *    serialise them. Results never depend on what an earlier call left in
 *    the array.
 * Every other argument, layout, result and error behaviour is dsa_forward's. */
#define DSA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
dsa_status dsa_forward_noalloc(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx,
                               const void* q, const void* k_cache, const void* v_cache, void* out,
                               float* lse, int32_t* indices, uint32_t* mask, void* stream);

/* fp8 reading of the indexer (a precision study: the pages keep the
 * indexer's tensors unquantised because top-k selection is sensitive to their
 * precision [aiaulis para 5; aiu "What happened"; devotd section 3]).
 *
 * dsa_quantize_fp8 turns bf16 indexer rows (idx_dim 128) into e4m3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest value 448)
 * with one float32 scale per row: scale = max|x| / 448 (1 for a zero row),
 * code = e4m3(x / scale), division correctly rounded in float32, rounding to
 * nearest with ties to the even mantissa.
 *   queries: qidx [B][T][idx_heads][128] bf16, w [B][T][idx_heads] float32
 *            -> qidx8 [B][T][idx_heads][128] codes, wq = w * scale [B][T][idx_heads]
 *   keys:    rows q_pos0 .. q_pos0+T-1 of kidx [B][kv_capacity][128] bf16 (the
 *            call's new tokens) -> the same rows of kidx8 [B][kv_capacity][128]
 *            codes and kscale [B][kv_capacity] float32; other rows untouched.
 * Pass NULL for all four query pointers or all three key pointers to skip
 * that half (at least one half is required). dims->dtype must be DSA_BF16
 * and idx_dim 128 (DSA_ERR_UNSUPPORTED otherwise).
 *
 * dsa_index_scores_fp8 is dsa_index_scores on the quantised tensors:
 *   scores[b][i][s] = kscale[b][s] * sum_h wq[b][i][h] * max(0, sum_d qidx8[b][i][h][d] * kidx8[b][s][d])
 * for s <= p (the products of codes summed in float32), -inf elsewhere; the
 * scale factors come out of the ReLU because they are positive. Reads key
 * rows and scales 0..n_kv-1. Same dims rules as the quantiser. */
dsa_status dsa_quantize_fp8(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx,
                            uint8_t* qidx8, float* wq, uint8_t* kidx8, float* kscale, void* stream);
dsa_status dsa_index_scores_fp8(const dsa_dims* dims, const uint8_t* qidx8, const float* wq,
                                const uint8_t* kidx8, const float* kscale, float* scores,
                                void* stream);

/* Problem sizes of the indexer front end (dsa_indexer_project). bf16 only.
 * Supported: hidden and q_rank multiples of 64; 1 <= idx_heads <= 32;
 * idx_dim in {32, 64, 128}; q_pos0 + n_q <= kv_capacity. */
typedef struct {
  int32_t batch;       /* B: independent sequences                          */
  int32_t n_q;         /* T: new tokens per sequence in this call           */
  int32_t q_pos0;      /* cache position of token 0                         */
  int32_t kv_capacity; /* L: token capacity of the index-key cache          */
  int32_t hidden;      /* width of the activations x                        */
  int32_t q_rank;      /* width of the compressed query q_lat               */
  int32_t idx_heads;   /* H_I                                               */
  int32_t idx_dim;     /* D_I                                               */
} dsa_proj_dims;

/* Indexer front end: the indexer's tensors q_b, k and projection [aiu "What
 * happened"; devotd section 3] applied to T new tokens of B sequences. The
 * pages name the tensors but give no formula; the reading implemented is
 * three linear maps (no bias, no norm, no RoPE, no scale):
 *   qidx[b][t][h][d] = sum_r q_lat[b][t][r] * w_qb[h*idx_dim + d][r]
 *   kidx_cache[b][q_pos0 + t][d] = sum_j x[b][t][j] * w_k[d][j]
 *   w[b][t][h] = sum_j x[b][t][j] * w_proj[h][j]
 * accumulated in float32; qidx and the cache rows are rounded to bf16, w is
 * float32. The outputs are exactly the inputs dsa_index_scores and
 * dsa_forward take (qidx, w, kidx with kv_capacity rows per sequence).
 * Layouts (bf16 unless stated, row-major, batch outermost):
 *   x [B][T][hidden], q_lat [B][T][q_rank],
 *   w_qb [idx_heads*idx_dim][q_rank], w_k [idx_dim][hidden],
 *   w_proj [idx_heads][hidden]             (weights are [out][in]),
 *   qidx [B][T][idx_heads][idx_dim], w [B][T][idx_heads] float32,
 *   kidx_cache [B][kv_capacity][idx_dim]: rows q_pos0 .. q_pos0+T-1 of each
 *   sequence are written, every other row is left untouched.
 * Needs dsa_indexer_project_workspace_size(dims) bytes of workspace (float32
 * partial sums of the thin products; `ws` may be NULL when that is 0).
 * Errors as for the other entry points (DSA_ERR_SHAPE / _UNSUPPORTED for
 * sizes outside the supported set). */
dsa_status dsa_indexer_project(const dsa_proj_dims* dims, const void* x, const void* q_lat,
                               const void* w_qb, const void* w_k, const void* w_proj,
                               void* qidx, float* w, void* kidx_cache, void* ws,
                               size_t ws_bytes, void* stream);

/* Workspace bytes dsa_indexer_project needs for `dims` (0 when none or when
 * dims are invalid). Host only. */
size_t dsa_indexer_project_workspace_size(const dsa_proj_dims* dims);

/* Workspace bytes `op` needs for `dims` (0 when none). Returns 0 for invalid
 * dims as well; the op itself then reports the error. Host only. */
size_t dsa_workspace_size(const dsa_dims* dims, int32_t op);

/* Static description of a status code. Host only. */
const char* dsa_status_string(int32_t status);

/* Detail of the last failing call on this thread ("" if none). Host only. */
const char* dsa_last_error(void);

/* DSA_ABI_VERSION of the built library. Host only. */
int32_t dsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
