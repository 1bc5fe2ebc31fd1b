// Host-side launchers of the gfx950 DSA kernels (internal to libdsa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Lightning-indexer scores for T queries of B sequences.
struct IndexerParams {
  const void* qidx;   // [B][T][HI][DI]
  const float* w;     // [B][T][HI]
  const void* kidx;   // [B][kv_cap][DI]
  float* scores;      // [B][T][Lpad]
  int B, T, q_pos0, n_kv, kv_cap, HI, Lpad;
  int key_chunk;      // keys per workgroup (multiple of 64)
  int write_upper;    // 1: write -inf for s > p; 0: leave those entries untouched
  const int32_t* seq_len;  // [B] per-sequence cache lengths (decode kernel only), or nullptr
  // Rows of qidx, w and scores in memory: sequence b's scored query t is
  // row b * T_ld + row0 + t (T_ld = 0 means T). A call that leaves the first
  // row0 rows of every sequence unscored passes T = rows - row0, T_ld = rows.
  int row0, T_ld;
  const float* kscale;     // fp8 keys: [B][kv_cap] per-key scales; nullptr otherwise
  // Streaming selection (prefill kernel only; zero / nullptr: plain scores).
  int kt_stride;              // > 1: score only key tiles kt_stride * j (a sample), stored
                              // compactly at column 64 j + (s mod 64)
  const uint32_t* guess;      // [B*T] survivor threshold on key >> 10; set: no scores are stored,
                              // survivors go to cand instead
  uint2* cand;                // [B*T][cand_cap] (orderable key, token) of the survivors
  uint32_t* cand_count;       // [B*T] survivors found (may exceed cand_cap; only cand_cap are written)
  int cand_cap;
  const uint32_t* tile_flag;  // [B][query tiles of 32]: a workgroup scores its range only when
                              // one of the range's query tiles is flagged; nullptr: always
};
constexpr int kIdxQueryTile = 32;  // queries per prefill indexer query tile
// dtype: 0 fp32, 1 bf16, kIndexerFp8 e4m3 codes (qidx, kidx; w holds the
// query-scaled weights, kscale the key scales; DI 128 only)
constexpr int kIndexerFp8 = 2;
hipError_t launch_indexer(const IndexerParams& p, int dtype, int DI, hipStream_t st);

// Per-row e4m3 quantisation (rows of 128 bf16 values): scale = max|x| / 448
// (1 for a zero row), code = e4m3(x / scale), round to nearest even.
struct QuantParams {
  const void* qidx;   // [B][T][HI][128] bf16, or nullptr (keys only)
  const float* w;     // [B][T][HI]
  const void* kidx;   // [B][kv_cap][128] bf16, or nullptr (queries only); rows q_pos0..q_pos0+T-1
  uint8_t* qidx8;     // [B][T][HI][128]
  float* wq;          // [B][T][HI] = w * query scale
  uint8_t* kidx8;     // [B][kv_cap][128], same rows as kidx
  float* kscale;      // [B][kv_cap]
  int B, T, q_pos0, kv_cap, HI;
};
hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t st);

// Indexer front end: one product C = X W^T (bf16 in, float32 accumulate),
// W the rows of w0 (outputs 0..N0-1) followed by those of w1 (N0..N0+N1-1).
struct ProjParams {
  const void* x;      // [M][K] bf16, token rows m = b * T + t
  const void* w0;     // [N0][K] bf16
  const void* w1;     // [N1][K] bf16 (mode 1), may be nullptr when N1 == 0
  int M, N0, N1, K;
  int mode;           // 0: out_bf16 = qidx [M][N0]; 1: out_bf16 = index-key cache rows, out_f32 = w [M][N1]
  void* out_bf16;
  float* out_f32;
  int T, q_pos0, kv_cap;  // mode 1: token m goes to cache row (m / T) * kv_cap + q_pos0 + m % T
  float* partial;     // K-split float32 partials (workspace) or nullptr: no split
  int k_split;        // set by the launcher
};
// Workspace bytes of the K-split partials launch_proj uses for an M x N x K
// product (0: no split).
size_t proj_partial_bytes(int M, int N, int K);
hipError_t launch_proj(const ProjParams& p, size_t ws_bytes, hipStream_t st);
// Both front-end products of one call (q_b, and k with projection), their
// launches arranged together where that saves launches; the workspace must
// hold proj_pair_partial_bytes (both products' partials share p.partial).
hipError_t launch_proj_pair(const ProjParams& q, const ProjParams& k, size_t ws_bytes, hipStream_t st);
size_t proj_pair_partial_bytes(int M, int Nq, int Kq, int Nk, int Kk);

// Top-k -> bitmask (+ ascending indices).
struct TopkParams {
  const float* scores;  // [B][T][Lpad]
  uint32_t* mask;       // [B][T][Lpad/32]
  int32_t* indices;     // [B][T][top_k] or nullptr
  int B, T, q_pos0, n_kv, Lpad, top_k;
  const int32_t* seq_len;  // [B] per-sequence cache lengths, or nullptr
  const uint32_t* row_flag;  // [B*T]: select only rows whose flag is nonzero; nullptr: all rows
  int pair_keep;  // set by launch_topk: rows [0, pair_keep) keep every candidate and ride along with others
};
hipError_t launch_topk(const TopkParams& p, hipStream_t st);

// Streaming selection for long prefill rows (topk.hip): the survivor
// threshold of each row from its sampled scores, and the exact selection
// from each row's survivor list. Rows the lists cannot decide are flagged
// (row_flag, and tile_flag of their query tile) for the materialised path.
struct StreamSelParams {
  const float* sample;      // [B*T][sample_ld] sampled scores (key tiles kt_stride * j)
  int sample_ld, kt_stride;
  uint32_t* guess;          // [B*T]
  const uint2* cand;        // [B*T][cand_cap]
  const uint32_t* cand_count;
  int cand_cap;
  uint32_t* row_flag;       // [B*T]
  uint32_t* tile_flag;      // [B][nqt]
  int nqt;
  uint32_t* mask;           // [B*T][Lpad/32]
  int32_t* indices;         // [B*T][top_k] or nullptr
  int B, T, q_pos0, n_kv, Lpad, top_k;
};
hipError_t launch_stream_guess(const StreamSelParams& p, hipStream_t st);
hipError_t launch_stream_select(const StreamSelParams& p, hipStream_t st);
// zeroes n words (counters and flags; a kernel, not a memset node)
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st);

// Masked flash attention over 64-key tiles (prefill-shaped calls).
struct AttnParams {
  const void* q;         // [B][T][H][D]
  const void* k;         // [B][kv_cap][Hkv][D]
  const void* v;
  const uint32_t* mask;  // [B][T][Lpad/32]
  void* out;             // [B][T][H][D]
  float* lse;            // [B][T][H] or nullptr
  int B, T, q_pos0, n_kv, kv_cap, H, Hkv, Lpad;
  float scale_log2;      // softmax scale * log2(e)
};
hipError_t launch_attn_prefill(const AttnParams& p, int dtype, int D, hipStream_t st);
// bf16, head dim 128: 32 queries per wave, register-transposed V (attn_prefill_bf16.hip).
bool attn_prefill_bf16_supported(int D);
hipError_t launch_attn_prefill_bf16(const AttnParams& p, hipStream_t st);

// Gather attention for few queries per sequence: kept-token lists -> split
// partials -> combine.
struct GatherParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* list;    // [B*T][list_stride] ascending kept tokens
  const int32_t* counts;  // [B*T] kept-token counts, or nullptr: min(top_k, p+1)
  int list_stride, top_k;
  float* part_o;          // [B*T][n_splits][H][D] float
  float* part_ml;         // [B*T][n_splits][H][2] float (max in log2 units, sum)
  void* out;              // [B][T][H][D]
  float* lse;             // [B][T][H] or nullptr
  int B, T, q_pos0, n_kv, kv_cap, H, Hkv, n_splits;
  float scale_log2;
  const int32_t* seq_len;  // [B] per-sequence cache lengths (gather kernels), or nullptr
};
#ifndef DSA_GATHER_SPLIT
#define DSA_GATHER_SPLIT 128
#endif
#ifndef DSA_GATHER_UNROLL
#define DSA_GATHER_UNROLL 4
#endif
constexpr int kGatherSplit = DSA_GATHER_SPLIT;    // kept tokens per split workgroup
constexpr int kGatherUnroll = DSA_GATHER_UNROLL;  // tokens per lane slot with loads in flight together
bool gather_supported(int H, int D);
hipError_t launch_attn_gather(const GatherParams& p, int dtype, int D, hipStream_t st);
// bf16, head dim 128, one K/V row per token (kv_heads == 1), prefill-shaped
// calls: one wave per query over its kept-token list (attn_mqa_bf16.hip);
// part_o / part_ml / n_splits are not used.
bool attn_mqa_bf16_supported(int H, int Hkv, int D);
hipError_t launch_attn_mqa_bf16(const GatherParams& p, hipStream_t st);

// Compacts mask rows (bits s <= p, s < n_kv) into ascending token lists.
struct CompactParams {
  const uint32_t* mask;  // [B][T][Lpad/32]
  int32_t* list;         // [B*T][list_stride]
  int32_t* counts;       // [B*T]
  int B, T, q_pos0, n_kv, Lpad, list_stride;
};
hipError_t launch_mask_compact(const CompactParams& p, hipStream_t st);

// Largest row length (p + 1) the top-k kernel holds in registers.
constexpr int kTopkMaxRow = 65536;
// Largest row length of all: longer rows than kTopkMaxRow are streamed.
constexpr int kTopkMaxRowBig = 262144;

}  // namespace dsa
