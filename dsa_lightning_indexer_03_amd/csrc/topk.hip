// Per-query top-k selection, written as a bitmask over the whole cache: one
// workgroup per query row (the selection routine is in topk_row.hpp).
//
// Each query keeps its top_k best-scored earlier tokens [aiaulis paras 2-3;
// devotd section 1 table, 2048 tokens] and the selection is applied as a
// mask over the whole cache rather than by gathering rows [aiaulis para 4;
// devotd section 2].
#include "topk_row.hpp"

namespace dsa {
namespace {

// Rows of up to 4096 candidates (EPT_R <= 16) keep eight workgroups per CU
// (at most 64 registers per lane).
template <int NW, int EPT_R, int EPT_L>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(EPT_R <= 16 ? 8 : 1)))
void topk_mask_kernel(TopkParams a) {
  // Last rows first: they have the most candidates. When the call's first
  // pair_keep rows keep every candidate (only writes), workgroup x also
  // writes keep-all row x, before its own row, so those writes overlap the
  // selections instead of running after them.
  const int x = (int)blockIdx.x, t = a.T - 1 - x;
  if (x < a.pair_keep) {
    const size_t row = (size_t)blockIdx.y * a.T + x;
    keep_all_row<NW * 64>(a, a.q_pos0 + x + 1, a.mask + row * (a.Lpad / 32),
                          a.indices ? a.indices + row * a.top_k : nullptr);
  }
  if (a.row_flag && a.row_flag[(size_t)blockIdx.y * a.T + t] == 0u) return;
  __shared__ TopkShared<NW, EPT_L> sh;
  topk_select_row<NW, EPT_R, EPT_L>(a, t, blockIdx.y, sh);
}


// Long rows (prefill chunks deep into a long cache): one 4-wave workgroup
// per row, four rows per CU (33 KiB of LDS and at most 128 registers each),
// the row streamed from memory, two 4096-token blocks ahead, instead of held
// on chip.
//
//  1. A threshold is guessed from a sample of the row (64-token segments
//     0, 16, 32, ...): the sample's (1.25 k ns / n + 16)-th largest score, so
//     that about 1.25 k + 256 of the row's scores reach it. The row's first
//     block of loads is already in flight meanwhile.
//  2. One pass over the row compacts every token whose score reaches the
//     guess into LDS, in index order (at most kLongCap tokens).
//  3. When between k and kLongCap tokens survived, the k-th largest score of
//     the row is the k-th largest survivor (every other score is below the
//     guess), so selecting among the survivors, ties to the lower index,
//     gives the row's selection exactly. The mask is assembled in LDS.
//  4. Otherwise (an unrepresentative sample, or heavy ties) the workgroup
//     finds the exact threshold by radix passes that re-read the row, and a
//     last pass writes the selection: slower, exact.
// Rows longer than the register-resident kernel holds (65537 to 262144
// tokens) always take a second instantiation, whatever the row count and
// top_k: 32-bit survivor indices, a sample of up to 128 segments at the
// smallest stride that fits (every 13th segment at 100000 tokens), and the
// mask bitmap laid over the survivor arrays once they are in registers.
constexpr int kLongNW = 4, kLongNT = kLongNW * 64;
constexpr int kLongCap = 4096;               // survivors held in LDS
constexpr int kLongEPT = 16;                 // row elements per thread per block
constexpr int kLongBlock = kLongNT * kLongEPT;  // 4096 tokens per block
constexpr int kLongSampleSeg = 16;  // the sample takes every 16th 64-token segment
constexpr int kLongSampleEPT = kTopkMaxRow / kLongSampleSeg / kLongNT;  // sample elements per thread (16)

// Rows of up to kTopkMaxRow tokens, or (BIG) up to kTopkMaxRowBig.
template <bool BIG> struct TopkLongShared;
template <> struct TopkLongShared<false> {
  float val[kLongCap];     // survivor scores
  uint16_t idx[kLongCap];  // token indices (rows hold at most 65536 tokens)
  SelectShared<kLongNW, 1> sel;  // its histogram is also the mask bitmap (<= 2048 words)
  uint32_t wcnt[2][64];  // per (element, wave) counts of one block, double-buffered
};
// Rows past 65536 tokens: 32-bit token indices, and the mask bitmap (up to
// 8192 words) overlays the survivors' scores and indices once they have been
// taken into registers.
template <> struct TopkLongShared<true> {
  uint32_t vi[2 * kLongCap];  // survivor scores (as float), then token indices; later the mask bitmap
  SelectShared<kLongNW, 1> sel;
  uint32_t wcnt[2][64];
};
static_assert(kTopkMaxRowBig / 32 <= 2 * kLongCap, "the bitmap fits over the survivor arrays");

// Exclusive position of this lane's flagged element e in (e, wave, lane)
// order, for kLongEPT elements per thread; returns the block total. wc is a
// 64-entry LDS array; one barrier inside.
__device__ __forceinline__ uint32_t ordered_positions(const uint64_t (&bal)[kLongEPT], uint32_t (&pos)[kLongEPT],
                                                      uint32_t* wc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  static_assert(kLongEPT * kLongNW == 64, "one count per lane");
  if (lane < kLongEPT) {
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < kLongEPT; ++e)
      if (lane == e) mine = (uint32_t)__popcll(bal[e]);
    wc[lane * kLongNW + wave] = mine;
  }
  __syncthreads();
  const uint32_t v = wc[lane];
  const uint32_t incl = wave_inclusive_sum(v);
  const uint32_t excl = incl - v;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int e = 0; e < kLongEPT; ++e)
    pos[e] = (uint32_t)__shfl((int)excl, e * kLongNW + wave, 64) + (uint32_t)__popcll(bal[e] & lt);
  return (uint32_t)__shfl((int)incl, 63, 64);
}

// Radix select of rank `rank` (1 = largest) over the keys that for_each
// visits: for_each(f) calls f(key) for every candidate key of this thread
// (key 0 = no token, never counted). Returns the threshold as (thr, shift):
// the tokens kept are key >> shift > thr, plus, among key >> shift == thr,
// all of them when all_eq, else the first `rem` in index order.
template <typename ForEach>
__device__ __forceinline__ void long_radix_select(ForEach for_each, uint32_t rank, uint32_t* hist, uint32_t* red,
                                                  uint32_t* found, uint32_t& thr, int& shift_out, uint32_t& rem,
                                                  bool& all_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, count_eq = 0;
  rem = rank;
  int thr_shift = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    const int pshift = pass == 0 ? 32 : (pass == 1 ? 21 : 10);
    for (int i = tid; i < nbins; i += kLongNT) hist[i] = 0;
    __syncthreads();
    for_each([&](uint32_t k) {
      const bool cand = k != 0u && (pass == 0 || (k >> pshift) == prefix);
      if (cand) atomicAdd(&hist[(k >> shift) & (nbins - 1)], 1u);
    });
    __syncthreads();
    const int bpt = nbins / kLongNT;
    const int top = nbins - tid * bpt;
    uint32_t local = 0;
    for (int d = top - 1; d >= top - bpt; --d) local += hist[d];
    const uint32_t incl = block_inclusive_sum<kLongNW>(local, red);
    uint32_t cum = incl - local;
    if (cum < rem && rem <= incl) {
      for (int d = top - 1; d >= top - bpt; --d) {
        const uint32_t h = hist[d];
        if (cum < rem && rem <= cum + h) {
          found[0] = (uint32_t)d;
          found[1] = cum;
          found[2] = h;
          break;
        }
        cum += h;
      }
    }
    __syncthreads();
    const uint32_t d = found[0];
    rem -= found[1];
    count_eq = found[2];
    prefix = pass == 0 ? d : ((prefix << (pass == 1 ? 11 : 10)) | d);
    __syncthreads();
    thr_shift = shift;
    if (rem == count_eq) break;  // the threshold's bin is kept whole
  }
  thr = prefix;
  shift_out = thr_shift;
  all_eq = rem == count_eq;
}

template <bool BIG>
__global__ __launch_bounds__(kLongNT) __attribute__((amdgpu_waves_per_eu(BIG ? 3 : 4))) void topk_long_kernel(TopkParams a) {
  const int t = a.T - 1 - (int)blockIdx.x, b = blockIdx.y;  // longest rows first
  if (a.row_flag && a.row_flag[(size_t)b * a.T + t] == 0u) return;
  __shared__ TopkLongShared<BIG> sh;
  float* lval;  // survivor scores in LDS
  if constexpr (BIG) lval = reinterpret_cast<float*>(sh.vi);
  else lval = sh.val;
  auto set_idx = [&](uint32_t at, uint32_t token) {
    if constexpr (BIG) sh.vi[kLongCap + at] = token;
    else sh.idx[at] = (uint16_t)token;
  };
  auto get_idx = [&](uint32_t at) -> int {
    if constexpr (BIG) return (int)sh.vi[kLongCap + at];
    else return (int)sh.idx[at];
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int q_pos0, n_kv;
  seq_extent(a.seq_len, b, a.T, a.q_pos0, a.n_kv, q_pos0, n_kv);
  const int p = q_pos0 + t, n = p + 1;
  const size_t row = (size_t)b * a.T + t;
  const int nwords = a.Lpad / 32;
  const float* srow = a.scores + row * a.Lpad;
  uint32_t* mrow = a.mask + row * nwords;
  int32_t* irow = a.indices ? a.indices + row * a.top_k : nullptr;
  const uint32_t k = (uint32_t)a.top_k;

  if (a.top_k >= n) {  // every candidate is kept
    for (int wi = tid; wi < nwords; wi += kLongNT) {
      const int lo = wi * 32;
      mrow[wi] = lo + 32 <= n ? 0xffffffffu : (lo < n ? (1u << (n - lo)) - 1u : 0u);
    }
    if (irow)
      for (int j = tid; j < a.top_k; j += kLongNT) irow[j] = j < n ? j : -1;
    return;
  }
  const int nblocks = (n + kLongBlock - 1) / kLongBlock;
  // element e of this thread in block blk is token blk * kLongBlock + e * kLongNT + tid
  auto load_block = [&](int blk, float (&v)[kLongEPT]) {
#pragma unroll
    for (int e = 0; e < kLongEPT; ++e) v[e] = srow[min(blk * kLongBlock + e * kLongNT + tid, n - 1)];
  };
  auto block_key = [&](int blk, int e, float v) -> uint32_t {
    return blk * kLongBlock + e * kLongNT + tid < n ? orderable_key(v) : 0u;
  };

  // The row's first block is requested before anything else, so that its
  // loads are in flight while the sample is selected (rows past 65536 tokens
  // need those registers for their larger sample).
  float cur[kLongEPT];
  if constexpr (!BIG) load_block(0, cur);

  // 1. Threshold guess from the sample (or none: every token survives). The
  // sample is every stride-th 64-token segment: stride 16 for rows of up to
  // 65536 tokens, else the smallest stride that keeps it within 128 segments.
  float guess = __uint_as_float(0xff800000u);  // survivors: score >= guess
  if (n > kLongCap) {
    constexpr int SEPT = BIG ? 2 * kLongSampleEPT : kLongSampleEPT;  // sample slots per thread
    const int nseg = (n + 63) / 64;
    int stride = kLongSampleSeg;
    if constexpr (BIG) stride = (nseg + SEPT * kLongNT / 64 - 1) / (SEPT * kLongNT / 64);
    const int span = 64 * stride;  // tokens from one sampled segment to the next
    const int ns = ((nseg + stride - 1) / stride) * 64;  // sample slots (the last segment may be partial)
    float sval[SEPT];
    {
      float v[SEPT];
#pragma unroll
      for (int e = 0; e < SEPT; ++e) {
        const int u = e * kLongNT + tid;
        v[e] = srow[min(span * (u >> 6) + (u & 63), n - 1)];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < SEPT; ++e) {
        const int u = e * kLongNT + tid, s = span * (u >> 6) + (u & 63);
        sval[e] = u < ns && s < n ? v[e] : no_token();
      }
    }
    const uint32_t nsv = (uint32_t)(64 * (n / span) + min(n % span, 64));  // tokens in the sample
    const uint32_t ks = min(nsv, (uint32_t)((1.25f * (float)k * (float)nsv) / (float)n) + 16u);
    guess = select_kth<kLongNW, 1>([&](auto f) {
#pragma unroll
      for (int e = 0; e < SEPT; ++e) f(sval[e], (uint32_t)(e * kLongNT + tid));
    }, ks, sh.sel).val;
  }
  if constexpr (BIG) load_block(0, cur);

  // 2. Survivors, in index order, into LDS.
  uint32_t total = 0;
  {
    float nxt[kLongEPT], nxt2[kLongEPT];
    if (nblocks > 1) load_block(1, nxt);
    for (int blk = 0; blk < nblocks; ++blk) {
      if (blk + 2 < nblocks) load_block(blk + 2, nxt2);
      uint64_t bal[kLongEPT];
      uint32_t pos[kLongEPT];
#pragma unroll
      for (int e = 0; e < kLongEPT; ++e)
        bal[e] = ballot64(blk * kLongBlock + e * kLongNT + tid < n && cur[e] >= guess);
      const uint32_t cnt = ordered_positions(bal, pos, sh.wcnt[blk & 1]);
#pragma unroll
      for (int e = 0; e < kLongEPT; ++e) {
        const uint32_t at = total + pos[e];
        if (((bal[e] >> lane) & 1ull) && at < (uint32_t)kLongCap) {
          lval[at] = cur[e];
          set_idx(at, (uint32_t)(blk * kLongBlock + e * kLongNT + tid));
        }
      }
      total += cnt;
#pragma unroll
      for (int e = 0; e < kLongEPT; ++e) {
        cur[e] = nxt[e];
        nxt[e] = nxt2[e];
      }
    }
  }
  __syncthreads();

  if (total >= k && total <= (uint32_t)kLongCap) {
    // 3. Exact selection among the survivors (index order = LDS order).
    constexpr int CE = kLongCap / kLongNT;  // survivor slots per thread (16)
    static_assert(CE == kLongEPT, "survivor slots use the block layout");
    const KthResult th = select_kth<kLongNW, 1>([&](auto f) {
#pragma unroll
      for (int e = 0; e < CE; ++e) {
        const uint32_t u = (uint32_t)(e * kLongNT + tid);
        f(u < total ? lval[u] : no_token(), u);
      }
    }, k, sh.sel);
    // tie ranks among threshold-equal survivors, then the kept flags
    uint64_t beq[kLongEPT], bsel[kLongEPT];
    float cval[kLongEPT];
    uint32_t pos[kLongEPT];
    int cid[BIG ? kLongEPT : 1];  // token ids, taken before the bitmap overwrites them
#pragma unroll
    for (int e = 0; e < CE; ++e) {
      const uint32_t u = (uint32_t)(e * kLongNT + tid);
      cval[e] = u < total ? lval[u] : no_token();  // NaN: compares false
      if constexpr (BIG) cid[e] = get_idx(u & (kLongCap - 1));
      beq[e] = ballot64(cval[e] == th.val);
    }
    ordered_positions(beq, pos, sh.wcnt[0]);  // its barrier ends every read of the survivor arrays
#pragma unroll
    for (int e = 0; e < CE; ++e) {
      const bool eq = (beq[e] >> lane) & 1ull;
      const bool gt = cval[e] > th.val;
      bsel[e] = ballot64(gt || (eq && (th.all_eq || pos[e] < th.rem)));
    }
    uint32_t* bitmap;
    if constexpr (BIG) bitmap = sh.vi;
    else bitmap = sh.sel.hist[0];
    const int nbw = (n + 31) / 32;  // bitmap words (the rest of the mask row is zero)
    for (int i = tid; i < nbw; i += kLongNT) bitmap[i] = 0;
    const uint32_t nsel = ordered_positions(bsel, pos, sh.wcnt[1]);
    (void)nsel;
#pragma unroll
    for (int e = 0; e < CE; ++e) {
      if ((bsel[e] >> lane) & 1ull) {
        int s;
        if constexpr (BIG) s = cid[e];
        else s = get_idx(e * kLongNT + tid);
        atomicOr(&bitmap[s >> 5], 1u << (s & 31));
        if (irow && pos[e] < k) irow[pos[e]] = s;
      }
    }
    __syncthreads();
    for (int i = tid; i < nwords; i += kLongNT) mrow[i] = i < nbw ? bitmap[i] : 0u;
    return;
  }

  // 4. Exact threshold by passes over the row, then the selection.
  uint32_t thr, rem;
  int shift;
  bool all_eq;
  long_radix_select([&](auto f) {
    for (int blk = 0; blk < nblocks; ++blk) {
      float v[kLongEPT];
      load_block(blk, v);
#pragma unroll
      for (int e = 0; e < kLongEPT; ++e) f(block_key(blk, e, v[e]));
    }
  }, k, sh.sel.hist[0], sh.sel.red, sh.sel.found, thr, shift, rem, all_eq);
  uint32_t eq_before = 0, sel_before = 0;
  for (int blk = 0; blk < nblocks; ++blk) {
    float v[kLongEPT];
    load_block(blk, v);
    uint64_t beq[kLongEPT], bsel[kLongEPT];
    uint32_t keys[kLongEPT], pos[kLongEPT];
#pragma unroll
    for (int e = 0; e < kLongEPT; ++e) {
      keys[e] = block_key(blk, e, v[e]);
      beq[e] = ballot64(keys[e] != 0u && (keys[e] >> shift) == thr);
    }
    const uint32_t neq = ordered_positions(beq, pos, sh.wcnt[0]);
#pragma unroll
    for (int e = 0; e < kLongEPT; ++e) {
      const bool eq = (beq[e] >> lane) & 1ull;
      const bool gt = keys[e] != 0u && (keys[e] >> shift) > thr;
      bsel[e] = ballot64(gt || (eq && (all_eq || eq_before + pos[e] < rem)));
    }
    const uint32_t nsel = ordered_positions(bsel, pos, sh.wcnt[1]);
#pragma unroll
    for (int e = 0; e < kLongEPT; ++e) {
      // the ballot of element e in wave w is mask word pair (blk * kLongBlock + e * kLongNT + 64 w) / 64
      const int s0 = blk * kLongBlock + e * kLongNT + 64 * wave;
      if (lane == 0 && s0 / 32 < nwords)
        *reinterpret_cast<uint2*>(mrow + s0 / 32) = make_uint2((uint32_t)bsel[e], (uint32_t)(bsel[e] >> 32));
      if (irow && ((bsel[e] >> lane) & 1ull) && sel_before + pos[e] < k) irow[sel_before + pos[e]] = s0 + lane;
    }
    eq_before += neq;
    sel_before += nsel;
    __syncthreads();  // wcnt reuse
  }
  for (int wp = nblocks * (kLongBlock / 64) + tid; 2 * wp < nwords; wp += kLongNT)
    *reinterpret_cast<uint2*>(mrow + 2 * wp) = make_uint2(0u, 0u);
}


// Streaming selection for long prefill rows: the indexer first scores a
// sample of each row (every kt_stride-th 64-key tile); stream_guess_kernel
// turns it into the row's survivor threshold (as the streamed top-k above
// does with its sample); the indexer then stores only the (key, token)
// pairs reaching it, and stream_select_kernel selects from that list. The
// list holds every token whose score can be among the row's top_k as soon
// as it has at least top_k entries, so the selection is exact; rows with
// fewer (an unrepresentative sample) or more than the list holds are
// flagged, with their query tile, for the materialised scores and top-k.
struct StreamShared {
  uint32_t hist[2048];  // radix histograms, then the mask bitmap
  uint32_t red[kLongNW];
  uint32_t found[3];
};

__global__ __launch_bounds__(kLongNT) void stream_guess_kernel(StreamSelParams a) {
  __shared__ StreamShared sh;
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)b * a.T + t;
  const int p = a.q_pos0 + t, n = p + 1;
  const uint32_t k = (uint32_t)a.top_k;
  if (k >= (uint32_t)n || n <= a.cand_cap) {  // every token survives (or every token is kept)
    if (tid == 0) a.guess[row] = 0u;
    return;
  }
  const int span = 64 * a.kt_stride;  // tokens between sampled tiles
  const float* srow = a.sample + row * a.sample_ld;
  uint32_t skey[kLongEPT];
#pragma unroll
  for (int e = 0; e < kLongEPT; ++e) {
    const int j = e * kLongNT + tid;
    const int s = (j >> 6) * span + (j & 63);
    skey[e] = j < a.sample_ld && s <= p ? orderable_key(srow[min(j, a.sample_ld - 1)]) : 0u;
  }
  const int kt0 = p / span;  // last sampled tile at or before p
  const uint32_t nsv = (uint32_t)(64 * kt0 + min(p - kt0 * span + 1, 64));  // sampled tokens
  const uint32_t ks = min(nsv, (uint32_t)((1.25f * (float)k * (float)nsv) / (float)n) + 16u);
  uint32_t thr, rem;
  int shift;
  bool all_eq;
  long_radix_select([&](auto f) {
#pragma unroll
    for (int e = 0; e < kLongEPT; ++e) f(skey[e]);
  }, ks, sh.hist, sh.red, sh.found, thr, shift, rem, all_eq);
  if (tid == 0) a.guess[row] = shift >= 10 ? thr << (shift - 10) : thr >> (10 - shift);
}

__global__ __launch_bounds__(kLongNT) void stream_select_kernel(StreamSelParams a) {
  __shared__ StreamShared sh;
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)b * a.T + t;
  const int p = a.q_pos0 + t, n = p + 1;
  const int nwords = a.Lpad / 32;
  uint32_t* mrow = a.mask + row * nwords;
  int32_t* irow = a.indices ? a.indices + row * a.top_k : nullptr;
  const uint32_t k = (uint32_t)a.top_k;
  if (k >= (uint32_t)n) {  // every candidate is kept
    for (int wi = tid; wi < nwords; wi += kLongNT) {
      const int lo = wi * 32;
      mrow[wi] = lo + 32 <= n ? 0xffffffffu : (lo < n ? (1u << (n - lo)) - 1u : 0u);
    }
    if (irow)
      for (int j = tid; j < a.top_k; j += kLongNT) irow[j] = j < n ? j : -1;
    return;
  }
  const uint32_t cnt = a.cand_count[row];
  if (cnt < k || cnt > (uint32_t)a.cand_cap) {
    if (tid == 0) {
      a.row_flag[row] = 1u;
      a.tile_flag[(size_t)b * a.nqt + t / kIdxQueryTile] = 1u;
    }
    return;
  }
  const uint2* lst = a.cand + row * a.cand_cap;
  // k-th largest key among the survivors
  uint32_t thr, rem;
  int shift;
  bool all_eq;
  long_radix_select([&](auto f) {
    for (uint32_t j = tid; j < cnt; j += kLongNT) f(lst[j].x);
  }, k, sh.hist, sh.red, sh.found, thr, shift, rem, all_eq);
  // ties at the threshold: the rem lowest tokens, i.e. the rem largest of
  // 65536 - token among the threshold-equal survivors (tokens are distinct)
  uint32_t tthr = 0;
  int tshift = 0;
  if (!all_eq) {
    uint32_t trem;
    bool tall;
    long_radix_select([&](auto f) {
      for (uint32_t j = tid; j < cnt; j += kLongNT) {
        const uint2 e = lst[j];
        f((e.x >> shift) == thr ? 65536u - e.y : 0u);
      }
    }, rem, sh.hist, sh.red, sh.found, tthr, tshift, trem, tall);
  }
  for (int i = tid; i < nwords; i += kLongNT) sh.hist[i] = 0u;  // bitmap
  __syncthreads();
  for (uint32_t j = tid; j < cnt; j += kLongNT) {
    const uint2 e = lst[j];
    const uint32_t hk = e.x >> shift;
    const bool sel = hk > thr || (hk == thr && (all_eq || ((65536u - e.y) >> tshift) >= tthr));
    if (sel) atomicOr(&sh.hist[e.y >> 5], 1u << (e.y & 31));
  }
  __syncthreads();
  for (int i = tid; i < nwords; i += kLongNT) mrow[i] = sh.hist[i];
  if (irow) {  // ascending: each thread takes a run of consecutive words
    constexpr int WPT = 2048 / kLongNT;
    const int w0 = tid * WPT;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) c += w0 + i < nwords ? (uint32_t)__popc(sh.hist[w0 + i]) : 0u;
    uint32_t pos = block_inclusive_sum<kLongNW>(c, sh.red) - c;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      uint32_t bits = w0 + i < nwords ? sh.hist[w0 + i] : 0u;
      while (bits) {
        const int bit = __ffs(bits) - 1;
        if (pos < k) irow[pos] = 32 * (w0 + i) + bit;
        ++pos;
        bits &= bits - 1u;
      }
    }
  }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t launch_topk(const TopkParams& p0, hipStream_t st) {
  TopkParams p = p0;
  const int nmax = p.q_pos0 + p.T;  // longest candidate row in the call
  // Rows t < top_k - q_pos0 keep every candidate. When they are at most half
  // of the call (and every sequence shares q_pos0, and every row is wanted),
  // each rides along with a selecting row: grid T - pair_keep.
  const int n_keep = std::min(std::max(p.top_k - p.q_pos0, 0), p.T);
  p.pair_keep = (!p.seq_len && !p.row_flag && n_keep > 0 && 2 * n_keep <= p.T) ? n_keep : 0;
  dim3 grid(p.T, p.B);
  // Many long rows: stream each row through a small workgroup (several rows
  // per CU) with a sampled threshold; its survivors fit the LDS for top_k up
  // to 2048.
  if (nmax > 16384 && nmax <= kTopkMaxRow && p.top_k <= 2048 && (long long)p.B * p.T >= 512) {
    p.pair_keep = 0;
    hipLaunchKernelGGL(topk_long_kernel<false>, grid, dim3(kLongNT), 0, st, p);
    return hipGetLastError();
  }
  // Rows past the register-resident limit always stream (any row count or
  // top_k: survivors beyond the LDS take the exact passes over the row).
  if (nmax > kTopkMaxRow) {
    if (nmax > kTopkMaxRowBig || p.Lpad > kTopkMaxRowBig) return hipErrorInvalidValue;
    p.pair_keep = 0;
    hipLaunchKernelGGL(topk_long_kernel<true>, grid, dim3(kLongNT), 0, st, p);
    return hipGetLastError();
  }
  grid.x = p.T - p.pair_keep;
  // Rows are latency-bound chains of barriers and LDS histograms, so the
  // smallest workgroup that holds a row (keys in registers) wins: more rows
  // are then in flight per CU.
  if (nmax <= 2048)
    hipLaunchKernelGGL((topk_mask_kernel<4, 8, 0>), grid, dim3(256), 0, st, p);
  else if (nmax <= 4096)
    hipLaunchKernelGGL((topk_mask_kernel<4, 16, 0>), grid, dim3(256), 0, st, p);
  else if (nmax <= 8192)
    hipLaunchKernelGGL((topk_mask_kernel<4, 32, 0>), grid, dim3(256), 0, st, p);
  else if (nmax <= 16384)
    hipLaunchKernelGGL((topk_mask_kernel<8, 32, 0>), grid, dim3(512), 0, st, p);
  else if (nmax <= 32768)
    hipLaunchKernelGGL((topk_mask_kernel<16, 32, 0>), grid, dim3(1024), 0, st, p);
  else if (nmax <= kTopkMaxRow)
    hipLaunchKernelGGL((topk_mask_kernel<16, 32, 32>), grid, dim3(1024), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_stream_guess(const StreamSelParams& p, hipStream_t st) {
  if (p.sample_ld > kLongEPT * kLongNT || p.q_pos0 + p.T > kTopkMaxRow) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_guess_kernel, dim3(p.T, p.B), dim3(kLongNT), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_stream_select(const StreamSelParams& p, hipStream_t st) {
  if (p.Lpad > 2048 * 32 || p.q_pos0 + p.T > kTopkMaxRow) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_select_kernel, dim3(p.T, p.B), dim3(kLongNT), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace dsa
