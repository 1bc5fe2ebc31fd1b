// Per-row top-k selection written as a bitmask over the whole cache (and an
// ascending index list): the workgroup-level routine shared by the top-k
// kernel and the fused decode kernel.
//
// Each query keeps its top_k best-scored earlier tokens [aiaulis paras 2-3;
// devotd section 1 table, 2048 tokens] and the selection is applied as a
// mask over the whole cache rather than by gathering rows [aiaulis para 4;
// devotd section 2]. Ties go to the lower token index; -0.0 equals +0.0.
//
// One workgroup per query row. The row's candidate scores (s <= p) are held
// on chip as order-preserving 32-bit keys (the first EPT_R per lane in
// registers, the rest, for the longest rows, in LDS): wave w owns tokens
// [w*EPT*64, (w+1)*EPT*64), element e of lane l is token w*EPT*64 + e*64 + l,
// so a wave ballot over element e is exactly one 64-bit mask word. A radix
// select (11 + 11 + 10 bits, LDS histograms) finds the key of the k-th
// largest score (or only its leading digits, once the bin holding it is
// kept whole) and how many of the tokens equal to it are kept; when only
// some of the equal tokens are kept, their ranks in index order come from
// ballots, a per-wave prefix and a workgroup scan. The row is read from HBM
// once.
#pragma once

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

template <int NW, int EPT_L> struct TopkShared {
  uint32_t hist[2048];
  uint32_t lkeys[EPT_L > 0 ? EPT_L * NW * 64 : 1];  // element e >= EPT_R of thread tid
  uint32_t red[NW];
  uint32_t found[3];
};

// Inclusive scan over the workgroup; red must hold NW words.
template <int NW>
__device__ __forceinline__ uint32_t block_inclusive_sum(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_inclusive_sum(v);
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) base += red[w];
  __syncthreads();
  return base + inc;
}

// Selects row t of sequence b (one workgroup of NW waves per row).
template <int NW, int EPT_R, int EPT_L>
__device__ __forceinline__ void topk_select_row(const TopkParams& a, int t, int b, TopkShared<NW, EPT_L>& sh) {
  constexpr int NT = NW * 64, EPT = EPT_R + EPT_L;
  static_assert(EPT_L % 16 == 0, "LDS-held elements load 16 at a time");
  uint32_t* hist = sh.hist;
  uint32_t* lkeys = sh.lkeys;
  uint32_t* red = sh.red;
  uint32_t* found = sh.found;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int q_pos0, n_kv;
  seq_extent(a.seq_len, b, a.T, a.q_pos0, a.n_kv, q_pos0, n_kv);
  const int p = q_pos0 + t, n = p + 1;
  const size_t row = (size_t)b * a.T + t;
  const int nwords = a.Lpad / 32;
  const float* srow = a.scores + row * a.Lpad;
  uint32_t* mrow = a.mask + row * nwords;
  int32_t* irow = a.indices ? a.indices + row * a.top_k : nullptr;

  if (a.top_k >= n) {  // every candidate is kept
    for (int wi = tid; wi < nwords; wi += NT) {
      const int lo = wi * 32;
      mrow[wi] = lo + 32 <= n ? 0xffffffffu : (lo < n ? (1u << (n - lo)) - 1u : 0u);
    }
    if (irow)
      for (int j = tid; j < a.top_k; j += NT) irow[j] = j < n ? j : -1;
    return;
  }

  // Loads are unconditional (positions past the row read its last candidate,
  // then become the "no token" key 0), so they all stay in flight together
  // instead of each waiting behind a branch.
  // The scheduling barriers keep each batch of loads together ahead of its
  // conversions, which the scheduler would otherwise pair one by one.
  const int base = wave * EPT * 64;
  auto to_key = [&](float v, int idx) -> uint32_t { return idx < n ? orderable_key(v) : 0u; };
  uint32_t rkey[EPT_R];
  if (EPT_L > 0) {  // LDS-held elements first, 16 loads in flight at a time
#pragma unroll 1
    for (int e0 = EPT_R; e0 < EPT; e0 += 16) {
      float v16[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v16[j] = srow[min(base + (e0 + j) * 64 + lane, n - 1)];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 16; ++j) lkeys[(e0 + j - EPT_R) * NT + tid] = to_key(v16[j], base + (e0 + j) * 64 + lane);
    }
  }
  {
    float v[EPT_R];
#pragma unroll
    for (int e = 0; e < EPT_R; ++e) v[e] = srow[min(base + e * 64 + lane, n - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < EPT_R; ++e) rkey[e] = to_key(v[e], base + e * 64 + lane);
  }
  // e is a compile-time constant at every use, so this picks a register or LDS.
  auto key = [&](int e) -> uint32_t { return e < EPT_R ? rkey[e < EPT_R ? e : 0] : lkeys[(e - EPT_R) * NT + tid]; };

  // Radix select of the k-th largest key.
  uint32_t prefix = 0;
  uint32_t rem = (uint32_t)a.top_k;  // rank of the threshold within the current candidates
  uint32_t count_eq = 0;
  int thr_shift = 0;  // the threshold is a prefix: keys compare as key >> thr_shift
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < nbins; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      // key 0 marks "no token" (no finite score maps to 0, and its high
      // digits never equal a selected prefix, which is a finite key's).
      const uint32_t k = key(e);
      const bool cand = pass == 0 ? k != 0u : (pass == 1 ? (k >> 21) == prefix : (k >> 10) == prefix);
      if (cand) atomicAdd(&hist[(k >> shift) & (nbins - 1)], 1u);
    }
    __syncthreads();
    // Thread tid owns bins [nbins - (tid+1)*bpt, nbins - tid*bpt), highest first.
    const int bpt = nbins / NT;
    const int top = nbins - tid * bpt;
    uint32_t local = 0;
    for (int d = top - 1; d >= top - bpt; --d) local += hist[d];
    const uint32_t incl = block_inclusive_sum<NW>(local, red);
    uint32_t cum = incl - local;  // tokens in bins above this thread's range
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
    // Every token of the threshold's bin is kept: the prefix already
    // separates kept from dropped tokens, and the later digits need not be
    // resolved (the usual case after 22 bits on continuous scores).
    if (pass < 2 && rem == count_eq) {
      thr_shift = shift;
      break;
    }
  }
  const uint32_t thr = prefix;
  const bool all_eq = rem == count_eq;  // every token equal to the threshold (prefix) is kept

  // Index-order rank base of this wave's threshold-equal tokens.
  uint32_t eq_base = 0;
  if (!all_eq) {
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) cnt += __popcll(ballot64((key(e) >> thr_shift) == thr));
    if (lane == 0) red[wave] = cnt;
    __syncthreads();
    for (int w = 0; w < wave; ++w) eq_base += red[w];
    __syncthreads();
  }

  // Selection of element e, in index order within the wave. The running
  // count of threshold-equal tokens gives each tie its rank.
  const uint64_t lt = lanemask_lt();
  auto select = [&](int e, uint32_t& running_eq) -> bool {
    const uint32_t k = key(e);
    // thr is a finite key's prefix: never that of the 0 sentinel, whose every
    // prefix is 0 (finite keys are at least 0x00800000)
    const bool eq = (k >> thr_shift) == thr;
    bool s = (k >> thr_shift) > thr;
    if (all_eq) return s || eq;
    const uint64_t be = ballot64(eq);
    s = s || (eq && running_eq + (uint32_t)__popcll(be & lt) < rem);
    running_eq += (uint32_t)__popcll(be);
    return s;
  };

  // Mask words: the ballot over element e is the word pair of tokens
  // [base + 64e, base + 64e + 64).
  // Lane e keeps the ballot of element e (one mask word pair), so the pairs
  // are stored by all lanes at once and the index list is built per word.
  static_assert(EPT <= 64, "one mask word pair per lane");
  uint32_t running_eq = eq_base, nsel = 0;
  uint64_t my_pair = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint64_t bs = ballot64(select(e, running_eq));
    nsel += (uint32_t)__popcll(bs);
    if (lane == e) my_pair = bs;
  }
  if (lane < EPT && 2 * (wave * EPT + lane) < nwords)
    *reinterpret_cast<uint2*>(mrow + 2 * (wave * EPT + lane)) = make_uint2((uint32_t)my_pair, (uint32_t)(my_pair >> 32));
  for (int wp = NW * EPT + tid; 2 * wp < nwords; wp += NT)
    *reinterpret_cast<uint2*>(mrow + 2 * wp) = make_uint2(0u, 0u);

  if (irow) {  // exactly top_k tokens are kept here
    if (lane == 0) red[wave] = nsel;
    __syncthreads();
    uint32_t off = 0;
    for (int w = 0; w < wave; ++w) off += red[w];
    if (4 * a.top_k < n) {
      // Sparse rows: word pair e = lane covers tokens base + 64 lane + (0..63);
      // each lane writes the few kept tokens of its own word.
      const uint32_t cnt = (uint32_t)__popcll(my_pair);
      uint32_t pos = off + wave_inclusive_sum(cnt) - cnt;
      uint64_t bits = my_pair;
      while (bits) {
        const int bit = __ffsll((unsigned long long)bits) - 1;
        if (pos < (uint32_t)a.top_k) irow[pos] = base + lane * 64 + bit;
        ++pos;
        bits &= bits - 1ull;
      }
    } else {
      // Dense rows: element by element, consecutive lanes writing consecutive
      // positions.
      running_eq = eq_base;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const bool sel = select(e, running_eq);
        const uint64_t bs = ballot64(sel);
        const uint32_t pos = off + (uint32_t)__popcll(bs & lt);
        if (sel && pos < (uint32_t)a.top_k) irow[pos] = base + e * 64 + lane;
        off += (uint32_t)__popcll(bs);
      }
    }
  }
}

}  // namespace dsa
