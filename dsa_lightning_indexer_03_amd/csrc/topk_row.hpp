// Per-row top-k selection written as a bitmask over the whole cache (and an
// ascending index list): the workgroup-level routines shared by the top-k
// kernels.
//
// Each query keeps its top_k best-scored earlier tokens [aiaulis paras 2-3;
// devotd section 1 table, 2048 tokens] and the selection is applied as a
// mask over the whole cache rather than by gathering rows [aiaulis para 4;
// devotd section 2]. Ties go to the lower token index; -0.0 equals +0.0.
//
// Scores are held and compared as floats (NaN marks "no token"; float
// comparison already treats -0.0 and +0.0 as equal). The k-th largest score
// of a row (select_kth) is found in two steps:
//  1. a histogram of 2048 bins laid linearly over the row's [min, max] score
//     (a monotone map of the value, so bins are ordered like the scores)
//     gives the bin holding the k-th largest score and its rank inside it;
//     on continuous scores that bin holds a few tokens, and the bins spread
//     the LDS atomics instead of piling them onto the handful of bins that a
//     float's top bits would give;
//  2. a bin of at most 64 tokens is resolved directly: its tokens are
//     gathered into one wave's lanes and each lane counts the tokens ranked
//     above its own (larger score, or equal score and lower index). A larger
//     bin (heavy ties, outliers, infinities) is resolved by exact radix
//     passes over the order-preserving 32-bit keys of its tokens (11, 11 and
//     10 bits), down to the full key.
// The result is the threshold score, how many of the tokens equal to it are
// kept and whether that is all of them; kept tokens are those above it plus,
// among those equal to it, the first ones in index order.
#pragma once

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

constexpr int kSelBins = 2048;   // histogram bins of one select pass
constexpr int kSelDirect = 64;   // largest threshold bin resolved by ranking its tokens

template <int NW, int NBUF> struct SelectShared {
  // NBUF = 2: a pass zeroes the next pass's histogram, saving a barrier.
  // The 64 words past the bins take the counts of lanes without a
  // candidate (one word per lane, never read), which keeps the counting
  // branch-free.
  alignas(16) uint32_t hist[NBUF][kSelBins + 64];
  uint32_t red[NW];               // scan partials
  float vmm[2][NW];               // per-wave min / max score
  uint32_t found[3];              // threshold bin, tokens in bins above it, tokens in it
  uint32_t ncand;
  uint2 cand[kSelDirect];         // (key, token) of the threshold bin's tokens
};

struct KthResult {
  float val;      // the k-th largest score
  uint32_t rem;   // tokens equal to val that are kept (the first rem in index order)
  bool all_eq;    // every token equal to val is kept
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

// Whole-wave reductions and scans on DPP lane moves (the device library's
// wave functions), cheaper than LDS-routed shuffles; every lane must be
// active. The reductions return a wave-uniform value; the float ones skip
// NaN.
extern "C" __device__ float __ockl_wfred_min_f32(float);
extern "C" __device__ float __ockl_wfred_max_f32(float);
extern "C" __device__ uint32_t __ockl_wfscan_add_u32(uint32_t, bool);
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) { return __ockl_wfscan_add_u32(v, true); }

// A value every lane holds alike, read from LDS: moved to a scalar register
// so that loops and branches on it are uniform.
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ float uniform_f32(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Lanes below this one whose bit is set in a wave ballot.
__device__ __forceinline__ uint32_t ballot_rank(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// The float value of a nonzero orderable key (inverse of orderable_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ float no_token() { return __uint_as_float(0x7fc00000u); }

// Word 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data format,
// no swizzle): loads past the descriptor's byte count return 0 and stores
// past it are dropped.
constexpr int kBufferWord3 = 0x00020000;

// k-th largest score (k = rank >= 1) over the scores for_each visits:
// for_each(f) calls f(score, token) for each of this thread's elements
// (NaN = no token), with tokens distinct and ordered like the token
// indices. At least `rank` tokens must exist. Every thread of the workgroup
// calls it; a barrier must separate it from earlier uses of sh, and waves
// may still read sh when it returns.
template <int NW, int NBUF, typename ForEach>
__device__ __forceinline__ KthResult select_kth(ForEach for_each, uint32_t rank, SelectShared<NW, NBUF>& sh) {
  constexpr int NT = NW * 64;
  constexpr int BPT = kSelBins / NT;  // histogram bins scanned per thread
  static_assert(BPT == 2 || BPT == 4 || BPT == 8, "bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t spare = (uint32_t)(kSelBins + lane);  // the count word of a lane without a candidate

  // Both histograms are cleared first (16-byte stores), while the caller's
  // loads of the scores may still be in flight.
  {
    constexpr int kWords = NBUF * (kSelBins + 64);
    static_assert(kWords % 4 == 0, "whole 16-byte stores");
    uint4* hz = reinterpret_cast<uint4*>(&sh.hist[0][0]);
    for (int i = tid; i < kWords / 4; i += NT) hz[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  // Score range of the row: three-operand min / max over pairs of
  // elements, one instruction per element for both bounds (IEEE mode: a
  // quiet NaN, the "no token" mark, loses to any number). Written as single
  // instructions because fminf / fmaxf first canonicalise every operand.
  float lo = __uint_as_float(0x7f800000u), hi = -lo;
  {
    float held = lo;
    int n_seen = 0;  // a compile-time count once for_each is unrolled
    for_each([&](float v, uint32_t) {
      if (n_seen & 1) {
        asm("v_min3_f32 %0, %1, %2, %3" : "=v"(lo) : "v"(lo), "v"(held), "v"(v));
        asm("v_max3_f32 %0, %1, %2, %3" : "=v"(hi) : "v"(hi), "v"(held), "v"(v));
      } else {
        held = v;
      }
      ++n_seen;
    });
    if (n_seen & 1) {
      asm("v_min_f32 %0, %1, %2" : "=v"(lo) : "v"(lo), "v"(held));
      asm("v_max_f32 %0, %1, %2" : "=v"(hi) : "v"(hi), "v"(held));
    }
  }
  lo = __ockl_wfred_min_f32(lo);
  hi = __ockl_wfred_max_f32(hi);
  if (tid == 0) sh.ncand = 0u;
  if (lane == 0) {
    sh.vmm[0][wave] = lo;
    sh.vmm[1][wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = fminf(lo, sh.vmm[0][w]);
    hi = fmaxf(hi, sh.vmm[1][w]);
  }
  lo = uniform_f32(lo);
  hi = uniform_f32(hi);
  // Bin of a score: linear over [min, max], v * scale - lo * scale as one
  // fused multiply-add, clamped to [0, 2047] by a median of three and
  // truncated. A rounded fma with a positive factor never reverses an order,
  // so the bins are ordered like the scores. A range that is empty or
  // overflows gives a factor of inf or 0 and the results NaN or 0 (the
  // median takes NaN to 0) or inf (bin 2047): still ordered, and the exact
  // passes decide.
  const float scale = (float)kSelBins / (hi - lo);
  const float offset = -lo * scale;
  auto bin_of = [offset, scale](float v) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_fmed3f(fmaf(v, scale, offset), 0.0f, (float)(kSelBins - 1));
  };
  // Each pass folds its own opaque zero into the scores, so the compiler
  // recomputes bins and keys where they are needed instead of keeping values
  // per element live in registers across the passes.
  auto opaque_zero = []() {
    uint32_t z = 0u;
    asm volatile("" : "+v"(z));
    return z;
  };

  uint32_t rem = rank, d0 = 0, prefix = 0, count_eq = 0;
  int shift = 0;  // key shift of the prefix matched so far (passes >= 1)
  int dpass = 0;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    // pass 0: score bins; passes 1-3: key bits 31..21, 20..10, 9..0 of the
    // threshold bin's tokens
    uint32_t* h = sh.hist[NBUF == 2 ? (pass & 1) : 0];
    if (pass > 0) {
      if (NBUF == 1) {
        for (int i = tid; i < kSelBins; i += NT) h[i] = 0u;
        __syncthreads();
      } else if (pass < 3) {  // the next pass's histogram (last read before this pass's first barrier)
        uint32_t* hn = sh.hist[(pass + 1) & 1];
        for (int i = tid; i < kSelBins; i += NT) hn[i] = 0u;
      }
    }
    const int dshift = pass == 1 ? 21 : (pass == 2 ? 10 : 0);
    const uint32_t dmask = pass == 3 ? 1023u : 2047u;
    const uint32_t z = opaque_zero();
    for_each([&](float v0, uint32_t) {
      // pass 0 takes the scores as they are (the later passes and the
      // gather below fold in their own zero)
      const float v = pass == 0 ? v0 : __uint_as_float(__float_as_uint(v0) ^ z);
      const bool tok = v == v;
      const uint32_t b = bin_of(v);
      if (pass == 0) {
        atomicAdd(&h[tok ? b : spare], 1u);
      } else {
        const uint32_t k = orderable_key(v);
        const bool c = tok && b == d0 && (pass == 1 || (k >> shift) == prefix);
        atomicAdd(&h[c ? (k >> dshift) & dmask : spare], 1u);
      }
    });
    __syncthreads();
    // Thread tid owns bins [kSelBins - (tid+1)*BPT, kSelBins - tid*BPT), highest first.
    const int b0 = kSelBins - (tid + 1) * BPT;
    uint32_t local = 0;
    if constexpr (BPT == 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(h + b0), y = *reinterpret_cast<const uint4*>(h + b0 + 4);
      local = x.x + x.y + x.z + x.w + y.x + y.y + y.z + y.w;
    } else if constexpr (BPT == 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(h + b0);
      local = x.x + x.y + x.z + x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(h + b0);
      local = x.x + x.y;
    }
    // workgroup scan (red is next written after this pass's last barrier)
    const uint32_t inc = wave_scan_u32(local);
    if (lane == 63) sh.red[wave] = inc;
    __syncthreads();
    uint32_t cum = inc - local;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) cum += sh.red[w];
    if (cum < rem && rem <= cum + local) {  // the one thread whose bins hold the rank
      for (int j = BPT - 1; j >= 0; --j) {
        const uint32_t hj = h[b0 + j];
        if (rem <= cum + hj) {
          sh.found[0] = (uint32_t)(b0 + j);
          sh.found[1] = cum;
          sh.found[2] = hj;
          break;
        }
        cum += hj;
      }
    }
    __syncthreads();
    const uint32_t d = uniform_u32(sh.found[0]);
    rem -= uniform_u32(sh.found[1]);
    count_eq = uniform_u32(sh.found[2]);
    if (pass == 0) {
      d0 = d;
    } else {
      prefix = pass == 1 ? d : ((prefix << (pass == 2 ? 11 : 10)) | d);
      shift = dshift;
    }
    if (pass == 3) return KthResult{key_value(prefix), rem, rem == count_eq};
    if (count_eq <= (uint32_t)kSelDirect) {
      dpass = pass;
      break;
    }
  }

  // Rank the threshold bin's tokens directly (dpass: the last pass taken).
  // Keys are formed only for the bin's tokens. The gather recomputes the
  // histogram's bins with the same arithmetic, so exactly count_eq tokens
  // arrive; the slot bound only keeps the writes inside the array.
  const uint32_t zc = opaque_zero();
  if (dpass == 0) {
    for_each([&](float v0, uint32_t id) {
      const float v = __uint_as_float(__float_as_uint(v0) ^ zc);
      if (v == v && bin_of(v) == d0) {
        const uint32_t slot = atomicAdd(&sh.ncand, 1u);
        if (slot < (uint32_t)kSelDirect) sh.cand[slot] = make_uint2(orderable_key(v), id);
      }
    });
  } else {
    for_each([&](float v0, uint32_t id) {
      const float v = __uint_as_float(__float_as_uint(v0) ^ zc);
      const uint32_t k = orderable_key(v);
      if (v == v && bin_of(v) == d0 && (k >> shift) == prefix) {
        const uint32_t slot = atomicAdd(&sh.ncand, 1u);
        if (slot < (uint32_t)kSelDirect) sh.cand[slot] = make_uint2(k, id);
      }
    });
  }
  __syncthreads();
  const bool mine = (uint32_t)lane < count_eq;
  const uint2 c = mine ? sh.cand[lane] : make_uint2(0u, 0xffffffffu);
  uint32_t above = 0;  // tokens of the bin ranked above this lane's
  for (uint32_t i = 0; i < count_eq; ++i) {
    const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)c.x, (int)i);
    const uint32_t ii = (uint32_t)__builtin_amdgcn_readlane((int)c.y, (int)i);
    above += (ki > c.x || (ki == c.x && ii < c.y)) ? 1u : 0u;
  }
  const uint64_t at = ballot64(mine && above == rem - 1u);
  const uint32_t tkey = (uint32_t)__builtin_amdgcn_readlane((int)c.x, (int)(__ffsll((unsigned long long)at) - 1));
  const uint32_t gt = (uint32_t)__popcll(ballot64(mine && c.x > tkey));
  const uint32_t eq = (uint32_t)__popcll(ballot64(mine && c.x == tkey));
  return KthResult{key_value(tkey), rem - gt, eq == rem - gt};
}

// A row whose candidates (n of them) are all kept: mask bits [0, n), and the
// index list 0 .. n-1 padded with -1.
template <int NT>
__device__ __forceinline__ void keep_all_row(const TopkParams& a, int n, uint32_t* mrow, int32_t* irow) {
  const int nwords = a.Lpad / 32;
  for (int wi = threadIdx.x; wi < nwords; wi += NT) {
    const int lo = wi * 32;
    mrow[wi] = lo + 32 <= n ? 0xffffffffu : (lo < n ? (1u << (n - lo)) - 1u : 0u);
  }
  if (irow)
    for (int j = threadIdx.x; j < a.top_k; j += NT) irow[j] = j < n ? j : -1;
}

template <int NW, int EPT_L> struct TopkShared {
  SelectShared<NW, 2> sel;
  float lvals[EPT_L > 0 ? EPT_L * NW * 64 : 1];  // element e >= EPT_R of thread tid
  uint32_t eqc[NW];   // per-wave threshold-equal counts
  uint32_t selc[NW];  // per-wave kept counts
};

// Selects row t of sequence b (one workgroup of NW waves per row). The row's
// candidate scores (s <= p) are held on chip: the first EPT_R per lane in
// registers, the rest, for the longest rows, in LDS. Wave w owns tokens
// [w*EPT*64, (w+1)*EPT*64), element e of lane l is token w*EPT*64 + e*64 + l,
// so a wave ballot over element e is exactly one 64-bit mask word. The row
// is read from HBM once.
template <int NW, int EPT_R, int EPT_L>
__device__ __forceinline__ void topk_select_row(const TopkParams& a, int t, int b, TopkShared<NW, EPT_L>& sh) {
  constexpr int NT = NW * 64, EPT = EPT_R + EPT_L;
  static_assert(EPT_L % 16 == 0, "LDS-held elements load 16 at a time");
  float* lvals = sh.lvals;

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
    keep_all_row<NT>(a, n, mrow, irow);
    return;
  }

  // Loads are unconditional (positions past the row read its last candidate,
  // then become "no token"), so they all stay in flight together instead of
  // each waiting behind a branch.
  // The scheduling barriers keep each batch of loads together ahead of its
  // conversions, which the scheduler would otherwise pair one by one.
  // The row is read through a buffer descriptor bounded to its n
  // candidates: one offset register per lane, each element's 256-byte step
  // in the instruction's immediate offset, and loads past the row return 0
  // (then marked "no token"), so every load is unconditional and they all
  // stay in flight together. The scheduling barriers keep each batch of
  // loads together ahead of its conversions, which the scheduler would
  // otherwise pair one by one.
  const int base = wave * EPT * 64;
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc((void*)srow, (short)0, n * 4, kBufferWord3);
  const int voff = (base + lane) * 4;
  auto to_val = [&](float v, int idx) -> float { return idx < n ? v : no_token(); };
  float rval[EPT_R];
  if (EPT_L > 0) {  // LDS-held elements first, 16 loads in flight at a time
#pragma unroll 1
    for (int e0 = EPT_R; e0 < EPT; e0 += 16) {
      float v16[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v16[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srsrc, voff + (e0 + j) * 256, 0, 0));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 16; ++j) lvals[(e0 + j - EPT_R) * NT + tid] = to_val(v16[j], base + (e0 + j) * 64 + lane);
    }
  }
  {
    float v[EPT_R];
#pragma unroll
    for (int e = 0; e < EPT_R; ++e) v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srsrc, voff + e * 256, 0, 0));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < EPT_R; ++e) rval[e] = to_val(v[e], base + e * 64 + lane);
  }
  // e is a compile-time constant at every use, so this picks a register or LDS.
  auto val = [&](int e) -> float { return e < EPT_R ? rval[e < EPT_R ? e : 0] : lvals[(e - EPT_R) * NT + tid]; };

  const KthResult th = select_kth<NW, 2>([&](auto f) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) f(val(e), (uint32_t)(base + e * 64 + lane));
  }, (uint32_t)a.top_k, sh.sel);

  // Index-order rank base of this wave's threshold-equal tokens.
  uint32_t eq_base = 0;
  if (!th.all_eq) {
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) cnt += __popcll(ballot64(val(e) == th.val));
    if (lane == 0) sh.eqc[wave] = cnt;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) eq_base += w < wave ? sh.eqc[w] : 0u;
  }

  // Selection of element e, in index order within the wave. The running
  // count of threshold-equal tokens gives each tie its rank. ("No token"
  // is NaN, which compares false.)
  auto select = [&](int e, uint32_t& running_eq) -> bool {
    const float v = val(e);
    if (th.all_eq) return v >= th.val;
    const bool eq = v == th.val;
    const uint64_t be = ballot64(eq);
    const bool s = v > th.val || (eq && running_eq + ballot_rank(be) < th.rem);
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
    if (lane == 0) sh.selc[wave] = nsel;
    __syncthreads();
    uint32_t off = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) off += w < wave ? sh.selc[w] : 0u;
    if (4 * a.top_k < n) {
      // Sparse rows: word pair e = lane covers tokens base + 64 lane + (0..63);
      // each lane writes the few kept tokens of its own word.
      const uint32_t cnt = (uint32_t)__popcll(my_pair);
      uint32_t pos = off + wave_scan_u32(cnt) - cnt;
      uint64_t bits = my_pair;
      while (bits) {
        const int bit = __ffsll((unsigned long long)bits) - 1;
        if (pos < (uint32_t)a.top_k) irow[pos] = base + lane * 64 + bit;
        ++pos;
        bits &= bits - 1ull;
      }
    } else {
      // Dense rows: element by element, consecutive lanes writing consecutive
      // positions, through a descriptor bounded to the list's top_k entries:
      // lanes that keep nothing store past its end, which the hardware drops.
      const __amdgpu_buffer_rsrc_t irsrc =
          __builtin_amdgcn_make_buffer_rsrc((void*)irow, (short)0, a.top_k * 4, kBufferWord3);
      running_eq = eq_base;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const bool sel = select(e, running_eq);
        const uint64_t bs = ballot64(sel);
        const uint32_t pos = sel ? off + ballot_rank(bs) : 0x3fffffffu;
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(base + e * 64 + lane), irsrc, (int)(pos * 4u), 0, 0);
        off += (uint32_t)__popcll(bs);
      }
    }
  }
}

}  // namespace dsa
