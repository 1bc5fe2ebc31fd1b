// Lightning-indexer scoring on gfx950 matrix cores.
//
//   scores[b][i][s] = sum_h w[b][i][h] * max(0, qidx[b][i][h] . kidx[b][s]),  s <= p = q_pos0 + i
//
// The indexer scores every earlier token for each query [aiaulis para 2]; 32
// heads of key dim 128, no RoPE [aiu "What happened"; devotd section 1 table];
// one key per cached token in the indexer-key cache [devotd section 2]. The
// pages print no formula: the ReLU-weighted head sum above is the reading
// this library implements.
//
// Per query the heads form the M dimension of an MFMA (two 16-row blocks
// cover 32 heads), keys the N dimension (16 per MFMA) and the indexer dim the
// K dimension. The ReLU * w head sum runs on the accumulators in registers:
// each lane owns 8 heads of one key, and two permlane swaps finish the sum
// over the four 16-lane rows while packing four queries into one wave-wide
// result (one score per lane), which is then stored.
//
// Two kernels share that inner step:
//  - indexer_prefill_kernel: 8 waves x 4 queries per workgroup; 64-key tiles
//    staged in LDS (double-buffered) and reused by all 32 queries.
//  - indexer_decode_kernel: few queries per sequence; each wave streams its
//    own 16-key subtiles straight from HBM into MFMA operands (every key is
//    used once per query group, so LDS staging would only add traffic).
#include <algorithm>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr int QPW = 4;  // queries per wave (the swap-based head sum packs up to four)

// max(x, 0) as one integer max on the bit pattern: negative floats (and -0)
// are negative as int32, so they become +0; non-negative floats pass
// unchanged. One instruction, where fmaxf also quiets NaNs first.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <typename T, int DI, int NQ>
struct QueryFrags {
  static constexpr int KSTEPS = DI / kStepElems<T>;
  frag_t<T> a[NQ][2][KSTEPS];  // A operands: heads 16*rb + (l%16), dims frag_off(kk, l/16) + e
  float w[NQ][2][4];           // weights of the heads this lane's accumulators hold
};

// Loads the A fragments and head weights of queries t_first .. t_first+NQ-1.
// Queries past T and heads past H_I read a valid row (finite data). Heads
// past H_I get weight 0, so they add exact zeros to their query's sum; a
// query past T only lands in lanes whose score is never stored, so its
// weights stay as loaded. Every load is unconditional and issued before any
// of them is used, so they all share one memory round trip; with 32 or more
// heads nothing waits for them here.
template <typename T, int DI, int NQ>
__device__ __forceinline__ void load_queries(QueryFrags<T, DI, NQ>& f, const IndexerParams& a, int b,
                                             int t_first, int c, int g) {
  const size_t row_b = (size_t)b * (a.T_ld > 0 ? a.T_ld : a.T) + a.row0;  // memory row of scored query 0
  const T* qb = static_cast<const T*>(a.qidx) + row_b * a.HI * DI;
  const float* wb = a.w + row_b * a.HI;
  float wr[NQ][2][4];
  // 32 heads: the four weights of heads 16*rb + 4*g + (0..3) are one aligned 16-byte load
  const bool all_heads = a.HI == 32 && ((reinterpret_cast<uintptr_t>(wb) & 15) == 0);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int tc = min(t_first + j, a.T - 1);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int head = min(16 * rb + c, a.HI - 1);
#pragma unroll
      for (int kk = 0; kk < QueryFrags<T, DI, NQ>::KSTEPS; ++kk)
        f.a[j][rb][kk] = load_frag<T>(qb + ((size_t)tc * a.HI + head) * DI + frag_off<T>(kk, g));
      // weights of heads 16*rb + 4*g + (0..3)
      if (all_heads) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(wb + (size_t)tc * 32 + 16 * rb + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) wr[j][rb][r] = w4[r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) wr[j][rb][r] = wb[(size_t)tc * a.HI + min(16 * rb + 4 * g + r, a.HI - 1)];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        f.w[j][rb][r] = all_heads ? wr[j][rb][r] : (16 * rb + 4 * g + r < a.HI ? wr[j][rb][r] : 0.f);
}

// Scores of the wave's (up to 4) queries against one 16-key subtile whose B
// operands (keys (l%16), dims 32*kk + 8*(l/16) + e) are in bf. Returns the
// score of query j(lane) = 2*(g&1) + (g>>1) and key (l%16).
// Queries past the end and heads past H_I have zero operands and zero
// weights, so they add exact zeros; every query and both head blocks are
// computed unconditionally, the 2*NQ accumulator chains interleaved per k-step.
template <typename T, int DI, int NQ>
__device__ __forceinline__ float score_subtile(const QueryFrags<T, DI, NQ>& f,
                                               const frag_t<T> (&bf)[DI / kStepElems<T>]) {
  f32x4 acc[NQ][2];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[j][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < DI / kStepElems<T>; ++kk) {
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) acc[j][rb] = mma_kstep(f.a[j][rb][kk], bf[kk], acc[j][rb]);
    // keep the 2*NQ independent chains interleaved (the scheduler would
    // otherwise run them one after another, exposing the MFMA latency)
    __builtin_amdgcn_sched_barrier(0);
  }
  float part[QPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    part[j] = 0.f;
    if (j < NQ) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[j] = fmaf(f.w[j][rb][r], relu(acc[j][rb][r]), part[j]);
    }
  }
  // Sum over the four 16-lane rows (head groups) and pack the 4 queries.
  swap32(part[0], part[1]);
  float x = part[0] + part[1];  // lanes 0-31: query 0, lanes 32-63: query 1 (half reduced)
  swap32(part[2], part[3]);
  float y = part[2] + part[3];  // queries 2, 3
  swap16(x, y);
  return (x + y) + 0.f;         // rows 0..3 -> queries 0, 2, 1, 3; "+0" turns -0 into +0
}

// Prefill work is cut into units (sequence b, 32-query tile qt, 64-key tile
// kt), kt covering keys 0..p_last of the query tile, ordered b, qt, kt. A
// fixed grid of workgroups (one per CU) takes equal contiguous ranges of
// units, so every CU gets the same amount of matrix work whatever the causal
// shape, and a workgroup reloads its queries' q fragments only when its range
// crosses into the next query tile.
#ifndef DSA_IDX_WAVES
#define DSA_IDX_WAVES 8
#endif
#ifndef DSA_IDX_WG_PER_CU
#define DSA_IDX_WG_PER_CU 1
#endif
constexpr int kIdxWaves = DSA_IDX_WAVES;      // waves per workgroup, 4 queries each
constexpr int kIdxQT = kIdxWaves * QPW;      // 32 queries per query tile
#ifndef DSA_IDX_KT
#define DSA_IDX_KT 64
#endif
constexpr int kIdxKT = DSA_IDX_KT;            // keys per key tile
static_assert(kIdxKT % kIdxQT == 0, "query tile divides key tile");
static_assert((kIdxKT & (kIdxKT - 1)) == 0 && (kIdxQT & (kIdxQT - 1)) == 0, "power-of-two tiles");

static_assert(kIdxQT == kIdxQueryTile, "query tile size shared with the host");

struct UnitMap {
  int T, q_pos0, nqt, nfull;
  int lk, lr;  // log2 of the keys one unit's key tile spans (kIdxKT x stride) and of that / query tile
  long long per_seq;
  __device__ __host__ int ntk(int qt) const { return ((q_pos0 + min(kIdxQT * qt + kIdxQT - 1, T - 1)) >> lk) + 1; }
  // sum over x < n of floor(x / R), R = 2^lr = key tile span / query tile
  __device__ __host__ long long floor_sum(long long n) const {
    const long long m = n >> lr;
    return ((m * (m - 1) / 2) << lr) + (n - (m << lr)) * m;
  }
  // units of query tiles 0..n-1. A full query tile qt has
  // floor((A + QT qt) / span) + 1 key tiles, A = q_pos0 + QT - 1; with
  // A = a0 span + rq QT + rr (rr < QT) that is a0 + 1 + floor((qt + rq) / R).
  __device__ __host__ long long prefix(int n) const {
    const int A = q_pos0 + kIdxQT - 1, a0 = A >> lk, rq = (A & ((1 << lk) - 1)) / kIdxQT;
    const long long k = min(n, nfull);
    long long s = k * (a0 + 1) + floor_sum(rq + k) - floor_sum(rq);
    if (n > nfull) s += ntk(nfull);
    return s;
  }
  // Query tiles are visited short and long alternately (position i holds
  // tile i/2 for even i, nqt-1-i/2 for odd i), so that any run of units
  // crosses few query tiles and the q-fragment reloads spread evenly over
  // the workgroups' equal ranges.
  __device__ __host__ int qt_at(int i) const { return (i & 1) ? nqt - 1 - (i >> 1) : (i >> 1); }
  // units of positions 0..n-1: tiles 0..ceil(n/2)-1 and nqt-floor(n/2)..nqt-1
  __device__ __host__ long long prefix_pos(int n) const {
    return prefix((n + 1) >> 1) + per_seq - prefix(nqt - (n >> 1));
  }
  // stride > 1 (a power of two): only every stride-th key tile (a sample of the keys)
  __device__ __host__ void init(int T_, int q_pos0_, int stride = 1) {
    T = T_;
    q_pos0 = q_pos0_;
    lk = 0;
    while ((1 << lk) < kIdxKT * (stride > 1 ? stride : 1)) ++lk;
    lr = lk;
    while ((1 << (lk - lr)) < kIdxQT) --lr;
    nqt = (T + kIdxQT - 1) / kIdxQT;
    nfull = T / kIdxQT;
    per_seq = prefix(nqt);
  }
  // (b, position, kt) of unit u
  __device__ void decode(long long u, int& b, int& pos, int& kt) const {
    b = (int)(u / per_seq);
    const long long v = u - (long long)b * per_seq;
    int lo = 0, hi = nqt - 1;  // largest position with prefix_pos(pos) <= v
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix_pos(mid) <= v) lo = mid;
      else hi = mid - 1;
    }
    pos = lo;
    kt = (int)(v - prefix_pos(lo));
  }
};

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_wave_base + 16 l (lds_wave_base is the same for the whole wave).
__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_wave_base, 16, 0, 0);
}
// The same with 4 bytes per lane (lane l's word lands at lds_wave_base + 4 l).
__device__ __forceinline__ void dma4(const void* src, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_wave_base, 4, 0, 0);
}

// B fragment (elements 32 kk + 8 g .. +7) of a key row stored with its
// 16-byte chunks permuted by XOR with sw.
template <typename T> __device__ __forceinline__ frag_t<T> lds_frag(const unsigned char* rowp, int kk, int g, int sw);
template <> __device__ __forceinline__ bf16x8 lds_frag<bf16>(const unsigned char* rowp, int kk, int g, int sw) {
  return *reinterpret_cast<const bf16x8*>(rowp + (((4 * kk + g) ^ sw) << 4));
}
template <> __device__ __forceinline__ i32x8 lds_frag<fp8e4m3>(const unsigned char* rowp, int kk, int g, int sw) {
  // codes 128 kk + 32 g .. +31: 16-byte chunks 8 kk + 2 g and 8 kk + 2 g + 1
  const u32x4 lo = *reinterpret_cast<const u32x4*>(rowp + (((8 * kk + 2 * g) ^ sw) << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(rowp + (((8 * kk + 2 * g + 1) ^ sw) << 4));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
template <> __device__ __forceinline__ f32x8 lds_frag<float>(const unsigned char* rowp, int kk, int g, int sw) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(rowp + (((8 * kk + 2 * g) ^ sw) << 4));
  const f32x4 hi = *reinterpret_cast<const f32x4*>(rowp + (((8 * kk + 2 * g + 1) ^ sw) << 4));
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

#ifndef DSA_IDX_STAGES
#define DSA_IDX_STAGES 3
#endif
constexpr int kIdxStages = DSA_IDX_STAGES;  // key tiles in the LDS ring (kIdxStages - 1 in flight)
static_assert(kIdxStages >= 2 && kIdxStages <= 6, "LDS ring depth");

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Key tiles go from HBM (L2 in practice: every tile is reused by all query
// tiles) straight into LDS with global_load_lds, 16 bytes per lane, through
// a ring of kIdxStages tiles: the tiles of the next kIdxStages-1 units are in
// flight while the current one is scored. Every iteration issues the same
// number of tile loads (past the end of the range the last tile is loaded
// again), after the score stores, so "tile u+1 has landed" is a count: at
// most (kIdxStages-2) x loads-per-tile operations may still be outstanding
// (a wave that loads nothing for a tile has nothing to wait for). The
// workgroup barrier carries no memory fence, so the scores stored earlier
// are not waited for. A tile's rows are stored unpadded, each row's 16-byte
// chunks permuted (physical chunk = chunk ^ (row mod CH16)) so that the 16
// lanes reading one chunk column of 16 consecutive rows hit distinct banks.
// The scores of a unit are stored one unit late, after the next tile loads
// are issued.
// STREAM: survivor lists instead of stored scores (a.guess set)
template <typename T, int DI, bool STREAM>
__global__ __launch_bounds__(64 * kIdxWaves) void indexer_prefill_kernel(IndexerParams a, UnitMap um,
                                                                          long long n_units) {
  constexpr int KT = kIdxKT, KSTEPS = DI / kStepElems<T>, NSUB = KT / 16, S = kIdxStages;
  constexpr int ROWB = DI * (int)sizeof(T), CH16 = ROWB / 16;
  constexpr int TILEB = KT * ROWB, NINST = TILEB / 1024;  // 1 KiB (64 lanes x 16 B) per instruction
  static_assert(TILEB % 1024 == 0 && (CH16 & (CH16 - 1)) == 0, "tile layout");
  // fp8 keys carry one float32 scale per key: every wave keeps its own copy
  // of the tile's 64 scales after the key rows (so every wave issues the
  // same number of loads per tile and waits for its own)
  constexpr bool kFp8 = kStepElems<T> == 128;
  constexpr int SLOT = TILEB + (kFp8 ? 256 * kIdxWaves : 0);
  static_assert(!kFp8 || KT == 64, "one 4-byte scale per lane per tile");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[S * SLOT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round-robin; the 1/8 of the unit
  // sequence an XCD works on is contiguous, so neighbouring ranges (which
  // share query tiles) share that XCD's L2.
  const int G = gridDim.x;
  const int r = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const long long u0 = (long long)r * n_units / G;
  const long long u1 = (long long)(r + 1) * n_units / G;
  if (u0 >= u1) return;
  if (a.tile_flag) {  // score the range only when one of its query tiles is flagged
    int fb, fpos, fkt;
    um.decode(u0, fb, fpos, fkt);
    bool any = false;
    for (long long tu = u0; tu < u1;) {
      any = any || a.tile_flag[fb * um.nqt + um.qt_at(fpos)] != 0u;
      tu = (long long)fb * um.per_seq + um.prefix_pos(fpos + 1);  // first unit of the next tile
      if (++fpos == um.nqt) {
        fpos = 0;
        ++fb;
      }
    }
    if (!any) return;
  }
  const int kstride = a.kt_stride > 1 ? a.kt_stride : 1;  // key tiles scored: kstride * kt
  const float ninf = fneg_inf();
  const int jl = ((g & 1) << 1) | (g >> 1);  // query of the wave whose score this lane ends up with

  // Loader: instruction j (waves take j = wave, wave + NW, ...) fills LDS
  // bytes [1024 j, 1024 j + 1024) of a ring slot; lane l writes physical
  // chunk L % CH16 of row L / CH16 (L = 64 j + l) and so fetches the logical
  // chunk the permutation puts there. Rows past n_kv read the last cached
  // key: finite data whose scores are never stored.
  constexpr int NJ = (NINST + kIdxWaves - 1) / kIdxWaves;
  constexpr bool kAllWavesLoad = NINST % kIdxWaves == 0;
  constexpr int NLD = NJ + (kFp8 ? 1 : 0);  // loads per wave per tile
  static_assert(kAllWavesLoad || NINST < kIdxWaves, "tile loads split evenly or fit in one round");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy, kept in a scalar register
  uint32_t dl_off[NJ];  // byte offset of this lane's 16 bytes from the tile's first key row
  int dl_row[NJ];
#pragma unroll
  for (int n = 0; n < NJ; ++n) {
    const int L = (wave_u + n * kIdxWaves) * 64 + lane;
    dl_row[n] = L / CH16;
    dl_off[n] = (uint32_t)(dl_row[n] * ROWB + (((L % CH16) ^ (dl_row[n] & (CH16 - 1))) << 4));
  }
  const char* kcache = static_cast<const char*>(a.kidx);
  auto dload = [&](int b, int kt, int slot) {
    const int s0 = kt * kstride * KT;
    const char* kb = kcache + ((size_t)b * a.kv_cap + s0) * ROWB;
    unsigned char* dst = lds + slot * SLOT;
    if constexpr (kFp8) dma4(a.kscale + (size_t)b * a.kv_cap + min(s0 + lane, a.n_kv - 1), dst + TILEB + wave_u * 256);
    if (s0 + KT <= a.n_kv) {
#pragma unroll
      for (int n = 0; n < NJ; ++n) {
        const int j = wave_u + n * kIdxWaves;
        if (kAllWavesLoad || j < NINST) dma16(kb + dl_off[n], dst + j * 1024);
      }
    } else {  // last tile of the cache: rows past n_kv read the last cached key
#pragma unroll
      for (int n = 0; n < NJ; ++n) {
        const int j = wave_u + n * kIdxWaves;
        const int over = max(s0 + dl_row[n] - (a.n_kv - 1), 0);
        if (kAllWavesLoad || j < NINST) dma16(kb + dl_off[n] - (size_t)over * ROWB, dst + j * 1024);
      }
    }
  };
  // B operand of key subtile sub: row 16 sub + c, elements 32 kk + 8 g .. +7
  auto load_b = [&](int slot, int sub, frag_t<T> (&bf)[KSTEPS]) {
    const int row = sub * 16 + c;
    const unsigned char* rowp = lds + slot * SLOT + row * ROWB;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) bf[kk] = lds_frag<T>(rowp, kk, g, row & (CH16 - 1));
  };
  // unit cursor: (b, position, kt) -> the next unit; qt = um.qt_at(position)
  auto advance = [&](int& b, int& pos, int& kt) {
    if (++kt == um.ntk(um.qt_at(pos))) {
      kt = 0;
      if (++pos == um.nqt) {
        pos = 0;
        ++b;
      }
    }
  };

  int b, qp, kt;
  um.decode(u0, b, qp, kt);
  QueryFrags<T, DI, QPW> f;
  int cur_b = -1, cur_qt = -1;
  int t_wave = 0, p_wave_last = -1, p_mine = 0;
  float* srow = nullptr;  // this lane's score row, or nullptr when its query is past T
  // scores of the previous unit, stored one unit late
  float pend[NSUB];
  float* pend_row = nullptr;
  int pend_s0 = 0, pend_c0 = 0, pend_p = 0;
  // streaming selection: this lane's row (or -1) and its survivor threshold
  int row_mine = -1, pend_rowid = -1;
  uint32_t guess_mine = 0, pend_guess = 0;
  // the queries of query tile qt of sequence b: this wave's q fragments,
  // head weights and output row
  auto switch_tile = [&](int b, int qt) {
    cur_b = b;
    cur_qt = qt;
    t_wave = qt * kIdxQT + wave * QPW;
    const int nq = max(0, min(QPW, a.T - t_wave));
    p_wave_last = a.q_pos0 + t_wave + nq - 1;
    load_queries<T, DI, QPW>(f, a, b, t_wave, c, g);
    const int t_mine = t_wave + jl;
    p_mine = a.q_pos0 + t_mine;
    srow = t_mine < a.T && !STREAM
               ? a.scores + ((size_t)b * (a.T_ld > 0 ? a.T_ld : a.T) + a.row0 + t_mine) * a.Lpad
               : nullptr;
    if constexpr (STREAM) {
      row_mine = t_mine < a.T ? b * a.T + t_mine : -1;
      guess_mine = row_mine >= 0 ? a.guess[row_mine] : 0u;
    }
  };
  // Prologue: tiles of units u0 .. u0+S-2 (clamped to the range's last
  // unit), then the first query tile's fragments, all in flight together.
  int pb = b, ppos = qp, pkt = kt;  // prefetch cursor: the unit whose tile was loaded last
  long long pu = u0;
  dload(pb, pkt, 0);
#pragma unroll
  for (int i = 1; i < S - 1; ++i) {
    if (pu + 1 < u1) {
      advance(pb, ppos, pkt);
      ++pu;
    }
    dload(pb, pkt, i);
  }
  switch_tile(b, um.qt_at(qp));

  auto flush = [&]() {
    if constexpr (STREAM) {
      // survivors (key prefix reaching the row's guess) appended to the row's
      // list: ranks within the 16 lanes of one query, one atomic per row and unit
      uint32_t keys[NSUB];
      uint32_t cnt = 0;
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        const int s = pend_s0 + sub * 16 + c;
        keys[sub] = orderable_key(pend[sub]);
        const bool sv = pend_rowid >= 0 && s <= pend_p && (keys[sub] >> 10) >= pend_guess;
        if (!sv) keys[sub] = 0u;
        cnt += sv ? 1u : 0u;
      }
      uint32_t incl = cnt;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)incl, off, 16);
        if (c >= off) incl += o;
      }
      const uint32_t total = (uint32_t)__shfl((int)incl, 15, 16);
      uint32_t base = 0;
      if (c == 15 && total > 0u) base = atomicAdd(a.cand_count + pend_rowid, total);
      base = (uint32_t)__shfl((int)base, 15, 16);
      uint32_t at = base + incl - cnt;
      uint2* lst = a.cand + (size_t)max(pend_rowid, 0) * a.cand_cap;
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        if (keys[sub] != 0u) {
          if (at < (uint32_t)a.cand_cap) lst[at] = make_uint2(keys[sub], (uint32_t)(pend_s0 + sub * 16 + c));
          ++at;
        }
      }
    } else if (pend_row) {
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        const int s = pend_s0 + sub * 16 + c, col = pend_c0 + sub * 16 + c;
        // scores are streamed out with non-temporal stores (read once, by top-k)
        if (s <= pend_p) __builtin_nontemporal_store(pend[sub], pend_row + col);
        else if (a.write_upper) __builtin_nontemporal_store(ninf, pend_row + col);
      }
    }
  };
  // Every prologue load landed: the query fragments (issued last) and so the
  // tiles before them. With no fragment load outstanding when the unit loop
  // starts, its matrix instructions wait for LDS only; a fragment load left
  // in flight would make the compiler wait for every load in flight (the
  // tile prefetches included) in front of every unit's matrix work.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  int slot = 0;
  for (long long u = u0; u < u1; ++u) {
    const int qt = um.qt_at(qp);
    if (b != cur_b || qt != cur_qt) {
      switch_tile(b, qt);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the new fragments, once (see the prologue)
    }
    // stores of unit u-1, then the tile of unit u+S-1 (or the range's last
    // one again) into the slot read at unit u-1: the newest S-2 tile loads
    // are then the last operations issued when tile u+1 is waited for
    flush();
    if (pu + 1 < u1) {
      advance(pb, ppos, pkt);
      ++pu;
    }
    dload(pb, pkt, slot == 0 ? S - 1 : slot - 1);

    const int s_tile = kt * kstride * KT;
    float cur[NSUB];
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      cur[sub] = ninf;
      if (t_wave < a.T && s_tile + sub * 16 <= p_wave_last) {
        frag_t<T> bf[KSTEPS];
        load_b(slot, sub, bf);
        cur[sub] = score_subtile<T, DI, QPW>(f, bf);
        if constexpr (kFp8)
          cur[sub] *= *reinterpret_cast<const float*>(lds + slot * SLOT + TILEB + wave * 256 + 4 * (sub * 16 + c));
      }
    }
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) pend[sub] = cur[sub];
    pend_row = srow;
    pend_s0 = s_tile;
    pend_c0 = kt * KT;
    pend_p = p_mine;
    pend_rowid = row_mine;
    pend_guess = guess_mine;

    // Tile u+1 has landed in every wave's part (each wave waits for its own
    // loads; the S-2 tiles issued after it may still be in flight) before
    // any wave reads it, and every wave is done with slot `slot` before it
    // is refilled.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * NLD));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    slot = slot == S - 1 ? 0 : slot + 1;
    advance(b, qp, kt);
  }
  flush();
  // no tile load may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);
}

// -inf for the columns past each query tile's last key tile (scores rows of
// index_scores are written in full; the prefill kernel writes key tiles
// 0..ntk(qt)-1 only). One workgroup per query row.
__global__ __launch_bounds__(256) void scores_upper_fill_kernel(IndexerParams a, UnitMap um) {
  const int row = blockIdx.x, t = row % a.T, b = row / a.T;
  const int s_from = um.ntk(t / kIdxQT) << um.lk;
  float* srow = a.scores + ((size_t)b * (a.T_ld > 0 ? a.T_ld : a.T) + a.row0 + t) * a.Lpad;
  const float ninf = fneg_inf();
  for (int s4 = s_from + 4 * threadIdx.x; s4 < a.Lpad; s4 += 4 * 256)
    *reinterpret_cast<f32x4*>(srow + s4) = f32x4{ninf, ninf, ninf, ninf};
}

// Few queries per sequence: grid (key chunks, ceil(T/NQ), B), 4 waves; wave w
// takes 16-key subtiles w, w+4, ... of the chunk, two at a time, loading the
// B operands directly from the key cache.
template <typename T, int DI, int NQ>
__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerParams a) {
  constexpr int NT = 256, KSTEPS = DI / kStepElems<T>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int b = blockIdx.z, t_first = blockIdx.y * NQ, s_begin = blockIdx.x * a.key_chunk;
  int q_pos0, n_kv;
  seq_extent(a.seq_len, b, a.T, a.q_pos0, a.n_kv, q_pos0, n_kv);
  const int nq = min(NQ, a.T - t_first);
  const int p_last = q_pos0 + t_first + nq - 1;
  const int s_chunk_end = min(s_begin + a.key_chunk, a.Lpad);
  const int s_stop = min(s_chunk_end, p_last + 1);
  float* scores_b = a.scores + ((size_t)b * (a.T_ld > 0 ? a.T_ld : a.T) + a.row0) * a.Lpad;
  const float ninf = fneg_inf();
  const int jl = ((g & 1) << 1) | (g >> 1);
  const int t_mine = jl < nq ? t_first + jl : a.T;  // a.T: this lane stores nothing
  const int p_mine = q_pos0 + t_mine;
  float* srow = scores_b + (size_t)t_mine * a.Lpad;

  if (s_begin < s_stop) {
    QueryFrags<T, DI, NQ> f;
    load_queries<T, DI, NQ>(f, a, b, t_first, c, g);
    const T* kb = static_cast<const T*>(a.kidx) + (size_t)b * a.kv_cap * DI;
    const int n_sub = (s_stop - s_begin + 15) / 16;
    auto load_b = [&](int sub, frag_t<T> (&bf)[KSTEPS]) {
      const int s = s_begin + sub * 16 + c;
      const bool sv = s < n_kv;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        bf[kk] = sv ? load_frag<T>(kb + (size_t)s * DI + frag_off<T>(kk, g)) : zero_frag<T>();
    };
    auto emit = [&](int sub, const frag_t<T> (&bf)[KSTEPS]) {
      float e = score_subtile<T, DI, NQ>(f, bf);
      const int s = s_begin + sub * 16 + c;
      if constexpr (kStepElems<T> == 128) e *= a.kscale[(size_t)b * a.kv_cap + min(s, n_kv - 1)];
      if (t_mine < a.T) {
        if (s <= p_mine) __builtin_nontemporal_store(e, srow + s);
        else if (a.write_upper) __builtin_nontemporal_store(ninf, srow + s);
      }
    };
    for (int sub = wave; sub < n_sub; sub += 8) {
      frag_t<T> b0[KSTEPS], b1[KSTEPS];
      load_b(sub, b0);
      const bool has1 = sub + 4 < n_sub;
      if (has1) load_b(sub + 4, b1);
      emit(sub, b0);
      if (has1) emit(sub + 4, b1);
    }
    if (a.write_upper && t_mine < a.T) {
      for (int s = s_begin + n_sub * 16 + tid % 16; s < s_chunk_end; s += 16)
        if (tid < 64) srow[s] = ninf;
    }
  } else if (a.write_upper) {
    const int ncol = s_chunk_end - s_begin;
    for (int i = tid; i < nq * ncol; i += NT)
      scores_b[(size_t)(t_first + i / ncol) * a.Lpad + s_begin + i % ncol] = ninf;
  }
}

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <typename T, int DI>
hipError_t launch_indexer_t(const IndexerParams& p, hipStream_t st) {
  IndexerParams q = p;
  if (p.T == 1) {
    q.key_chunk = 512;
    dim3 grid((p.Lpad + q.key_chunk - 1) / q.key_chunk, p.T, p.B);
    hipLaunchKernelGGL((indexer_decode_kernel<T, DI, 1>), grid, dim3(256), 0, st, q);
  } else if (p.T <= 8) {
    q.key_chunk = 512;
    dim3 grid((p.Lpad + q.key_chunk - 1) / q.key_chunk, (p.T + QPW - 1) / QPW, p.B);
    hipLaunchKernelGGL((indexer_decode_kernel<T, DI, QPW>), grid, dim3(256), 0, st, q);
  } else {
    UnitMap um;
    um.init(p.T, p.q_pos0, p.kt_stride);
    const long long n_units = um.per_seq * p.B;
    if (p.write_upper) {
      hipLaunchKernelGGL(scores_upper_fill_kernel, dim3(p.B * p.T), dim3(256), 0, st, q, um);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int n_wg = (int)std::min<long long>(n_units, (long long)device_cu_count() * DSA_IDX_WG_PER_CU);
    if (p.guess)
      hipLaunchKernelGGL((indexer_prefill_kernel<T, DI, true>), dim3(n_wg), dim3(64 * kIdxWaves), 0, st, q, um, n_units);
    else
      hipLaunchKernelGGL((indexer_prefill_kernel<T, DI, false>), dim3(n_wg), dim3(64 * kIdxWaves), 0, st, q, um,
                         n_units);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerParams& p, int dtype, int DI, hipStream_t st) {
  if (dtype == kIndexerFp8) return DI == 128 && p.kscale ? launch_indexer_t<fp8e4m3, 128>(p, st) : hipErrorInvalidValue;
  if (dtype == 1) {
    if (DI == 128) return launch_indexer_t<bf16, 128>(p, st);
    if (DI == 64) return launch_indexer_t<bf16, 64>(p, st);
    if (DI == 32) return launch_indexer_t<bf16, 32>(p, st);
  } else {
    if (DI == 64) return launch_indexer_t<float, 64>(p, st);
    if (DI == 32) return launch_indexer_t<float, 32>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
