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
  static constexpr int KSTEPS = DI / 32;
  frag_t<T> a[NQ][2][KSTEPS];  // A operands: heads 16*rb + (l%16), dims 32*kk + 8*(l/16) + e
  float w[NQ][2][4];           // weights of the heads this lane's accumulators hold
};

// Loads the A fragments and head weights of queries t_first .. t_first+NQ-1.
template <typename T, int DI, int NQ>
__device__ __forceinline__ void load_queries(QueryFrags<T, DI, NQ>& f, const IndexerParams& a, int b,
                                             int t_first, int c, int g) {
  const T* qb = static_cast<const T*>(a.qidx) + (size_t)b * a.T * a.HI * DI;
  const float* wb = a.w + (size_t)b * a.T * a.HI;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int t = t_first + j;
    const bool tv = t < a.T;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int head = 16 * rb + c;
      const bool hv = tv && head < a.HI;
#pragma unroll
      for (int kk = 0; kk < QueryFrags<T, DI, NQ>::KSTEPS; ++kk)
        f.a[j][rb][kk] = hv ? load_frag<T>(qb + ((size_t)t * a.HI + head) * DI + 32 * kk + 8 * g)
                            : zero_frag<T>();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h2 = 16 * rb + 4 * g + r;
        f.w[j][rb][r] = (tv && h2 < a.HI) ? wb[(size_t)t * a.HI + h2] : 0.f;
      }
    }
  }
}

// Scores of the wave's (up to 4) queries against one 16-key subtile whose B
// operands (keys (l%16), dims 32*kk + 8*(l/16) + e) are in bf. Returns the
// score of query j(lane) = 2*(g&1) + (g>>1) and key (l%16).
// Queries past the end and heads past H_I have zero operands and zero
// weights, so they add exact zeros; every query and both head blocks are
// computed unconditionally, the 2*NQ accumulator chains interleaved per k-step.
template <typename T, int DI, int NQ>
__device__ __forceinline__ float score_subtile(const QueryFrags<T, DI, NQ>& f,
                                               const frag_t<T> (&bf)[DI / 32]) {
  f32x4 acc[NQ][2];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[j][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < DI / 32; ++kk) {
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

// Launch shape of the prefill kernel: waves per workgroup (4 queries each),
// keys per LDS tile and keys per workgroup.
#ifndef DSA_IDX_WAVES
#define DSA_IDX_WAVES 8
#endif
#ifndef DSA_IDX_KT
#define DSA_IDX_KT 64
#endif
#ifndef DSA_IDX_CHUNK
#define DSA_IDX_CHUNK 2048
#endif
constexpr int kIdxWaves = DSA_IDX_WAVES, kIdxKT = DSA_IDX_KT, kIdxChunk = DSA_IDX_CHUNK;
static_assert(kIdxChunk % kIdxKT == 0 && kIdxKT % 16 == 0, "key chunk is whole tiles of 16-key subtiles");

template <typename T, int DI>
__global__ __launch_bounds__(64 * kIdxWaves) void indexer_prefill_kernel(IndexerParams a) {
  constexpr int NT = 64 * kIdxWaves, QT = kIdxWaves * QPW, KT = kIdxKT, KSTEPS = DI / 32;
  constexpr int ROWB = DI * (int)sizeof(T), PITCH = ROWB + 16, CH16 = ROWB / 16;
  constexpr int TOT16 = KT * CH16, N16 = (TOT16 + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * KT * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int b = blockIdx.z, t0 = blockIdx.y * QT, s_begin = blockIdx.x * a.key_chunk;
  const int t_end = min(t0 + QT, a.T);
  const int p_last = a.q_pos0 + t_end - 1;
  const int s_chunk_end = min(s_begin + a.key_chunk, a.Lpad);
  const int s_stop = min(s_chunk_end, p_last + 1);
  float* scores_b = a.scores + (size_t)b * a.T * a.Lpad;
  const float ninf = fneg_inf();
  int s_filled = s_begin;

  if (s_begin < s_stop) {
    const int t_wave = t0 + wave * QPW;
    const int nq = max(0, min(QPW, a.T - t_wave));
    const int p_wave_last = a.q_pos0 + t_wave + nq - 1;
    QueryFrags<T, DI, QPW> f;
    load_queries<T, DI, QPW>(f, a, b, t_wave, c, g);
    const int jl = ((g & 1) << 1) | (g >> 1);
    const int t_mine = t_wave + jl;
    const int p_mine = a.q_pos0 + t_mine;
    float* srow = scores_b + (size_t)t_mine * a.Lpad;

    const T* kb = static_cast<const T*>(a.kidx) + (size_t)b * a.kv_cap * DI;
    const int n_tiles = (s_stop - s_begin + KT - 1) / KT;
    u32x4 stg[N16];
    auto gload = [&](int tile) {
      const int s0 = s_begin + tile * KT;
#pragma unroll
      for (int n = 0; n < N16; ++n) {
        const int i = tid + n * NT;
        if (i < TOT16) {
          const int s = s0 + i / CH16;
          stg[n] = s < a.n_kv ? *reinterpret_cast<const u32x4*>(
                                    reinterpret_cast<const char*>(kb + (size_t)s * DI) + (i % CH16) * 16)
                              : u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int n = 0; n < N16; ++n) {
        const int i = tid + n * NT;
        if (i < TOT16)
          *reinterpret_cast<u32x4*>(lds + buf * KT * PITCH + (i / CH16) * PITCH + (i % CH16) * 16) = stg[n];
      }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int it = 0; it < n_tiles; ++it) {
      const int buf = it & 1;
      if (it + 1 < n_tiles) gload(it + 1);
      const int s_tile = s_begin + it * KT;
      auto load_b = [&](int sub, frag_t<T> (&bf)[KSTEPS]) {
        const unsigned char* rowp = lds + buf * KT * PITCH + (sub * 16 + c) * PITCH;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
          bf[kk] = load_frag<T>(reinterpret_cast<const T*>(rowp + (32 * kk + 8 * g) * (int)sizeof(T)));
      };
      auto store = [&](int s, float e) {
        if (t_mine < a.T) {
          if (s <= p_mine) srow[s] = e;
          else if (a.write_upper) srow[s] = ninf;
        }
      };
      if (nq > 0 && s_tile + KT - 1 <= p_wave_last) {
        // Whole tile below the wave's last query: the next subtile's key
        // fragments are read from LDS while this one's MFMAs run.
        frag_t<T> bf[2][KSTEPS];
        load_b(0, bf[0]);
#pragma unroll
        for (int sub = 0; sub < KT / 16; ++sub) {
          if (sub + 1 < KT / 16) load_b(sub + 1, bf[(sub + 1) & 1]);
          store(s_tile + sub * 16 + c, score_subtile<T, DI, QPW>(f, bf[sub & 1]));
        }
      } else {
#pragma unroll
        for (int sub = 0; sub < KT / 16; ++sub) {
          const int s_sub = s_tile + sub * 16;
          const int s = s_sub + c;
          if (nq > 0 && s_sub <= p_wave_last) {
            frag_t<T> bf[KSTEPS];
            load_b(sub, bf);
            store(s, score_subtile<T, DI, QPW>(f, bf));
          } else if (a.write_upper && t_mine < a.T) {
            srow[s] = ninf;
          }
        }
      }
      if (it + 1 < n_tiles) lstore(buf ^ 1);
      __syncthreads();
    }
    s_filled = s_begin + n_tiles * KT;
  }
  if (a.write_upper && s_filled < s_chunk_end) {
    // rows t0..t_end-1, columns s_filled..s_chunk_end-1 (a multiple of 16): one
    // wave per row, 4 floats per lane
    for (int t = t0 + wave; t < t_end; t += NT / 64)
      for (int s4 = s_filled + 4 * lane; s4 < s_chunk_end; s4 += 256)
        *reinterpret_cast<f32x4*>(scores_b + (size_t)t * a.Lpad + s4) = f32x4{ninf, ninf, ninf, ninf};
  }
}

// Few queries per sequence: grid (key chunks, ceil(T/NQ), B), 4 waves; wave w
// takes 16-key subtiles w, w+4, ... of the chunk, two at a time, loading the
// B operands directly from the key cache.
template <typename T, int DI, int NQ>
__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerParams a) {
  constexpr int NT = 256, KSTEPS = DI / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int b = blockIdx.z, t_first = blockIdx.y * NQ, s_begin = blockIdx.x * a.key_chunk;
  const int nq = min(NQ, a.T - t_first);
  const int p_last = a.q_pos0 + t_first + nq - 1;
  const int s_chunk_end = min(s_begin + a.key_chunk, a.Lpad);
  const int s_stop = min(s_chunk_end, p_last + 1);
  float* scores_b = a.scores + (size_t)b * a.T * a.Lpad;
  const float ninf = fneg_inf();
  const int jl = ((g & 1) << 1) | (g >> 1);
  const int t_mine = jl < nq ? t_first + jl : a.T;  // a.T: this lane stores nothing
  const int p_mine = a.q_pos0 + t_mine;
  float* srow = scores_b + (size_t)t_mine * a.Lpad;

  if (s_begin < s_stop) {
    QueryFrags<T, DI, NQ> f;
    load_queries<T, DI, NQ>(f, a, b, t_first, c, g);
    const T* kb = static_cast<const T*>(a.kidx) + (size_t)b * a.kv_cap * DI;
    const int n_sub = (s_stop - s_begin + 15) / 16;
    auto load_b = [&](int sub, frag_t<T> (&bf)[KSTEPS]) {
      const int s = s_begin + sub * 16 + c;
      const bool sv = s < a.n_kv;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        bf[kk] = sv ? load_frag<T>(kb + (size_t)s * DI + 32 * kk + 8 * g) : zero_frag<T>();
    };
    auto emit = [&](int sub, const frag_t<T> (&bf)[KSTEPS]) {
      const float e = score_subtile<T, DI, NQ>(f, bf);
      const int s = s_begin + sub * 16 + c;
      if (t_mine < a.T) {
        if (s <= p_mine) srow[s] = e;
        else if (a.write_upper) srow[s] = ninf;
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
    q.key_chunk = kIdxChunk;
    dim3 grid((p.Lpad + q.key_chunk - 1) / q.key_chunk, (p.T + kIdxWaves * QPW - 1) / (kIdxWaves * QPW), p.B);
    hipLaunchKernelGGL((indexer_prefill_kernel<T, DI>), grid, dim3(64 * kIdxWaves), 0, st, q);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerParams& p, int dtype, int DI, hipStream_t st) {
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
