// Indexer front end: the indexer's three tensors q_b, k and projection
// [aiu "What happened"; devotd section 3] turn a token's compressed query
// q_lat and its activations x into the indexer's inputs, read as linear maps
// with output-major ([out][in]) bf16 weights:
//   qidx[m][n] = sum_r q_lat[m][r] w_qb[n][r]      n = h * D_I + d
//   kidx[m][d] = sum_j x[m][j] w_k[d][j]           written into the index-key cache
//   w[m][h]    = sum_j x[m][j] w_proj[h][j]        float32
// (m = b * T + t). k and projection share their input, so they run as one
// product over the concatenated weights [w_k; w_proj].
//
// proj_gemm_kernel<Shape>: C^T = W X^T on v_mfma_f32_16x16x32_bf16. Wide
// products (many tokens, q_b) use 128 x 128 tiles of 4 waves, each wave 64
// tokens x 64 outputs (every 16-byte fragment read from LDS feeds 4 MFMAs);
// thin ones 128 x 32 tiles of 4 waves. K advances 64 at a time
// through a ring of LDS stages that global_load_lds fills straight from
// memory (one 16-byte piece per lane, 128-byte rows whose pieces are
// XOR-swizzled by row so that the fragment reads are free of bank
// conflicts). Weight rows are the MFMA A operand (outputs as M), token rows
// the B operand, so each lane ends with four consecutive outputs of one
// token: one 8-byte (bf16) or 16-byte (float32) store. Workgroups are mapped
// to tiles XCD by XCD in groups of token tiles (tile_of), so the operands a
// workgroup shares with its neighbours are in its XCD's L2.
//
// Thin products (few tokens, or only D_I + H_I outputs) split K over
// blockIdx.z into float32 partials, which proj_reduce_kernel sums in split
// order (deterministic) before the same epilogue. Calls of at most 64 tokens
// run both products' tiles in one launch and both products' sums in a
// second.
#include <algorithm>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr int kBK = 64;         // K per LDS stage
constexpr int kRowB = kBK * 2;  // bytes per tile row

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds_wave_base + 16 l.
__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

// Byte offset of 16-byte piece `piece` (0..7) of tile row `row`.
__device__ __forceinline__ int tile_off(int row, int piece) { return row * kRowB + ((piece ^ (row & 7)) << 4); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16 a = (bf16)lo, b = (bf16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return ua | ((uint32_t)ub << 16);
}

// Final store of outputs n .. n+3 (n % 4 == 0) of token m.
__device__ __forceinline__ void store_out(const ProjParams& a, int m, int n, f32x4 v) {
  if (a.mode == 0) {  // qidx [M][N0]
    if (n < a.N0)
      *reinterpret_cast<uint2*>(static_cast<bf16*>(a.out_bf16) + (size_t)m * a.N0 + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    return;
  }
  if (n < a.N0) {  // kidx into cache row (b, q_pos0 + t)
    const int b = m / a.T, t = m - b * a.T;
    bf16* dst = static_cast<bf16*>(a.out_bf16) + ((size_t)b * a.kv_cap + a.q_pos0 + t) * a.N0 + n;
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    return;
  }
  const int h = n - a.N0;  // w [M][N1]
  float* dst = a.out_f32 + (size_t)m * a.N1 + h;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (h + j < a.N1) dst[j] = v[j];
}

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// Waits until at most `newer` stages of PS loads each are outstanding
// (newer <= N; the immediate has to be a constant, hence one case each).
template <int PS, int N>
__device__ __forceinline__ void wait_stages(int newer) {
  if constexpr (N > 0) {
    if (newer >= N) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(N * PS));
      return;
    }
    wait_stages<PS, N - 1>(newer);
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

// Tile of workgroup `bid` in a 1-D grid of 8 * per_xcd: workgroups are
// dealt to the 8 XCDs round-robin (bid % 8), so each XCD gets one contiguous
// run of the tile order, and that order walks groups of kGroupM token tiles
// output-tile by output-tile: the tiles an XCD has in flight share their
// token rows and weight rows in its L2. Returns false past the last tile.
constexpr int kGroupM = 8;
__device__ __forceinline__ bool tile_of(int bid, int m_tiles, int n_tiles, int n_split, int per_xcd, int& mt, int& nt,
                                        int& z) {
  const int L = (bid & 7) * per_xcd + (bid >> 3);
  const int per_split = m_tiles * n_tiles;
  if (L >= per_split * n_split) return false;
  z = L / per_split;
  const int r = L - z * per_split;
  const int group = r / (kGroupM * n_tiles);
  const int gm = min(kGroupM, m_tiles - group * kGroupM);
  const int within = r - group * kGroupM * n_tiles;
  mt = group * kGroupM + within % gm;
  nt = within / gm;
  return true;
}

// Workgroup shape: WGM x WGN waves, each owning MB 16-token blocks x NB
// 16-output blocks; STAGES LDS buffers in the load ring.
template <int WGM_, int WGN_, int MB_, int NB_, int STAGES_>
struct ProjShape {
  static constexpr int WGM = WGM_, WGN = WGN_, MB = MB_, NB = NB_, STAGES = STAGES_;
  static constexpr int WAVES = WGM * WGN;
  static constexpr int BM = WGM * MB * 16;  // tokens per workgroup
  static constexpr int BN = WGN * NB * 16;  // outputs per workgroup
};
// 128 x 128 tiles, 4 waves of 64 x 64, two workgroups per CU (measured
// faster than 256 x 256 tiles of 8 waves of 128 x 64)
using WideShape = ProjShape<2, 2, 4, 4, 2>;
// 128 tokens x 32 outputs, 4 waves of 64 x 16, for few-token products
using ThinShape = ProjShape<2, 2, 4, 1, 3>;
// 128 tokens x 160 outputs, 4 waves of 32 x 160: every output of the k and
// projection product (D_I + H_I <= 160) in one tile; one workgroup per CU
// with three stages in flight, as these run one wave of workgroups deep
using AllOutShape = ProjShape<4, 1, 2, 10, 4>;
// Calls of at most 64 tokens (decode): 64 tokens x 64 outputs, 4 waves of
// 32 x 32, three stages (48 KiB of LDS, three workgroups per CU). Every
// workgroup reads the whole token tile for its K range, so the tile is made
// wide and K split instead (q_b: 64 output tiles x 4 splits read a quarter
// of the activation bytes that 256 tiles of 16 outputs do).
using FewShape = ProjShape<2, 2, 2, 2, 3>;
constexpr int kFewMaxM = FewShape::BM;

// One product's tiles in a launch.
struct ProjTask {
  ProjParams p;
  int m_tiles, n_tiles, n_split, per_xcd;  // workgroups 8 * per_xcd (0: no task)
};

// Sums the K-split partials of four outputs (quad i of the product) in
// split order.
__device__ __forceinline__ void reduce_quad(const ProjParams& a, int n_split, int Npad, long long i) {
  const int quads = Npad / 4;
  if (i >= (long long)a.M * quads) return;
  const int m = (int)(i / quads), n = (int)(i % quads) * 4;
  if (n >= a.N0 + a.N1) return;
  const float* src = a.partial + (size_t)m * Npad + n;
  const size_t zstride = (size_t)a.M * Npad;
  f32x4 s = *reinterpret_cast<const f32x4*>(src);
#pragma unroll 8
  for (int z = 1; z < n_split; ++z) s += *reinterpret_cast<const f32x4*>(src + z * zstride);
  store_out(a, m, n, s);
}

// Tile `bid` of one product.
template <class S>
__device__ __forceinline__ void proj_tile(const ProjParams& a, int m_tiles, int n_tiles, int n_split, int per_xcd,
                                          int bid) {
  constexpr int MB = S::MB, NB = S::NB, BM = S::BM, BN = S::BN, STAGES = S::STAGES;
  constexpr int A_BYTES = BM * kRowB;      // token tile
  constexpr int STAGE = A_BYTES + BN * kRowB;
  constexpr int A_DL = BM / 8 / S::WAVES;  // tile-load instructions per wave (8 rows each)
  constexpr int B_DL = BN / 8 / S::WAVES;
  static_assert(A_DL * 8 * S::WAVES == BM && B_DL * 8 * S::WAVES == BN, "whole 8-row loads per wave");
  constexpr int PER_STAGE = A_DL + B_DL;   // loads per wave per stage
  __shared__ __attribute__((aligned(16))) unsigned char lds[STAGES * STAGE];

  int mt, nt, z;
  if (!tile_of(bid, m_tiles, n_tiles, n_split, per_xcd, mt, nt, z)) return;  // whole workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int n0 = nt * BN, m0 = mt * BM;
  const int k0 = z * a.k_split;
  const int nk = a.k_split / kBK;
  const int N = a.N0 + a.N1;

  // Loader: instruction i of wave w fills tile rows 8 (w * DL + i) + lane / 8;
  // lane l writes physical piece l % 8, which holds logical piece
  // (l % 8) ^ (row % 8) = (l % 8) ^ (l / 8). Rows past the end read the last
  // valid row (finite data whose outputs are never stored).
  const int lp = (lane & 7) ^ (lane >> 3);
  const bf16* asrc[A_DL];
#pragma unroll
  for (int i = 0; i < A_DL; ++i) {
    const int m = min(m0 + 8 * (wave * A_DL + i) + (lane >> 3), a.M - 1);
    asrc[i] = static_cast<const bf16*>(a.x) + (size_t)m * a.K + k0 + 8 * lp;
  }
  const bf16* bsrc[B_DL];
#pragma unroll
  for (int i = 0; i < B_DL; ++i) {
    const int n = min(n0 + 8 * (wave * B_DL + i) + (lane >> 3), N - 1);
    const bf16* row = n < a.N0 ? static_cast<const bf16*>(a.w0) + (size_t)n * a.K
                               : static_cast<const bf16*>(a.w1) + (size_t)(n - a.N0) * a.K;
    bsrc[i] = row + k0 + 8 * lp;
  }
  auto dload = [&](int kt) {
    unsigned char* st = lds + (kt % STAGES) * STAGE;
#pragma unroll
    for (int i = 0; i < A_DL; ++i) dma16(asrc[i] + kt * kBK, st + (wave * A_DL + i) * 8 * kRowB);
#pragma unroll
    for (int i = 0; i < B_DL; ++i) dma16(bsrc[i] + kt * kBK, st + A_BYTES + (wave * B_DL + i) * 8 * kRowB);
  };

  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Ring of STAGES buffers, STAGES - 1 stages in flight ahead of the one
  // being multiplied.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) dload(s);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most the loads of the stages issued after
    // it (min(STAGES - 2, nk - 1 - kt) of them) are still outstanding
    const int newer = min(STAGES - 2, nk - 1 - kt);
    static_assert((STAGES - 2) * PER_STAGE <= 63, "outstanding loads fit the counter");
    wait_stages<PER_STAGE, STAGES - 2>(newer);
    // every wave's share of stage kt is visible, and every wave is done with
    // the buffer the next load overwrites (it held stage kt - 1)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES - 1 < nk) dload(kt + STAGES - 1);
    // the scheduler's small-GEMM strategy interleaves the fragment reads
    // with the MFMAs (6% faster on the 4096-token call)
    __builtin_amdgcn_iglp_opt(0);
    const unsigned char* sa = lds + (kt % STAGES) * STAGE;
    const unsigned char* sb = sa + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[MB], wf[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8*>(sa + tile_off(16 * (MB * wm + mb) + c, 4 * ks + g));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        wf[nb] = *reinterpret_cast<const bf16x8*>(sb + tile_off(16 * (NB * wn + nb) + c, 4 * ks + g));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mma_kstep(wf[nb], af[mb], acc[nb][mb]);
    }
  }

  // lane (c, g) holds outputs n = 16 nb + 4 g + r of token m = 16 mb + c
  const int Npad = n_tiles * BN;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + 16 * (MB * wm + mb) + c;
    if (m >= a.M) continue;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = n0 + 16 * (NB * wn + nb) + 4 * g;
      if (a.partial)
        *reinterpret_cast<f32x4*>(a.partial + ((size_t)z * a.M + m) * Npad + n) = acc[nb][mb];
      else if (n < N)
        store_out(a, m, n, acc[nb][mb]);
    }
  }
}

// The tiles of task t0, then (kTwo) those of task t1, in one launch.
template <class S, bool kTwo>
__global__ __launch_bounds__(64 * S::WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void proj_gemm_kernel(ProjTask t0, ProjTask t1) {
  const int bid = (int)blockIdx.x;
  if (!kTwo || bid < 8 * t0.per_xcd) {
    proj_tile<S>(t0.p, t0.m_tiles, t0.n_tiles, t0.n_split, t0.per_xcd, bid);
    return;
  }
  if constexpr (kTwo) proj_tile<S>(t1.p, t1.m_tiles, t1.n_tiles, t1.n_split, t1.per_xcd, bid - 8 * t0.per_xcd);
}

// Sums the K-split partials of four outputs per thread, in split order:
// the a_threads quads of product a first, then those of product b (b.M = 0:
// none).
__global__ __launch_bounds__(256) void proj_reduce_kernel(ProjParams a, int n_split, int Npad, ProjParams b,
                                                          int b_split, int b_Npad, long long a_threads) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < a_threads) reduce_quad(a, n_split, Npad, i);
  else reduce_quad(b, b_split, b_Npad, i - a_threads);
}

// Splits of K (a divisor of K / 64) so that the grid has at least `target`
// workgroups, or 1 when the tiles alone do; each split keeps at least 4
// stages of 64 (so the load ring has something to overlap).
int choose_split(long long tiles, int K, int target) {
  const int steps = K / kBK;
  int s = 1;
  while (tiles * s < target && 4 * (s + 1) <= steps) {
    int t = s + 1;
    while (4 * t <= steps && steps % t != 0) ++t;
    if (4 * t > steps) break;
    s = t;
  }
  return s;
}

// How one product is run: tile shape, tile counts and K splits. The same
// plan sizes the workspace and drives the launch.
enum ShapeId { kWide, kAllOut, kThin, kFew };
struct Plan {
  ShapeId shape;
  int BM, BN;
  long long m_tiles, n_tiles;
  int split;
};
template <class S>
Plan make_plan(ShapeId id, int M, int N, int K, int split_target) {
  Plan pl{id, S::BM, S::BN, (M + S::BM - 1) / S::BM, (N + S::BN - 1) / S::BN, 1};
  if (split_target > 0) pl.split = choose_split(pl.m_tiles * pl.n_tiles, K, split_target);
  return pl;
}
Plan plan_for(int M, int N, int K) {
  // at most 64 tokens: one token tile, K split to fill the chip
  if (M <= kFewMaxM) return make_plan<FewShape>(kFew, M, N, K, 256);
  // many tokens, wide output (q_b): square tiles, no split
  if (M >= 1024 && N % WideShape::BN == 0) return make_plan<WideShape>(kWide, M, N, K, 0);
  // many tokens, narrow output (k and projection): one tile spans every
  // output, so each token row is read once; K split to fill the chip
  if (M >= 1024 && N <= AllOutShape::BN) return make_plan<AllOutShape>(kAllOut, M, N, K, 256);
  // few tokens (decode): narrow output tiles, K split to fill the chip
  return make_plan<ThinShape>(kThin, M, N, K, 512);
}

// The task of a product under plan pl, its partials (when split) at
// p.partial, which must hold partial_bytes(pl, M).
size_t partial_bytes(const Plan& pl, int M) { return pl.split > 1 ? (size_t)pl.split * M * pl.n_tiles * pl.BN * 4 : 0; }
hipError_t make_task(ProjParams p, const Plan& pl, size_t avail, ProjTask& t) {
  if (pl.m_tiles > 65535) return hipErrorInvalidValue;
  if (pl.split > 1 && (!p.partial || partial_bytes(pl, p.M) > avail)) return hipErrorInvalidValue;
  if (pl.split == 1) p.partial = nullptr;
  p.k_split = p.K / pl.split;
  const long long total = pl.n_tiles * pl.m_tiles * pl.split;
  const long long per_xcd = (total + 7) / 8;
  if (8 * per_xcd > 0x3fffffffll) return hipErrorInvalidValue;
  t = ProjTask{p, (int)pl.m_tiles, (int)pl.n_tiles, pl.split, (int)per_xcd};
  return hipSuccess;
}
// Sums of the split tasks among t0 and t1 (t1.per_xcd = 0: no second task).
hipError_t launch_reduce(const ProjTask& t0, const Plan& p0, const ProjTask& t1, const Plan& p1, hipStream_t st) {
  const bool r0 = p0.split > 1, r1 = t1.per_xcd > 0 && p1.split > 1;
  if (!r0 && !r1) return hipSuccess;
  const ProjParams none{};
  const ProjParams& a = r0 ? t0.p : t1.p;
  const Plan& pa = r0 ? p0 : p1;
  const ProjParams& b = r0 && r1 ? t1.p : none;
  const long long a_threads = (long long)a.M * (pa.n_tiles * pa.BN / 4);
  const long long b_threads = r0 && r1 ? (long long)b.M * (p1.n_tiles * p1.BN / 4) : 0;
  const long long blocks = (a_threads + b_threads + 255) / 256;
  hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, pa.split,
                     (int)(pa.n_tiles * pa.BN), b, p1.split, (int)(p1.n_tiles * p1.BN), a_threads);
  return hipGetLastError();
}
template <class S>
hipError_t launch_plan(const ProjParams& p, const Plan& pl, size_t ws_bytes, hipStream_t st) {
  ProjTask t{};
  hipError_t e = make_task(p, pl, ws_bytes, t);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((proj_gemm_kernel<S, false>), dim3((unsigned)(8 * t.per_xcd)), dim3(64 * S::WAVES), 0, st, t,
                     ProjTask{});
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce(t, pl, ProjTask{}, pl, st);
}

}  // namespace

size_t proj_partial_bytes(int M, int N, int K) { return partial_bytes(plan_for(M, N, K), M); }

size_t proj_pair_partial_bytes(int M, int Nq, int Kq, int Nk, int Kk) {
  const size_t bq = proj_partial_bytes(M, Nq, Kq), bk = proj_partial_bytes(M, Nk, Kk);
  if (M <= kFewMaxM) return (bq + 255) / 256 * 256 + bk;  // both products' partials at once
  return std::max(bq, bk);
}

hipError_t launch_proj(const ProjParams& p, size_t ws_bytes, hipStream_t st) {
  if (p.K % kBK != 0 || p.M < 1 || p.N0 % 4 != 0) return hipErrorInvalidValue;
  const Plan pl = plan_for(p.M, p.N0 + p.N1, p.K);
  switch (pl.shape) {
    case kWide: return launch_plan<WideShape>(p, pl, ws_bytes, st);
    case kAllOut: return launch_plan<AllOutShape>(p, pl, ws_bytes, st);
    case kFew: return launch_plan<FewShape>(p, pl, ws_bytes, st);
    default: return launch_plan<ThinShape>(p, pl, ws_bytes, st);
  }
}

hipError_t launch_proj_pair(const ProjParams& q, const ProjParams& k, size_t ws_bytes, hipStream_t st) {
  if (q.K % kBK != 0 || k.K % kBK != 0 || q.M < 1 || q.M != k.M || q.N0 % 4 != 0 || k.N0 % 4 != 0)
    return hipErrorInvalidValue;
  if (q.M > kFewMaxM) {  // one product after the other, sharing the workspace
    hipError_t e = launch_proj(q, ws_bytes, st);
    if (e != hipSuccess) return e;
    return launch_proj(k, ws_bytes, st);
  }
  // Few tokens: both products' tiles in one launch, their partials side by
  // side in the workspace, both sums in a second launch.
  const Plan pq = plan_for(q.M, q.N0 + q.N1, q.K), pk = plan_for(k.M, k.N0 + k.N1, k.K);
  const size_t bq = (partial_bytes(pq, q.M) + 255) / 256 * 256;
  if (bq > ws_bytes) return hipErrorInvalidValue;
  ProjParams kk = k;
  if (k.partial) kk.partial = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(k.partial) + bq);
  ProjTask tq{}, tk{};
  hipError_t e = make_task(q, pq, ws_bytes, tq);
  if (e != hipSuccess) return e;
  e = make_task(kk, pk, ws_bytes - bq, tk);
  if (e != hipSuccess) return e;
  const long long blocks = 8ll * tq.per_xcd + 8ll * tk.per_xcd;
  hipLaunchKernelGGL((proj_gemm_kernel<FewShape, true>), dim3((unsigned)blocks), dim3(64 * FewShape::WAVES), 0, st,
                     tq, tk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce(tq, pq, tk, pk, st);
}

}  // namespace dsa
