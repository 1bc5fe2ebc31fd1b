// Masked flash attention for prefill-shaped calls, bf16 inputs, head dim 128.
//
// Computes, for every query i at position p and head h, attention over the
// keys its mask row keeps (s <= p, s < n_kv, bit s set); unkept keys get
// exactly zero weight. The selection is a mask over the whole cache and the
// attention is the masked flash-attention path it feeds [aiaulis paras 2 and
// 4; devotd section 2].
//
// Work split. A workgroup is 8 waves of one (sequence, head); each wave owns
// 32 query rows (two blocks of 16, Q^T fragments in registers) and 64-key
// tiles of K and V stream through LDS, double-buffered. Every K and V
// fragment a wave reads from LDS is used for both of its query blocks (512 B
// of LDS reads per key per wave against 32 * 512 flops of matrix work). At
// at most 256 registers per lane one workgroup fills a CU, two waves per
// SIMD, so one wave's softmax can overlap the other's matrix work; its 256
// queries share each tile loaded into LDS. With the operand reads free of
// bank conflicts LDS is about half busy; the exp2 and masking work of the
// softmax (VALU, exp2 at quarter rate) and the matrix work of the two waves
// on a SIMD overlap only partly, and that is what bounds the kernel. (Waves
// of 64 queries halve the LDS traffic but need more than 256 registers:
// their accumulators then live in AGPRs, which the compiler copies around
// every tile, and they measured slower; waves of 16 queries, four per SIMD,
// measured slower too.)
//
// Matrix layout (v_mfma_f32_16x16x32_bf16, see dsa_device.hpp):
//   S^T = K Q^T   A = K rows from LDS, B = Q^T; lane (c, g) ends up holding
//                 keys 16*kb + 4*g + r (r = 0..3) of query c.
//   O^T += V^T P^T  the S^T accumulators, exponentiated and rounded to bf16,
//                 are used in place as the B operand.
// K and V tiles go from HBM straight into LDS (global_load_lds, 16 bytes per
// lane, no registers), row-major with each row's 16-byte columns XOR-swizzled
// (see swz) so that both operand reads are free of bank conflicts. The V^T operand of P V is read from the row-major V tile
// with LDS transpose reads (ds_read_b64_tr_b16): within a 16-lane group, lane
// c receives element c % 4 of the 8-byte pieces lanes 4k + c/4 point at, so
// pointing lane 4r + j at dims 4j..4j+3 of key r gives each lane one dim of
// four consecutive keys.
//
// Softmax. Scores are masked with one sign-extending bit extract and one
// bitfield insert per element and exponentiated with exp2 against a per-row
// offset. The offset is the exact maximum of the row's first tile with a
// kept key; later tiles take no maximum at all. A lane's share of a tile's
// row sum bounds every probability in it, so when no share exceeds 2^40 the
// tile is accepted as computed; otherwise (scores that rose by about 36 log2
// units or more) the tile's exact maxima are taken, the offset raised, O and
// the sums rescaled, and the probabilities computed again. Probabilities thus
// stay <= 2^40 (float32 sums and bf16 P carry them without loss, and O stays
// finite for |v| < 2^70), and since the offset never exceeds the row's true
// maximum the largest probability is >= 1, so nothing that matters
// underflows. The row sum is taken over the bf16 probabilities that enter
// P V (two per dot2 instruction), and the final normalisation divides by it,
// so the result is softmax over the kept keys.
//
// Scheduling. Workgroup ids are mapped so that all query tiles of one
// (sequence, head) pair land on the same XCD (id mod 8), sharing its L2 for
// the K/V stream, and the query tiles with the most keys are dispatched first.
#include "attn_bf16_common.hpp"
#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

using namespace attn_bf16;

constexpr int kStage = 2 * kTileBytes;       // K tile then V tile
constexpr float kSumCap = 1099511627776.0f;  // 2^40: largest accepted lane share of a tile's row sum
constexpr int kQB = 2;               // 16-query blocks per wave
constexpr int kQW = 16 * kQB;        // queries per wave
#ifndef DSA_ATTN_WAVES
#define DSA_ATTN_WAVES 8
#endif
constexpr int kWaves = DSA_ATTN_WAVES;  // waves per workgroup
constexpr int kQT = kWaves * kQW;     // queries per workgroup
constexpr int kDL = kKT / (4 * kWaves);  // tile-load instructions per wave per K (or V) tile
static_assert(kKT % (4 * kWaves) == 0, "each wave loads whole groups of four key rows");

__device__ __forceinline__ float mask_elem(float s, uint32_t word, int bit) {
  // all-ones when bit `bit` of word is set, else zero; then keep s or -inf
  const int m = (int)(word << (31 - bit)) >> 31;
  return __int_as_float((m & __float_as_int(s)) | (~m & (int)0xff800000u));
}

__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_bf16_kernel(AttnParams a, int n_qtiles, int pairs_per_xcd) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kStage];

  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int qi = slot / pairs_per_xcd, pair = (slot % pairs_per_xcd) * 8 + xcd;
  if (pair >= a.B * a.H || qi >= n_qtiles) return;
  const int qt = n_qtiles - 1 - qi;
  const int b = pair / a.H, h = pair % a.H, hk = h / (a.H / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int t0 = qt * kQT;
  const int t_end = min(t0 + kQT, a.T);
  const int n_tiles = (a.q_pos0 + t_end - 1) / kKT + 1;
  const int nwords = a.Lpad / 32;
  const int tw = t0 + wave * kQW;                // first query of this wave
  const bool wave_live = tw < a.T;
  const int pw_first = a.q_pos0 + tw;
  const int pw_last = a.q_pos0 + min(tw + kQW, a.T) - 1;

  const size_t kv_tok = (size_t)a.Hkv * kD;        // elements per cached token
  const bf16* kbase = static_cast<const bf16*>(a.k) + (size_t)b * a.kv_cap * kv_tok + (size_t)hk * kD;
  const bf16* vbase = static_cast<const bf16*>(a.v) + (size_t)b * a.kv_cap * kv_tok + (size_t)hk * kD;
  // Query rows past the end read the last row (finite data, never stored).
  const bf16* qsrc = static_cast<const bf16*>(a.q) + ((size_t)b * a.T * a.H + h) * kD;

  // Q^T operands: query 16*qb + c of the wave, dims 32*kk + 8*g + e.
  bf16x8 qreg[kQB][kKS];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const bf16* qp = qsrc + (size_t)min(tw + 16 * qb + c, a.T - 1) * a.H * kD;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) qreg[qb][kk] = load_frag<bf16>(qp + 32 * kk + 8 * g);
  }
  int tq[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) tq[qb] = tw + 16 * qb + c;
  // Mask row of query block 0; block qb is 16 * qb rows further.
  const uint32_t* mrow0 = a.mask + ((size_t)b * a.T + min(tw + c, a.T - 1)) * nwords;
  const int last_row_off = a.T - 1 - min(tw + c, a.T - 1);  // rows to the last valid one

  f32x4 o[kDB][kQB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // exponent offset (log2 units; -inf until the row has a kept key), its
  // negation (0 until then), and the row sum
  float m_run[kQB], nm_run[kQB], l_run[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m_run[qb] = fneg_inf();
    nm_run[qb] = 0.f;
    l_run[qb] = 0.f;
  }

  // Tile loader: wave w fills key rows 4 kDL w .. 4 kDL (w+1) - 1 of the K and
  // V tiles, four rows (1 KiB) per instruction; lane l writes physical column l % 16 of
  // row l / 16, so it fetches the logical column that the swizzle puts
  // there. Keys past n_kv (last tile only) read the last cached row instead:
  // finite data the mask gives zero weight.
  int dl_row[kDL], dl_col[kDL];  // row of the tile and logical column this lane fetches, per instruction
  uint32_t dl_off[kDL];          // element offset of that row/column from the tile's first key
#pragma unroll
  for (int n = 0; n < kDL; ++n) {
    dl_row[n] = 4 * kDL * wave + 4 * n + (lane >> 4);
    dl_col[n] = (lane & 15) ^ swz(dl_row[n]);
    dl_off[n] = (uint32_t)(dl_row[n] * kv_tok + dl_col[n] * 8);
  }
  auto dload = [&](int tile, int buf) {
    const int s0 = tile * kKT;
    unsigned char* st = lds + buf * kStage;
    const size_t tbase = (size_t)s0 * kv_tok;
    if (s0 + kKT <= a.n_kv) {
#pragma unroll
      for (int n = 0; n < kDL; ++n) {
        const int r0 = 4 * kDL * wave + 4 * n;
        __builtin_amdgcn_global_load_lds(kbase + tbase + dl_off[n], (lds_void*)(st + r0 * kRow), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + tbase + dl_off[n], (lds_void*)(st + kTileBytes + r0 * kRow), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int n = 0; n < kDL; ++n) {
        const int r0 = 4 * kDL * wave + 4 * n;
        const size_t off = (size_t)min(s0 + dl_row[n], a.n_kv - 1) * kv_tok + dl_col[n] * 8;
        __builtin_amdgcn_global_load_lds(kbase + off, (lds_void*)(st + r0 * kRow), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + off, (lds_void*)(st + kTileBytes + r0 * kRow), 16, 0, 0);
      }
    }
  };

  // Mask words (64 keys = 2 words) of tile `tile` for this lane's queries.
  uint2 mw_next[kQB];
  auto mload = [&](int tile) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      mw_next[qb] = *reinterpret_cast<const uint2*>(mrow0 + (size_t)min(16 * qb, last_row_off) * nwords + 2 * tile);
  };

  const float sl2 = a.scale_log2;
  dload(0, 0);
  mload(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    uint2 mw[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) mw[qb] = mw_next[qb];
    if (it + 1 < n_tiles) {
      dload(it + 1, buf ^ 1);
      mload(it + 1);
    }
    const int s0 = it * kKT;
    const unsigned char* kl = lds + buf * kStage;
    const unsigned char* vl = kl + kTileBytes;

    if (wave_live && s0 <= pw_last) {
      // Causal limit folded into the mask words on diagonal tiles.
      const bool diag = s0 + kKT - 1 > pw_first;
      bool any = false, full = !diag;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        uint32_t lo = mw[qb].x, hi = mw[qb].y;
        if (diag) {
          const int lim = a.q_pos0 + tq[qb] - s0;  // keys kl <= lim are causal
          const uint32_t clo = lim >= 31 ? 0xffffffffu : (lim < 0 ? 0u : (2u << lim) - 1u);
          const uint32_t chi = lim >= 63 ? 0xffffffffu : (lim < 32 ? 0u : (2u << (lim - 32)) - 1u);
          lo &= clo;
          hi &= chi;
        }
        if (tq[qb] >= a.T) lo = hi = 0u;
        mw[qb] = make_uint2(lo, hi);
        any = any || (lo | hi) != 0u;
        full = full && (lo & hi) == 0xffffffffu;
      }
      if (ballot64(any) != 0ull) {
        // S^T = K Q^T (the scheduler's small-GEMM strategy interleaves the K
        // fragment reads with the MFMAs; measured 2-3% faster per call)
        __builtin_amdgcn_iglp_opt(0);
        f32x4 sacc[4][kQB];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) sacc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kKS; ++kk) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + tile_off(16 * kb + c, 4 * kk + g));
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) sacc[kb][qb] = mma_kstep(kf, qreg[qb][kk], sacc[kb][qb]);
          }
        }
        // Unkept keys to -inf (no masking when every query of the wave keeps
        // the whole tile).
        const bool plain = ballot64(!full) == 0ull;
        if (!plain) {
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) {
            const uint32_t wlo = mw[qb].x >> (4 * g), whi = mw[qb].y >> (4 * g);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                sacc[kb][qb][r] = mask_elem(sacc[kb][qb][r], kb < 2 ? wlo : whi, 16 * (kb & 1) + r);
          }
        }
        // P^T in bf16 against the current exponent offset, in the accumulator
        // layout; lt = this lane's share of the tile's row sums.
        bf16x8 pf[kQB][2];
        float lt[kQB];
        auto probs = [&]() {
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) {
            lt[qb] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              bf16x8 pv;
#pragma unroll
              for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  pv[4 * hf + r] = (bf16)__builtin_amdgcn_exp2f(fmaf(sacc[2 * ks + hf][qb][r], sl2, nm_run[qb]));
              pf[qb][ks] = pv;
              lt[qb] = sum8_bf16(pv, lt[qb]);
            }
          }
        };
        // The offset of a row is set to the exact maximum of its first tile
        // with a kept key and raised only when a lane's share of a tile's sum
        // exceeds 2^40 (then every probability so far is <= 2^40).
        bool first = false;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) first = first || (m_run[qb] == fneg_inf() && (mw[qb].x | mw[qb].y) != 0u);
        bool exact = ballot64(first) != 0ull;
        if (!exact) {
          probs();
          bool over = false;
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) over = over || lt[qb] > kSumCap;
          exact = ballot64(over) != 0ull;
        }
        if (exact) {
          float mx_all[kQB];
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) {
            float mx = fneg_inf();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
            mx_all[qb] = rows4_max(mx) * sl2;
          }
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) {
            const bool need = mx_all[qb] > m_run[qb] + kLazyMax;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run[qb] - mx_all[qb]) : 1.f;
            if (need) {
              m_run[qb] = mx_all[qb];
              nm_run[qb] = -mx_all[qb];
            }
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < kDB; ++db) o[db][qb] *= alpha;
          }
          probs();
        }
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) l_run[qb] += lt[qb];
        // O^T += V^T P^T (same strategy)
        __builtin_amdgcn_iglp_opt(0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            const bf16x8 vf = vt_frag(vl, ks, db, c, g);
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) o[db][qb] = mma_kstep(vf, pf[qb][ks], o[db][qb]);
          }
      }
    }
    // the next tile's direct loads (and mask words) have landed in this
    // wave; the barrier makes every wave's share visible
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (!wave_live) return;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float l_tot = rows4_sum(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (tq[qb] < a.T) {
      bf16* orow = static_cast<bf16*>(a.out) + (((size_t)b * a.T + tq[qb]) * a.H + h) * kD;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const f32x4 v = o[db][qb] * inv;
        const bf16 v0 = (bf16)v[0], v1 = (bf16)v[1], v2 = (bf16)v[2], v3 = (bf16)v[3];
        uint16_t u[4];
        __builtin_memcpy(&u[0], &v0, 2);
        __builtin_memcpy(&u[1], &v1, 2);
        __builtin_memcpy(&u[2], &v2, 2);
        __builtin_memcpy(&u[3], &v3, 2);
        *reinterpret_cast<uint2*>(orow + 16 * db + 4 * g) =
            make_uint2(u[0] | ((uint32_t)u[1] << 16), u[2] | ((uint32_t)u[3] << 16));
      }
      if (a.lse && g == 0) {
        const float m_use = m_run[qb] == fneg_inf() ? 0.f : m_run[qb];
        a.lse[((size_t)b * a.T + tq[qb]) * a.H + h] = l_tot > 0.f ? (m_use + __log2f(l_tot)) * kLn2f : fneg_inf();
      }
    }
  }
}

}  // namespace

bool attn_prefill_bf16_supported(int D) { return D == kD; }

hipError_t launch_attn_prefill_bf16(const AttnParams& p, hipStream_t st) {
  const int n_qtiles = (p.T + kQT - 1) / kQT;
  const int pairs = p.B * p.H;
  const int pairs_per_xcd = (pairs + 7) / 8;
  const long long nblocks = 8ll * n_qtiles * pairs_per_xcd;
  if (nblocks > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_prefill_bf16_kernel, dim3((unsigned)nblocks), dim3(64 * kWaves), 0, st, p, n_qtiles,
                     pairs_per_xcd);
  return hipGetLastError();
}

}  // namespace dsa
