// Masked flash attention for prefill-shaped calls, bf16 inputs, head dim 128.
//
// Computes, for every query i at position p and head h, attention over the
// keys its mask row keeps (s <= p, s < n_kv, bit s set); unkept keys get
// exactly zero weight. The selection is a mask over the whole cache and the
// attention is the masked flash-attention path it feeds [aiaulis paras 2 and
// 4; devotd section 2].
//
// Work split. A workgroup is 4 waves of one (sequence, head); each wave owns
// 32 query rows (two blocks of 16, Q^T fragments in registers) and 64-key
// tiles of K and V stream through LDS, double-buffered. Every K and V
// fragment a wave reads from LDS is used for both of its query blocks (512 B
// of LDS reads per key per wave against 32 * 512 flops of matrix work). At
// at most 256 registers per lane two workgroups share a CU, two waves per
// SIMD, so one wave's softmax overlaps the other's matrix work. (Waves of 64
// queries halve the LDS traffic but need more than 256 registers: their
// accumulators then live in AGPRs, which the compiler copies around every
// tile, and they measured slower.)
//
// Matrix layout (v_mfma_f32_16x16x32_bf16, see dsa_device.hpp):
//   S^T = K Q^T   A = K rows from LDS, B = Q^T; lane (c, g) ends up holding
//                 keys 16*kb + 4*g + r (r = 0..3) of query c.
//   O^T += V^T P^T  the S^T accumulators, exponentiated and rounded to bf16,
//                 are used in place as the B operand; V^T is stored in LDS so
//                 that the 8 keys a lane feeds per k-step are contiguous.
// V is transposed in registers on its way into LDS (4 keys x 8 dims per
// thread, byte permutes), and the V^T rows are XOR-swizzled in 16-byte units
// so both the transposing writes and the fragment reads avoid bank conflicts.
//
// Softmax. Scores are masked with one sign-extending bit extract and one
// bitfield insert per element, exponentiated with exp2 against a running
// maximum that is only raised (and O rescaled) when a tile's maximum exceeds
// it by more than 2^8; until then probabilities stay <= 256, which float32
// sums and bf16 P carry without loss. The row sum is taken over the bf16
// probabilities that enter P V (two per dot2 instruction), and the final
// normalisation divides by it, so the result is softmax over the kept keys.
//
// Scheduling. Workgroup ids are mapped so that all query tiles of one
// (sequence, head) pair land on the same XCD (id mod 8), sharing its L2 for
// the K/V stream, and the query tiles with the most keys are dispatched first.
#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr int kD = 128;             // head dim
constexpr int kKT = 64;             // keys per tile
constexpr int kKS = kD / 32;        // k-steps of S^T (head dim / 32)
constexpr int kDB = kD / 16;        // 16-dim blocks of O^T
constexpr int kKPitch = kD * 2 + 16;         // bytes per K row in LDS (padded)
constexpr int kKBytes = kKT * kKPitch;
constexpr int kVBytes = kD * kKT * 2;        // V^T: kD rows of 64 keys, 128 B each
constexpr int kStage = kKBytes + kVBytes;
constexpr float kLazyMax = 8.0f;             // log2 units
constexpr float kLn2f = 0.69314718055994530942f;

constexpr int kQB = 2;               // 16-query blocks per wave
constexpr int kQW = 16 * kQB;        // queries per wave
constexpr int kQT = 4 * kQW;        // queries per workgroup

// 16-byte column of V^T row d that holds logical column `chunk` (0..7).
__device__ __forceinline__ int vt_chunk(int d, int chunk) { return chunk ^ ((d ^ (d >> 3)) & 7); }

// Logical V^T column (16-B unit, 0..7) and 8-byte half of the 4 keys 4*kq..4*kq+3.
// The PV k-step ks covers keys 32*ks + 16*hf + 4*g + r; lane group g reads
// column 4*ks + g, whose two halves are hf = 0 and hf = 1.
__device__ __forceinline__ int vt_col_of_quad(int kq) { return 4 * (kq >> 3) + (kq & 3); }
__device__ __forceinline__ int vt_half_of_quad(int kq) { return (kq >> 2) & 1; }

__device__ __forceinline__ float mask_elem(float s, uint32_t word, int bit) {
  // all-ones when bit `bit` of word is set, else zero; then keep s or -inf
  const int m = (int)(word << (31 - bit)) >> 31;
  return __int_as_float((m & __float_as_int(s)) | (~m & (int)0xff800000u));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float sum8_bf16(const bf16x8& p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[2 * i], p[2 * i + 1]}, one, acc, false);
  return acc;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
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
  float m_run[kQB], l_run[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m_run[qb] = fneg_inf();
    l_run[qb] = 0.f;
  }

  // Tile loaders. K: 1024 16-B chunks, 4 per thread (chunk i = tid + 256 n:
  // key i / 16, column i % 16). V: thread (kq = tid / 16, dc = tid % 16)
  // loads dims 8*dc..8*dc+7 of keys 4*kq..4*kq+3. Keys past n_kv (last tile
  // only) read the last cached row instead: finite data the mask gives zero
  // weight.
  const int v_kq = tid >> 4, v_dc = tid & 15;
  const size_t tile_stride = (size_t)kKT * kv_tok;
  const bf16* kp = kbase + (size_t)(tid >> 4) * kv_tok + (tid & 15) * 8;  // + 16 keys per n
  const bf16* vp = vbase + (size_t)(4 * v_kq) * kv_tok + v_dc * 8;         // + 1 key per j
  u32x4 kst[4], vst[4];
  auto gload = [&](int tile) {
    const int s0 = tile * kKT;
    if (s0 + kKT <= a.n_kv) {
      const bf16* kt = kp + tile * tile_stride;
      const bf16* vt = vp + tile * tile_stride;
#pragma unroll
      for (int n = 0; n < 4; ++n) kst[n] = *reinterpret_cast<const u32x4*>(kt + (size_t)(16 * n) * kv_tok);
#pragma unroll
      for (int j = 0; j < 4; ++j) vst[j] = *reinterpret_cast<const u32x4*>(vt + (size_t)j * kv_tok);
    } else {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int s = min(s0 + (tid >> 4) + 16 * n, a.n_kv - 1);
        kst[n] = *reinterpret_cast<const u32x4*>(kbase + (size_t)s * kv_tok + (tid & 15) * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = min(s0 + 4 * v_kq + j, a.n_kv - 1);
        vst[j] = *reinterpret_cast<const u32x4*>(vbase + (size_t)s * kv_tok + v_dc * 8);
      }
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* kl = lds + buf * kStage;
    unsigned char* vl = kl + kKBytes;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int i = tid + n * 256, key = i >> 4, ch = i & 15;
      *reinterpret_cast<u32x4*>(kl + key * kKPitch + ch * 16) = kst[n];
    }
    const int col = vt_col_of_quad(v_kq), half = vt_half_of_quad(v_kq);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // dims 8*dc + 2m (low halves) and 8*dc + 2m + 1 (high halves) of the 4 keys
      const uint32_t lo01 = __builtin_amdgcn_perm(vst[1][m], vst[0][m], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(vst[3][m], vst[2][m], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(vst[1][m], vst[0][m], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(vst[3][m], vst[2][m], 0x07060302u);
      const int d0 = 8 * v_dc + 2 * m, d1 = d0 + 1;
      *reinterpret_cast<uint2*>(vl + d0 * 128 + vt_chunk(d0, col) * 16 + half * 8) = make_uint2(lo01, lo23);
      *reinterpret_cast<uint2*>(vl + d1 * 128 + vt_chunk(d1, col) * 16 + half * 8) = make_uint2(hi01, hi23);
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
  gload(0);
  mload(0);
  lstore(0);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    uint2 mw[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) mw[qb] = mw_next[qb];
    if (it + 1 < n_tiles) {
      gload(it + 1);
      mload(it + 1);
    }
    const int s0 = it * kKT;
    const unsigned char* kl = lds + buf * kStage;
    const unsigned char* vl = kl + kKBytes;

    if (wave_live && s0 <= pw_last) {
      // Causal limit folded into the mask words on diagonal tiles.
      const bool diag = s0 + kKT - 1 > pw_first;
      bool any = false;
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
      }
      if (ballot64(any) != 0ull) {
        // S^T = K Q^T
        f32x4 sacc[4][kQB];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) sacc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kKS; ++kk) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + (16 * kb + c) * kKPitch + (4 * kk + g) * 16);
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) sacc[kb][qb] = mma_kstep(kf, qreg[qb][kk], sacc[kb][qb]);
          }
        }
        // Masked maxima; the running maximum is raised lazily.
        bool need_any = false;
        float mx_all[kQB];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          const uint32_t wlo = mw[qb].x >> (4 * g), whi = mw[qb].y >> (4 * g);
          float mx = fneg_inf();
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = mask_elem(sacc[kb][qb][r], kb < 2 ? wlo : whi, 16 * (kb & 1) + r);
              sacc[kb][qb][r] = v;
              mx = fmaxf(mx, v);
            }
          mx = rows4_max(mx) * sl2;
          mx_all[qb] = mx;
          need_any = need_any || mx > m_run[qb] + kLazyMax;
        }
        if (ballot64(need_any) != 0ull) {
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) {
            const bool need = mx_all[qb] > m_run[qb] + kLazyMax;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run[qb] - mx_all[qb]) : 1.f;
            if (need) m_run[qb] = mx_all[qb];
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < kDB; ++db) o[db][qb] *= alpha;
          }
        }
        // P^T in bf16, in the accumulator layout; row sums over the bf16 values.
        bf16x8 pf[kQB][2];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          const float m_use = m_run[qb] == fneg_inf() ? 0.f : m_run[qb];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 pv;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                pv[4 * hf + r] = (bf16)__builtin_amdgcn_exp2f(fmaf(sacc[2 * ks + hf][qb][r], sl2, -m_use));
            pf[qb][ks] = pv;
            l_run[qb] = sum8_bf16(pv, l_run[qb]);
          }
        }
        // O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            const int d = 16 * db + c;
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vl + d * 128 + vt_chunk(d, 4 * ks + g) * 16);
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) o[db][qb] = mma_kstep(vf, pf[qb][ks], o[db][qb]);
          }
      }
    }
    if (it + 1 < n_tiles) lstore(buf ^ 1);
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
  hipLaunchKernelGGL(attn_prefill_bf16_kernel, dim3((unsigned)nblocks), dim3(256), 0, st, p, n_qtiles,
                     pairs_per_xcd);
  return hipGetLastError();
}

}  // namespace dsa
