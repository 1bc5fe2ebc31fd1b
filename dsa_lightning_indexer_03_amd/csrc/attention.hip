// Attention over the kept keys only.
//
// The selection is a mask over the whole cache; attention keeps exactly the
// masked-in keys, so unkept keys get zero weight [aiaulis paras 2 and 4;
// devotd section 2]. For every query i at position p and head h:
//   out[i][h] = sum_{s in S_i} softmax_s(scale * q[i][h] . k[s][g]) v[s][g],
//   S_i = {s <= p, s < n_kv, mask bit s set}, g = h / (H / H_kv).
//
// attn_prefill_kernel - masked flash attention for prefill-shaped calls.
//   Workgroup = 4 waves x 32 queries of one head. 64-key tiles of K (row
//   major) and V (transposed, keys permuted, see vt_pos) are staged in LDS,
//   double-buffered. The kernel computes S^T = K Q^T, so each lane's
//   accumulators hold 16 keys of one query; after the online softmax they
//   are, unchanged in place, the B operand P^T of O^T = V^T P^T. The mask is
//   read one 64-bit word per (query, tile); tiles where every query of the
//   wave keeps every key skip the masking arithmetic, and tiles no query of
//   the wave keeps anything of are skipped outright.
//   Workgroups of the same (sequence, head) are placed on the same XCD
//   (workgroup id mod 8) so its L2 serves their shared K/V stream, and the
//   longest query tiles are dispatched first.
//
// attn_gather_kernel - few queries per sequence (decode). Each workgroup
//   takes up to 128 kept tokens of one query (a split), streams their whole
//   K/V rows (contiguous across heads) through a per-lane online softmax and
//   writes a partial (max, sum, unnormalised output) per head;
//   attn_gather_combine_kernel merges the partials. Kept tokens are read
//   once per query.
#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;

// Position of key kl (0..63 in a tile) inside a transposed V row, chosen so
// that the 8 keys a lane feeds to one PV k-step are contiguous: PV k-step ks
// covers keys 32*ks + 16*hf + 4*gg + r (hf, r in 0..1 / 0..3), which S^T's
// accumulator layout puts in lane group gg, slot 4*hf + r.
__device__ __forceinline__ int vt_pos(int kl) {
  const int ks = kl >> 5, rem = kl & 31, hf = rem >> 4, gg = (rem >> 2) & 3, r = rem & 3;
  return 32 * ks + 8 * gg + 4 * hf + r;
}

template <typename T> struct PFrag;
template <> struct PFrag<bf16> {
  static __device__ __forceinline__ bf16x8 make(const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
    return v;
  }
};
template <> struct PFrag<float> {
  static __device__ __forceinline__ f32x8 make(const float (&x)[8]) {
    return f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnParams a, int n_qtiles, int pairs_per_xcd) {
  constexpr int NT = 256, QB = 2, QT = 128, KT = 64, KSTEPS = D / 32, DB = D / 16;
  constexpr int ES = (int)sizeof(T);
  constexpr int KPITCH = D * ES + 16, VPITCH = KT * ES + 16;
  constexpr int KBYTES = KT * KPITCH, VBYTES = D * VPITCH, STAGE = KBYTES + VBYTES;
  constexpr int CH = D * ES / 16;         // 16-B chunks per key row
  constexpr int EPC = 16 / ES;            // elements per chunk
  constexpr int NCH = KT * CH / NT;       // chunks per thread per tile (K and V each)
  static_assert(KT * CH % NT == 0, "tile chunks divide evenly");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE];

  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int qi = slot / pairs_per_xcd, pair = (slot % pairs_per_xcd) * 8 + xcd;
  if (pair >= a.B * a.H || qi >= n_qtiles) return;
  const int qt = n_qtiles - 1 - qi;
  const int b = pair / a.H, h = pair % a.H, hk = h / (a.H / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int t0 = qt * QT;
  const int t_end = min(t0 + QT, a.T);
  const int n_tiles = (a.q_pos0 + t_end - 1) / KT + 1;
  const int nwords = a.Lpad / 32;
  const int tw = t0 + wave * 32;                 // first query of this wave
  const bool wave_live = tw < a.T;
  const int pw_first = a.q_pos0 + tw;
  const int pw_last = a.q_pos0 + min(tw + 32, a.T) - 1;

  const T* qbase = static_cast<const T*>(a.q);
  const size_t kv_tok = (size_t)a.Hkv * D;       // elements per cached token
  const T* kbase = static_cast<const T*>(a.k) + (size_t)b * a.kv_cap * kv_tok + (size_t)hk * D;
  const T* vbase = static_cast<const T*>(a.v) + (size_t)b * a.kv_cap * kv_tok + (size_t)hk * D;

  // Q^T operands: query tw + 16*qb + c, dims 32*kk + 8*g + e.
  frag_t<T> qf[QB][KSTEPS];
  int tq[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    tq[qb] = tw + 16 * qb + c;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf[qb][kk] = tq[qb] < a.T ? load_frag<T>(qbase + (((size_t)b * a.T + tq[qb]) * a.H + h) * D + 32 * kk + 8 * g)
                                : zero_frag<T>();
  }

  f32x4 o[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = fneg_inf();
    l_run[qb] = 0.f;
  }

  u32x4 kst[NCH], vst[NCH];
  auto gload = [&](int tile) {
    const int s0 = tile * KT;
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int i = tid + n * NT, key = i / CH, ch = i % CH, s = s0 + key;
      const bool sv = s < a.n_kv;
      kst[n] = sv ? *reinterpret_cast<const u32x4*>(kbase + (size_t)s * kv_tok + ch * EPC) : u32x4{0u, 0u, 0u, 0u};
      vst[n] = sv ? *reinterpret_cast<const u32x4*>(vbase + (size_t)s * kv_tok + ch * EPC) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* kl = lds + buf * STAGE;
    unsigned char* vl = kl + KBYTES;
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int i = tid + n * NT, key = i / CH, ch = i % CH;
      *reinterpret_cast<u32x4*>(kl + key * KPITCH + ch * 16) = kst[n];
      const int pos = vt_pos(key);
      if (ES == 2) {
        const uint32_t w4[4] = {vst[n][0], vst[n][1], vst[n][2], vst[n][3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t hv = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
          *reinterpret_cast<uint16_t*>(vl + (ch * EPC + e) * VPITCH + pos * 2) = hv;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint32_t*>(vl + (ch * EPC + e) * VPITCH + pos * 4) = vst[n][e];
      }
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_tiles) gload(it + 1);
    const int s0 = it * KT;
    const unsigned char* kl = lds + buf * STAGE;
    const unsigned char* vl = kl + KBYTES;

    if (wave_live && s0 <= pw_last) {
      // Mask words of this tile for the wave's queries.
      uint32_t mlo[QB], mhi[QB];
      bool any = false, full = true;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        uint2 mw = make_uint2(0u, 0u);
        if (tq[qb] < a.T) mw = *reinterpret_cast<const uint2*>(a.mask + ((size_t)b * a.T + tq[qb]) * nwords + 2 * it);
        mlo[qb] = mw.x;
        mhi[qb] = mw.y;
        any = any || (mw.x | mw.y) != 0u;
        full = full && (tq[qb] < a.T) && (mw.x & mw.y) == 0xffffffffu;
      }
      const bool wave_any = ballot64(any) != 0ull;
      const bool diag = s0 + KT - 1 > pw_first;
      const bool plain = !diag && ballot64(!full) == 0ull;
      if (wave_any) {
        // S^T = K Q^T: key block kb (keys 16*kb + 4*g + r), query block qb.
        f32x4 sacc[4][QB];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const frag_t<T> kf = load_frag<T>(reinterpret_cast<const T*>(kl + (16 * kb + c) * KPITCH + (32 * kk + 8 * g) * ES));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = mma_kstep(kf, qf[qb][kk], sacc[kb][qb]);
          }
        }
        frag_t<T> pf[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float x[4][4];
          const int lim = a.q_pos0 + tq[qb] - s0;  // keys kl <= lim are causal
          const uint32_t wlo = mlo[qb] >> (4 * g), whi = mhi[qb] >> (4 * g);
          float mx = fneg_inf();
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float v = sacc[kb][qb][r] * a.scale_log2;
              if (!plain) {
                const uint32_t wd = kb < 2 ? wlo : whi;
                const bool keep = ((wd >> (16 * (kb & 1) + r)) & 1u) && (16 * kb + 4 * g + r <= lim);
                v = keep ? v : fneg_inf();
              }
              x[kb][r] = v;
              mx = fmaxf(mx, v);
            }
          mx = rows4_max(mx);
          const float m_new = fmaxf(m_run[qb], mx);
          const float m_use = m_new == fneg_inf() ? 0.f : m_new;
          const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
          m_run[qb] = m_new;
          float ps = 0.f;
          float pv[2][8];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float e = __builtin_amdgcn_exp2f(x[kb][r] - m_use);
              ps += e;
              pv[kb >> 1][4 * (kb & 1) + r] = e;
            }
          l_run[qb] = l_run[qb] * alpha + ps;
          if (ballot64(alpha != 1.f) != 0ull) {
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db][qb] *= alpha;
          }
          pf[qb][0] = PFrag<T>::make(pv[0]);
          pf[qb][1] = PFrag<T>::make(pv[1]);
        }
        // O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const frag_t<T> vf = load_frag<T>(reinterpret_cast<const T*>(vl + (16 * db + c) * VPITCH + (32 * ks + 8 * g) * ES));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[db][qb] = mma_kstep(vf, pf[qb][ks], o[db][qb]);
          }
      }
    }
    if (it + 1 < n_tiles) lstore(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = rows4_sum(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (tq[qb] < a.T) {
      T* orow = static_cast<T*>(a.out) + (((size_t)b * a.T + tq[qb]) * a.H + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        T* dst = orow + 16 * db + 4 * g;
        if (ES == 2) {
          const bf16 v0 = (bf16)(o[db][qb][0] * inv), v1 = (bf16)(o[db][qb][1] * inv);
          const bf16 v2 = (bf16)(o[db][qb][2] * inv), v3 = (bf16)(o[db][qb][3] * inv);
          uint16_t u[4];
          __builtin_memcpy(&u[0], &v0, 2);
          __builtin_memcpy(&u[1], &v1, 2);
          __builtin_memcpy(&u[2], &v2, 2);
          __builtin_memcpy(&u[3], &v3, 2);
          *reinterpret_cast<uint2*>(dst) = make_uint2(u[0] | ((uint32_t)u[1] << 16), u[2] | ((uint32_t)u[3] << 16));
        } else {
          *reinterpret_cast<f32x4*>(dst) = o[db][qb] * inv;
        }
      }
      if (a.lse && g == 0)
        a.lse[((size_t)b * a.T + tq[qb]) * a.H + h] =
            l_tot > 0.f ? (m_run[qb] + __log2f(l_tot)) * kLn2 : fneg_inf();
    }
  }
}

// --------------------------------------------------------------------------------------------
// Gather path (few queries per sequence).
//
// Workgroup = 4 waves; wave w owns query heads [w*HW, (w+1)*HW), HW = H/4, for
// all kept tokens of its split. A token's K (or V) row for those heads is
// HW*D*sizeof(T) contiguous bytes when H == H_kv; lanes take 16-B chunks:
// NCHK = HW * D*sizeof(T)/16 chunks per token, TPI = max(1, 64/NCHK) tokens
// per load instruction, NIT = max(1, NCHK/64) instructions per token.

template <typename T, int D, int HW>
struct GatherCfg {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int CHH = D * ES / 16;     // chunks per head
  static constexpr int EPC = 16 / ES;         // elements per chunk
  static constexpr int NCHK = HW * CHH;       // chunks per token per wave
  static constexpr int TPI = NCHK >= 64 ? 1 : 64 / NCHK;
  static constexpr int NIT = NCHK >= 64 ? NCHK / 64 : 1;
  static constexpr int SPLIT = kGatherSplit;
};

template <typename T> __device__ __forceinline__ void chunk_to_float(const u32x4& v, float* f);
template <> __device__ __forceinline__ void chunk_to_float<bf16>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}
template <> __device__ __forceinline__ void chunk_to_float<float>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}

// One workgroup per (query row, split of up to SPLIT kept tokens). Each lane
// keeps an online softmax (running max in log2 units, sum, unnormalised
// output) for the head chunk(s) it holds and streams the split's tokens U at
// a time, with all of their K and V loads in flight together; token slots of
// a wave (TPI > 1) are merged at the end, and the workgroup writes its
// partial. A row with no kept token still gets split 0, which writes the
// empty partial (max -inf, sum 0).
template <typename T, int D, int HW>
__global__ __launch_bounds__(256) void attn_gather_kernel(GatherParams a) {
  using C = GatherCfg<T, D, HW>;
  constexpr int SPLIT = C::SPLIT, EPC = C::EPC, CHH = C::CHH, TPI = C::TPI, NIT = C::NIT, U = kGatherUnroll;
  constexpr int LPS = 64 / TPI;  // lanes per token slot
  __shared__ int tok[SPLIT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.y, split = blockIdx.x;
  const int b = row / a.T, t = row % a.T;
  int q_pos0, n_kv;
  seq_extent(a.seq_len, b, a.T, a.q_pos0, a.n_kv, q_pos0, n_kv);
  const int p = q_pos0 + t;
  const int count = a.counts ? a.counts[row] : min(a.top_k, p + 1);
  const int ns = max(1, (count + SPLIT - 1) / SPLIT);  // an empty row still gets one split
  if (split >= ns) return;
  const int start = split * SPLIT;
  const int ntok = max(0, min(SPLIT, count - start));
  // Kept-token lists come from the library's own top-k or mask compaction and
  // hold tokens in [0, n_kv); the clamp only guarantees that a corrupted list
  // can never address memory outside the caches.
  for (int i = tid; i < ntok; i += 256) tok[i] = min(max(a.list[(size_t)row * a.list_stride + start + i], 0), n_kv - 1);
  __syncthreads();

  const int group = a.H / a.Hkv;
  const int h0 = wave * HW;
  const int tslot = lane / LPS, lane_c = lane % LPS;
  const size_t kv_tok = (size_t)a.Hkv * D;
  const T* kb = static_cast<const T*>(a.k) + (size_t)b * a.kv_cap * kv_tok;
  const T* vb = static_cast<const T*>(a.v) + (size_t)b * a.kv_cap * kv_tok;

  // Query values of the chunks this lane handles (in float), and the offsets
  // of those chunks inside a token's K/V row.
  float qv[NIT][EPC];
  size_t coff[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int cc = it * 64 + lane_c, hl = cc / CHH, part = cc % CHH;
    const T* qp = static_cast<const T*>(a.q) + (((size_t)b * a.T + t) * a.H + h0 + hl) * D + part * EPC;
    chunk_to_float<T>(*reinterpret_cast<const u32x4*>(qp), qv[it]);
    coff[it] = (size_t)((h0 + hl) / group) * D + part * EPC;
  }

  float m[NIT], l[NIT], acc[NIT][EPC];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    m[it] = fneg_inf();
    l[it] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[it][e] = 0.f;
  }

  for (int i0 = 0; i0 < ntok; i0 += U * TPI) {
    u32x4 kc[U][NIT], vc[U][NIT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t off = (size_t)tok[min(i0 + u * TPI + tslot, ntok - 1)] * kv_tok;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        kc[u][it] = *reinterpret_cast<const u32x4*>(kb + off + coff[it]);
        vc[u][it] = *reinterpret_cast<const u32x4*>(vb + off + coff[it]);
      }
    }
    float sc[U][NIT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = i0 + u * TPI + tslot < ntok;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        float kf[EPC];
        chunk_to_float<T>(kc[u][it], kf);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) d = fmaf(qv[it][e], kf[e], d);
#pragma unroll
        for (int off = 1; off < CHH; off <<= 1) d += __shfl_xor(d, off, 64);
        sc[u][it] = valid ? d * a.scale_log2 : fneg_inf();
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float mx = m[it];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][it]);
      const float mref = mx == fneg_inf() ? 0.f : mx;  // no finite score yet: every weight is 0
      const float alpha = __builtin_amdgcn_exp2f(m[it] - mref);
      l[it] *= alpha;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[it][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pr = __builtin_amdgcn_exp2f(sc[u][it] - mref);
        l[it] += pr;
        float vf[EPC];
        chunk_to_float<T>(vc[u][it], vf);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[it][e] = fmaf(pr, vf[e], acc[it][e]);
      }
      m[it] = mx;
    }
  }
  // Merge the token slots of the wave (lanes LPS apart hold the same chunk).
#pragma unroll
  for (int off = LPS; off < 64; off <<= 1) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const float mo = __shfl_xor(m[it], off, 64), lo = __shfl_xor(l[it], off, 64);
      const float mx = fmaxf(m[it], mo);
      const float mref = mx == fneg_inf() ? 0.f : mx;
      const float fa = __builtin_amdgcn_exp2f(m[it] - mref), fb = __builtin_amdgcn_exp2f(mo - mref);
      l[it] = l[it] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[it][e] = acc[it][e] * fa + __shfl_xor(acc[it][e], off, 64) * fb;
      m[it] = mx;
    }
  }
  if (tslot == 0) {
    float* po = a.part_o + ((size_t)row * a.n_splits + split) * a.H * D;
    float* pml = a.part_ml + ((size_t)row * a.n_splits + split) * a.H * 2;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int cc = it * 64 + lane_c, hl = cc / CHH, part = cc % CHH;
      float* dst = po + (size_t)(h0 + hl) * D + part * EPC;
#pragma unroll
      for (int e = 0; e < EPC; e += 4)
        *reinterpret_cast<f32x4*>(dst + e) = f32x4{acc[it][e], acc[it][e + 1], acc[it][e + 2], acc[it][e + 3]};
      if (part == 0) {
        pml[2 * (h0 + hl)] = m[it];
        pml[2 * (h0 + hl) + 1] = l[it];
      }
    }
  }
}

// One workgroup per (head, query row), one thread per output dim: the split
// partials of that head are merged by their log-sum-exp. Splits are taken 16
// at a time with all their loads issued together (one memory round trip per
// 16 splits instead of one per split). A row with no kept token gets a zero
// output and lse = -inf.
template <typename T, int D>
__global__ __launch_bounds__(D) void attn_gather_combine_kernel(GatherParams a) {
  constexpr int CH = 16;
  const int h = blockIdx.x, row = blockIdx.y, d = threadIdx.x;
  const int b = row / a.T, t = row % a.T;
  int q_pos0, n_kv;
  seq_extent(a.seq_len, b, a.T, a.q_pos0, a.n_kv, q_pos0, n_kv);
  const int p = q_pos0 + t;
  const int count = a.counts ? a.counts[row] : min(a.top_k, p + 1);
  const int ns = max(1, (count + kGatherSplit - 1) / kGatherSplit);
  const float* ml = a.part_ml + (size_t)row * a.n_splits * a.H * 2 + 2 * h;
  const float* po = a.part_o + (size_t)row * a.n_splits * a.H * D + (size_t)h * D + d;
  const size_t mls = (size_t)a.H * 2, pos = (size_t)a.H * D;  // strides between splits
  float M = fneg_inf(), L = 0.f, O = 0.f;
  for (int j0 = 0; j0 < ns; j0 += CH) {
    float m[CH], l[CH], o[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int j = min(j0 + i, ns - 1);  // past the last split: a valid split, weighted 0 below
      m[i] = ml[j * mls];
      l[i] = ml[j * mls + 1];
      o[i] = po[j * pos];
    }
    float mc = M;
#pragma unroll
    for (int i = 0; i < CH; ++i) mc = j0 + i < ns ? fmaxf(mc, m[i]) : mc;
    const float mr = mc == fneg_inf() ? 0.f : mc;
    const float alpha = __builtin_amdgcn_exp2f(M - mr);
    L *= alpha;
    O *= alpha;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const float f = j0 + i < ns ? __builtin_amdgcn_exp2f(m[i] - mr) : 0.f;
      L = fmaf(f, l[i], L);
      O = fmaf(f, o[i], O);
    }
    M = mc;
  }
  static_cast<T*>(a.out)[(((size_t)b * a.T + t) * a.H + h) * D + d] = from_float<T>(L > 0.f ? O / L : 0.f);
  if (a.lse && d == 0) a.lse[((size_t)b * a.T + t) * a.H + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : fneg_inf();
}

// One workgroup per row: tokens s <= p (and < n_kv) whose mask bit is set,
// ascending.
__global__ __launch_bounds__(256) void mask_compact_kernel(CompactParams a) {
  __shared__ uint32_t red[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = row % a.T, p = a.q_pos0 + t;
  const int n = min(p + 1, a.n_kv);
  const int nw = (n + 31) / 32;
  const uint32_t* mrow = a.mask + (size_t)row * (a.Lpad / 32);
  const int wpt = (nw + 255) / 256;
  const int w0 = tid * wpt;
  uint32_t local = 0;
  for (int w = w0; w < min(w0 + wpt, nw); ++w) {
    uint32_t bits = mrow[w];
    if (w * 32 + 32 > n) bits &= (n - w * 32 >= 32) ? 0xffffffffu : ((1u << (n - w * 32)) - 1u);
    local += __popc(bits);
  }
  uint32_t inc = wave_inclusive_sum(local);
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  uint32_t off = inc - local;
  for (int w = 0; w < wave; ++w) off += red[w];
  int32_t* lrow = a.list + (size_t)row * a.list_stride;
  for (int w = w0; w < min(w0 + wpt, nw); ++w) {
    uint32_t bits = mrow[w];
    if (w * 32 + 32 > n) bits &= (n - w * 32 >= 32) ? 0xffffffffu : ((1u << (n - w * 32)) - 1u);
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      lrow[off++] = w * 32 + bpos;
      bits &= bits - 1u;
    }
  }
  if (tid == 255) a.counts[row] = (int32_t)(off);
}

template <typename T, int D>
hipError_t launch_prefill_t(const AttnParams& p, hipStream_t st) {
  const int n_qtiles = (p.T + 127) / 128;
  const int pairs = p.B * p.H;
  const int pairs_per_xcd = (pairs + 7) / 8;
  const int nblocks = 8 * n_qtiles * pairs_per_xcd;
  hipLaunchKernelGGL((attn_prefill_kernel<T, D>), dim3(nblocks), dim3(256), 0, st, p, n_qtiles, pairs_per_xcd);
  return hipGetLastError();
}

template <typename T, int D, int HW>
hipError_t launch_gather_hw(const GatherParams& p, hipStream_t st) {
  hipLaunchKernelGGL((attn_gather_kernel<T, D, HW>), dim3(p.n_splits, p.B * p.T), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_gather_combine_kernel<T, D>), dim3(p.H, p.B * p.T), dim3(D), 0, st, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_gather_t(const GatherParams& p, hipStream_t st) {
  switch (p.H / 4) {
    case 1: return launch_gather_hw<T, D, 1>(p, st);
    case 2: return launch_gather_hw<T, D, 2>(p, st);
    case 4: return launch_gather_hw<T, D, 4>(p, st);
    case 8: return launch_gather_hw<T, D, 8>(p, st);
    case 16: return launch_gather_hw<T, D, 16>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gather_supported(int H, int D) {
  return (D == 64 || D == 128) && H % 4 == 0 && (H / 4 == 1 || H / 4 == 2 || H / 4 == 4 || H / 4 == 8 || H / 4 == 16);
}

hipError_t launch_attn_prefill(const AttnParams& p, int dtype, int D, hipStream_t st) {
  if (dtype == 1) {
    if (attn_prefill_bf16_supported(D)) return launch_attn_prefill_bf16(p, st);
    if (D == 128) return launch_prefill_t<bf16, 128>(p, st);
    if (D == 64) return launch_prefill_t<bf16, 64>(p, st);
  } else {
    if (D == 128) return launch_prefill_t<float, 128>(p, st);
    if (D == 64) return launch_prefill_t<float, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_gather(const GatherParams& p, int dtype, int D, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_gather_t<bf16, 128>(p, st);
    if (D == 64) return launch_gather_t<bf16, 64>(p, st);
  } else {
    if (D == 128) return launch_gather_t<float, 128>(p, st);
    if (D == 64) return launch_gather_t<float, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mask_compact(const CompactParams& p, hipStream_t st) {
  hipLaunchKernelGGL(mask_compact_kernel, dim3(p.B * p.T), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
