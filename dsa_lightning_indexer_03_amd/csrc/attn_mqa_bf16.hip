// Sparse attention over gathered kept keys when every head shares one K/V
// row per token (kv_heads == 1; a key-only latent cache passes the same
// buffer as K and V, and its rows are then gathered once), bf16, head dim
// 128, prefill-shaped calls.
//
// The selection is shared by all heads of a query [aiaulis paras 2-4; devotd
// section 2], so with one K/V row per token the kept rows serve every head:
// gathering them turns the attention of one query into a dense product with
// the heads as the MFMA M dimension, and the work done is exactly the kept
// (query, key) pairs instead of the masked-dense causal square.
//
// One wave per query row (four per workgroup, no workgroup barriers). The
// query's ascending kept-token list is walked 64 tokens at a time:
//   S^T = K Q^T    A = the 64 gathered K rows, loaded straight from memory
//                  into MFMA operands (key 16 kb + (lane % 16), dims
//                  32 kk + 8 (lane / 16) .. +7 are 16 contiguous bytes),
//                  B = Q^T of all heads (registers);
//   softmax        per head over the tile's keys, running max raised lazily;
//   O^T += V^T P^T the gathered V rows go straight to the wave's own LDS
//                  tile (global_load_lds, swizzled rows) and are read back
//                  transposed; P^T is the S^T accumulators in place.
// Positions past the end of the list read the last kept token again and
// get -inf scores.
#include "attn_bf16_common.hpp"
#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

using namespace attn_bf16;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds_wave_base + 16 l (lds_wave_base is the same for the whole wave).
__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_wave_base, 16, 0, 0);
}

constexpr int kMqaWaves = 4;  // query rows per workgroup

// SHARED: K and V are one buffer (a key-only cache): each kept row is
// gathered once, into the LDS tile, and the K operand is read back from it.
template <int HB, bool SHARED>  // heads = 16 HB
__global__ __launch_bounds__(64 * kMqaWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_mqa_bf16_kernel(GatherParams a) {
  constexpr int H = 16 * HB;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kMqaWaves][kTileBytes];

  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * kMqaWaves + wave;  // b * T + t
  if (row >= a.B * a.T) return;                   // whole wave; no barriers below
  const int b = row / a.T, t = row % a.T, p = a.q_pos0 + t;
  const int count = a.counts ? a.counts[row] : min(a.top_k, p + 1);
  const int32_t* list = a.list + (size_t)row * a.list_stride;
  const bf16* kbase = static_cast<const bf16*>(a.k) + (size_t)b * a.kv_cap * kD;
  const bf16* vbase = static_cast<const bf16*>(a.v) + (size_t)b * a.kv_cap * kD;
  unsigned char* vl = lds[wave];

  // Q^T operands: head 16 hb + c, dims 32 kk + 8 g + e.
  const bf16* qrow = static_cast<const bf16*>(a.q) + (size_t)row * H * kD;
  bf16x8 qreg[HB][kKS];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) qreg[hb][kk] = load_frag<bf16>(qrow + (16 * hb + c) * kD + 32 * kk + 8 * g);

  f32x4 o[kDB][HB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) o[db][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[HB], l_run[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m_run[hb] = fneg_inf();
    l_run[hb] = 0.f;
  }
  const float sl2 = a.scale_log2;

  for (int j0 = 0; j0 < count; j0 += kKT) {
    const int nk = min(kKT, count - j0);
    // Token of tile row `lane`; lists come from the library's own top-k and
    // hold tokens in [0, n_kv): the clamp only keeps a corrupted list inside
    // the caches.
    const int tok = min(max(list[j0 + min(lane, nk - 1)], 0), a.n_kv - 1);

    // V rows into this wave's LDS tile: instruction i fills rows 4i..4i+3,
    // lane l physical column l % 16 of row 4i + l / 16.
#pragma unroll
    for (int i = 0; i < kKT / 4; ++i) {
      const int r = 4 * i + (lane >> 4);
      const int tr_ = __shfl(tok, r, 64);
      dma16(vbase + (size_t)tr_ * kD + (((lane & 15) ^ swz(r)) << 3), vl + i * 1024);
    }
    // K fragments: key 16 kb + c (from the LDS tile when K is V: the rows
    // landed once this wave's loads are done; no other wave writes it).
    bf16x8 kf[4][kKS];
    if constexpr (SHARED) {
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int kk = 0; kk < kKS; ++kk)
          kf[kb][kk] = *reinterpret_cast<const bf16x8*>(vl + tile_off(16 * kb + c, 4 * kk + g));
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int tk = __shfl(tok, 16 * kb + c, 64);
#pragma unroll
        for (int kk = 0; kk < kKS; ++kk) kf[kb][kk] = load_frag<bf16>(kbase + (size_t)tk * kD + 32 * kk + 8 * g);
      }
    }

    // S^T = K Q^T: lane (c, g) holds keys 16 kb + 4 g + r of head 16 hb + c.
    f32x4 sacc[4][HB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) sacc[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) sacc[kb][hb] = mma_kstep(kf[kb][kk], qreg[hb][kk], sacc[kb][hb]);
    if (nk < kKT) {  // the list's last, partial tile
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + 4 * g + r >= nk) sacc[kb][hb][r] = fneg_inf();
    }

    // Tile maxima per head; the running maximum is raised lazily.
    float mx_all[HB];
    bool need_any = false;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float mx = fneg_inf();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb][hb][r]);
      mx_all[hb] = rows4_max(mx) * sl2;
      need_any = need_any || mx_all[hb] > m_run[hb] + kLazyMax;
    }
    if (ballot64(need_any) != 0ull) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const bool need = mx_all[hb] > m_run[hb] + kLazyMax;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run[hb] - mx_all[hb]) : 1.f;
        if (need) m_run[hb] = mx_all[hb];
        l_run[hb] *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; ++db) o[db][hb] *= alpha;
      }
    }
    // P^T in bf16, in the accumulator layout; row sums over the bf16 values.
    bf16x8 pf[HB][2];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const float m_use = m_run[hb] == fneg_inf() ? 0.f : m_run[hb];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 pv;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            pv[4 * hf + r] = (bf16)__builtin_amdgcn_exp2f(fmaf(sacc[2 * ks + hf][hb][r], sl2, -m_use));
        pf[hb][ks] = pv;
        l_run[hb] = sum8_bf16(pv, l_run[hb]);
      }
    }
    // O^T += V^T P^T (the V tile loads are waited for before the first read).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const bf16x8 vf = vt_frag(vl, ks, db, c, g);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) o[db][hb] = mma_kstep(vf, pf[hb][ks], o[db][hb]);
      }
  }
  // no tile load may still be writing the LDS tile when the wave exits
  __builtin_amdgcn_s_waitcnt(0);

  // O^T[dim 16 db + 4 g + r][head 16 hb + c]
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const float l_tot = rows4_sum(l_run[hb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16* orow = static_cast<bf16*>(a.out) + ((size_t)row * H + 16 * hb + c) * kD;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const f32x4 v = o[db][hb] * inv;
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
      const float m_use = m_run[hb] == fneg_inf() ? 0.f : m_run[hb];
      a.lse[(size_t)row * H + 16 * hb + c] = l_tot > 0.f ? (m_use + __log2f(l_tot)) * kLn2f : fneg_inf();
    }
  }
}

}  // namespace

bool attn_mqa_bf16_supported(int H, int Hkv, int D) { return D == kD && Hkv == 1 && (H == 16 || H == 32); }

hipError_t launch_attn_mqa_bf16(const GatherParams& p, hipStream_t st) {
  const long long rows = (long long)p.B * p.T;
  const long long nblocks = (rows + kMqaWaves - 1) / kMqaWaves;
  if (nblocks > 0x7fffffffll || !attn_mqa_bf16_supported(p.H, p.Hkv, kD)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblocks), block(64 * kMqaWaves);
  if (p.k == p.v) {
    if (p.H == 16) hipLaunchKernelGGL((attn_mqa_bf16_kernel<1, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((attn_mqa_bf16_kernel<2, true>), grid, block, 0, st, p);
  } else {
    if (p.H == 16) hipLaunchKernelGGL((attn_mqa_bf16_kernel<1, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((attn_mqa_bf16_kernel<2, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace dsa
