// Per-row e4m3 quantisation of the indexer's queries and keys (the fp8
// reading of the indexer; the pages keep these tensors unquantised because
// selection is sensitive to their precision [aiaulis para 5; devotd section
// 3], and this path exists to measure that).
//
// One wave per row of 128 values, two per lane: scale = max|x| / 448 (1 for
// an all-zero row), code = e4m3(x / scale) rounded to nearest even, every
// division correctly rounded in float32. Query rows also store
// wq = w * scale, the query scale folded into the head weight; key rows store
// their scale, which the scoring kernels apply after the head sum
// (max(0, a b z) = a b max(0, z) for positive scales).
#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {
namespace {

constexpr float kE4m3Max = 448.f;

// e4m3 code of r (|r| <= 448 up to float32 rounding): 1 sign bit, exponent
// bias 7, 3 mantissa bits, subnormal step 2^-9; ties to the even mantissa;
// magnitudes from 448 up map to 448.
__device__ __forceinline__ uint32_t e4m3_code(float r) {
  const uint32_t sign = (__float_as_uint(r) >> 31) << 7;
  const float a = fabsf(r);
  uint32_t code;
  if (!(a < kE4m3Max)) {
    code = 0x7e;  // 1.75 * 2^8
  } else if (a < 0.015625f) {
    // subnormal: a multiple of 2^-9 (2^-6 itself rounds up into code 8, the
    // smallest normal)
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;   // -6..8
    const float m = __builtin_rintf(a * __builtin_ldexpf(1.f, 3 - e));  // 8..16, exact scaling
    code = (uint32_t)((e + 7) << 3) + (uint32_t)m - 8u;            // m = 16 carries into the exponent
  }
  return sign | code;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Rows 0 .. nq-1: query head rows (b, t, h); rows nq .. nq+nk-1: key rows of
// the call's tokens (b, t) at cache position q_pos0 + t.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(QuantParams a, int nq, int nk) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)nq + nk) return;  // whole wave
  const bool is_q = row < nq;
  size_t src_row, dst_row;
  if (is_q) {
    src_row = dst_row = (size_t)row;
  } else {
    const int kr = (int)(row - nq), b = kr / a.T, t = kr - b * a.T;
    src_row = dst_row = (size_t)b * a.kv_cap + a.q_pos0 + t;
  }
  const uint32_t pair = reinterpret_cast<const uint32_t*>(is_q ? a.qidx : a.kidx)[src_row * 64 + lane];
  const float x0 = bf16_lo(pair), x1 = bf16_hi(pair);
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float scale = amax > 0.f ? amax / kE4m3Max : 1.f;
  const uint32_t c0 = e4m3_code(x0 / scale), c1 = e4m3_code(x1 / scale);
  uint16_t* dst = reinterpret_cast<uint16_t*>(is_q ? a.qidx8 : a.kidx8);
  dst[dst_row * 64 + lane] = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) {
    if (is_q) a.wq[row] = a.w[row] * scale;
    else a.kscale[dst_row] = scale;
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t st) {
  const long long nq = p.qidx ? (long long)p.B * p.T * p.HI : 0;
  const long long nk = p.kidx ? (long long)p.B * p.T : 0;
  const long long blocks = (nq + nk + 3) / 4;
  if (nq + nk > 0x7fffffffll || blocks == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, (int)nq, (int)nk);
  return hipGetLastError();
}

}  // namespace dsa
