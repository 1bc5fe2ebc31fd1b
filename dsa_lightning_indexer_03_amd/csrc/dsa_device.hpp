// Device-side building blocks for the gfx950 DSA kernels: fragment types, the
// MFMA k-step, cross-lane swaps and orderable float keys.
//
// Matrix-core conventions (checked on an MI355X with an in-bounds probe):
//   v_mfma_f32_16x16x32_bf16  A: lane l holds A[l%16][8*(l/16)+e], e=0..7
//                             B: lane l holds B[8*(l/16)+e][l%16]
//                             C: lane l holds C[4*(l/16)+r][l%16], r=0..3
//   v_mfma_f32_16x16x4f32     A: lane l holds A[l%16][l/16]; B: B[l/16][l%16];
//                             C as above.
// A "k-step" here covers 32 reduction indices: lane group g = l/16 owns the 8
// indices 8g..8g+7 of it. For bf16 that is one 16x16x32 MFMA; for fp32 it is
// eight 16x16x4 MFMAs, the e-th of which takes element e of every lane, so
// both element types use the same data-to-lane assignment.
//   permlane32_swap(x, y) -> (x', y') = ([x_lo, y_lo], [x_hi, y_hi])  (32-lane halves)
//   permlane16_swap(x, y) -> (x', y') = ([x0, y0, x2, y2], [x1, y1, x3, y3])  (16-lane rows)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One e4m3 code (1 sign, 4 exponent, 3 mantissa bits): the storage type of
// the fp8 indexer's queries and keys.
struct fp8e4m3 {
  uint8_t bits;
};
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };
template <> struct Frag<fp8e4m3> { typedef i32x8 type; };
template <typename T> using frag_t = typename Frag<T>::type;

// Reduction indices one k-step covers: 32 for bf16 and fp32, 128 for fp8
// (one v_mfma_scale_f32_16x16x128_f8f6f4). Lane group g = l/16 owns a quarter
// of them; frag_off is the first element lane group g holds in k-step kk.
template <typename T> inline constexpr int kStepElems = 32;
template <> inline constexpr int kStepElems<fp8e4m3> = 128;
template <typename T> __device__ __forceinline__ int frag_off(int kk, int g) {
  return kStepElems<T> * kk + (kStepElems<T> / 4) * g;
}

// 8 contiguous elements (16 B for bf16, 32 B for fp32) from 16-B aligned memory.
template <typename T> __device__ __forceinline__ frag_t<T> load_frag(const T* p);
template <> __device__ __forceinline__ bf16x8 load_frag<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ f32x8 load_frag<float>(const float* p) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <> __device__ __forceinline__ i32x8 load_frag<fp8e4m3>(const fp8e4m3* p) {  // 32 codes, 32-B aligned
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <typename T> __device__ __forceinline__ frag_t<T> zero_frag() { return frag_t<T>{}; }

// acc += A(16 x 32) * B(32 x 16) for one k-step.
__device__ __forceinline__ f32x4 mma_kstep(const bf16x8& a, const bf16x8& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// fp8: A 16 x 128, B 128 x 16, e4m3 codes with unit scales (exponent byte
// 127). Lane l holds 32 codes of row (A) or column (B) l % 16; A and B use
// the same assignment of reduction indices to lanes, which is all a dot
// product needs (checked against a CPU product on an MI355X).
__device__ __forceinline__ f32x4 mma_kstep(const i32x8& a, const i32x8& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x4 mma_kstep(const f32x8& a, const f32x8& b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ void swap32(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// v_max_f32 as one instruction: fmaxf would first quiet both operands when
// they come from a lane swap (the compiler cannot see that they are never
// NaN), three instructions instead of one.
__device__ __forceinline__ float max_plain(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Max / sum of x over the four 16-lane rows (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float rows4_max(float x) {
  float y = x;
  swap32(x, y);
  x = max_plain(x, y);
  y = x;
  swap16(x, y);
  return max_plain(x, y);
}
__device__ __forceinline__ float rows4_sum(float x) {
  float y = x;
  swap32(x, y);
  x = x + y;
  y = x;
  swap16(x, y);
  return x + y;
}

// Unsigned key with the order of the float value; -0.0 maps to +0.0.
__device__ __forceinline__ uint32_t orderable_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ float fneg_inf() { return __uint_as_float(0xff800000u); }

// Cache extent of sequence b: the call's (q_pos0, n_kv), or, for a batch of
// different lengths, its own length len (clamped to [T, n_kv]) with its T
// queries at positions len - T .. len - 1.
__device__ __forceinline__ void seq_extent(const int32_t* seq_len, int b, int T, int q_pos0, int n_kv, int& q0,
                                           int& nkv) {
  if (seq_len) {
    nkv = min(max(seq_len[b], T), n_kv);
    q0 = nkv - T;
  } else {
    nkv = n_kv;
    q0 = q_pos0;
  }
}

// bf16 <-> f32 on raw 16-bit patterns.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> __device__ __forceinline__ T from_float(float x);
template <> __device__ __forceinline__ float from_float<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_float<bf16>(float x) { return (bf16)x; }

}  // namespace dsa
