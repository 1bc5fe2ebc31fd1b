// Shared pieces of the bf16 (head dim 128) attention kernels: tile layout in
// LDS, the swizzle of key rows, and small math helpers.
#pragma once

#include "dsa_device.hpp"

namespace dsa {
namespace attn_bf16 {

constexpr int kD = 128;             // head dim
constexpr int kKT = 64;             // keys per tile
constexpr int kKS = kD / 32;        // k-steps of S^T (head dim / 32)
constexpr int kDB = kD / 16;        // 16-dim blocks of O^T
constexpr int kRow = kD * 2;                 // bytes per key row in LDS (K and V)
constexpr int kTileBytes = kKT * kRow;       // one 64-key tile of K or V
constexpr float kLazyMax = 8.0f;             // log2 units
constexpr float kLn2f = 0.69314718055994530942f;

// Swizzle of a key row's 16-byte columns: physical column = col ^ swz(row).
// LDS serves 256 bytes (64 four-byte banks) per pass, so the 16-byte pieces
// that 16 lanes of a K fragment read (16 rows, one column) and that 32 lanes
// of a V^T transpose read (two groups of four rows, two columns each) must
// all fall in different 16-byte slots of a 256-byte window. swz is a
// bijection on row mod 16 (the K read); within an aligned group of four rows
// its bits 1-2 take all four values (eight slots for one 16-lane group of the
// transpose read), and bit 3 is row bit 2 ^ row bit 3, so the neighbouring
// group of four rows lands in the other eight slots. (Bit 3 equal to row
// bit 3 alone put both groups in the same slots: a two-way conflict on
// every transpose read, measured as half of the kernel's LDS cycles.)
__device__ __forceinline__ int swz(int row) {
  return ((row & 3) << 1) | ((row >> 2) & 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 3);
}
// Byte offset of 16-byte column `col` of key row `row` in a swizzled tile.
__device__ __forceinline__ int tile_off(int row, int col) { return row * kRow + ((col ^ swz(row)) << 4); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float sum8_bf16(const bf16x8& p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[2 * i], p[2 * i + 1]}, one, acc, false);
  return acc;
}

// V^T fragment (dims 16 db + (lane % 16), keys 32 ks + 16 hf + 4 g + (0..3)
// for hf = 0, 1 -- the key order of the S^T accumulators) from a row-major,
// swizzled V tile, with two LDS transpose reads: within a 16-lane group lane
// c receives element c % 4 of the 8-byte pieces lanes 4k + c/4 point at, so
// pointing lane 4r + j at dims 4j..4j+3 of key r gives each lane one dim of
// four consecutive keys.
__device__ __forceinline__ bf16x8 vt_frag(const unsigned char* vl, int ks, int db, int c, int g) {
  v4i16 t[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int row = 32 * ks + 16 * hf + 4 * g + (c >> 2), j = c & 3;
    t[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + tile_off(row, 2 * db + (j >> 1)) + 8 * (j & 1)));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace attn_bf16
}  // namespace dsa
