// fa_tiles.h — LDS layout of K/V-style tiles shared by the forward and backward kernels.
#pragma once

namespace fa {

// Tiles of rows of d bf16 values are stored row-major in LDS with the 16-byte chunks of row
// r permuted by an XOR. Two read patterns are served without bank conflicts (gfx950 LDS:
// 128-bit reads are served 16 lanes at a time over a 256-byte bank window):
//   k_xor — 128-bit reads by 16 lanes = 16 consecutive rows, same logical chunk: every row
//   of a 16-row group lands on a different 16-byte slot;
//   v_xor — transposed 64-bit reads (ds_read_b64_tr_b16), where a 16-lane group touches 4
//   consecutive rows x one 32-byte chunk pair, two groups per access: the 8 (row, pair)
//   slots of an access differ.
template <int D>
__device__ __forceinline__ int k_xor(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_xor(int r) {
  const int j = r & 3;
  return D == 128 ? 2 * (j ^ ((j & 1) << 2)) : ((j & 2) << 1);
}

// kv_xor — one layout that serves both patterns, for tiles the backward reads both ways
// (rows for products over d, transposed for products over rows):
//   128-bit row reads: the 16 consecutive rows of a 16-lane group get 16 different values
//   of the permutation (d = 128), or 8 different ones among the even and among the odd rows,
//   which share a bank window two rows at a time (d = 64);
//   transposed reads: 4 consecutive rows x 4 consecutive chunks per 32 lanes; the rows of
//   such a group differ in bits 2..3 of the permutation (d = 128), or the two rows of the
//   group that share a bank window differ in bit 2 (d = 64), so the 16 slots are distinct.
template <int D>
__device__ __forceinline__ int kv_xor(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

}  // namespace fa
