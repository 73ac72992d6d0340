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

// Query tile and (batch, head) of prefill tile id `hw` (ntq query tiles per head, nwg tiles),
// heaviest tile first. Tile id i is meant for XCD i % 8 as that XCD's slot i / 8: it is the
// hardware workgroup id when every tile is a workgroup (hardware id i runs on XCD i % 8), and
// tile_of_program keeps a persistent workgroup on the XCD its tile ids belong to.
// When the (batch, head) count is a multiple of 8, head bh belongs to XCD bh % 8, so every
// XCD gets the same mix of sequences (equal work even when lengths vary) and its L2 serves
// the K/V of its own heads only. An XCD goes through its heads in groups of just enough
// heads to fill its 32 CUs with query tiles, heaviest tile first across the group: one head
// at a time when a head has 32 or more tiles (its CUs then share that head's K/V in L2;
// walking all of an XCD's heads at once multiplied HBM re-reads 2.3x at B=1, H=32,
// L=16384), several when heads are short (one head at a time would start the heaviest tiles
// of later heads too late). Otherwise each XCD takes a contiguous range of logical ids,
// heaviest tile first within a head.
__device__ __forceinline__ void xcd_tile_order(int hw, int nwg, int ntq, int& bh, int& qt) {
  const int xcd = hw & 7, slot = hw >> 3;
  const int nheads = nwg / ntq;
  if ((nheads & 7) == 0) {
    const int per_xcd = nheads >> 3;
    const int group = min(max(1, (32 + ntq - 1) / ntq), per_xcd);
    const int g = slot / (group * ntq);
    const int in_group = min(group, per_xcd - g * group);  // the last group may be smaller
    const int idx = slot - g * group * ntq;
    qt = ntq - 1 - idx / in_group;
    bh = xcd + 8 * (g * group + idx % in_group);
  } else {
    const int per = nwg >> 3, extra = nwg & 7;
    const int logical = xcd * per + min(xcd, extra) + slot;
    bh = logical / ntq;
    qt = ntq - 1 - (logical - bh * ntq);
  }
}

// Tile id (as numbered for xcd_tile_order) that workgroup p of nprog takes in its round r, or
// -1 when it has no more. With one workgroup per tile (nprog == ntiles) workgroup p takes tile
// p. Otherwise nprog is a multiple of 8: workgroup p stays on XCD p % 8 (the tiles whose ids
// are p mod 8, which xcd_tile_order lists heaviest first) and takes one of them in each round
// of nprog / 8, forward through the round in even rounds and backward in odd ones, so that
// the workgroup with a round's heaviest tile gets the next round's lightest.
__device__ __forceinline__ int tile_of_program(int p, int r, int nprog, int ntiles) {
  if (nprog == ntiles) return r == 0 ? p : -1;
  const int x = p & 7, s = p >> 3, S = nprog >> 3;
  const int slot = S * r + ((r & 1) ? S - 1 - s : s);
  const int id = 8 * slot + x;
  return id < ntiles ? id : -1;
}

}  // namespace fa
