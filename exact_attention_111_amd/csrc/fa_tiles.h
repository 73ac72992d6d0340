// fa_tiles.h — LDS layouts of K/V-style tiles and the order of query tiles, shared by the
// forward and backward kernels.
#pragma once

#include <algorithm>

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

// Division by a value fixed for a whole launch, as one 64-bit product and a shift (the
// invariant-divisor method of Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): for 0 <= n < 2^31 and 1 <= d < 2^31, with l = ceil(log2 d) and
// m = ceil(2^(31 + l) / d), which is below 2^32, m d - 2^(31 + l) < d <= 2^l and so
// floor(n / d) = floor(m n / 2^(31 + l)). A signed division by a launch argument costs the
// scalar unit about fifteen instructions after a reciprocal, and all the waves of a
// workgroup decode their tile at once on the compute unit's one scalar unit.
struct Divisor {
  unsigned m;
  int shift;  // 31 + l
  int d;
};

inline Divisor make_divisor(int d) {  // host side; 1 <= d < 2^31
  int l = 0;
  while ((1LL << l) < d) ++l;
  const unsigned long long m = ((1ULL << (31 + l)) + (unsigned long long)d - 1) / (unsigned long long)d;
  return Divisor{(unsigned)m, 31 + l, d};
}

__device__ __forceinline__ int div_by(int n, const Divisor& v) {
  return (int)(((unsigned long long)v.m * (unsigned)n) >> v.shift);
}

// Order of the query tiles of a prefill-style launch: nwg tiles, ntq per head (or per
// (batch, KV head) pair), heaviest tile first. Tile id i is meant for XCD i % 8 as that XCD's
// slot i / 8: it is the hardware workgroup id when every tile is a workgroup (hardware id i
// runs on XCD i % 8), and tile_of_program keeps a persistent workgroup on the XCD its tile
// ids belong to.
// When the head count is a multiple of 8, head bh belongs to XCD bh % 8, so every XCD gets
// the same mix of sequences (equal work even when lengths vary) and its L2 serves the K/V of
// its own heads only. An XCD goes through its heads in groups of just enough heads to fill
// its 32 CUs with query tiles, heaviest tile first across the group: one head at a time when
// a head has 32 or more tiles (its CUs then share that head's K/V in L2; walking all of an
// XCD's heads at once multiplied HBM re-reads 2.3x at B=1, H=32, L=16384), several when
// heads are short (one head at a time would start the heaviest tiles of later heads too
// late). Otherwise each XCD takes a contiguous range of tile ids, heaviest tile first within
// a head.
// The host computes the launch's constants once (make_tile_order); tile_order decodes a tile
// id with products and shifts only.
struct TileOrder {
  int ntq;
  int grouped;     // the head count is a multiple of 8: heads go to the XCDs in groups
  int g_last;      // grouped: index of an XCD's last head group
  Divisor span;    // grouped: tiles of one head group (heads per group x ntq)
  Divisor grp;     // grouped: heads per group
  Divisor last;    // grouped: heads in the last group (it may be smaller)
  int per, extra;  // otherwise: tiles per XCD, and how many XCDs take one more
  Divisor tiles;   // otherwise: ntq
};

inline TileOrder make_tile_order(int nwg, int ntq) {  // host side; nwg >= 1, ntq >= 1
  TileOrder t{};
  t.ntq = ntq;
  const int nheads = nwg / ntq;
  t.grouped = (nheads & 7) == 0;
  if (t.grouped) {
    const int per_xcd = nheads >> 3;
    const int group = std::min(std::max(1, (32 + ntq - 1) / ntq), per_xcd);
    t.g_last = (per_xcd - 1) / group;
    t.span = make_divisor(group * ntq);
    t.grp = make_divisor(group);
    t.last = make_divisor(per_xcd - t.g_last * group);
  } else {
    t.per = nwg >> 3;
    t.extra = nwg & 7;
    t.tiles = make_divisor(ntq);
  }
  return t;
}

// Head (or pair) bh and query tile qt of tile id hw.
__device__ __forceinline__ void tile_order(const TileOrder& t, int hw, int& bh, int& qt) {
  const int xcd = hw & 7, slot = hw >> 3;
  if (t.grouped) {
    const int g = div_by(slot, t.span);
    const int idx = slot - g * t.span.d;
    const bool lg = g == t.g_last;
    const Divisor in_group{lg ? t.last.m : t.grp.m, lg ? t.last.shift : t.grp.shift, lg ? t.last.d : t.grp.d};
    const int i = div_by(idx, in_group);
    qt = t.ntq - 1 - i;
    bh = xcd + 8 * (g * t.grp.d + idx - i * in_group.d);
  } else {
    const int logical = xcd * t.per + min(xcd, t.extra) + slot;
    bh = div_by(logical, t.tiles);
    qt = t.ntq - 1 - (logical - bh * t.ntq);
  }
}

// Tile id (as numbered for tile_order) that workgroup p of nprog takes in its round r, or
// -1 when it has no more. With one workgroup per tile (nprog == ntiles) workgroup p takes tile
// p. Otherwise nprog is a multiple of 8: workgroup p stays on XCD p % 8 (the tiles whose ids
// are p mod 8, which tile_order lists heaviest first) and takes one of them in each round
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
