// fa_fwd_fp8.hip — prefill attention on FP8 (E4M3) Q, K, V for gfx950 (MI355X), d = 128.
//
// The low-precision step of FlashAttention-3 ("FlashAttention 与长上下文：先分清三张账", section
// on FlashAttention-2/3; the pages give no scaling scheme). The scheme used:
//   * q, k, v are OCP E4M3 codes with one fp32 descale per (batch, head); scores are
//     t = s * (scale * log2(e) * descale_q * descale_k) with s = q8 . k8 from the FP8 matrix
//     cores (fp32 accumulation of exact products);
//   * each row keeps an integer base-2 reference m (raised to ceil(tile max) when a tile's
//     scores pass it);
//   * x = 2^(t - m + 8) <= 256 enters the P V product as E4M3 (v_cvt_pk_fp8_f32, round to
//     nearest even) while the row sum l adds the unrounded x;
//   * o and l are kept relative to a frame mf <= m (the row's first reference, moved up only
//     when m passes it by more than 64): a tile's x enters with the factor 2^(m - mf), applied
//     to P through the product's E8M0 scale operand and to l with an fma, so a rising
//     reference costs no pass over the output accumulators. Every factor is a power of two;
//   * O = descale_v * o / l (bf16) and LSE = ln(2) (mf - 8 + log2 l).
// E4M3 rounding commutes with power-of-two scaling, so the result does not depend on the
// tiling: it is the whole-row definition with the final reference.
//
// gfx950 mapping (v_mfma_scale_f32_32x32x64_f8f6f4; unit scales except the per-row scale of P):
//   * Workgroup: 256 query rows of one (batch, head) at a time (dense inputs: a persistent grid
//     taking tiles in rounds, as the bf16 prefill), 8 waves of 32 rows, two per SIMD. Each
//     wave keeps its Q rows as B operands: lane (half, col) holds dims 64 ks + 32 half ..
//     + 31 of query row col (the operands' byte t of half h pair up in the product). On the
//     causal diagonal a wave stops computing after the last tile its rows can see; the two
//     waves of a SIMD hold a top and a bottom row block.
//   * 64-key K and V tiles (8 KB each) stream through a 4-stage LDS ring filled by direct
//     buffer-to-LDS loads three tiles ahead, one barrier per tile. The S products of the next
//     tile are issued before the softmax of the current one (software pipeline).
//   * S^T = K Q^T: K rows read 32 bytes at a time (two 128-bit reads); accumulator element
//     r of key block kb is key 32 kb + 8 (r / 4) + 4 half + r % 4 of query col.
//   * P^T as the B operand of O^T += V^T P^T: byte 16 kb + r of a lane is that element's
//     E4M3 value. V^T comes from ds_read_b64_tr_b8: output lane 16 g + j gets byte j % 8 of
//     the 8-byte addresses of lanes 16 g + j / 8 + 2 t (t = 0..7), so lane 16 g + p points
//     at the key of byte 8 u + p / 2 and the 8 dims starting 32 nb + 16 (g % 2) + 8 (p % 2).
//   * LDS layout: K chunk ^ ((row >> 1) & 7) (128-bit row reads: 16 rows of 128 bytes per
//     read); V chunk ^ 2 ((row >> 1 & 1) | (row >> 3 & 1) << 1) (transposed reads: 8 rows x
//     32 bytes per 32 lanes); both conflict-free.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kF8D = 128;              // head dim
constexpr int kF8NW = 8;               // waves per workgroup (two per SIMD)
constexpr int kF8NT = 64 * kF8NW;
constexpr int kF8BM = 32 * kF8NW;      // query rows per workgroup
constexpr int kF8BN = 64;              // keys per tile
constexpr int kF8Tile = kF8BN * kF8D;  // bytes of a K or V tile
constexpr int kF8Stage = 2 * kF8Tile;  // K | V
constexpr int kF8NS = 4;               // stages in the ring
constexpr int kF8KS = kF8D / 64;       // 32x32x64 k-steps over d
constexpr int kF8NB = kF8D / 32;       // 32-wide blocks of O^T
static_assert(kF8Tile == 1024 * kF8NW, "one 1 KB direct load per wave and tile");
constexpr int kF8RS = 2 * kF8D + 16;   // bytes per row of staged O (the pad spreads rows over banks)
constexpr int kF8Smem = kF8NS * kF8Stage > kF8NW * 32 * kF8RS ? kF8NS * kF8Stage : kF8NW * 32 * kF8RS;

__device__ __forceinline__ int f8_kxor(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int f8_vxor(int r) { return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)); }

// Key of P^T byte T (0..31) in lane half h: accumulator element r = T % 16 of key block T / 16.
__device__ __forceinline__ int f8_key(int h, int T) { return 32 * (T >> 4) + 8 * ((T & 15) >> 2) + 4 * h + (T & 3); }

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The same product with the B operand scaled by 2^(sb - 127) (E8M0, one per lane: the lane's
// 32 values of B along K, here one query row's P for half of the tile's keys).
__device__ __forceinline__ f32x16 mfma_f8_bscaled(i32x8 a, i32x8 b, f32x16 c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

struct Fp8Args {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  const float* q_descale;  // [B, H]
  const float* k_descale;  // [B, Hkv]
  const float* v_descale;  // [B, Hkv]
  __bf16* o;
  float* lse;
  int B, H, Hkv, Lq, Lk;
  int group, ntq, nwg;
  int nprog;                   // workgroups launched (tile_of_program)
  TileOrder order;             // tile_order over (batch, KV head) pairs, group x ntq tiles each
  Divisor group_div, hkv_div;  // H / Hkv and Hkv as divisors
  float scale_log2;
  int causal, window;
  const int32_t* seqlens;
};

__global__ __launch_bounds__(kF8NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_fp8_kernel(const Fp8Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) char smem[kF8Smem];

  // Tiles of this workgroup, one per round (tile_of_program, as in the bf16 prefill).
  for (int round = 0;; ++round) {
    const int tile_id = tile_of_program(blockIdx.x, round, a.nprog, a.nwg);
    if (tile_id < 0) break;
    // Per-lane values are rebuilt in every round rather than hoisted out of the round loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;

    // Workgroup order as in the bf16 prefill: (batch, KV head) pairs with group x ntq tiles
    // each, so the query heads that share a KV head run side by side on one XCD.
    int pair, u;
    tile_order(a.order, tile_id, pair, u);
    const int qt = div_by(u, a.group_div);
    const int b = div_by(pair, a.hkv_div), kvh = pair - b * a.Hkv;
    const int h = kvh * a.group + (u - qt * a.group);
    int n_kv = a.Lk, n_q = a.Lq;
    if (a.seqlens != nullptr) {
      const int n = min(max(load_const(a.seqlens + b), 0), a.Lk);
      n_kv = n;
      n_q = n;
    }
    const int delta = a.Lk - a.Lq;
    const int q0 = qt * kF8BM;
    // Waves w and w + 4 share a SIMD; they take row blocks s and 7 - s, a top block of the tile
    // with a bottom one, so that every SIMD is left the same work on causal diagonal tiles.
    const int rblk = w < kF8NW / 2 ? w : 3 * kF8NW / 2 - 1 - w;
    const int qw0 = q0 + 32 * rblk;
    const int my_q = qw0 + col;

    int kv_end = 0;
    if (q0 < n_q) {
      kv_end = n_kv;
      if (a.causal) kv_end = min(kv_end, min(q0 + kF8BM, n_q) + delta);
      kv_end = max(kv_end, 0);
    }
    kv_end = __builtin_amdgcn_readfirstlane(kv_end);
    const int kbase = __builtin_amdgcn_readfirstlane(
        a.window > 0 ? (max(q0 + delta - a.window + 1, 0) / kF8BN) * kF8BN : 0);
    const int ntk = max((kv_end - kbase + kF8BN - 1) / kF8BN, 0);
    // Tiles this wave has keys in (causal: up to its last row's newest key); past them it only
    // moves its share of the tiles into LDS and meets the barriers.
    const int ntw = __builtin_amdgcn_readfirstlane(
        a.causal ? min(ntk, max((qw0 + 31 + delta - kbase) / kF8BN + 1, 1)) : ntk);

    // Combined score factor (base 2) and the output descale.
    const float c = a.scale_log2 * a.q_descale[b * a.H + h] * a.k_descale[b * a.Hkv + kvh];
    const float dv = a.v_descale[b * a.Hkv + kvh];

    // Q rows as B operands (read from LDS in the prologue below).
    i32x8 qf[kF8KS];

    f32x16 oacc[kF8NB];
#pragma unroll
    for (int nb = 0; nb < kF8NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.f;
    float m = kNegInf, l = 0.f;
    float mf = kNegInf;  // the frame of o and l: the row's first reference, or the one of their last rescale

    // LDS addresses. K: lane (half, col) reads row 32 kb + col, logical chunks 4 ks + 2 half
    // (+1); kv rows of the two key blocks share the swizzle, so kb is an immediate offset.
    int kaddr[kF8KS][2];
#pragma unroll
    for (int ks = 0; ks < kF8KS; ++ks)
#pragma unroll
      for (int p = 0; p < 2; ++p) kaddr[ks][p] = col * kF8D + (((4 * ks + 2 * half + p) ^ f8_kxor(col)) << 4);
    // V^T: lane 16 g + p, read u (keys of bytes 8 u .. 8 u + 7), block nb; reads u + 2 are
    // 32 rows further on with the same swizzle.
    int vaddr[2][kF8NB];
    {
      const int g = lane >> 4, p = lane & 15;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = f8_key(half, 8 * u + (p >> 1));
#pragma unroll
        for (int nb = 0; nb < kF8NB; ++nb)
          vaddr[u][nb] = key * kF8D + (((2 * nb + (g & 1)) ^ f8_vxor(key)) << 4) + 8 * (p & 1);
      }
    }
    // Direct-load source offsets of this wave's 1 KB of each tile.
    const int lrow = w * 8 + (lane >> 3), pch = lane & 7;
    const unsigned koff = (unsigned)(lrow * kF8D + ((pch ^ f8_kxor(lrow)) << 4));
    const unsigned voff = (unsigned)(lrow * kF8D + ((pch ^ f8_vxor(lrow)) << 4));
    const size_t kv_row0 = (size_t)(b * a.Hkv + kvh) * a.Lk;
    const char* const ksrc = reinterpret_cast<const char*>(a.k) + kv_row0 * kF8D;
    const char* const vsrc = reinterpret_cast<const char*>(a.v) + kv_row0 * kF8D;
    auto issue = [&](int t) {
      const int k0 = kbase + t * kF8BN;
      const unsigned nrows = (unsigned)max(kv_end - k0, 0);
      char* st = smem + (t % kF8NS) * kF8Stage;
      serial_fence();
      lds_dma16_buf(raw_buffer_rsrc(ksrc + (size_t)k0 * kF8D, nrows * kF8D), koff, lds_addr(st + w * 1024));
      lds_dma16_buf(raw_buffer_rsrc(vsrc + (size_t)k0 * kF8D, nrows * kF8D), voff, lds_addr(st + kF8Tile + w * 1024));
      serial_fence();
    };

    // The tile's Q rows come through LDS as well, into stages 2 and 3 (refilled only after
    // every wave has read its rows): row r at byte 128 r, 16-byte chunk c at c ^ (r & 7), so
    // that the 16 rows of a 128-bit read hit distinct banks. With no Q row loaded directly into
    // registers, the compiler tracks no load on the tile path; otherwise it cannot tell, past
    // the direct loads it does not see, that the Q loads are done, and waits for every load
    // before the first score product of each tile (the stage just issued included).
    constexpr int kQBase = 2 * kF8Stage;
    static_assert(kF8BM * kF8D <= (kF8NS - 2) * kF8Stage, "the Q tile fits in stages 2 and 3");
    auto issue_q = [&] {
      const u32x4 rq = raw_buffer_rsrc(a.q + ((size_t)(b * a.H + h) * a.Lq + q0) * kF8D,
                                       (unsigned)max(min(n_q, a.Lq) - q0, 0) * kF8D);
      serial_fence();
#pragma unroll
      for (int i = 0; i < kF8BM * kF8D / 1024 / kF8NW; ++i) {  // wave w: rows 32 w .. 32 w + 31
        const int seg = (kF8BM * kF8D / 1024 / kF8NW) * w + i;
        const int row = 8 * seg + (lane >> 3), pch = lane & 7;
        lds_dma16_buf(rq, (unsigned)(row * kF8D + ((pch ^ (row & 7)) << 4)), lds_addr(smem + kQBase + seg * 1024));
      }
      serial_fence();
    };

    if (ntk > 0) {
      for (int i = tid; i < kF8NS * kF8Stage / 16; i += kF8NT) reinterpret_cast<u32x4*>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
      lds_barrier();  // the zero fill is done before any direct load lands
      issue_q();
      issue(0);
      wait_vmcnt<0>();
      lds_barrier();  // everyone's Q rows and stage 0 have landed
      const int rr = qw0 - q0 + col;  // this lane's row of the tile (rows past n_q are zero)
#pragma unroll
      for (int ks = 0; ks < kF8KS; ++ks) {
        const char* qr = smem + kQBase + rr * kF8D;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(qr + (((4 * ks + 2 * half) ^ (rr & 7)) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(qr + (((4 * ks + 2 * half + 1) ^ (rr & 7)) << 4));
        qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      lds_barrier();  // every wave holds its Q rows before stages 2 and 3 are refilled
#pragma unroll
      for (int t = 1; t < kF8NS - 1; ++t)
        if (t < ntk) issue(t);
    } else {
#pragma unroll
      for (int ks = 0; ks < kF8KS; ++ks) qf[ks] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }

    // S^T of tile t (K from its slot) and its mask on boundary tiles (selects).
    auto scores = [&](int t, f32x16 (&s)[2]) {
      const char* kt = smem + (t % kF8NS) * kF8Stage;
      // K operand f = (key block f / KS, k-step f % KS); operand f + 1 is read before the
      // product of operand f, so each product waits for one LDS round trip less.
      auto read_k = [&](int f) {
        const int kb = f / kF8KS, ks = f % kF8KS;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(kt + kaddr[ks][0] + 32 * kb * kF8D);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(kt + kaddr[ks][1] + 32 * kb * kF8D);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };
      // (A scheduling fence per step keeps that order; left alone, the scheduler moves each
      // read behind the previous product.)
      i32x8 buf[2];
      buf[0] = read_k(0);
#pragma unroll
      for (int f = 0; f < 2 * kF8KS; ++f) {
        __builtin_amdgcn_sched_barrier(0);
        if (f + 1 < 2 * kF8KS) buf[(f + 1) & 1] = read_k(f + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = f / kF8KS, ks = f % kF8KS;
        s[kb] = mfma_f8(buf[f & 1], qf[ks], ks == 0 ? f32x16{} : s[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto mask = [&](int t, f32x16 (&s)[2]) {
      const int k0 = kbase + t * kF8BN;
      const bool need_mask = (k0 + kF8BN > n_kv) || (a.causal && k0 + kF8BN - 1 > qw0 + delta) ||
                             (a.window > 0 && k0 < qw0 + 32 + delta - a.window);
      if (!need_mask) return;
      // visible: lo <= (key - base) < lim, with base the lane's first key of the tile
      const int base = k0 + 4 * half;
      const int lim = min(n_kv - base, a.causal ? my_q + delta + 1 - base : n_kv - base);
      const int lo = a.window > 0 ? my_q + delta - a.window + 1 - base : -kF8BN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
          s[kb][r] = (off >= lim || off < lo) ? kNegInf : s[kb][r];
        }
    };

    // Software pipeline: iteration t issues the S products of tile t + 1 before the softmax of
    // tile t, so a wave's own matrix-core work runs under its VALU work; then P V of tile t.
    // Tile t + 1's K|V stage must have landed at iteration t, and the slot refilled there (of
    // tile t + 3) was last read at iteration t - 1.
    f32x16 sc[2], sn[2];
    int pk[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // P words (each fully rewritten per tile; no zeroing)
    if (ntk > 0) {
      scores(0, sc);
      mask(0, sc);
    }
    // One tile: its softmax and P V from `cur`, the next tile's scores into `nxt`. The loop
    // runs two tiles per trip with the buffers swapped, so no scores are copied.
    auto tile = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
      const bool more = t + 1 < ntk;   // another tile for the workgroup
      const bool mine = t + 1 < ntw;   // and this wave has keys in it
      if (more) {
        if (t + 2 < ntk) wait_vmcnt<2>();  // stage t + 2 may stay in flight
        else wait_vmcnt<0>();
        lds_barrier();
        if (t + kF8NS - 1 < ntk) issue(t + kF8NS - 1);
        if (mine) scores(t + 1, nxt);
      }
      const char* vt = smem + (t % kF8NS) * kF8Stage + kF8Tile;

      // Integer reference: raised to ceil(tile max) when the tile passes it.
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[kb][r]);
      mx = max_of_halves(mx) * c;
      const float m_new = mx > m ? ceilf(mx) : m;
      // o and l stay in the frame mf instead of being rescaled whenever the reference rises:
      // this tile's x (relative to m_new, so that it fits E4M3) enters P V scaled by
      // 2^(m_new - mf) through the product's scale of P, and l by the same factor; all of it
      // exact powers of two. The frame is the row's first reference, and moves up (o and l
      // rescaled) only when the reference passes it by more than 64, which keeps o and l far
      // from overflow.
      float frame = mf == kNegInf ? m_new : mf;
      if (__builtin_amdgcn_ballot_w64(m_new - frame > 64.f) != 0) {
        const bool up = m_new - frame > 64.f;
        const float f = up ? __builtin_amdgcn_ldexpf(1.f, (int)(frame - m_new)) : 1.f;
        l *= f;
#pragma unroll
        for (int nb = 0; nb < kF8NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[nb][r] *= f;
        frame = up ? m_new : frame;
      }
      mf = frame;
      m = m_new;
      const int kf = m == kNegInf ? 0 : (int)(m - mf);  // 0 .. 64
      const float sk = __builtin_amdgcn_ldexpf(1.f, kf);
      // x = 2^(t - m + 8) <= 256; a row with no reference yet has only masked scores here.
      const float off = m == kNegInf ? 0.f : 8.f - m;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // bytes 4 i .. 4 i + 3 = elements (kb, r) with 16 kb + r = 4 i .. 4 i + 3
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int T = 4 * i + e;
          x[e] = exp2_hw(fmaf(cur[T >> 4][T & 15], c, off));
          l = fmaf(x[e], sk, l);
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], pk[i], false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], word, true);
        pk[i] = word;
      }
      const i32x8 pb = {pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
      // O^T += V^T P^T.
#pragma unroll
      for (int nb = 0; nb < kF8NB; ++nb) {
        const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vt + vaddr[0][nb]));
        const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vt + vaddr[1][nb]));
        const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vt + vaddr[0][nb] + 32 * kF8D));
        const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vt + vaddr[1][nb] + 32 * kF8D));
        const i32x8 va = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
        oacc[nb] = mfma_f8_bscaled(va, pb, oacc[nb], 127 + kf);
      }
      if (mine) mask(t + 1, nxt);
    };
    int t = 0;
    while (t < ntw) {
      tile(t, sc, sn);
      if (++t >= ntw) break;
      tile(t, sn, sc);
      ++t;
    }
    for (; t < ntk; ++t) {  // tiles past this wave's rows: loads and barriers only
      if (t + 1 < ntk) {
        if (t + 2 < ntk) wait_vmcnt<2>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (t + kF8NS - 1 < ntk) issue(t + kF8NS - 1);
      }
    }
    if (ntk > 0) wait_vmcnt<0>();

    // Epilogue: O = descale_v * o / l, LSE = ln(2) (m - 8 + log2 l); rows that saw nothing
    // (and padding rows) get O = 0 and LSE = -inf. O leaves through LDS as whole rows (as in
    // the bf16 prefill): every wave has waited for its loads, so LDS is free once all have
    // returned their last reads.
    lds_barrier();
    unsigned lo_bits, hi_bits;
    wave_halves(__builtin_bit_cast(unsigned, l), lo_bits, hi_bits);
    const float lt = __builtin_bit_cast(float, lo_bits) + __builtin_bit_cast(float, hi_bits);
    const bool row_ok = my_q < n_q && lt > 0.f;
    const float inv = row_ok ? dv / lt : 0.f;
    char* const stage_o = smem + w * 32 * kF8RS;
#pragma unroll
    for (int nb = 0; nb < kF8NB; ++nb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * nb + 8 * jj + 4 * half;
        Store4<__bf16>::store(reinterpret_cast<__bf16*>(stage_o + col * kF8RS) + d0, oacc[nb][4 * jj] * inv,
                              oacc[nb][4 * jj + 1] * inv, oacc[nb][4 * jj + 2] * inv, oacc[nb][4 * jj + 3] * inv);
      }
    __bf16* const ob = a.o + (size_t)(b * a.H + h) * a.Lq * kF8D;
#pragma unroll
    for (int i = 0; i < 32 * (kF8D / 8) / 64; ++i) {
      const int idx = 64 * i + lane, r = idx / (kF8D / 8), c16 = idx - r * (kF8D / 8);
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage_o + r * kF8RS + 16 * c16);
      if (qw0 + r < a.Lq) *reinterpret_cast<u32x4*>(ob + (size_t)(qw0 + r) * kF8D + 8 * c16) = val;
    }
    if (my_q < a.Lq && half == 0)
      a.lse[(size_t)(b * a.H + h) * a.Lq + my_q] = row_ok ? (mf - 8.f + __log2f(lt)) * kLn2 : kNegInf;
    // The next tile clears and refills LDS: every wave's staged-O reads must have returned.
    lds_barrier();
  }
#endif
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream) {
  Fp8Args a;
  a.q = static_cast<const unsigned char*>(p.q);
  a.k = static_cast<const unsigned char*>(p.k);
  a.v = static_cast<const unsigned char*>(p.v);
  a.q_descale = p.q_descale;
  a.k_descale = p.k_descale;
  a.v_descale = p.v_descale;
  a.o = static_cast<__bf16*>(p.o);
  a.lse = p.lse;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.Lq = p.Lq; a.Lk = p.Lk;
  a.group = p.H / p.Hkv;
  a.ntq = (p.Lq + kF8BM - 1) / kF8BM;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.window = p.window;
  a.seqlens = p.seqlens;
  const long long nwg = (long long)a.ntq * p.B * p.H;
  if (nwg > 0x7fffffffLL || (long long)p.Lk * kF8D > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  a.nwg = (int)nwg;
  if (a.nwg == 0) return hipSuccess;
  a.order = make_tile_order(a.nwg, a.group * a.ntq);
  a.group_div = make_divisor(a.group);
  a.hkv_div = make_divisor(p.Hkv);
  // Dense inputs on a persistent grid, variable lengths one workgroup per tile (as for bf16).
  const int P = p.seqlens == nullptr ? persistent_programs(reinterpret_cast<const void*>(&fwd_fp8_kernel), kF8NT) : 0;
  a.nprog = (P > 0 && a.nwg > P) ? P : a.nwg;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_fp8_kernel), dim3((unsigned)a.nprog), dim3(kF8NT), args,
                         0, stream);
}

}  // namespace fa
