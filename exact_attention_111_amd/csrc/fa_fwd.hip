// fa_fwd.hip — prefill attention forward for gfx950 (MI355X).
//
// The method ("FlashAttention 与长上下文：先分清三张账", section "FlashAttention 的关键是
// online softmax"; "2.1 FlashAttention-2 的核心思想" §2.1.2–§2.1.3): the queries are cut
// into row tiles and the keys/values into column tiles; each tile pair is scored on chip
// and thrown away, while every query row carries a running maximum m, a running sum l of
// exponentials relative to m, and an unnormalised output o. When a new key tile raises
// the maximum, l and o are multiplied by exp(m_old - m_new) first. At the end O = o / l
// and the row's log-sum-exp is written. The score and probability tiles never leave the
// compute unit.
//
// gfx950 mapping (one workgroup = 4 wave64s = one 128-row query tile of one head):
//   * Each wave owns 32 query rows. Its Q rows stay in VGPRs for the whole kernel as the
//     B operand of v_mfma_f32_32x32x16_bf16.
//   * Key/value tiles of 64 rows are staged HBM -> VGPR (prefetched one tile ahead, so the
//     loads of tile j+1 are in flight while tile j is computed) -> LDS. K is kept row
//     major (rows padded by 16 bytes so a 128-bit read by 8 lanes hits 8 distinct bank
//     groups); V is written transposed with a XOR swizzle so the PV operand is one
//     128-bit LDS read per lane.
//   * The wave computes S^T = K Q^T (keys down, queries across). In the 32x32 MFMA
//     accumulator layout a lane then holds one query column: all per-row softmax state
//     (m, l, the rescale factor) lives in that lane and needs one cross-lane exchange
//     (lane ^ 32) per tile for the maximum and one at the end for the sum.
//   * O^T = V^T P^T uses the probabilities straight from the accumulator registers as the
//     B operand (converted to bf16); the contraction index is permuted to match the
//     accumulator layout, and V^T in LDS is stored in that permuted key order.
//   * Exponentials are 2^x on v_exp_f32 with scale*log2(e) folded into one FMA.
//   * Causal and padding masks are applied element-wise only on tiles that straddle the
//     diagonal or the sequence end; tiles no row of a wave can see are skipped, and key
//     tiles beyond the last visible key of the query tile are never loaded.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;                 // query rows per workgroup
  static constexpr int BN = 64;                  // keys per tile
  static constexpr int NT = 256;                 // threads (4 waves)
  static constexpr int NCH = D / 8;              // 16-byte chunks per K/V row
  static constexpr int RPP = NT / NCH;           // key rows loaded per pass
  static constexpr int PASSES = BN / RPP;        // passes per tile
  static constexpr int KSTR = D + 8;             // LDS K row stride in bf16 (16-byte pad)
  static constexpr int QKS = D / 16;             // 32x32x16 k-steps over d
  static constexpr int NB = D / 32;              // 32-row blocks of O^T
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Lq, Lk;
  int group;        // H / Hkv
  int ntq;          // query tiles per head
  float scale_log2; // scale * log2(e)
  int causal;
  const int32_t* seqlens;
};

// Position of key u (within a 64-key tile) in a transposed V row: swap bits 2 and 3, so
// that the 8 keys one lane needs for a PV k-step are 8 consecutive bf16 (16 bytes).
__device__ __forceinline__ int vt_pos(int u) { return (u & ~0xC) | ((u & 4) << 1) | ((u & 8) >> 1); }

// Element index of (d, position p) in the transposed V tile [D][64] with a XOR swizzle of
// the 16-byte chunk index by the row, which spreads both the transposing writes and the
// MFMA-operand reads over the LDS banks.
__device__ __forceinline__ int vt_index(int d, int p) {
  const int swz = (d ^ (d >> 3)) & 7;
  return d * 64 + ((((p >> 3) ^ swz) << 3) | (p & 7));
}

template <int D, typename IT, typename OT>
__global__ __launch_bounds__(256) void fwd_kernel(const FwdArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[C::BN * C::KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[D * C::BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane & 31;   // this lane's query row within the wave
  const int half = lane >> 5;  // which 8-element half of a 16-wide k-step

  // Heaviest query tiles (the last ones under a causal mask) are dispatched first.
  const int BH = a.B * a.H;
  const int wg = blockIdx.x;
  const int qt = a.ntq - 1 - wg / BH;
  const int bh = wg - (wg / BH) * BH;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int kvh = h / a.group;

  int n_kv = a.Lk, n_q = a.Lq;
  if (a.seqlens != nullptr) {
    const int n = min(max(a.seqlens[b], 0), a.Lk);
    n_kv = n;
    n_q = n;
  }
  const int delta = a.Lk - a.Lq;  // bottom-right causal alignment
  const int q0 = qt * C::BM;
  const int qw0 = q0 + 32 * w;
  const int my_q = qw0 + col;

  // Keys this query tile can see: [0, kv_end).
  int kv_end = 0;
  if (q0 < n_q) {
    kv_end = n_kv;
    if (a.causal) kv_end = min(kv_end, min(q0 + C::BM, n_q) - 1 + delta + 1);
    kv_end = max(kv_end, 0);
  }
  const int ntk = (kv_end + C::BN - 1) / C::BN;

  const IT* __restrict__ qp = static_cast<const IT*>(a.q) + (size_t)(b * a.H + h) * a.Lq * D;
  const IT* __restrict__ kp = static_cast<const IT*>(a.k) + (size_t)(b * a.Hkv + kvh) * a.Lk * D;
  const IT* __restrict__ vp = static_cast<const IT*>(a.v) + (size_t)(b * a.Hkv + kvh) * a.Lk * D;

  // Q rows of this lane as MFMA B operands: element t of k-step ks is d = 16*ks + 8*half + t.
  bf16x8 qf[C::QKS];
#pragma unroll
  for (int ks = 0; ks < C::QKS; ++ks) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (my_q < n_q && ntk > 0) u = Load8<IT>::load(qp + (size_t)my_q * D + 16 * ks + 8 * half);
    qf[ks] = as_bf16x8(u);
  }

  f32x16 oacc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.f;
  float m = kNegInf;  // running max of scale*log2(e)*s for this lane's row
  float l = 0.f;      // this lane's part of the running sum (the other part is in lane ^ 32)

  // Tile staging: thread tid loads 16 bytes of key row (pass*RPP + ld_row), chunk ld_ch.
  const int ld_row = tid / C::NCH;
  const int ld_ch = tid - ld_row * C::NCH;
  u32x4 kreg[C::PASSES], vreg[C::PASSES];

  auto load_tile = [&](int t) {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int key = t * C::BN + p * C::RPP + ld_row;
      u32x4 ku = {0u, 0u, 0u, 0u}, vu = {0u, 0u, 0u, 0u};
      if (key < kv_end) {  // zero-fill past the last visible key: never read padding
        ku = Load8<IT>::load(kp + (size_t)key * D + ld_ch * 8);
        vu = Load8<IT>::load(vp + (size_t)key * D + ld_ch * 8);
      }
      kreg[p] = ku;
      vreg[p] = vu;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int r = p * C::RPP + ld_row;
      *reinterpret_cast<u32x4*>(&Ks[r * C::KSTR + ld_ch * 8]) = kreg[p];
      const int pos = vt_pos(r);
      uint16_t* vt16 = reinterpret_cast<uint16_t*>(Vt);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t word = vreg[p][e >> 1];
        vt16[vt_index(ld_ch * 8 + e, pos)] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
      }
    }
  };

  if (ntk > 0) load_tile(0);
  for (int t = 0; t < ntk; ++t) {
    if (t > 0) __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < ntk) load_tile(t + 1);  // next tile's HBM loads overlap this tile's math

    const int k0 = t * C::BN;
    // Skip the tile when no row of this wave sees any of its keys.
    if (qw0 >= n_q) continue;
    if (a.causal && k0 > qw0 + 31 + delta) continue;
    const bool need_mask = (k0 + C::BN > n_kv) || (a.causal && k0 + C::BN - 1 > qw0 + delta);

    // S^T = K Q^T for the two 32-key halves of the tile.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::QKS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + col) * C::KSTR + 16 * ks + 8 * half]);
        s[kb] = mfma_32x32x16(kf, qf[ks], s[kb]);
      }
    }
    // Accumulator element r of half kb is key k0 + 32*kb + 8*(r/4) + 4*half + r%4, query my_q.
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = key < n_kv && (!a.causal || key <= my_q + delta);
          if (!vis) s[kb][r] = kNegInf;
        }
    }

    // Online softmax update (base 2): m' = max(m, max S_j); alpha = 2^(m - m').
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx * a.scale_log2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // no -inf - -inf
    const float alpha = exp2_hw(m - m_use);
    const float neg_m = -m_use;

    bf16x8 pb[4];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2_hw(fmaf(s[kb][8 * hh + e], a.scale_log2, neg_m));
          rs += p;
          pb[2 * kb + hh][e] = (__bf16)p;
        }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nb][r] *= alpha;

    // O^T += V^T P^T. k-step ks covers accumulator registers 8*(ks%2) .. +7 of half ks/2,
    // i.e. keys 16*ks + 8*(e/4) + 4*half + e%4; V^T stores exactly that order.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&Vt[vt_index(32 * nb + col, 16 * ks + 8 * half)]);
        oacc[nb] = mfma_32x32x16(vf, pb[ks], oacc[nb]);
      }
  }

  // Epilogue: O = o / l and LSE = ln(2) * (m + log2 l); padding rows and rows that saw
  // no key get O = 0 and LSE = -inf.
  const float lt = l + __shfl_xor(l, 32);
  const bool row_ok = (my_q < n_q) && (lt > 0.f);
  const float inv = row_ok ? 1.f / lt : 0.f;
  if (my_q < a.Lq) {
    OT* op = static_cast<OT*>(a.o) + ((size_t)(b * a.H + h) * a.Lq + my_q) * D;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * nb + 8 * j + 4 * half;
        float x0 = oacc[nb][4 * j + 0] * inv, x1 = oacc[nb][4 * j + 1] * inv;
        float x2 = oacc[nb][4 * j + 2] * inv, x3 = oacc[nb][4 * j + 3] * inv;
        if (!row_ok) x0 = x1 = x2 = x3 = 0.f;
        Store4<OT>::store(op + d0, x0, x1, x2, x3);
      }
    if (half == 0)
      a.lse[(size_t)(b * a.H + h) * a.Lq + my_q] = row_ok ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

template <int D, typename IT, typename OT>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  using C = FwdCfg<D>;
  FwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.Lq = p.Lq; a.Lk = p.Lk;
  a.group = p.H / p.Hkv;
  a.ntq = (p.Lq + C::BM - 1) / C::BM;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.seqlens = p.seqlens;
  const long long nwg = (long long)a.ntq * p.B * p.H;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_kernel<D, IT, OT>), dim3((unsigned)nwg), dim3(C::NT),
                         args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return launch<64, __bf16, __bf16>(p, stream);
  return launch<128, __bf16, __bf16>(p, stream);
}

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return launch<64, float, float>(p, stream);
  return launch<128, float, float>(p, stream);
}

}  // namespace fa
