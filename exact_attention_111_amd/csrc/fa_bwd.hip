// fa_bwd.hip — attention backward for gfx950 (MI355X).
//
// The method ("FlashAttention 与长上下文：先分清三张账", section "FlashAttention 的关键是
// online softmax"): the backward pass keeps only the forward's per-row statistic (the LSE)
// and recomputes the score tiles it needs instead of storing them, trading compute for HBM
// traffic. The gradients are the derivative of the forward definition: with
// P = softmax(scale Q K^T + M),
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q        (dK, dV summed over a GQA group),
// and P is recomputed as exp2(s * scale*log2(e) - LSE*log2(e)) from the natural-log LSE.
//
// gfx950 mapping (all products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation):
//   * bwd_dot: D per query row (0 on padding rows); d / 8 lanes per row.
//   * bwd_dkdv: one workgroup per (batch, KV head, 128 keys): 4 waves x 32 keys. A wave
//     keeps its keys' K and V rows in registers as B operands. Blocks of 32 query rows of
//     every query head of the group go through LDS, each tile stored twice (swizzled for
//     128-bit row reads and for transposed reads). Per block: S = Q K^T and dP = dO V^T
//     (row reads; the accumulators hold one key column per lane), P and dS from them, then
//     dV^T += dO^T P and dK^T += Q^T dS (transposed reads; P and dS go from the
//     accumulators straight into B operands).
//   * bwd_dq: one workgroup per (batch, head, 128 query rows): 4 waves x 32 rows with their
//     Q and dO rows in registers; 64-key K/V tiles go through LDS. S^T = K Q^T and
//     dP^T = V dO^T leave one query column per lane, then dQ^T += K^T dS^T.
//   Rows and keys outside the sequence are loaded as zeros and masked entries get P = 0 and
//   dP = 0, so dS is exactly 0 there: nothing outside the sequence is read or contributes.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct BwdCfg {
  static constexpr int NW = 4;                // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int ROWB = 2 * D;          // bytes per row
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int QKS = D / 16;          // 32x32x16 k-steps over d
  static constexpr int NB = D / 32;           // 32-row blocks over d
  static constexpr int KEYS = 32 * NW;        // keys per dK/dV workgroup
  static constexpr int QROWS = 32 * NW;       // query rows per dQ workgroup
  static constexpr int QBLK = 32;             // query rows per dK/dV step
  static constexpr int KT = 64;               // keys per dQ step
};

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* ws_d;
  int B, H, Hkv, Lq, Lk;
  int group;
  float scale, scale_log2;
  int causal;
  const int32_t* seqlens;
};

// Valid query rows / keys of batch entry b.
__device__ __forceinline__ void seq_extent(const BwdArgs& a, int b, int& n_q, int& n_kv) {
  n_q = a.Lq;
  n_kv = a.Lk;
  if (a.seqlens != nullptr) {
    const int n = min(max(a.seqlens[b], 0), a.Lk);
    n_q = n;
    n_kv = n;
  }
}

// rows [row0, row0 + NR) of a row-major [*, D] bf16 matrix (zero past n_valid) into an
// LDS tile, chunks of row r permuted by `swz`; one or two destination layouts.
template <int D, int NR>
__device__ __forceinline__ void stage_rows(char* dst_k, char* dst_v, const __bf16* src, int row0, int n_valid,
                                           int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int i = tid; i < NR * C::CH; i += C::NT) {
    const int r = i / C::CH, c = i - r * C::CH;
    u32x4 u = {0u, 0u, 0u, 0u};
    if (row0 + r < n_valid) u = *reinterpret_cast<const u32x4*>(src + (size_t)(row0 + r) * D + 8 * c);
    if (dst_k != nullptr) *reinterpret_cast<u32x4*>(dst_k + r * C::ROWB + ((c ^ k_xor<D>(r)) << 4)) = u;
    if (dst_v != nullptr) *reinterpret_cast<u32x4*>(dst_v + r * C::ROWB + ((c ^ v_xor<D>(r)) << 4)) = u;
  }
}

// Per-lane operand addresses inside a tile. Row reads: lane (col, half) reads row
// 32 * blk + col, logical chunk 2 ks + half (the A operand of a 32x32x16 product over d).
// Transposed reads: lane (g, sl) = (lane / 16, lane % 16) reads rows 16 ks + 4 (g / 2) +
// sl / 4 (+ 8), dims 32 nb + 16 (g % 2) + 4 (sl % 4): output lane l then holds dim
// 32 nb + l % 32 and rows 16 ks + 8 (t / 4) + 4 (l / 32) + t % 4, t = 0..7, the order of
// accumulator elements 8 ks .. 8 ks + 7 used as a B operand.
template <int D>
struct TileAddr {
  int row[BwdCfg<D>::QKS];
  int tr[BwdCfg<D>::NB];
  __device__ __forceinline__ void init(int lane) {
    using C = BwdCfg<D>;
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < C::QKS; ++ks) row[ks] = col * C::ROWB + (((2 * ks + half) ^ k_xor<D>(col)) << 4);
    const int g = lane >> 4, sl = lane & 15;
    const int vrow = 4 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      const int dim = 32 * nb + 16 * (g & 1) + 4 * (sl & 3);
      tr[nb] = vrow * C::ROWB + (((dim >> 3) ^ v_xor<D>(vrow)) << 4) + ((dim & 4) << 1);
    }
  }
  __device__ __forceinline__ bf16x8 read_row(const char* tile, int blk, int ks) const {
    return *reinterpret_cast<const bf16x8*>(tile + row[ks] + blk * 32 * BwdCfg<D>::ROWB);
  }
  __device__ __forceinline__ bf16x8 read_tr(const char* tile, int ks, int nb) const {
    constexpr int RB = BwdCfg<D>::ROWB;
    const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + tr[nb] + 16 * ks * RB));
    const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + tr[nb] + (16 * ks + 8) * RB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// exp2 offset of a query row: LSE * log2(e), or +inf for a row that sees nothing (P = 0).
__device__ __forceinline__ float row_offset(float lse) { return lse == kNegInf ? __builtin_inff() : lse * kLog2e; }

// ---------------------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic for every query row (0 on padding rows).
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const long long rows = (long long)a.B * a.H * a.Lq;
  const int c = threadIdx.x % LPR;
  const long long rr = row < rows ? row : rows - 1;  // every lane computes, so the group reduces fully
  const u32x4 uo = *reinterpret_cast<const u32x4*>(a.o + rr * D + 8 * c);
  const u32x4 ud = *reinterpret_cast<const u32x4*>(a.dout + rr * D + 8 * c);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s = fmaf(bf16_bits_lo(uo[j]), bf16_bits_lo(ud[j]), s);
    s = fmaf(bf16_bits_hi(uo[j]), bf16_bits_hi(ud[j]), s);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
  if (row < rows && c == 0) {
    const int b = (int)(row / ((long long)a.H * a.Lq));
    const int i = (int)(row % a.Lq);
    int n_q, n_kv;
    seq_extent(a, b, n_q, n_kv);
    a.ws_d[row] = i < n_q ? s : 0.f;
  }
}

// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(BwdCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = BwdCfg<D>;
  constexpr int QT = C::QBLK * C::ROWB;  // bytes of one 32-row tile
  __shared__ __attribute__((aligned(1024))) char smem[4 * QT];  // Q rows | Q transposed | dO rows | dO transposed
  __shared__ __attribute__((aligned(16))) float rowv[2][C::QBLK];  // exp2 offset, D
  char* const q_row = smem;
  char* const q_tr = smem + QT;
  char* const d_row = smem + 2 * QT;
  char* const d_tr = smem + 3 * QT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // Key blocks in order of decreasing work under a causal mask (the first keys are seen by
  // the most rows), all (batch, KV head) pairs of one key block together.
  const int nbk = a.B * a.Hkv;
  const int kbi = blockIdx.x / nbk;
  const int bk = blockIdx.x - kbi * nbk;
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  int n_q, n_kv;
  seq_extent(a, b, n_q, n_kv);
  const int delta = a.Lk - a.Lq;
  const int k0 = kbi * C::KEYS;
  const int kw0 = k0 + 32 * w;  // this wave's first key
  const int my_key = kw0 + col;

  const size_t kv_off = (size_t)(b * a.Hkv + kvh) * a.Lk * D;
  bf16x8 kf[C::QKS], vf[C::QKS];
#pragma unroll
  for (int ks = 0; ks < C::QKS; ++ks) {
    u32x4 uk = {0u, 0u, 0u, 0u}, uv = {0u, 0u, 0u, 0u};
    if (my_key < n_kv) {
      uk = *reinterpret_cast<const u32x4*>(a.k + kv_off + (size_t)my_key * D + 16 * ks + 8 * half);
      uv = *reinterpret_cast<const u32x4*>(a.v + kv_off + (size_t)my_key * D + 16 * ks + 8 * half);
    }
    kf[ks] = as_bf16x8(uk);
    vf[ks] = as_bf16x8(uv);
  }
  f32x16 dka[C::NB], dva[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[nb][r] = dva[nb][r] = 0.f;

  TileAddr<D> ta;
  ta.init(lane);
  // The first query row that sees key k0 (bottom-right causal alignment: j <= i + delta).
  const int q_first = (k0 < n_kv) ? (a.causal ? max(0, k0 - delta) : 0) : n_q;
  const int qb_first = q_first / C::QBLK;
  const int nqb = (n_q + C::QBLK - 1) / C::QBLK;

  for (int hq = kvh * a.group; hq < (kvh + 1) * a.group; ++hq) {
    const size_t q_off = (size_t)(b * a.H + hq) * a.Lq;
    for (int qb = qb_first; qb < nqb; ++qb) {
      const int q0 = qb * C::QBLK;
      __syncthreads();  // the previous block's reads are done
      stage_rows<D, C::QBLK>(q_row, q_tr, a.q + q_off * D, q0, n_q, tid);
      stage_rows<D, C::QBLK>(d_row, d_tr, a.dout + q_off * D, q0, n_q, tid);
      if (tid < C::QBLK) {
        const int i = q0 + tid;
        rowv[0][tid] = i < n_q ? row_offset(a.lse[q_off + i]) : __builtin_inff();
        rowv[1][tid] = i < n_q ? a.ws_d[q_off + i] : 0.f;
      }
      __syncthreads();

      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < C::QKS; ++ks) {
        s = mfma_32x32x16(ta.read_row(q_row, 0, ks), kf[ks], s);
        dp = mfma_32x32x16(ta.read_row(d_row, 0, ks), vf[ks], dp);
      }
      // Accumulator element r: query row q0 + 8 (r / 4) + 4 half + r % 4, key my_key.
      const bool need_mask = (q0 + C::QBLK > n_q) || (kw0 + 32 > n_kv) || (a.causal && kw0 + 31 > q0 + delta);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = q0 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = i < n_q && my_key < n_kv && (!a.causal || my_key <= i + delta);
          s[r] = vis ? s[r] : kNegInf;
          dp[r] = vis ? dp[r] : 0.f;
        }
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 off = *reinterpret_cast<const f32x4*>(&rowv[0][8 * m + 4 * half]);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(&rowv[1][8 * m + 4 * half]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * m + t;
          const float p = exp2_hw(fmaf(s[r], a.scale_log2, -off[t]));
          const float ds = p * (dp[r] - dd[t]);
          pb[r >> 3][r & 7] = (__bf16)p;
          dsb[r >> 3][r & 7] = (__bf16)ds;
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          dva[nb] = mfma_32x32x16(ta.read_tr(d_tr, kk, nb), pb[kk], dva[nb]);
          dka[nb] = mfma_32x32x16(ta.read_tr(q_tr, kk, nb), dsb[kk], dka[nb]);
        }
    }
  }

  // dK = scale * dK^T-accumulator, dV: lane holds key my_key, dims 32 nb + 8 (r / 4) +
  // 4 half + r % 4.
  if (my_key < a.Lk) {
    __bf16* dkp = a.dk + kv_off + (size_t)my_key * D;
    __bf16* dvp = a.dv + kv_off + (size_t)my_key * D;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = 32 * nb + 8 * m + 4 * half;
        Store4<__bf16>::store(dkp + d0, dka[nb][4 * m] * a.scale, dka[nb][4 * m + 1] * a.scale,
                              dka[nb][4 * m + 2] * a.scale, dka[nb][4 * m + 3] * a.scale);
        Store4<__bf16>::store(dvp + d0, dva[nb][4 * m], dva[nb][4 * m + 1], dva[nb][4 * m + 2], dva[nb][4 * m + 3]);
      }
  }
#endif
}

// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(BwdCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(const BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = BwdCfg<D>;
  constexpr int KTB = C::KT * C::ROWB;  // bytes of one 64-row tile
  __shared__ __attribute__((aligned(1024))) char smem[3 * KTB];  // K rows | K transposed | V rows
  char* const k_row = smem;
  char* const k_tr = smem + KTB;
  char* const v_row = smem + 2 * KTB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // Query blocks in order of decreasing work under a causal mask (the last rows see the
  // most keys), all (batch, head) pairs of one block together.
  const int nbh = a.B * a.H;
  const int ntq = (a.Lq + C::QROWS - 1) / C::QROWS;
  const int qt = ntq - 1 - (int)(blockIdx.x / nbh);
  const int bh = blockIdx.x % nbh;
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / a.group;
  int n_q, n_kv;
  seq_extent(a, b, n_q, n_kv);
  const int delta = a.Lk - a.Lq;
  const int q0 = qt * C::QROWS;
  const int qw0 = q0 + 32 * w;
  const int my_q = qw0 + col;
  const size_t q_off = (size_t)(b * a.H + h) * a.Lq;
  const size_t kv_off = (size_t)(b * a.Hkv + kvh) * a.Lk * D;

  bf16x8 qf[C::QKS], dof[C::QKS];
#pragma unroll
  for (int ks = 0; ks < C::QKS; ++ks) {
    u32x4 uq = {0u, 0u, 0u, 0u}, ud = {0u, 0u, 0u, 0u};
    if (my_q < n_q) {
      uq = *reinterpret_cast<const u32x4*>(a.q + (q_off + my_q) * D + 16 * ks + 8 * half);
      ud = *reinterpret_cast<const u32x4*>(a.dout + (q_off + my_q) * D + 16 * ks + 8 * half);
    }
    qf[ks] = as_bf16x8(uq);
    dof[ks] = as_bf16x8(ud);
  }
  const float off = my_q < n_q ? row_offset(a.lse[q_off + my_q]) : __builtin_inff();
  const float dd = my_q < n_q ? a.ws_d[q_off + my_q] : 0.f;
  f32x16 dqa[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[nb][r] = 0.f;

  TileAddr<D> ta;
  ta.init(lane);
  // Keys any row of this block can see: [0, kv_end).
  int kv_end = 0;
  if (q0 < n_q) {
    kv_end = n_kv;
    if (a.causal) kv_end = min(kv_end, min(q0 + C::QROWS, n_q) + delta);
    kv_end = max(kv_end, 0);
  }
  const int ntk = (kv_end + C::KT - 1) / C::KT;
  for (int t = 0; t < ntk; ++t) {
    const int k0 = t * C::KT;
    __syncthreads();  // the previous tile's reads are done
    stage_rows<D, C::KT>(k_row, k_tr, a.k + kv_off, k0, kv_end, tid);
    stage_rows<D, C::KT>(v_row, nullptr, a.v + kv_off, k0, kv_end, tid);
    __syncthreads();

    // S^T and dP^T for the two 32-key halves: element r of half kb is key
    // k0 + 32 kb + 8 (r / 4) + 4 half + r % 4, query my_q.
    f32x16 sx[2], dpx[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sx[kb] = f32x16{};
      dpx[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::QKS; ++ks) {
        sx[kb] = mfma_32x32x16(ta.read_row(k_row, kb, ks), qf[ks], sx[kb]);
        dpx[kb] = mfma_32x32x16(ta.read_row(v_row, kb, ks), dof[ks], dpx[kb]);
      }
    }
    const bool need_mask = (k0 + C::KT > n_kv) || (qw0 + 32 > n_q) || (a.causal && k0 + C::KT - 1 > qw0 + delta);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = my_q < n_q && j < n_kv && (!a.causal || j <= my_q + delta);
          sx[kb][r] = vis ? sx[kb][r] : kNegInf;
          dpx[kb][r] = vis ? dpx[kb][r] : 0.f;
        }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(fmaf(sx[kb][r], a.scale_log2, -off));
        dsb[2 * kb + (r >> 3)][r & 7] = (__bf16)(p * (dpx[kb][r] - dd));
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) dqa[nb] = mfma_32x32x16(ta.read_tr(k_tr, ks, nb), dsb[ks], dqa[nb]);
  }

  // dQ = scale * accumulator: lane holds query my_q, dims 32 nb + 8 jj + 4 half + (0..3).
  if (my_q < a.Lq) {
    __bf16* dqp = a.dq + (q_off + my_q) * D;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * nb + 8 * jj + 4 * half;
        Store4<__bf16>::store(dqp + d0, dqa[nb][4 * jj] * a.scale, dqa[nb][4 * jj + 1] * a.scale,
                              dqa[nb][4 * jj + 2] * a.scale, dqa[nb][4 * jj + 3] * a.scale);
      }
  }
#endif
}

template <int D>
hipError_t launch_b(const BwdParams& p, hipStream_t stream) {
  using C = BwdCfg<D>;
  BwdArgs a;
  a.q = static_cast<const __bf16*>(p.q);
  a.k = static_cast<const __bf16*>(p.k);
  a.v = static_cast<const __bf16*>(p.v);
  a.o = static_cast<const __bf16*>(p.o);
  a.dout = static_cast<const __bf16*>(p.dout);
  a.lse = p.lse;
  a.dq = static_cast<__bf16*>(p.dq);
  a.dk = static_cast<__bf16*>(p.dk);
  a.dv = static_cast<__bf16*>(p.dv);
  a.ws_d = p.ws_d;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.Lq = p.Lq; a.Lk = p.Lk;
  a.group = p.H / p.Hkv;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.seqlens = p.seqlens;
  void* args[] = {&a};
  const long long rows = (long long)p.B * p.H * p.Lq;
  const long long ndot = (rows + (256 / (D / 8)) - 1) / (256 / (D / 8));
  const long long nkv = (long long)p.B * p.Hkv * ((p.Lk + C::KEYS - 1) / C::KEYS);
  const long long nq = (long long)p.B * p.H * ((p.Lq + C::QROWS - 1) / C::QROWS);
  if (ndot > 0x7fffffffLL || nkv > 0x7fffffffLL || nq > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipError_t e = hipSuccess;
  if (ndot > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dot_kernel<D>), dim3((unsigned)ndot), dim3(256), args, 0,
                        stream);
    if (e != hipSuccess) return e;
  }
  if (nkv > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D>), dim3((unsigned)nkv), dim3(C::NT), args,
                        0, stream);
    if (e != hipSuccess) return e;
  }
  if (nq > 0)
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<D>), dim3((unsigned)nq), dim3(C::NT), args, 0,
                        stream);
  return e;
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.d == 64) return launch_b<64>(p, stream);
  return launch_b<128>(p, stream);
}

}  // namespace fa
