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
//   * bwd_dot: per query row, the exp2 offset LSE*log2(e) and D, as one (offset, D) pair
//     (+inf and 0 on padding rows); d / 8 lanes per row.
//   * bwd_dkdv: one workgroup per (batch, KV head, 128 keys): 4 waves x 32 keys, whose K
//     and V rows stay in registers as B operands; two workgroups per CU (two waves per SIMD).
//     Steps of 32 query rows of every query head of the group stream through a 4-stage ring
//     of LDS stages (Q tile, dO tile, the rows' pairs), filled by direct buffer-to-LDS loads
//     issued three steps ahead. Per step: S = Q K^T and dP = dO V^T (row reads; the
//     accumulators hold one key column per lane), P and dS, then dV^T += dO^T P and
//     dK^T += Q^T dS (transposed reads; P and dS go from the accumulators straight into B
//     operands). Operands are read one (rows) and two (transposed) products ahead.
//   * bwd_dq: one workgroup per (batch, head, 128 query rows): 4 waves x 32 rows, with their
//     Q and dO rows in registers. 32-key K/V tiles stream through a 4-stage ring loaded
//     three steps ahead. S^T = K Q^T and dP^T = V dO^T leave one query column per lane, then
//     dQ^T += K^T dS^T. Operands are read four (rows) and three (transposed) products ahead.
//   Each tile sits in LDS once, in a layout (kv_xor) that serves both its row and its
//   transposed reads without bank conflicts. Rows past the sequence are not read: their LDS
//   rows keep earlier input rows or the zeros the kernels start from, and the mask gives
//   them P = 0 and dP = 0, so dS is exactly 0 there and nothing outside a sequence counts.
//   Every wave computes every step of its workgroup, masked or not: the step's barrier holds
//   a wave that skipped anyway, and a skip branch makes the compiler copy the loop-carried
//   accumulators between register files on every step.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct BwdCfg {
  static constexpr int NW = 4;        // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int WAVES_PER_SIMD = 2;  // two waves share a SIMD (256 registers each)
  static constexpr int ROWB = 2 * D;  // bytes per row
  static constexpr int QKS = D / 16;  // 32x32x16 k-steps over d
  static constexpr int NB = D / 32;   // 32-wide blocks over d
  // dK/dV: 32 keys per wave, RB blocks of 32 query rows per step.
  static constexpr int KEYS = 32 * NW;
  static constexpr int RB = 1;
  static constexpr int QSTEP = 32 * RB;
  static constexpr int QTILE = QSTEP * ROWB;              // bytes of a Q or dO tile
  static constexpr int KV_STAGE = 2 * QTILE + QSTEP * 8;  // Q | dO | (offset, D) per row
  static constexpr int KV_NS = 4;                         // stages in the ring
  static constexpr int KV_SEGS = QTILE / 1024 / NW;       // 1 KB direct loads per wave and tile
  static constexpr int RV_LANES = QSTEP / NW / 2;         // lanes loading two rows' pairs each
  static constexpr int KV_LOADS = 2 * KV_SEGS + 1;        // direct loads per wave and stage
  // dQ: QB blocks of 32 query rows per wave, 32 keys per step.
  static constexpr int QB = 1;
  static constexpr int WROWS = 32 * QB;
  static constexpr int QROWS = WROWS * NW;
  static constexpr int KSTEP = 32;
  static constexpr int KTILE = KSTEP * ROWB;  // bytes of a K or V tile
  static constexpr int Q_STAGE = 2 * KTILE;   // K | V
  static constexpr int Q_NS = 4;
  static constexpr int Q_SEGS = KTILE / 1024 / NW;
  static constexpr int Q_LOADS = 2 * Q_SEGS;
  static_assert(KV_SEGS >= 1 && Q_SEGS >= 1, "tile smaller than one load per wave");
  static_assert(RV_LANES >= 1 && RV_LANES * 2 * NW == QSTEP, "pair loads cover the step's rows");
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
  float* ws;  // [B, H, Lq] x (offset, D)
  int B, H, Hkv, Lq, Lk;
  int group;
  float scale, scale_log2;
  int causal;
  int window;  // sliding window W (0: none): key j needs j > i + Lk - Lq - W
  const int32_t* seqlens;
  TileOrder order;             // tile_order of the launch (used with GQA)
  Divisor group_div, hkv_div;  // H / Hkv and Hkv as divisors
};

// Valid query rows / keys of batch entry b.
__device__ __forceinline__ void seq_extent(const BwdArgs& a, int b, int& n_q, int& n_kv) {
  n_q = a.Lq;
  n_kv = a.Lk;
  if (a.seqlens != nullptr) {
    const int n = min(max(load_const(a.seqlens + b), 0), a.Lk);
    n_q = n;
    n_kv = n;
  }
}

// Zero a workgroup's LDS buffer (so rows that are never loaded hold finite values).
template <int BYTES, int NT>
__device__ __forceinline__ void zero_lds(char* smem, int tid) {
  static_assert(BYTES % 16 == 0, "16-byte stores");
#pragma unroll 4
  for (int i = tid; i < BYTES / 16; i += NT) reinterpret_cast<u32x4*>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
}

// Byte offsets, relative to a tile's first row, that direct-load segment i of wave w reads
// so that LDS byte (w * SEGS + i) * 1024 + 16 * lane receives row r's logical chunk
// (physical chunk ^ kv_xor(r)).
template <int D, int SEGS>
__device__ __forceinline__ void tile_load_offsets(unsigned (&off)[SEGS], int w, int lane) {
  constexpr int ROWB = 2 * D;
#pragma unroll
  for (int i = 0; i < SEGS; ++i) {
    const int byte = (w * SEGS + i) * 1024 + lane * 16;
    const int r = byte / ROWB;
    const int cp = (byte - r * ROWB) >> 4;
    off[i] = (unsigned)(r * ROWB + ((cp ^ kv_xor<D>(r)) << 4));
  }
}

// Per-lane operand addresses inside a kv_xor tile. Row reads: lane (col, half) reads row
// 32 blk + col, logical chunk 2 ks + half (the A operand of a 32x32x16 product over d).
// Transposed reads: lane (g, sl) = (lane / 16, lane % 16) reads rows 16 ks + 4 (g / 2) +
// sl / 4 (+ 8), dims 32 nb + 16 (g % 2) + 4 (sl % 4): output lane l then holds dim
// 32 nb + l % 32 and rows 16 ks + 8 (t / 4) + 4 (l / 32) + t % 4, t = 0..7, the order of
// accumulator elements 8 ks .. 8 ks + 7 used as a B operand.
template <int D>
struct TileAddr {
  int row[BwdCfg<D>::QKS];
  int tr[BwdCfg<D>::NB];  // rows 16 ks + 4 (g / 2) + sl / 4
  int tr_hi;              // + this for the same dims 8 rows further on
  __device__ __forceinline__ void init(int lane) {
    using C = BwdCfg<D>;
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < C::QKS; ++ks) row[ks] = col * C::ROWB + (((2 * ks + half) ^ kv_xor<D>(col)) << 4);
    const int g = lane >> 4, sl = lane & 15;
    const int vrow = 4 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      const int dim = 32 * nb + 16 * (g & 1) + 4 * (sl & 3);
      tr[nb] = vrow * C::ROWB + (((dim >> 3) ^ kv_xor<D>(vrow)) << 4) + ((dim & 4) << 1);
    }
    // kv_xor(vrow + 8) = kv_xor(vrow) ^ 2 (vrow < 8), so the chunk moves by +-2 the same
    // way for every nb: its bit 1 is (g & 1) ^ bit 1 of kv_xor(vrow).
    const int bit1 = ((g & 1) ^ (kv_xor<D>(vrow) >> 1)) & 1;
    tr_hi = 8 * C::ROWB + (bit1 ? -32 : 32);
  }
  __device__ __forceinline__ bf16x8 read_row(const char* tile, int blk, int ks) const {
    return *reinterpret_cast<const bf16x8*>(tile + row[ks] + blk * 32 * BwdCfg<D>::ROWB);
  }
  // `hi`: tr_hi passed through the loop so that the sums are formed per step instead of
  // being held in registers across it.
  __device__ __forceinline__ bf16x8 read_tr(const char* tile, int ks, int nb, int hi) const {
    constexpr int RB = BwdCfg<D>::ROWB;
    const char* p = tile + tr[nb] + 16 * ks * RB;
    const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + hi));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// A wave's 32 x D result block, held in the accumulator layout (lane (col, half): row col,
// dims 32 nb + 8 m + 4 half + (0..3) in acc[nb][4 m .. 4 m + 3]), times `mul`, stored as
// whole rows: it goes through this wave's LDS region `stage` (32 rows of 2 D + 16 bytes, the
// pad spreading the rows over the banks) and out 16 contiguous bytes per lane, rows below
// `nrows` only. Stored straight from the accumulators, each store instruction would write 8
// bytes into each of 32 rows. LDS must be free; the same region may be used again at once.
template <int D>
__device__ __forceinline__ void store_block_rows(char* stage, const f32x16 (&acc)[D / 32], float mul, __bf16* out,
                                                 int nrows, int lane) {
  constexpr int RS = 2 * D + 16, CPR = D / 8;
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      Store4<__bf16>::store(reinterpret_cast<__bf16*>(stage + col * RS) + 32 * nb + 8 * m + 4 * half,
                            acc[nb][4 * m] * mul, acc[nb][4 * m + 1] * mul, acc[nb][4 * m + 2] * mul,
                            acc[nb][4 * m + 3] * mul);
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int idx = 64 * i + lane, r = idx / CPR, c = idx - r * CPR;
    const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * RS + 16 * c);
    if (r < nrows) *reinterpret_cast<u32x4*>(out + (size_t)r * D + 8 * c) = val;
  }
}

// ---------------------------------------------------------------------------------------
// Per query row: exp2 offset LSE * log2(e) (+inf for a row that sees nothing, so P = 0)
// and D = sum_c dO_ic O_ic; (+inf, 0) on padding rows.
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
    float2 out = make_float2(__builtin_inff(), 0.f);
    if (i < n_q) {
      const float lse = a.lse[row];
      out = make_float2(lse == kNegInf ? __builtin_inff() : lse * kLog2e, s);
    }
    reinterpret_cast<float2*>(a.ws)[row] = out;
  }
}

// ---------------------------------------------------------------------------------------
// XCD_ORDER: workgroups in the prefill's XCD order (used with GQA, see below).
template <int D, bool XCD_ORDER>
__global__ __launch_bounds__(BwdCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(BwdCfg<D>::WAVES_PER_SIMD, BwdCfg<D>::WAVES_PER_SIMD)))
void bwd_dkdv_kernel(const BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::KV_NS * C::KV_STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // Key blocks in order of decreasing work under a causal mask (the first keys are seen by
  // the most rows). Without GQA: all (batch, KV head) pairs of one key block together. With
  // GQA (XCD_ORDER) a workgroup streams the Q and dO rows of every query head of its group,
  // so the order of the prefill is used instead (tile_order): pairs dealt to the XCDs,
  // each XCD working through its pairs a few at a time, so that the key blocks it runs at
  // once share those rows in its L2.
  const int nbk = a.B * a.Hkv;
  int kbi, bk;
  if constexpr (XCD_ORDER) {
    int qt;
    tile_order(a.order, blockIdx.x, bk, qt);  // a.order.ntq key blocks per pair
    kbi = a.order.ntq - 1 - qt;
  } else {
    kbi = blockIdx.x / nbk;
    bk = blockIdx.x - kbi * nbk;
  }
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  int n_q, n_kv;
  seq_extent(a, b, n_q, n_kv);
  const int delta = a.Lk - a.Lq;
  const int k0 = kbi * C::KEYS;
  const int kw0 = k0 + 32 * w;  // this wave's first key
  const int my_key = kw0 + col;

  zero_lds<C::KV_NS * C::KV_STAGE, C::NT>(smem, tid);

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
  unsigned toff[C::KV_SEGS];
  tile_load_offsets<D, C::KV_SEGS>(toff, w, lane);

  // Steps: (query head of the group, 64-row block) pairs, head-major. The first row that
  // sees key k0 is k0 - delta (bottom-right causal alignment: j <= i + delta).
  // With a sliding window the last row that sees key k0 + KEYS - 1 is k0 + KEYS - 2 - delta + W.
  const int q_first = (k0 < n_kv) ? (a.causal ? max(0, k0 - delta) : 0) : n_q;
  const int q_end = a.window > 0 ? min(n_q, k0 + C::KEYS - 1 - delta + a.window) : n_q;  // exclusive
  const int qs_first = q_first / C::QSTEP;
  const int nqs = max((q_end + C::QSTEP - 1) / C::QSTEP, qs_first);  // end of the step range
  const int per_head = nqs - qs_first;
  const int T = a.group * per_head;

  // Stage the next step (ihq, iqs) into ring slot `slot`: the Q and dO tiles through
  // buffer resources that end at row n_q (rows past it read nothing), and the rows'
  // (offset, D) pairs, QSTEP / NW rows per wave from its first RV_LANES lanes.
  const char* const qsrc = reinterpret_cast<const char*>(a.q);
  const char* const dsrc = reinterpret_cast<const char*>(a.dout);
  const char* const wsrc = reinterpret_cast<const char*>(a.ws);
  int ihq = kvh * a.group, iqs = qs_first;
  auto issue = [&](int slot) {
    const int q0 = iqs * C::QSTEP;
    const size_t row0 = (size_t)(b * a.H + ihq) * a.Lq + q0;
    const unsigned nrows = (unsigned)max(n_q - q0, 0);
    char* st = smem + slot * C::KV_STAGE;
    const u32x4 rq = raw_buffer_rsrc(qsrc + row0 * C::ROWB, nrows * C::ROWB);
    const u32x4 rd = raw_buffer_rsrc(dsrc + row0 * C::ROWB, nrows * C::ROWB);
    serial_fence();
#pragma unroll
    for (int i = 0; i < C::KV_SEGS; ++i) lds_dma16_buf(rq, toff[i], lds_addr(st + (w * C::KV_SEGS + i) * 1024));
#pragma unroll
    for (int i = 0; i < C::KV_SEGS; ++i)
      lds_dma16_buf(rd, toff[i], lds_addr(st + C::QTILE + (w * C::KV_SEGS + i) * 1024));
    const u32x4 rr = raw_buffer_rsrc(wsrc + row0 * 8, nrows * 8);
    if (lane < C::RV_LANES)
      lds_dma16_buf(rr, (unsigned)(16 * (C::RV_LANES * w + lane)), lds_addr(st + 2 * C::QTILE + 16 * C::RV_LANES * w));
    serial_fence();
    if (++iqs == nqs) {
      iqs = qs_first;
      ++ihq;
    }
  };

  __syncthreads();  // the zero fill is done before any direct load lands
#pragma unroll
  for (int t = 0; t < C::KV_NS - 1; ++t)
    if (t < T) issue(t);
  // Wait for every load once here, on every path into the step loop. The K and V rows were
  // loaded into registers above; the compiler does not see the ring's direct loads, so unless
  // it sees a complete wait after those register loads it waits for all loads before their
  // first use in every step, the ring stages just issued for later steps included.
  wait_vmcnt<0>();

  int qs = qs_first;  // block of the step being computed
  for (int t = 0; t < T; ++t) {
    // Step t's loads are done when at most the later staged steps' loads are outstanding.
    if (t + C::KV_NS - 1 <= T) wait_vmcnt<(C::KV_NS - 2) * C::KV_LOADS>();
    else wait_vmcnt<0>();
    lds_barrier();  // every wave's loads of step t landed; step t - 1's reads are done
    if (t + C::KV_NS - 1 < T) issue((t + C::KV_NS - 1) % C::KV_NS);

    const int q0 = qs * C::QSTEP;
    if (++qs == nqs) qs = qs_first;
    int hi = ta.tr_hi;
    asm volatile("" : "+v"(hi));  // a per-step value: tile + tr + hi is not hoisted out of the loop
    const char* qt = smem + (t % C::KV_NS) * C::KV_STAGE;
    const char* dt = qt + C::QTILE;
    const float* rv = reinterpret_cast<const float*>(qt + 2 * C::QTILE);

    // S and dP of the step (one row block): operand f is the Q (f even) or dO (f odd) row chunk
    // of k-step f / 2, read one product ahead; the operands of the dV and dK products below are
    // read two products ahead. Scheduling fences keep each read ahead of the product it
    // precedes (left alone, the scheduler puts every read right before its product, which then
    // waits for a whole LDS round trip). Deeper read-ahead of the row chunks does not fit the
    // 256 registers at d = 128.
    static_assert(C::RB == 1, "one row block of queries per step");
    constexpr int kRowPF = 1, kTrPF = 2;
    f32x16 s[C::RB], dp[C::RB];
    {
      constexpr int NF = 2 * C::QKS;
      auto read_rowop = [&](int f) { return (f & 1) ? ta.read_row(dt, 0, f >> 1) : ta.read_row(qt, 0, f >> 1); };
      bf16x8 rbuf[kRowPF];
#pragma unroll
      for (int f = 0; f < kRowPF; ++f) rbuf[f] = read_rowop(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 x = rbuf[f % kRowPF];
        if (f + kRowPF < NF) rbuf[f % kRowPF] = read_rowop(f + kRowPF);
        __builtin_amdgcn_sched_barrier(0);
        const int ks = f >> 1;
        if (f & 1) dp[0] = mfma_32x32x16(x, vf[ks], ks == 0 ? f32x16{} : dp[0]);
        else s[0] = mfma_32x32x16(x, kf[ks], ks == 0 ? f32x16{} : s[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Element r of block rb: query row q0 + 32 rb + 8 (r / 4) + 4 half + r % 4, key my_key.
    const bool need_mask = (q0 + C::QSTEP > n_q) || (kw0 + 32 > n_kv) || (a.causal && kw0 + 31 > q0 + delta) ||
                           (a.window > 0 && kw0 <= q0 + C::QSTEP - 1 + delta - a.window);
    if (need_mask) {
      // The rows my_key is visible to, as bounds on the element's row offset from
      // q0 + 4 half: row i sees the key when i < n_q, i >= my_key - delta (causal) and
      // i < my_key - delta + W (window), and the key exists (my_key < n_kv). Compares and
      // selects only: the same test written with && and || compiled to a branch per element.
      const bool key_ok = my_key < n_kv;
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = q0 + 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = key_ok & (i < n_q) & (!a.causal | (my_key <= i + delta)) &
                           ((a.window <= 0) | (my_key > i + delta - a.window));
          s[rb][r] = vis ? s[rb][r] : kNegInf;
          dp[rb][r] = vis ? dp[rb][r] : 0.f;
        }
    }
    bf16x8 pb[2 * C::RB], dsb[2 * C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float* pr = rv + 2 * (32 * rb + 8 * m + 4 * half);  // (offset, D) of 4 rows
        const f32x4 lo = *reinterpret_cast<const f32x4*>(pr);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(pr + 4);
        const float off[4] = {lo[0], lo[2], hi[0], hi[2]};
        const float dd[4] = {lo[1], lo[3], hi[1], hi[3]};
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const int r = 4 * m + t4;
          const float p = exp2_hw(fmaf(s[rb][r], a.scale_log2, -off[t4]));
          const float ds = p * (dp[rb][r] - dd[t4]);
          pb[2 * rb + (r >> 3)][r & 7] = (__bf16)p;
          dsb[2 * rb + (r >> 3)][r & 7] = (__bf16)ds;
        }
      }
    // dV^T += dO^T P and dK^T += Q^T dS: product f is dV (f even) or dK (f odd) of block
    // (f / 2) % NB at k-step (f / 2) / NB.
    {
      constexpr int NT = 2 * 2 * C::RB * C::NB;
      auto read_trop = [&](int f) {
        const int g = f >> 1, kk = g / C::NB, nb = g % C::NB;
        return (f & 1) ? ta.read_tr(qt, kk, nb, hi) : ta.read_tr(dt, kk, nb, hi);
      };
      bf16x8 tbuf[kTrPF];
#pragma unroll
      for (int f = 0; f < kTrPF; ++f) tbuf[f] = read_trop(f);
#pragma unroll
      for (int f = 0; f < NT; ++f) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 x = tbuf[f % kTrPF];
        if (f + kTrPF < NT) tbuf[f % kTrPF] = read_trop(f + kTrPF);
        __builtin_amdgcn_sched_barrier(0);
        const int g = f >> 1, kk = g / C::NB, nb = g % C::NB;
        if (f & 1) dka[nb] = mfma_32x32x16(x, dsb[kk], dka[nb]);
        else dva[nb] = mfma_32x32x16(x, pb[kk], dva[nb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // dK = scale * dK^T-accumulator, dV: lane holds key my_key, dims 32 nb + 8 (r / 4) +
  // 4 half + r % 4. Every wave's loads landed at its last step; once all have done their
  // last reads, LDS holds the blocks on their way out.
  static_assert(C::NW * 32 * (2 * D + 16) <= (int)sizeof(smem), "staged blocks fit in LDS");
  lds_barrier();
  {
    char* const stage = smem + w * 32 * (2 * D + 16);
    const int nrows = min(a.Lk - kw0, 32);
    store_block_rows<D>(stage, dka, a.scale, a.dk + kv_off + (size_t)kw0 * D, nrows, lane);
    store_block_rows<D>(stage, dva, 1.f, a.dv + kv_off + (size_t)kw0 * D, nrows, lane);
  }
#endif
}

// ---------------------------------------------------------------------------------------
// XCD_ORDER: workgroups grouped by KV head on the XCDs (used with GQA, see below).
template <int D, bool XCD_ORDER>
__global__ __launch_bounds__(BwdCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(BwdCfg<D>::WAVES_PER_SIMD, BwdCfg<D>::WAVES_PER_SIMD)))
void bwd_dq_kernel(const BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::Q_NS * C::Q_STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // Query blocks in order of decreasing work under a causal mask (the last rows see the
  // most keys). Without GQA: all (batch, head) pairs of one block together. With GQA
  // (XCD_ORDER) the query heads of a group read the same K and V rows, so the order of the
  // prefill (tile_order) is applied to (batch, KV head) pairs, each with `group` x ntq
  // blocks: a pair's blocks run on one XCD, and the group's heads take the same query block
  // next to each other, so their K/V tiles are shared in that XCD's L2.
  const int ntq = (a.Lq + C::QROWS - 1) / C::QROWS;
  int qt, b, h;
  if constexpr (XCD_ORDER) {
    int pair, u;
    tile_order(a.order, blockIdx.x, pair, u);
    qt = div_by(u, a.group_div);
    b = div_by(pair, a.hkv_div);
    h = (pair - b * a.Hkv) * a.group + (u - qt * a.group);
  } else {
    const int nbh = a.B * a.H;
    qt = ntq - 1 - (int)(blockIdx.x / nbh);
    const int bh = blockIdx.x % nbh;
    b = bh / a.H;
    h = bh - b * a.H;
  }
  const int kvh = h / a.group;
  int n_q, n_kv;
  seq_extent(a, b, n_q, n_kv);
  const int delta = a.Lk - a.Lq;
  const int q0 = qt * C::QROWS;
  const int qw0 = q0 + C::WROWS * w;  // this wave's first row
  const size_t q_off = (size_t)(b * a.H + h) * a.Lq;
  const size_t kv_row0 = (size_t)(b * a.Hkv + kvh) * a.Lk;

  zero_lds<C::Q_NS * C::Q_STAGE, C::NT>(smem, tid);

  bf16x8 qf[C::QB][C::QKS], dof[C::QB][C::QKS];
  float off[C::QB], dd[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int my_q = qw0 + 32 * qb + col;
#pragma unroll
    for (int ks = 0; ks < C::QKS; ++ks) {
      u32x4 uq = {0u, 0u, 0u, 0u}, ud = {0u, 0u, 0u, 0u};
      if (my_q < n_q) {
        uq = *reinterpret_cast<const u32x4*>(a.q + (q_off + my_q) * D + 16 * ks + 8 * half);
        ud = *reinterpret_cast<const u32x4*>(a.dout + (q_off + my_q) * D + 16 * ks + 8 * half);
      }
      qf[qb][ks] = as_bf16x8(uq);
      dof[qb][ks] = as_bf16x8(ud);
    }
    float2 od = make_float2(__builtin_inff(), 0.f);
    if (my_q < n_q) od = reinterpret_cast<const float2*>(a.ws)[q_off + my_q];
    off[qb] = od.x;
    dd[qb] = od.y;
  }
  f32x16 dqa[C::QB][C::NB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqa[qb][nb][r] = 0.f;

  TileAddr<D> ta;
  ta.init(lane);
  unsigned toff[C::Q_SEGS];
  tile_load_offsets<D, C::Q_SEGS>(toff, w, lane);

  // Keys any row of this block can see: [0, kv_end).
  int kv_end = 0;
  if (q0 < n_q) {
    kv_end = n_kv;
    if (a.causal) kv_end = min(kv_end, min(q0 + C::QROWS, n_q) + delta);
    kv_end = max(kv_end, 0);
  }
  kv_end = __builtin_amdgcn_readfirstlane(kv_end);
  // With a sliding window the block's first row sees nothing before q0 + delta - W + 1:
  // step t holds keys kbase + KSTEP t ...
  const int kbase = __builtin_amdgcn_readfirstlane(
      a.window > 0 ? (max(q0 + delta - a.window + 1, 0) / C::KSTEP) * C::KSTEP : 0);
  const int T = max((kv_end - kbase + C::KSTEP - 1) / C::KSTEP, 0);

  // Stage key tile t into ring slot t % Q_NS through buffer resources that end at key
  // kv_end (keys past it read nothing).
  const char* const ksrc = reinterpret_cast<const char*>(a.k) + kv_row0 * C::ROWB;
  const char* const vsrc = reinterpret_cast<const char*>(a.v) + kv_row0 * C::ROWB;
  auto issue = [&](int t) {
    const int k0 = kbase + t * C::KSTEP;
    const unsigned nrows = (unsigned)max(kv_end - k0, 0);
    char* st = smem + (t % C::Q_NS) * C::Q_STAGE;
    const u32x4 rk = raw_buffer_rsrc(ksrc + (size_t)k0 * C::ROWB, nrows * C::ROWB);
    const u32x4 rv = raw_buffer_rsrc(vsrc + (size_t)k0 * C::ROWB, nrows * C::ROWB);
    serial_fence();
#pragma unroll
    for (int i = 0; i < C::Q_SEGS; ++i) lds_dma16_buf(rk, toff[i], lds_addr(st + (w * C::Q_SEGS + i) * 1024));
#pragma unroll
    for (int i = 0; i < C::Q_SEGS; ++i)
      lds_dma16_buf(rv, toff[i], lds_addr(st + C::KTILE + (w * C::Q_SEGS + i) * 1024));
    serial_fence();
  };

  __syncthreads();  // the zero fill is done before any direct load lands
#pragma unroll
  for (int t = 0; t < C::Q_NS - 1; ++t)
    if (t < T) issue(t);
  // One complete wait on every path into the step loop, for the reason given in bwd_dkdv
  // (here the Q and dO rows were loaded into registers above).
  wait_vmcnt<0>();

  for (int t = 0; t < T; ++t) {
    if (t + C::Q_NS - 1 <= T) wait_vmcnt<(C::Q_NS - 2) * C::Q_LOADS>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (t + C::Q_NS - 1 < T) issue(t + C::Q_NS - 1);

    const int k0 = kbase + t * C::KSTEP;
    int hi = ta.tr_hi;
    asm volatile("" : "+v"(hi));  // a per-step value: tile + tr + hi is not hoisted out of the loop
    const char* kt = smem + (t % C::Q_NS) * C::Q_STAGE;
    const char* vt = kt + C::KTILE;

    // S^T and dP^T of both row blocks: element r is key k0 + 8 (r / 4) + 4 half + r % 4,
    // query qw0 + 32 qb + col.
    // Operand f of these products is the K (f even) or V (f odd) row chunk of k-step f / 2,
    // read kRowPF operands ahead; the operands of the dQ products after them are read kTrPF
    // ahead, the first ones before the softmax work. Scheduling fences keep each read ahead of
    // the product it precedes: left alone, the scheduler puts every read right before its
    // product and each product waits for a whole LDS round trip.
    constexpr int kRowPF = 4, kTrPF = 3;
    constexpr int NF = 2 * C::QKS, NT = 2 * C::NB;
    auto read_rowop = [&](int f) { return (f & 1) ? ta.read_row(vt, 0, f >> 1) : ta.read_row(kt, 0, f >> 1); };
    auto read_trop = [&](int f) { return ta.read_tr(kt, f / C::NB, f % C::NB, hi); };
    f32x16 sx[C::QB], dpx[C::QB];
    bf16x8 rbuf[kRowPF], tbuf[kTrPF];
#pragma unroll
    for (int f = 0; f < kRowPF; ++f) rbuf[f] = read_rowop(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 x = rbuf[f % kRowPF];
      if (f + kRowPF < NF) rbuf[f % kRowPF] = read_rowop(f + kRowPF);
      else if (f + kRowPF - NF < kTrPF) tbuf[f + kRowPF - NF] = read_trop(f + kRowPF - NF);
      __builtin_amdgcn_sched_barrier(0);
      const int ks = f >> 1;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        if (f & 1) dpx[qb] = mfma_32x32x16(x, dof[qb][ks], ks == 0 ? f32x16{} : dpx[qb]);
        else sx[qb] = mfma_32x32x16(x, qf[qb][ks], ks == 0 ? f32x16{} : sx[qb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool need_mask = (k0 + C::KSTEP > n_kv) || (qw0 + C::WROWS > n_q) ||
                           (a.causal && k0 + C::KSTEP - 1 > qw0 + delta) ||
                           (a.window > 0 && k0 <= qw0 + C::WROWS - 1 + delta - a.window);
    if (need_mask) {
      // The keys row my_q sees, as bounds on the element's key offset from k0 + 4 half: key j
      // is visible when j < n_kv, j <= my_q + delta (causal) and j > my_q + delta - W
      // (window), and the row exists (my_q < n_q). Compares and selects only, as above.
      const int base = k0 + 4 * half;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const int my_q = qw0 + 32 * qb + col;
        const int lo = (a.window > 0 ? my_q + delta - a.window + 1 : -(1 << 30)) - base;
        int hi = a.causal ? min(n_kv, my_q + delta + 1) : n_kv;
        hi = my_q < n_q ? hi - base : -(1 << 30);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          const bool vis = (off >= lo) & (off < hi);
          sx[qb][r] = vis ? sx[qb][r] : kNegInf;
          dpx[qb][r] = vis ? dpx[qb][r] : 0.f;
        }
      }
    }
    bf16x8 dsb[C::QB][2];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(fmaf(sx[qb][r], a.scale_log2, -off[qb]));
        dsb[qb][r >> 3][r & 7] = (__bf16)(p * (dpx[qb][r] - dd[qb]));
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < NT; ++f) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 x = tbuf[f % kTrPF];
      if (f + kTrPF < NT) tbuf[f % kTrPF] = read_trop(f + kTrPF);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) dqa[qb][f % C::NB] = mfma_32x32x16(x, dsb[qb][f / C::NB], dqa[qb][f % C::NB]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // dQ = scale * accumulator: lane holds query qw0 + 32 qb + col, dims 32 nb + 8 jj +
  // 4 half + (0..3); out through LDS as whole rows once every wave has done its last reads.
  static_assert(C::NW * 32 * (2 * D + 16) <= (int)sizeof(smem), "staged blocks fit in LDS");
  lds_barrier();
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
    store_block_rows<D>(smem + w * 32 * (2 * D + 16), dqa[qb], a.scale, a.dq + (q_off + qw0 + 32 * qb) * D,
                        min(a.Lq - qw0 - 32 * qb, 32), lane);
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
  a.ws = p.ws;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.Lq = p.Lq; a.Lk = p.Lk;
  a.group = p.H / p.Hkv;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.window = p.window;
  a.seqlens = p.seqlens;
  a.group_div = make_divisor(a.group);
  a.hkv_div = make_divisor(p.Hkv);
  void* args[] = {&a};
  const long long rows = (long long)p.B * p.H * p.Lq;
  const long long ndot = (rows + (256 / (D / 8)) - 1) / (256 / (D / 8));
  const long long nkv = (long long)p.B * p.Hkv * ((p.Lk + C::KEYS - 1) / C::KEYS);
  const long long nq = (long long)p.B * p.H * ((p.Lq + C::QROWS - 1) / C::QROWS);
  if (ndot > 0x7fffffffLL || nkv > 0x7fffffffLL || nq > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // Buffer resources address a sequence's rows with 32-bit byte counts.
  if ((long long)p.Lq * C::ROWB > 0x7fffffffLL || (long long)p.Lk * C::ROWB > 0x7fffffffLL)
    return hipErrorInvalidConfiguration;
  hipError_t e = hipSuccess;
  if (ndot > 0) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dot_kernel<D>), dim3((unsigned)ndot), dim3(256), args, 0,
                        stream);
    if (e != hipSuccess) return e;
  }
  if (nkv > 0) {
    // The XCD order pays with GQA (GQA varlen workload 10.8 -> 8.5 ms) and costs up to 10%
    // without it (B=4, H=16, L=2048, d=64), so it is used with GQA only.
    const void* kfn = p.H > p.Hkv ? reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, true>)
                                  : reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, false>);
    BwdArgs ak = a;
    ak.order = make_tile_order((int)nkv, (p.Lk + C::KEYS - 1) / C::KEYS);
    void* kargs[] = {&ak};
    e = hipLaunchKernel(kfn, dim3((unsigned)nkv), dim3(C::NT), kargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  if (nq > 0) {
    BwdArgs aq = a;
    aq.order = make_tile_order((int)nq, a.group * ((p.Lq + C::QROWS - 1) / C::QROWS));
    void* qargs[] = {&aq};
    e = hipLaunchKernel(p.H > p.Hkv ? reinterpret_cast<const void*>(&bwd_dq_kernel<D, true>)
                                    : reinterpret_cast<const void*>(&bwd_dq_kernel<D, false>),
                        dim3((unsigned)nq), dim3(C::NT), qargs, 0, stream);
  }
  return e;
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.d == 64) return launch_b<64>(p, stream);
  return launch_b<128>(p, stream);
}

}  // namespace fa
