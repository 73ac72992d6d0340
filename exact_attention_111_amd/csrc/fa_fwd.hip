// fa_fwd.hip — prefill attention forward for gfx950 (MI355X).
//
// The method ("FlashAttention 与长上下文：先分清三张账", section "FlashAttention 的关键是
// online softmax"; "2.1 FlashAttention-2 的核心思想" §2.1.2–§2.1.3): the queries are cut
// into row tiles and the keys/values into column tiles; each tile pair is scored on chip
// and thrown away, while every query row carries a running maximum m, a running sum l of
// exponentials relative to m, and an unnormalised output o. When the maximum grows, l and
// o are multiplied by exp(m_old - m_new). At the end O = o / l and the row's log-sum-exp
// is written. Score and probability tiles never leave the compute unit.
//
// gfx950 mapping. One workgroup = 8 wave64s = one 256-row query tile of one head; wave w
// owns 32 query rows and runs on SIMD w % 4, so waves w and w + 4 share a SIMD.
//   * The two wave groups (waves 0-3 and 4-7) run one phase apart ("ping-pong"): in every
//     phase one group issues matrix products — P V of tile j-1, then S of tile j — while
//     the other group runs the softmax of its latest S tile on the VALU; a workgroup
//     barrier separates phases, and the roles swap each phase. The softmax, which costs
//     about as much issue time as the products at d = 128 (one exp per score element runs
//     at a quarter of the FMA rate), is thus hidden behind the other wave's MFMAs. The
//     wave in its product phase raises its issue priority.
//   * Q rows stay in VGPRs as the B operand of v_mfma_f32_32x32x16_bf16.
//   * K/V tiles of 64 keys go HBM -> LDS with 16-byte direct-to-LDS loads
//     (global_load_lds_dwordx4; no VGPR staging, no VALU work). K runs one tile ahead of V;
//     both are double buffered and loads have two phases to land.
//   * S^T = K Q^T (keys down, queries across): in the 32x32 accumulator layout a lane holds
//     one query column, so a row's max, sum and rescale factor live in that lane (plus
//     lane ^ 32, one exchange per tile for the max).
//   * O^T = V^T P^T with P taken straight from the accumulators (converted to bf16) and the
//     V^T operand read from the row-major V tile with ds_read_b64_tr_b16 (its 16-lane
//     transpose turns 4 rows x 4 dims into the 4-keys-per-lane operand layout). The
//     contraction index of that product is ordered to match the accumulator layout.
//   * LDS rows are XOR-swizzled in 16-byte chunks so that both operand reads are free of
//     bank conflicts on gfx950's LDS (128-bit reads are served 16 lanes at a time); every
//     operand address is computed once per lane and reused with immediate offsets.
//   * exp is 2^x on v_exp_f32 with scale*log2(e) folded into one FMA. A row's reference
//     maximum is raised only when a tile's maximum exceeds it by more than 2^8 (then o and
//     l are rescaled); o / l does not depend on the reference, so this only skips work.
//   * Causal and padding masks are applied element-wise only on tiles that straddle the
//     diagonal or the sequence end; a wave skips tiles none of its rows can see, and key
//     tiles past the query tile's last visible key are never loaded.
//   * Workgroups are renumbered so that the ones dispatched to the same XCD (dispatch is
//     round-robin over the 8 XCDs) work on the same head at the same time and share its
//     K/V through that XCD's L2; within a head the heaviest (latest) query tiles go first.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct FwdCfg {
  static constexpr int BM = 256;                  // query rows per workgroup
  static constexpr int BN = 64;                   // keys per tile
  static constexpr int NW = 8;                    // waves
  static constexpr int NT = NW * 64;              // threads
  static constexpr int ROWB = D * 2;              // bytes per K/V row
  static constexpr int TILE_BYTES = BN * ROWB;    // one K (or V) tile
  static constexpr int SEGS = TILE_BYTES / 1024;  // 1 KB direct-load segments per tile
  static constexpr int SEGS_PER_WAVE = SEGS / NW;
  static constexpr int QKS = D / 16;              // 32x32x16 k-steps over d
  static constexpr int NB = D / 32;               // 32-row blocks of O^T
  static_assert(SEGS % NW == 0, "tile must split evenly over the waves");
};

constexpr float kLazyRescale = 8.0f;  // log2 of the largest probability allowed before rescaling

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Lq, Lk;
  int group;        // H / Hkv
  int ntq;          // query tiles per head
  int nwg;          // workgroups
  float scale_log2; // scale * log2(e)
  int causal;
  const int32_t* seqlens;
};

// XOR applied to the 16-byte chunk index of tile row r.
//   K (read by 16 lanes = 16 consecutive rows, same logical chunk): every row of a 16-row
//   group must land on a different 16-byte bank slot of the 256-byte bank window.
//   V (read transposed: a 16-lane group touches 4 consecutive rows x one 32-byte chunk pair,
//   two groups per access): the 8 (row, pair) slots of an access must differ.
template <int D>
__device__ __forceinline__ int k_xor(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_xor(int r) {
  const int j = r & 3;
  return D == 128 ? 2 * (j ^ ((j & 1) << 2)) : ((j & 2) << 1);
}

template <int D, typename IT, typename OT>
__global__ __launch_bounds__(512) void fwd_kernel(const FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = FwdCfg<D>;
  // [K slot 0 | K slot 1 | V slot 0 | V slot 1 | V slot 2]
  __shared__ __attribute__((aligned(1024))) char smem[5 * C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, provably uniform
  const int grp = w >> 2;                                  // ping-pong group
  const int col = lane & 31;   // this lane's query row within the wave
  const int half = lane >> 5;  // which 8-element half of a 16-wide k-step

  // XCD-aware renumbering: hardware id i runs on XCD i % 8; give each XCD a contiguous
  // range of logical ids so its CUs work through one head at a time.
  const int hw = blockIdx.x;
  const int xcd = hw & 7, slot = hw >> 3;
  const int per = a.nwg >> 3, extra = a.nwg & 7;
  const int logical = xcd * per + min(xcd, extra) + slot;
  const int bh = logical / a.ntq;
  const int qt = a.ntq - 1 - (logical - bh * a.ntq);  // heaviest first within a head
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
    if (a.causal) kv_end = min(kv_end, min(q0 + C::BM, n_q) + delta);
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

  // Operand addresses, computed once. K: lane reads row kb*32 + col, logical chunk
  // 2*ks + half. V (transposed read): lane (g, sl) = (lane / 16, lane % 16) reads row
  // 16*ks + 8*rr + 4*(g/2) + sl/4, dims 32*nb + 16*(g%2) + 4*(sl%4) .. +3.
  int kaddr[C::QKS];
#pragma unroll
  for (int ks = 0; ks < C::QKS; ++ks) kaddr[ks] = col * C::ROWB + (((2 * ks + half) ^ k_xor<D>(col)) << 4);
  const int g = lane >> 4, sl = lane & 15;
  const int vrow = 4 * (g >> 1) + (sl >> 2);
  int vaddr[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const int dim = 32 * nb + 16 * (g & 1) + 4 * (sl & 3);
    vaddr[nb] = vrow * C::ROWB + (((dim >> 3) ^ v_xor<D>(vrow)) << 4) + ((dim & 4) << 1);
  }

  f32x16 oacc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.f;
  float m = kNegInf;  // reference max (scaled, base 2) of this lane's row
  float l = 0.f;      // this lane's part of the running sum (the other part is in lane ^ 32)
  f32x16 s[2];        // S^T of the latest tile, two 32-key halves
  bf16x8 pb[4];       // P^T of the latest tile as PV operands
  float alpha = 1.f;  // rescale of o decided by the softmax phase, applied by the next product phase
  bool rescale = false;

  // LDS: K tiles double buffered (K tile t in slot t % 2), V tiles triple buffered (slot
  // t % 3), so that V tile t is resident one phase before the product phase that reads it.
  auto k_slot = [&](int t) { return (t & 1) * C::TILE_BYTES; };
  auto v_slot = [&](int t) { return (2 + t % 3) * C::TILE_BYTES; };

  // Stage K tile t (which = 0) or V tile t (which = 1). Keys past kv_end read row
  // kv_end - 1 instead (a visible, finite row); the mask gives them p = 0.
  auto stage = [&](int t, int which) {
    const int k0 = t * C::BN;
    char* dst = smem + (which ? v_slot(t) : k_slot(t));
    const IT* src = which ? vp : kp;
    if constexpr (sizeof(IT) == 2) {
#pragma unroll
      for (int i = 0; i < C::SEGS_PER_WAVE; ++i) {
        const int seg = w * C::SEGS_PER_WAVE + i;
        const int byte = seg * 1024 + lane * 16;
        const int r = byte / C::ROWB;
        const int cp = (byte - r * C::ROWB) >> 4;  // physical chunk this lane fills
        const int key = min(k0 + r, kv_end - 1);
        const int cl = cp ^ (which ? v_xor<D>(r) : k_xor<D>(r));
        __builtin_amdgcn_global_load_lds(src + (size_t)key * D + (cl << 3), (lds_void*)(dst + seg * 1024), 16, 0, 0);
      }
    } else {
      // fp32 input: load, round to bf16 (RNE) in registers, store into the same layout.
      constexpr int CH = D / 8;
#pragma unroll
      for (int i = 0; i < C::BN * CH / C::NT; ++i) {
        const int idx = i * C::NT + tid;
        const int r = idx / CH;
        const int c = idx - r * CH;
        const int key = min(k0 + r, kv_end - 1);
        const int cp = c ^ (which ? v_xor<D>(r) : k_xor<D>(r));
        *reinterpret_cast<u32x4*>(dst + r * C::ROWB + (cp << 4)) = Load8<IT>::load(src + (size_t)key * D + 8 * c);
      }
    }
  };

  // Does this wave see any key of tile t?
  auto active = [&](int t) { return (qw0 < n_q) && !(a.causal && t * C::BN > qw0 + 31 + delta); };

  // Operand reads. PV product i (k-step i / NB, block i % NB) of a tile whose V sits in
  // slot `vs`: two transposed 64-bit reads. S product i of a tile whose K sits in slot
  // `ksl`: one 128-bit read of half i / QKS, k-step i % QKS.
  auto read_v = [&](int vs, int i) {
    const int ks = i / C::NB, nb = i % C::NB;
    const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(smem + vaddr[nb] + vs + (16 * ks) * C::ROWB));
    const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(smem + vaddr[nb] + vs + (16 * ks + 8) * C::ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_k = [&](int ksl, int i) {
    return *reinterpret_cast<const bf16x8*>(smem + kaddr[i % C::QKS] + ksl + (i / C::QKS) * 32 * C::ROWB);
  };

  // Product phase for tile j: one chain of MFMAs, O^T += V^T P^T of tile j - 1 (NPV
  // products) followed by S^T = K Q^T of tile j (NSP products), with every operand read
  // PF products ahead and the first PF V operands already read at the end of the
  // previous softmax phase (vpre). Scheduling groups pin the interleaving. The chain always
  // runs whole: where tile j - 1 gives this wave nothing (j = 0, or no visible key) P is
  // zero and V is a resident tile of finite values, so the products add exact zeros; where
  // tile j does not exist or is invisible, S is computed and never read.
  constexpr int PF = 4;
  constexpr int NPV = 4 * C::NB;   // 16 at d = 128
  constexpr int NSP = 2 * C::QKS;  // 16 at d = 128
  constexpr int N = NPV + NSP;
  bf16x8 vpre[PF];
  auto product_phase = [&](int j) {
    // Keep the per-lane operand bases opaque to loop-invariant code motion: otherwise every
    // (base + immediate offset) pair is hoisted out of the phase loop into its own VGPR.
#pragma unroll
    for (int ks = 0; ks < C::QKS; ++ks) asm volatile("" : "+v"(kaddr[ks]));
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) asm volatile("" : "+v"(vaddr[nb]));
    __builtin_amdgcn_s_setprio(1);
    if (rescale) {  // wave-uniform; rare once a row's maximum has settled
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[nb][r] *= alpha;
      rescale = false;
    }
    const int vs = v_slot(max(j - 1, 0));
    const int ksl = k_slot(j);
    bf16x8 buf[PF];
#pragma unroll
    for (int f = 0; f < PF; ++f) buf[f] = vpre[f];
    const f32x16 zero = {};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bf16x8 x = buf[i % PF];
      const int nx = i + PF;
      if (nx < N) buf[i % PF] = nx < NPV ? read_v(vs, nx) : read_k(ksl, nx - NPV);
      if (i < NPV) {
        oacc[i % C::NB] = mfma_32x32x16(x, pb[i / C::NB], oacc[i % C::NB]);
      } else {
        const int ii = i - NPV, kb = ii / C::QKS, ks = ii % C::QKS;
        s[kb] = mfma_32x32x16(x, qf[ks], ks == 0 ? zero : s[kb]);
      }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int nx = i + PF;
      if (nx < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // two transposed reads
      else if (nx < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one 128-bit read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // one MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  // Softmax phase for tile j: mask, online max / rescale, P = 2^(S*c - m), row sums.
  auto softmax_phase = [&](int j) {
    if (!(j >= 0 && j < ntk && active(j))) {  // nothing visible: the next PV chain adds zeros
#pragma unroll
      for (int q = 0; q < 4; ++q) pb[q] = bf16x8{};
      return;
    }
    const int k0 = j * C::BN;
    const bool need_mask = (k0 + C::BN > n_kv) || (a.causal && k0 + C::BN - 1 > qw0 + delta);
    // Accumulator element r of half kb is key k0 + 4*half + (32*kb + 8*(r/4) + r%4), query
    // my_q; it is visible when that constant offset is below both per-lane limits.
    if (need_mask) {
      const int base = k0 + 4 * half;
      const int lim = min(n_kv - base, a.causal ? my_q + delta + 1 - base : n_kv - base);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = kNegInf;
    }
    // Row max and row sum are taken as four independent partial chains (short dependency
    // chains; the order of a max does not matter, the sum's grouping is fixed here).
    float mp[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], s[kb][r]);
    float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
    {  // lanes l and l ^ 32 hold the same row: exchange halves with v_permlane32_swap
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mx), __builtin_bit_cast(unsigned, mx),
                                                       false, false);
      mx = fmaxf(__builtin_bit_cast(float, sw[0]), __builtin_bit_cast(float, sw[1])) * a.scale_log2;
    }
    const bool raise = mx > m + kLazyRescale;  // also true for the first visible tile
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mx : m;
      alpha = raise ? exp2_hw(m - m_new) : 1.f;
      l *= alpha;
      m = m_new;
      rescale = true;
    }
    const float neg_m = (m == kNegInf) ? 0.f : -m;  // a row that has seen nothing keeps p = 0
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2_hw(fmaf(s[kb][8 * hh + e], a.scale_log2, neg_m));
          rs[e & 3] += p;
          pb[2 * kb + hh][e] = (__bf16)p;
        }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };

  // First V operands of the PV chain of tile i (read at the end of its softmax phase).
  auto pre_read_v = [&](int i) {
#pragma unroll
    for (int f = 0; f < PF; ++f) vpre[f] = read_v(v_slot(i), f);
  };

  if (ntk > 0) {
    stage(0, 0);
    stage(0, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) pb[q] = bf16x8{};
    pre_read_v(0);
    // Global phases are separated by workgroup barriers. Every wave runs the same body per
    // tile i: its product phase, a barrier, its softmax phase, a barrier. Group 1 starts one
    // phase late (a leading barrier) and so runs each softmax beside group 0's next product
    // phase. K and V tile i + 1 are loaded in global phase 2i (group 0: before product i;
    // group 1: before softmax i - 1) and every wave waits for its own loads at the end of
    // phase 2i + 1, before the barrier that opens phase 2i + 2.
    if (grp == 1) {
      if (1 < ntk) { stage(1, 0); stage(1, 1); }
      lds_barrier();
    }
    for (int i = 0; i <= ntk; ++i) {
      if (grp == 0 && i + 1 < ntk) { stage(i + 1, 0); stage(i + 1, 1); }
      product_phase(i);
      if (grp == 1) __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
      if (grp == 1 && i + 2 < ntk) { stage(i + 2, 0); stage(i + 2, 1); }
      softmax_phase(i);
      if (i < ntk) pre_read_v(i);
      if (grp == 0) __builtin_amdgcn_s_waitcnt(0);
      if (grp == 0 || i < ntk) lds_barrier();
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
#endif
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
  a.nwg = (int)nwg;
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
