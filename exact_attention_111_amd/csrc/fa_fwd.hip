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
// gfx950 mapping (one workgroup = 8 wave64s = one 256-row query tile of one head, so two
// waves share each SIMD and one wave's softmax overlaps the other's matrix products):
//   * Each wave owns 32 query rows, held in VGPRs as the B operand of
//     v_mfma_f32_32x32x16_bf16 for the whole kernel.
//   * K/V tiles of 64 keys go HBM -> LDS with 16-byte direct-to-LDS loads
//     (global_load_lds_dwordx4; no VGPR staging, no VALU work), double buffered so the
//     next tile streams in while the current one is used; one barrier per tile.
//     Both tiles stay row major; 16-byte chunks are XOR-swizzled per row so that the
//     operand reads below spread over the LDS banks.
//   * S^T = K Q^T (keys down, queries across): in the 32x32 accumulator layout a lane
//     holds one query column, so a row's max, sum and rescale factor live in that lane
//     (plus lane ^ 32, one exchange per tile for the max).
//   * O^T = V^T P^T with P taken straight from the accumulators (converted to bf16) and
//     V^T operands read from the row-major V tile with ds_read_b64_tr_b16, whose 16-lane
//     transpose turns 4 rows x 4 dims into the 4-keys-per-lane operand layout. The
//     contraction index of that product is ordered to match the accumulator layout.
//   * exp is 2^x on v_exp_f32 with scale*log2(e) folded into one FMA.
//   * A row's reference maximum is raised only when a tile's maximum exceeds it by more
//     than 2^8 (then o and l are rescaled); otherwise the tile's probabilities are taken
//     against the old reference and can be up to 256. The result o / l does not depend on
//     the reference, so this only skips rescaling work.
//   * Causal and padding masks are applied element-wise only on tiles that straddle the
//     diagonal or the sequence end; a wave skips tiles none of its rows can see, and key
//     tiles past the query tile's last visible key are never loaded.
//   * Workgroups are renumbered so that the ones dispatched to the same XCD (dispatch is
//     round-robin over the 8 XCDs) work on the same head at the same time and share its
//     K/V through that XCD's L2; within a head the heaviest (latest) query tiles go first.
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

// Byte offset of 16-byte chunk `c` of tile row `r`; K and V use different XOR swizzles.
//   K: chunk ^ (r & 7): the 8 lanes of a 128-bit read (8 consecutive rows, same chunk)
//      hit 8 different bank groups.
//   V: chunk ^ 2 (r & 3): a 16-lane transposed read touches 4 consecutive rows x one
//      32-byte chunk pair; the swizzle keeps the pair together and moves it per row.
template <int D>
__device__ __forceinline__ int k_off(int r, int c) { return r * (D * 2) + ((c ^ (r & 7)) << 4); }
template <int D>
__device__ __forceinline__ int v_off(int r, int c) { return r * (D * 2) + ((c ^ ((r & 3) << 1)) << 4); }

template <int D, typename IT, typename OT>
__global__ __launch_bounds__(512) void fwd_kernel(const FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][C::TILE_BYTES];  // [buffer][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, provably uniform
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

  f32x16 oacc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.f;
  float m = kNegInf;  // reference max (scaled, base 2) of this lane's row
  float l = 0.f;      // this lane's part of the running sum (the other part is in lane ^ 32)

  // Stage key tile t into buffer `buf`. Keys past kv_end read row kv_end - 1 instead (always
  // a visible, finite row); the mask gives them probability 0.
  auto stage = [&](int t, int buf) {
    const int k0 = t * C::BN;
    if constexpr (sizeof(IT) == 2) {
#pragma unroll
      for (int i = 0; i < C::SEGS_PER_WAVE; ++i) {
        const int seg = w * C::SEGS_PER_WAVE + i;
        const int byte = seg * 1024 + lane * 16;
        const int r = byte / C::ROWB;
        const int cp = (byte - r * C::ROWB) >> 4;  // physical chunk this lane fills
        const int key = min(k0 + r, kv_end - 1);
        const IT* ksrc = kp + (size_t)key * D + ((cp ^ (r & 7)) << 3);
        const IT* vsrc = vp + (size_t)key * D + ((cp ^ ((r & 3) << 1)) << 3);
        __builtin_amdgcn_global_load_lds(ksrc, (lds_void*)(&smem[buf][0][seg * 1024]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vsrc, (lds_void*)(&smem[buf][1][seg * 1024]), 16, 0, 0);
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
        *reinterpret_cast<u32x4*>(&smem[buf][0][k_off<D>(r, c)]) = Load8<IT>::load(kp + (size_t)key * D + 8 * c);
        *reinterpret_cast<u32x4*>(&smem[buf][1][v_off<D>(r, c)]) = Load8<IT>::load(vp + (size_t)key * D + 8 * c);
      }
    }
  };

  if (ntk > 0) {
    stage(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int t = 0; t < ntk; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntk) stage(t + 1, buf ^ 1);  // streams in while this tile is used

    const int k0 = t * C::BN;
    const bool active = (qw0 < n_q) && !(a.causal && k0 > qw0 + 31 + delta);
    if (active) {
      const char* Kt = smem[buf][0];
      const char* Vt = smem[buf][1];
      const bool need_mask = (k0 + C::BN > n_kv) || (a.causal && k0 + C::BN - 1 > qw0 + delta);

      // S^T = K Q^T for the two 32-key halves of the tile. All 2*QKS operand reads are
      // issued before the first product so LDS latency is paid once per tile.
      bf16x8 kf[2][C::QKS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < C::QKS; ++ks)
          kf[kb][ks] = *reinterpret_cast<const bf16x8*>(Kt + k_off<D>(kb * 32 + col, 2 * ks + half));
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::QKS; ++ks) s[kb] = mfma_32x32x16(kf[kb][ks], qf[ks], s[kb]);
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

      // Online softmax with a lazily raised reference max (base 2, scaled).
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
      const bool raise = mx > m + kLazyRescale;  // also true for the first visible tile
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float m_new = raise ? mx : m;
        const float alpha = raise ? exp2_hw(m - m_new) : 1.f;
        l *= alpha;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[nb][r] *= alpha;
        m = m_new;
      }
      const float neg_m = (m == kNegInf) ? 0.f : -m;  // a row that has seen nothing keeps p = 0

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
      l += rs;

      // O^T += V^T P^T. k-step ks uses accumulator registers 8*(ks%2) .. +7 of half ks/2,
      // i.e. keys 16*ks + 8*(e/4) + 4*half + e%4 for element e. The transposed read gives
      // lane (16 g + j) the 4 keys 16*ks + 8*rr + 4*(g/2) + u at dim 32*nb + 16*(g%2) + j
      // when its source lanes s = 0..15 point at row 16*ks + 8*rr + 4*(g/2) + s/4,
      // dims 32*nb + 16*(g%2) + 4*(s%4) .. +3.
      const int g = lane >> 4, sl = lane & 15;
      auto read_v = [&](int ks, int nb) {
        s16x4 part[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int row = 16 * ks + 8 * rr + 4 * (g >> 1) + (sl >> 2);
          const int dim = 32 * nb + 16 * (g & 1) + 4 * (sl & 3);
          const int off = v_off<D>(row, dim >> 3) + ((dim & 4) << 1);
          part[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + off));
        }
        const s16x4 p0 = part[0], p1 = part[1];
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      // Operands of k-step ks + 1 are read while k-step ks multiplies.
      bf16x8 vf[2][C::NB];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) vf[0][nb] = read_v(0, nb);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks + 1 < 4) {
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) vf[(ks + 1) & 1][nb] = read_v(ks + 1, nb);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) oacc[nb] = mfma_32x32x16(vf[ks & 1][nb], pb[ks], oacc[nb]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile have landed
    __syncthreads();                // ... everyone's have, and nobody reads `buf` any more
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
