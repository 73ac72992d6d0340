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
// gfx950 mapping. A workgroup computes 256-row query tiles of one head at a time: 8 wave64s of
// 32 query rows, two waves per SIMD, so a wave fits in 256 VGPRs (d = 64 and 128).
//   * One body per 64-key tile j, one workgroup barrier each, in two regions: (X) the MFMAs
//     of S for tile j + 1 beside exp / row sum / bf16 conversion of most of tile j, then
//     (Y) the MFMAs of P V for tile j beside the rest of tile j's exps and the scale-and-
//     shift of tile j + 1. Each region is written out one step per MFMA (operand read four
//     steps ahead, a fixed slice of softmax work, a scheduling fence), so the matrix cores
//     run while the wave issues its softmax arithmetic.
//   * Q rows stay in registers as the B operand of v_mfma_f32_32x32x16_bf16.
//   * K/V tiles go HBM -> LDS with 16-byte buffer loads straight into LDS (no VGPR staging,
//     no VALU work), three slots each, two tiles ahead. The buffer resource ends at the
//     last visible key, so the loads need no bounds branch. They are issued so that the
//     compiler does not see them (it would otherwise make every LDS read wait for them);
//     each wave waits for its own loads before the barrier that closes a tile.
//   * S^T = K Q^T (keys down, queries across): in the 32x32 accumulator layout a lane holds
//     one query column, so a row's reference, sum and rescale factor live in that lane
//     (plus lane ^ 32, combined with v_permlane32_swap).
//   * O^T = V^T P^T with P taken straight from the accumulators (converted to bf16) and the
//     V^T operand read from the row-major V tile with ds_read_b64_tr_b16 (its 16-lane
//     transpose turns 4 rows x 4 dims into the 4-keys-per-lane operand layout). The
//     contraction index of that product is ordered to match the accumulator layout.
//   * LDS rows are XOR-swizzled in 16-byte chunks so that both operand reads are free of
//     bank conflicts on gfx950's LDS (128-bit reads are served 16 lanes at a time); every
//     operand address is computed once per lane and reused with immediate offsets.
//   * exp is 2^x on v_exp_f32 with scale*log2(e) folded into one FMA. Tiles are shifted by
//     the row's current reference m without computing their maximum; only a part after
//     which a row-sum chain passes 2^40 (or, with a window, a row's first visible keys)
//     raises m and rescales l and o. o / l does not depend on the reference, so this only
//     skips work.
//   * Causal and padding masks are applied element-wise only on tiles that straddle the
//     diagonal or the sequence end, and key tiles past the query tile's last visible key are
//     never loaded. On the causal diagonal a wave stops computing after the last tile its
//     own rows can see; the two waves of a SIMD hold a top and a bottom row block, so every
//     SIMD is left the same work there.
//   * Heads are dealt round-robin to the 8 XCDs (dispatch is round-robin over them), and
//     each XCD works through its heads one at a time, heaviest query tile first, so that its
//     CUs share that head's K/V in the XCD's L2. Dense inputs run on a persistent grid (one
//     workgroup per CU taking its XCD's tiles in rounds); with per-sequence lengths each tile
//     is a workgroup of its own and the hardware hands them out.
//   * O leaves through LDS as whole rows (16 contiguous bytes per lane).
#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tiles.h"

namespace fa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct FwdCfg {
  // 32 rows per wave and 8 waves, two per SIMD: a wave fits in 256 registers, which also
  // keeps the compiler's MFMA results in VGPRs (with a 512-register budget it picks the
  // AGPR form and copies every score tile into VGPRs for the softmax). A workgroup covers
  // 256 query rows, which sets how often each K/V tile is streamed from L2 into LDS.
  static constexpr int QB = 1;                    // 32-row query blocks per wave
  static constexpr int NW = 8;                    // waves per workgroup (waves w, w + 4 share a SIMD)
  static constexpr int BM = 32 * QB * NW;         // query rows per workgroup (256)
  static constexpr int WAVES_PER_SIMD = NW / 4;
  static constexpr int NS = 3;                    // LDS slots for K tiles (and as many for V)
  static constexpr int BN = 64;                   // keys per tile
  static constexpr int NT = NW * 64;              // threads
  static constexpr int ROWB = D * 2;              // bytes per K/V row
  static constexpr int TILE_BYTES = BN * ROWB;    // one K (or V) tile
  static constexpr int SEGS = TILE_BYTES / 1024;  // 1 KB direct-load segments per tile
  static constexpr int SEGS_PER_WAVE = SEGS / NW;
  static constexpr int QKS = D / 16;              // 32x32x16 k-steps over d
  static constexpr int NB = D / 32;               // 32-row blocks of O^T
  static constexpr int NKF = 2 * QKS;             // K operands per tile (2 key halves x QKS)
  static constexpr int NVF = 4 * NB;              // V operands per tile (4 k-steps x NB)
  static_assert(SEGS % NW == 0, "tile must split evenly over the waves");
};

constexpr int kPF = 4;                // operand reads issued this many operands ahead
constexpr int kDmaStep = 2;           // step of each region at which its tile loads are issued

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Lq, Lk;
  int group;        // H / Hkv
  int ntq;          // query tiles per head
  int nwg;          // query tiles (ids of tile_order)
  int nprog;        // workgroups launched (tile_of_program)
  TileOrder order;  // tile_order over (batch, KV head) pairs, group x ntq tiles each
  Divisor group_div, hkv_div;  // H / Hkv and Hkv as divisors
  float scale_log2; // scale * log2(e)
  int causal;
  int window;       // sliding window W (0: none): key j needs j > i + Lk - Lq - W
  const int32_t* seqlens;
};

// WIN: a sliding window is in force (a.window > 0). Only then can a row meet its first
// visible key after the first tile; the window-free kernel leaves that test out.
template <int D, typename IT, typename OT, bool WIN>
__global__ __launch_bounds__(FwdCfg<D>::NT)
__attribute__((amdgpu_waves_per_eu(FwdCfg<D>::WAVES_PER_SIMD, FwdCfg<D>::WAVES_PER_SIMD))) void fwd_kernel(const FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = FwdCfg<D>;
  constexpr int QB = C::QB;
  // [K slots 0-2 | V slots 0-2]
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::NS * C::TILE_BYTES];

  // Tiles of this workgroup, one per round (tile_of_program); each round is the whole tile.
  // fp32 inputs take one tile per workgroup (the host launches one per tile), which leaves
  // their staging registers to the single tile.
  constexpr bool kRounds = sizeof(IT) == 2;
  for (int round = 0; kRounds || round == 0; ++round) {
    const int tile = tile_of_program(blockIdx.x, round, a.nprog, a.nwg);
    if (tile < 0) break;
    // Per-lane values are rebuilt in every round rather than hoisted out of the round loop,
    // where they would hold registers through the whole tile.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, provably uniform
    const int col = lane & 31;   // this lane's query row within a 32-row block
    const int half = lane >> 5;  // which 8-element half of a 16-wide k-step
    // Workgroup order: tile_order over (batch, KV head) pairs with group x ntq tiles
    // each, so the query heads that share a KV head run on one XCD and take the same query
    // tile side by side (their K/V tiles are then shared in that XCD's L2). Without GQA the
    // pairs are the heads themselves.
    int pair, u;
    tile_order(a.order, tile, pair, u);
    const int qt = div_by(u, a.group_div);
    const int b = div_by(pair, a.hkv_div);
    const int kvh = pair - b * a.Hkv;
    const int h = kvh * a.group + (u - qt * a.group);

    int n_kv = a.Lk, n_q = a.Lq;
    if (a.seqlens != nullptr) {
      const int n = min(max(load_const(a.seqlens + b), 0), a.Lk);
      n_kv = n;
      n_q = n;
    }
    const int delta = a.Lk - a.Lq;  // bottom-right causal alignment
    const int q0 = qt * C::BM;
    // Row block of this wave. Waves w and w + NW/2 share a SIMD; giving them blocks s and
    // NW - 1 - s pairs a top block of the tile with a bottom one, so that on causal diagonal
    // tiles every SIMD has the same amount of work left after its waves' last visible keys.
    const int rblk = w < C::NW / 2 ? w : 3 * C::NW / 2 - 1 - w;
    const int qw0 = q0 + 32 * QB * rblk;  // first query row of this wave
    int my_q[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) my_q[qb] = qw0 + 32 * qb + col;

    // Keys this query tile can see: [kv_begin, kv_end). With a sliding window the first row
    // of the tile sees nothing before q0 + delta - W + 1, so the tiles before the one holding
    // that key are never loaded; pipeline tile t holds keys kbase + 64 t ...
    int kv_end = 0;
    if (q0 < n_q) {
      kv_end = n_kv;
      if (a.causal) kv_end = min(kv_end, min(q0 + C::BM, n_q) + delta);
      kv_end = max(kv_end, 0);
    }
    kv_end = __builtin_amdgcn_readfirstlane(kv_end);  // uniform: keeps load setup in SGPRs
    const int kbase = __builtin_amdgcn_readfirstlane(
        WIN ? (max(q0 + delta - a.window + 1, 0) / C::BN) * C::BN : 0);
    const int ntk = max((kv_end - kbase + C::BN - 1) / C::BN, 0);
    // Newest key any row of this wave can see (every key of the tile range without a causal mask)
    const int wave_last_key = __builtin_amdgcn_readfirstlane(a.causal ? qw0 + 32 * QB - 1 + delta : kv_end);

    const IT* __restrict__ qp = static_cast<const IT*>(a.q) + (size_t)(b * a.H + h) * a.Lq * D;
    const IT* __restrict__ kp = uniform_ptr(static_cast<const IT*>(a.k) + (size_t)(b * a.Hkv + kvh) * a.Lk * D);
    const IT* __restrict__ vp = uniform_ptr(static_cast<const IT*>(a.v) + (size_t)(b * a.Hkv + kvh) * a.Lk * D);

    // Q rows of this lane as MFMA B operands: element t of k-step ks is d = 16*ks + 8*half + t.
    bf16x8 qf[QB][C::QKS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < C::QKS; ++ks) {
        u32x4 u = {0u, 0u, 0u, 0u};
        if (my_q[qb] < n_q && ntk > 0) u = Load8<IT>::load(qp + (size_t)my_q[qb] * D + 16 * ks + 8 * half);
        qf[qb][ks] = as_bf16x8(u);
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
      vaddr[nb] = C::NS * C::TILE_BYTES + vrow * C::ROWB + (((dim >> 3) ^ v_xor<D>(vrow)) << 4) + ((dim & 4) << 1);
    }
    // Direct-load source offsets within a tile (bytes from the tile's first row): segment i
    // of this wave puts 16 bytes at LDS byte seg * 1024 + 16 * lane, holding row r's logical
    // chunk (physical chunk ^ swizzle).
    unsigned koff[C::SEGS_PER_WAVE], voff[C::SEGS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::SEGS_PER_WAVE; ++i) {
      const int byte = (w * C::SEGS_PER_WAVE + i) * 1024 + lane * 16;
      const int r = byte / C::ROWB;
      const int cp = (byte - r * C::ROWB) >> 4;
      koff[i] = r * C::ROWB + ((cp ^ k_xor<D>(r)) << 4);
      voff[i] = r * C::ROWB + ((cp ^ v_xor<D>(r)) << 4);
    }

    f32x16 oacc[QB][C::NB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][nb][r] = 0.f;
    // Per row: the reference m (scaled, base 2), the shift nm applied before each exp (-m, or
    // 0 while the row has no reference), and this lane's part of the row sum l as two
    // interleaved chains of adds (elements of even and of odd index).
    float m[QB], nm[QB], lc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m[qb] = kNegInf;
      nm[qb] = 0.f;
      lc[qb][0] = lc[qb][1] = 0.f;
    }
    f32x16 sa[QB][2], sb[QB][2];  // S^T (then scaled, shifted scores) of two consecutive tiles
    bf16x8 pb[QB][4];              // P^T of the tile whose P V runs next

    // K and V tile t live in slot t % 3 (K slots first, then V slots), so loads can run two
    // tiles ahead of their use.
    auto k_slot = [&](int t) { return (t % C::NS) * C::TILE_BYTES; };
    auto v_slot = [&](int t) { return (C::NS + t % C::NS) * C::TILE_BYTES; };

    // Stage K tile t (which = 0) or V tile t (which = 1) into the slot at byte `slot` of the
    // LDS buffer. bf16 input: branch-free direct loads through a buffer resource that ends at
    // key kv_end, so rows past it (and whole tiles past it) read no memory; their LDS rows are
    // masked (K) or multiplied by p = 0 (V) and only need to be finite, which they are (the
    // buffers start zeroed and only ever hold input rows). fp32 input: rows past kv_end read
    // row kv_end - 1 instead.
    auto stage = [&](int t, int which, int slot) {
      const int k0 = kbase + t * C::BN;
      char* dst = smem + slot;
      const IT* src = which ? vp : kp;
      serial_fence();
      if constexpr (sizeof(IT) == 2) {
        const u32x4 rsrc = raw_buffer_rsrc(reinterpret_cast<const char*>(src) + (size_t)k0 * C::ROWB,
                                           (unsigned)max(kv_end - k0, 0) * C::ROWB);
#pragma unroll
        for (int i = 0; i < C::SEGS_PER_WAVE; ++i)
          lds_dma16_buf(rsrc, which ? voff[i] : koff[i], lds_addr(dst + (w * C::SEGS_PER_WAVE + i) * 1024));
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
      serial_fence();
    };

    // Operand reads: K operand f = (half kb = f / QKS, k-step f % QKS) of the tile at byte
    // `ksl` of the K slots; V operand f = (k-step f / NB, block f % NB) of the tile at byte
    // `vs` of the V slots (two transposed 64-bit reads). Slot offsets are compile-time
    // constants, so they become immediate offsets of the LDS reads.
    auto read_k = [&](int ksl, int f) {
      return *reinterpret_cast<const bf16x8*>(smem + kaddr[f % C::QKS] + ksl + (f / C::QKS) * 32 * C::ROWB);
    };
    auto read_v = [&](int vs, int f) {
      const int ks = f / C::NB, nb = f % C::NB;
      const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + vaddr[nb] + vs + (16 * ks) * C::ROWB));
      const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + vaddr[nb] + vs + (16 * ks + 8) * C::ROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // S^T = K Q^T of the tile in K slot `ksl` into `sx`: each K operand feeds both row blocks.
    auto s_mfmas = [&](int ksl, f32x16 (&sx)[QB][2]) {
      const f32x16 zero = {};
      bf16x8 buf[kPF];
#pragma unroll
      for (int f = 0; f < kPF; ++f) buf[f] = read_k(ksl, f);
#pragma unroll
      for (int f = 0; f < C::NKF; ++f) {
        const bf16x8 x = buf[f % kPF];
        if (f + kPF < C::NKF) buf[f % kPF] = read_k(ksl, f + kPF);
        const int kb = f / C::QKS, ks = f % C::QKS;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sx[qb][kb] = mfma_32x32x16(x, qf[qb][ks], ks == 0 ? zero : sx[qb][kb]);
      }
    };
    // Mask of tile t (uniform branch; only boundary tiles). Accumulator element r of half kb
    // is key k0 + 4*half + (32*kb + 8*(r/4) + r%4) for query my_q[qb].
    auto mask_tile = [&](int t, f32x16 (&sx)[QB][2]) {
      const int k0 = kbase + t * C::BN;
      if (!((k0 + C::BN > n_kv) || (a.causal && k0 + C::BN - 1 > qw0 + delta) ||
            (WIN && k0 < qw0 + 32 * QB + delta - a.window)))
        return;  // uniform
      const int base = k0 + 4 * half;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // visible: lo <= (offset from base) < lim
        const int lim = min(n_kv - base, a.causal ? my_q[qb] + delta + 1 - base : n_kv - base);
        const int lo = WIN ? my_q[qb] + delta - a.window + 1 - base : -C::BN;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
            if (off >= lim || off < lo) sx[qb][kb][r] = kNegInf;
          }
      }
    };

    // First tile only: the row's reference m is its maximum (exact), then the shift
    // t = s * scale*log2(e) - m in place. A row that sees nothing keeps m = -inf and t = s.
    auto first_shift = [&](f32x16 (&sx)[QB][2]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mp[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], sx[qb][kb][r]);
        float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
        // lanes l and l ^ 32 hold the same row
        m[qb] = max_of_halves(mx) * a.scale_log2;
        nm[qb] = (m[qb] == kNegInf) ? 0.f : -m[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sx[qb][kb][r] = fmaf(sx[qb][kb][r], a.scale_log2, nm[qb]);
      }
    };
    // The two halves of a body, written out step by step. A region is one step per MFMA
    // operand: step f takes the operand read kPF steps earlier, issues the read for step
    // f + kPF, runs its MFMA(s) and a fixed slice of the softmax arithmetic. A scheduling
    // fence between steps keeps that order; left to itself the scheduler either reads each
    // operand just before its MFMA (a full LDS round trip per MFMA) or gathers the softmax
    // work into stretches with no MFMA beside them. `mid` runs at step kDmaStep (tile loads).

    // The exp work of a tile is split between the two regions so that both carry about the
    // same VALU load: region X takes elements [0, kExpX), region Y the rest (their operands
    // belong to the last P V k-steps, which region Y reaches only in its second half). At
    // d = 128 region X takes three quarters; at d = 64, whose regions have half the steps,
    // 20 of 32 (measured: 2.5-3% faster than 24 on B=4, L=2048; 18 did as well, 16 and 22
    // less). Accumulator element r of key half h of row block qb is element e = 32 qb + 16 h
    // + r; P^T operand 2 h + r / 8 (k-step) holds its elements r % 8.
    constexpr int kElems = 32 * QB;
    constexpr int kExpX = D == 64 ? 20 : kElems - kElems / 4;
    auto elem = [](const f32x16 (&x)[QB][2], int e) { return x[e / 32][(e % 32) / 16][e % 16]; };
    // Keep running sums where they are computed: without this, chains of adds are linearised
    // after the region's last MFMA, where nothing else overlaps them.
    auto pin_sums = [&] {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(lc[qb][i]));
    };
    // Row-sum add and bf16 P^T operand of element e, whose p is in pv[e].
    auto sum_elem = [&](const float (&pv)[kElems], int e) {
      const int qb = e / 32, h = (e % 32) / 16, r = e % 16;
      lc[qb][e & 1] += pv[e];
      pb[qb][2 * h + (r >> 3)][r & 7] = (__bf16)pv[e];
      if (e & 1) {
        // The pair (e - 1, e) is complete: convert it here, beside this step's MFMA, rather
        // than after the part's check (where nothing overlaps the conversions).
        u32x4 u = as_u32x4(pb[qb][2 * h + (r >> 3)]);
        unsigned wd = u[(r & 7) >> 1];
        asm volatile("" : "+v"(wd));
        u[(r & 7) >> 1] = wd;
        pb[qb][2 * h + (r >> 3)] = as_bf16x8(u);
      }
    };
    // The rows' sums as they stood before a part was added (kept for the rare rescale).
    auto snapshot = [&](float (&lo)[QB][2]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lo[qb][0] = lc[qb][0], lo[qb][1] = lc[qb][1];
    };

    // Softmax without a per-tile maximum. Scores are shifted by the row's current reference m
    // before anyone looks at the tile, p = 2^(s*scale*log2(e) - m) is formed and added to the
    // row sum, and only then is the part checked: it stands unless a chain of the row sum went
    // past kMaxL (or is not a number: some p overflowed), or, with a sliding window, the row
    // has no reference yet and the tile holds keys it can see. Otherwise (rare after a row's
    // first tile; a wave-uniform branch) the row's reference is raised to the part's maximum,
    // l and o are rescaled at once, and the part's p are recomputed. A chain at or below 2^40
    // bounds every p and l far from fp32 overflow, and its test costs two compares per part.
    // Elements [E0, E1) of `cu` have been exponentiated (added to lc, which held `lo` before);
    // [E1, E2) are still to be, and are shifted along with them. Elements [EP, E0) belong to
    // an earlier part whose P^T operands are still waiting for their P V k-steps: a rescale
    // re-derives them against the new reference (o already holds the k-steps that ran, and
    // is rescaled). k0: the tile's first key.
    constexpr float kMaxL = 1099511627776.f;  // 2^40
    auto fix_part = [&](f32x16 (&cu)[QB][2], auto epc, auto e0c, auto e1c, auto e2c, const float (&lo)[QB][2],
                        int k0) {
      constexpr int EP = decltype(epc)::value, E0 = decltype(e0c)::value, E1 = decltype(e1c)::value,
                    E2 = decltype(e2c)::value;
      bool need[QB], any = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        need[qb] = !(lc[qb][0] <= kMaxL) || !(lc[qb][1] <= kMaxL);
        if constexpr (WIN) {
          // A row's first visible keys may all give p = 0 against the provisional shift of 0
          // (scores far below zero), so the test is on the keys, not on the sum.
          const int last = my_q[qb] + delta;  // the row's newest visible key
          need[qb] = need[qb] || (m[qb] == kNegInf && last - a.window + 1 < k0 + C::BN && last >= k0 && k0 < n_kv);
        }
        any |= need[qb];
      }
      if (__builtin_amdgcn_ballot_w64(any) == 0) return;  // the fast path holds for every row
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = kNegInf;
#pragma unroll
        for (int e = E0; e < E1; ++e)
          if (e / 32 == qb) mx = fmaxf(mx, elem(cu, e));
        // lanes l and l ^ 32 hold the same row: combine their halves
        mx = max_of_halves(mx);
        const bool row_need = any_of_halves(need[qb]) && mx != kNegInf;
        float d = 0.f, al = 1.f;
        if (row_need) {
          if (m[qb] == kNegInf) {  // first reference: the scores were shifted by 0; l, o are 0
            m[qb] = mx;
            d = mx;
            al = 0.f;
          } else if (mx > 0.f) {   // raise only: the scores were shifted by -m
            m[qb] += mx;
            d = mx;
            al = exp2_hw(-mx);
          }
          nm[qb] = -m[qb];
        }
        lc[qb][0] = lo[qb][0] * al;
        lc[qb][1] = lo[qb][1] * al;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][nb][r] *= al;
#pragma unroll
        for (int e = EP; e < E0; ++e) {
          if (e / 32 != qb) continue;
          const int h = (e % 32) / 16, r = e % 16;
          pb[qb][2 * h + (r >> 3)][r & 7] = (__bf16)exp2_hw(cu[qb][h][r] - d);
        }
#pragma unroll
        for (int e = E0; e < E2; ++e) {
          if (e / 32 != qb) continue;
          const int h = (e % 32) / 16, r = e % 16;
          cu[qb][h][r] -= d;
          if (e < E1) {
            const float pe = exp2_hw(cu[qb][h][r]);
            lc[qb][e & 1] += pe;
            pb[qb][2 * h + (r >> 3)][r & 7] = (__bf16)pe;
          }
        }
      }
    };

    // Region X: S^T of the next tile into `nx`, beside p = 2^t, the row sums and the bf16 P^T
    // operands of most of the current tile `cu` (whose scores were shifted in region Y), and
    // the check of that part.
    auto region_x = [&](int ksl, f32x16 (&nx)[QB][2], f32x16 (&cu)[QB][2], int k0, auto&& mid) {
      constexpr int NF = C::NKF;
      const f32x16 zero = {};
      float pv[kElems];  // p of element e, between its exp and its sum / conversion
      float lo[QB][2];
      snapshot(lo);
      bf16x8 buf[kPF];
#pragma unroll
      for (int f = 0; f < kPF; ++f) buf[f] = read_k(ksl, f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 x = buf[f % kPF];
        if (f + kPF < NF) buf[f % kPF] = read_k(ksl, f + kPF);
        const int kb = f / C::QKS, ks = f % C::QKS;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) nx[qb][kb] = mfma_32x32x16(x, qf[qb][ks], ks == 0 ? zero : nx[qb][kb]);
        // This step's exps; the sums and conversions of the previous step's (their results
        // are ready by now, so the wave does not stall on them).
#pragma unroll
        for (int e = (f - 1) * kExpX / NF; f > 0 && e < f * kExpX / NF; ++e) sum_elem(pv, e);
#pragma unroll
        for (int e = f * kExpX / NF; e < (f + 1) * kExpX / NF; ++e) pv[e] = exp2_hw(elem(cu, e));
        pin_sums();
        if (f == kDmaStep) mid();
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = (NF - 1) * kExpX / NF; e < kExpX; ++e) sum_elem(pv, e);
      fix_part(cu, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
               std::integral_constant<int, kExpX>{}, std::integral_constant<int, kElems>{}, lo, k0);
      pin_sums();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)  // operands completed here (the rest are written in region Y)
          if (32 * qb + 8 * i + 8 <= kExpX) asm volatile("" : "+v"(pb[qb][i]));
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // Region Y: O^T += V^T P^T of the current tile `cu` (V tile at byte `vs` of the V slots),
    // beside the rest of `cu`'s exp work and its check (first half of the steps), then
    // t = s * scale*log2(e) - m in place for the next tile `nx` (second half).
    auto region_y = [&](int vs, f32x16 (&nx)[QB][2], f32x16 (&cu)[QB][2], int k0, auto&& mid) {
      constexpr int NF = C::NVF;
      constexpr int NM = NF / 2;                       // steps of the leftover exps; the check
      constexpr int NS = NF - NM - 1;                  // steps of the shift
      constexpr int EPF = (32 * QB + NS - 1) / NS;     // elements per shift step
      constexpr int NE = kElems - kExpX;               // exp elements left over from region X
      // P^T operands not yet consumed when the leftover part is checked (operand i holds
      // elements 8 i .. 8 i + 7 and feeds k-step i, which starts at step i * NB)
      constexpr int kPend = 8 * (NM / C::NB);
      static_assert(QB == 1 && NM % C::NB == 0 && kPend <= kExpX, "pending operands of region X");
      float pv[kElems], lo[QB][2];
      snapshot(lo);
      bf16x8 buf[kPF];
#pragma unroll
      for (int f = 0; f < kPF; ++f) buf[f] = read_v(vs, f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        __builtin_amdgcn_sched_barrier(0);
        if (f == NM) {
          // The leftover part is complete: check it before the P V k-steps that read it.
#pragma unroll
          for (int e = kExpX + (NM - 1) * NE / NM; e < kElems; ++e) sum_elem(pv, e);
          fix_part(cu, std::integral_constant<int, kPend>{}, std::integral_constant<int, kExpX>{},
                   std::integral_constant<int, kElems>{}, std::integral_constant<int, kElems>{}, lo, k0);
          pin_sums();
          __builtin_amdgcn_sched_barrier(0);
        }
        const bf16x8 x = buf[f % kPF];
        if (f + kPF < NF) buf[f % kPF] = read_v(vs, f + kPF);
        const int ks = f / C::NB, nb = f % C::NB;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][nb] = mfma_32x32x16(x, pb[qb][ks], oacc[qb][nb]);
        if (f < NM) {
#pragma unroll
          for (int e = kExpX + (f - 1) * NE / NM; f > 0 && e < kExpX + f * NE / NM; ++e) sum_elem(pv, e);
#pragma unroll
          for (int e = kExpX + f * NE / NM; e < kExpX + (f + 1) * NE / NM; ++e) pv[e] = exp2_hw(elem(cu, e));
          pin_sums();
        } else if (f > NM) {
          const int s0 = (f - NM - 1) * EPF;
#pragma unroll
          for (int e = s0; e < s0 + EPF && e < kElems; ++e) {
            const int qb = e / 32, h = (e % 32) / 16, r = e % 16;
            nx[qb][h][r] = fmaf(nx[qb][h][r], a.scale_log2, nm[qb]);
          }
        }
        if (f == kDmaStep) mid();
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        asm volatile("" : "+v"(lc[qb][0]), "+v"(lc[qb][1]), "+v"(m[qb]), "+v"(nm[qb]));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+v"(nx[qb][kb]));
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // Tile j: region X = S of tile j + 1 beside the exp half of tile j's softmax; region Y =
    // P V of tile j beside the rest of tile j's exps and the shift of tile j + 1. Loads of K tile
    // j + 3 and V tile j + 2 stream in meanwhile. `uc` is j mod 6 as a compile-time constant (the
    // loop is unrolled six times, the period of the 3 slots and the 2 score buffers), which
    // makes every slot offset an immediate.
    // End of iteration j: wait for this wave's loads of K tile j + 2 and V tile j + 1 (issued
    // one iteration ago; the ones just issued may stay in flight), then the barrier makes
    // everyone's visible and frees the slots read in it.
    auto close_tile = [&](bool ld_k, bool ld_v) {
      if (ld_k && ld_v) wait_vmcnt<2 * C::SEGS_PER_WAVE>();
      else if (ld_k || ld_v) wait_vmcnt<C::SEGS_PER_WAVE>();
      else wait_vmcnt<0>();
      lds_barrier();
    };
    auto body = [&](auto uc, int j, f32x16 (&cur)[QB][2], f32x16 (&nxt)[QB][2]) {
      constexpr int u = decltype(uc)::value;
      constexpr int NS = C::NS;
      constexpr int ksl_next = ((u + 1) % NS) * C::TILE_BYTES;  // K slot of tile j + 1
      constexpr int vsl_cur = (u % NS) * C::TILE_BYTES;         // V slot of tile j
      // Keep the per-lane operand bases opaque to loop-invariant code motion: otherwise every
      // (base + immediate offset) pair is hoisted out of the loop into its own VGPR.
#pragma unroll
      for (int ks = 0; ks < C::QKS; ++ks) asm volatile("" : "+v"(kaddr[ks]));
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) asm volatile("" : "+v"(vaddr[nb]));
      // Loads two tiles ahead: K tile j + 3 (read by the S products of iteration j + 2) and V
      // tile j + 2 (read by the P V products of iteration j + 2), issued inside the regions
      // so that the workgroup's waves do not all queue on the load path at once. bf16 loads
      // are issued even past the last tile (they read nothing), which keeps the regions free
      // of branches; fp32 staging keeps its bounds.
      constexpr bool kAll = sizeof(IT) == 2;
      const bool ld_k = kAll || j + NS < ntk, ld_v = kAll || j + NS - 1 < ntk;
      auto load_k = [&] { if (ld_k) stage(j + NS, 0, (u % NS) * C::TILE_BYTES); };                 // tile j + NS
      auto load_v = [&] { if (ld_v) stage(j + NS - 1, 1, (NS + (u + NS - 1) % NS) * C::TILE_BYTES); };  // j + NS - 1
      __builtin_amdgcn_sched_barrier(0);
      const int k0 = kbase + j * C::BN;  // tile j's first key
      region_x(ksl_next, nxt, cur, k0, load_k);
      if (j + 1 < ntk) mask_tile(j + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      if (w >= C::NW / 2) __builtin_amdgcn_s_setprio(1);  // the wave that finished region X later goes first
      region_y(vsl_cur, nxt, cur, k0, load_v);
      __builtin_amdgcn_s_setprio(0);
      close_tile(ld_k, ld_v);
    };
    // A wave whose remaining tiles lie wholly past its rows (causal diagonal) computes nothing
    // more; it still moves its share of those tiles into LDS and meets every barrier.
    auto tail_body = [&](int j) {
      constexpr bool kAll = sizeof(IT) == 2;
      const bool ld_k = kAll || j + C::NS < ntk, ld_v = kAll || j + C::NS - 1 < ntk;
      if (ld_k) stage(j + C::NS, 0, k_slot(j + C::NS));
      if (ld_v) stage(j + C::NS - 1, 1, v_slot(j + C::NS - 1));
      close_tile(ld_k, ld_v);
    };

    if (ntk > 0) {
      // Zero the buffers at the start of every tile, so that operand reads of a slot or rows
      // not written for this tile (dummy work at the end of the pipeline, rows past kv_end)
      // see finite values.
      for (int i = tid; i < (int)sizeof(smem) / 16; i += C::NT) *reinterpret_cast<u32x4*>(smem + 16 * i) = u32x4{0u, 0u, 0u, 0u};
      // Only the LDS writes must be done before the loads land: a full __syncthreads() would
      // also wait for this wave's Q loads and put their latency before the K/V loads' own.
      lds_barrier();
      stage(0, 0, k_slot(0));
      stage(0, 1, v_slot(0));
      if (1 < ntk) stage(1, 0, k_slot(1));
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // Tiles the first iteration does not read yet, kept in flight: K tile 2 and V tile 1.
      if (2 < ntk) stage(2, 0, k_slot(2));
      if (1 < ntk) stage(1, 1, v_slot(1));
      s_mfmas(0, sa);
      mask_tile(0, sa);
      first_shift(sa);
      // The first body loads into K slot 0, which every wave has just read.
      lds_barrier();
      // Six bodies per trip, leaving after the body of the last tile this wave has keys in.
      using std::integral_constant;
      const int ntw = __builtin_amdgcn_readfirstlane(
          min(ntk, max((wave_last_key - kbase) / C::BN + 1, 1)));  // tiles with keys for this wave
      int j = 0;
      for (;; j += 6) {
        body(integral_constant<int, 0>{}, j, sa, sb);
        if (j + 1 >= ntw) { j += 1; break; }
        body(integral_constant<int, 1>{}, j + 1, sb, sa);
        if (j + 2 >= ntw) { j += 2; break; }
        body(integral_constant<int, 2>{}, j + 2, sa, sb);
        if (j + 3 >= ntw) { j += 3; break; }
        body(integral_constant<int, 3>{}, j + 3, sb, sa);
        if (j + 4 >= ntw) { j += 4; break; }
        body(integral_constant<int, 4>{}, j + 4, sa, sb);
        if (j + 5 >= ntw) { j += 5; break; }
        body(integral_constant<int, 5>{}, j + 5, sb, sa);
        if (j + 6 >= ntw) { j += 6; break; }
      }
      for (; j < ntk; ++j) tail_body(j);
      wait_vmcnt<0>();  // loads issued by the last bodies must land before the workgroup ends
    }

    // Epilogue: O = o / l and LSE = ln(2) * (m + log2 l); padding rows and rows that saw
    // no key get O = 0 and LSE = -inf. A bf16 O leaves through LDS: each wave puts its 32 x D
    // block there in the accumulator layout (8 bytes per lane, one row per lane), then stores
    // whole rows, 16 contiguous bytes per lane. Stored straight from the accumulators, every
    // store instruction would write 16 bytes into each of 32 rows, and the last wave of a tile
    // would spend several thousand cycles issuing them while the others wait for the next tile.
    constexpr bool kStaged = sizeof(OT) == 2;
    constexpr int RS = 2 * D + 16;  // bytes per staged row; the pad spreads the rows over the banks
    static_assert(!kStaged || C::NW * 32 * QB * RS <= (int)sizeof(smem), "staged O must fit in LDS");
    // Every wave has waited for its own loads, so once all have returned their last operand
    // reads LDS is free (an LDS-only barrier: the O stores need not wait for anything else).
    if constexpr (kStaged) lds_barrier();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lh = lc[qb][0] + lc[qb][1];
      const float lt = lh + __shfl_xor(lh, 32);
      const bool row_ok = (my_q[qb] < n_q) && (lt > 0.f);
      const float inv = row_ok ? 1.f / lt : 0.f;
      OT* const ob = static_cast<OT*>(a.o) + (size_t)(b * a.H + h) * a.Lq * D;  // this head's O
      char* const stage_o = smem + (w * QB + qb) * 32 * RS;                         // this block's rows
      if (kStaged || my_q[qb] < a.Lq) {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int d0 = 32 * nb + 8 * jj + 4 * half;
            float x0 = oacc[qb][nb][4 * jj + 0] * inv, x1 = oacc[qb][nb][4 * jj + 1] * inv;
            float x2 = oacc[qb][nb][4 * jj + 2] * inv, x3 = oacc[qb][nb][4 * jj + 3] * inv;
            if (!row_ok) x0 = x1 = x2 = x3 = 0.f;
            if constexpr (kStaged) Store4<OT>::store(reinterpret_cast<OT*>(stage_o + col * RS) + d0, x0, x1, x2, x3);
            else Store4<OT>::store(ob + (size_t)my_q[qb] * D + d0, x0, x1, x2, x3);
          }
      }
      if constexpr (kStaged) {
        constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
        for (int i = 0; i < 32 * CPR / 64; ++i) {
          const int idx = 64 * i + lane, r = idx / CPR, c = idx - r * CPR;
          const int row = qw0 + 32 * qb + r;
          const u32x4 val = *reinterpret_cast<const u32x4*>(stage_o + r * RS + 16 * c);
          if (row < a.Lq) *reinterpret_cast<u32x4*>(ob + (size_t)row * D + 8 * c) = val;
        }
      }
      if (my_q[qb] < a.Lq && half == 0)
        a.lse[(size_t)(b * a.H + h) * a.Lq + my_q[qb]] = row_ok ? (m[qb] + __log2f(lt)) * kLn2 : kNegInf;
    }
    // The next tile clears and refills the LDS buffers: every wave must be done with them (its
    // loads landed before the epilogue, its staged-O reads returned) first. The O stores may
    // still be in flight.
    lds_barrier();
  }
#endif
}

template <int D, typename IT, typename OT, bool WIN>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  using C = FwdCfg<D>;
  FwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.Lq = p.Lq; a.Lk = p.Lk;
  a.group = p.H / p.Hkv;
  a.ntq = (p.Lq + C::BM - 1) / C::BM;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.window = p.window;
  a.seqlens = p.seqlens;
  const long long nwg = (long long)a.ntq * p.B * p.H;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  a.nwg = (int)nwg;
  if (a.nwg == 0) return hipSuccess;
  a.order = make_tile_order(a.nwg, a.group * a.ntq);
  a.group_div = make_divisor(a.group);
  a.hkv_div = make_divisor(p.Hkv);
  // Dense inputs run on a persistent grid, one workgroup per compute unit: the hardware hands
  // workgroups to each XCD's shader engines in a fixed turn, so with one tile per workgroup a
  // compute unit that finishes early idles until its engine's turn comes round. Variable lengths
  // keep one workgroup per tile: their tiles' work is only known on the device, and the
  // hardware's dynamic dispatch balances it.
  const void* fn = reinterpret_cast<const void*>(&fwd_kernel<D, IT, OT, WIN>);
  const int P = p.seqlens == nullptr && sizeof(IT) == 2 ? persistent_programs(fn, C::NT) : 0;
  a.nprog = (P > 0 && a.nwg > P) ? P : a.nwg;
  void* args[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)a.nprog), dim3(C::NT), args, 0, stream);
}

}  // namespace

int persistent_programs(const void* kernel, int block_threads) {
  struct Entry {
    int dev;
    const void* kernel;
    int programs;
  };
  constexpr int kMaxEntries = 64;
  static std::mutex mu;
  static Entry cache[kMaxEntries];
  static int used = 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].dev == dev && cache[i].kernel == kernel) return cache[i].programs;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess) per_cu = 0;
  const int n = cus * per_cu;
  const int programs = n >= 8 ? n - n % 8 : 0;
  if (used < kMaxEntries) cache[used++] = Entry{dev, kernel, programs};
  return programs;
}

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.window > 0) {
    if (p.d == 64) return launch<64, __bf16, __bf16, true>(p, stream);
    return launch<128, __bf16, __bf16, true>(p, stream);
  }
  if (p.d == 64) return launch<64, __bf16, __bf16, false>(p, stream);
  return launch<128, __bf16, __bf16, false>(p, stream);
}

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  if (p.window > 0) return hipErrorInvalidValue;  // the fp32 entry point has no window
  if (p.d == 64) return launch<64, float, float, false>(p, stream);
  return launch<128, float, float, false>(p, stream);
}

}  // namespace fa
