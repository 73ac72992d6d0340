// fa_decode.hip — single-token decode over a long KV cache for gfx950 (MI355X).
//
// Decode has one query row per head and a long history of keys ("FlashAttention 与长上下文：
// 先分清三张账", section "Prefill 和 decode 是两类问题"): every step reads the whole KV cache
// once, so the kernel is bound by HBM bandwidth, not by the matrix cores. The keys of a
// request are cut into ranges; a workgroup produces the online-softmax state (m, l, o) of
// each of its ranges for the query heads that share a KV head, and a second kernel
// merges the range states of each (request, head) with the merge rule of
// "2.1 FlashAttention-2 的核心思想" §2.1.3 (rescale each state by exp(m_c - max m)).
//
// gfx950 mapping of the split kernel (one wave64 per workgroup):
//   * Every K and V byte of the chunk is loaded once, 16 bytes per lane per instruction,
//     and reused by up to 4 query heads of the GQA group (more heads are split over grid
//     slots of 4).
//   * Scores use v_mfma_f32_16x16x32_bf16 with K as the B operand straight from the
//     loaded registers (16 keys as columns) and the 4 query heads replicated 4 times over
//     the 16 A rows, so each lane ends up holding all 4 heads' scores of one key.
//   * Probabilities are passed through 512 bytes of LDS to the lanes holding the
//     matching V rows, and P V is accumulated in fp32 on the VALU (8 dims x 4 heads per
//     lane), so P is not rounded before the product.
//   * The chunk's K/V for the next 32 keys are loaded before the current 32 are used.
//   * K/V are read with non-temporal loads: each byte is used by exactly one workgroup, so
//     keeping it in the caches only evicts lines that are still wanted (measured: +4-7%).
//   * Caches longer than 2048 keys, without a window or with one of 2048 keys or more: a
//     balanced partition. The launch has one workgroup per split slot of the GPU (2048),
//     and each takes an equal run of the 32-key steps with visible keys of all (request, KV
//     head) units, cut where a unit ends. With fixed-size chunks, 2.6 chunks per slot left
//     some slots a whole chunk longer than others (measured: +11% K/V rate, contiguous or
//     paged, with or without a window).
//   * Otherwise chunks of 2048 keys, one workgroup each. With a window they are counted
//     from the one holding the window's first key and shortened (down to 512 keys) when
//     the window leaves too few to fill the GPU.
//   * Paged cache (PagedAttention's layout, which the same page names): position j of a
//     request is row j % P of page table[j / P] of a pool [pages, Hkv, P, d]. With P a power
//     of two >= 16, each 16-key half of a step lies in one page. A workgroup holds the page
//     numbers of up to 128 pages (two per lane; a balanced run reloads them when it moves
//     past them) and takes each step's page with a uniform readlane, so the K/V loads stay
//     16-byte row loads.
#include <mutex>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kHeadsPerPass = 4;
constexpr int kKeysPerStep = 32;
constexpr int kDecodeChunkShift = 11;        // kDecodeChunk keys: the workspace's slot unit
constexpr int kDecodeMinChunkShift = 9;      // shortest chunk a sliding window may use
constexpr long long kDecodeTargetWG = 4096;  // split workgroups that fill the GPU
constexpr int kBalancedWG = 2048;            // split slots of the GPU: 256 CUs x 4 SIMDs x 2 waves
static_assert((1 << kDecodeChunkShift) == kDecodeChunk, "workspace slots are kDecodeChunk keys");

struct DecArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int B, H, Hkv, Lmax;
  int group;   // H / Hkv
  int nsg;     // head slots of 4 per KV head
  int nchunk;  // workspace slots per (request, head): chunks of kDecodeChunk keys at capacity
  int cshift;  // log2 of the keys per chunk of this launch (kDecodeChunk, or less for short windows)
  float scale_log2;
  int window;  // sliding window W (0: none): the last W keys of the context
  const int32_t* ctx;
  const int32_t* table;  // paged cache: [B, max_pages] page of each P-key span
  int page_shift;        // log2(P)
  int max_pages;
  int num_pages;
  float* ws_o;
  float* ws_ml;
  int nwg;   // balanced partition: split workgroups of the launch
  int qmin;  // balanced partition: fewest 32-key steps per workgroup (keeps slots < nchunk)
};

// Visible keys of request b: [first, n), first > 0 only with a sliding window.
__device__ __forceinline__ int decode_ctx(const DecArgs& a, int b) { return min(max(a.ctx[b], 0), a.Lmax); }
__device__ __forceinline__ int decode_first_key(const DecArgs& a, int n) {
  return a.window > 0 ? max(n - a.window, 0) : 0;
}
// 32-key steps of request b that hold visible keys: from the one holding its first visible
// key to the one holding its last (0 for an empty context or b >= B).
__device__ __forceinline__ int decode_steps(const DecArgs& a, int b) {
  if (b >= a.B) return 0;
  const int n = decode_ctx(a, b);
  return n > 0 ? (n + kKeysPerStep - 1) / kKeysPerStep - decode_first_key(a, n) / kKeysPerStep : 0;
}

// A value every lane holds alike, moved to scalar registers.
__device__ __forceinline__ long long wave_uniform(long long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Balanced partition of a decode. The 32-key steps with visible keys of all (request, KV
// head, head slot) units, taken in that order, form one sequence of T steps; workgroup w
// takes steps [w Qs, (w + 1) Qs), Qs = max(ceil(T / nwg), qmin), cut at unit boundaries
// into segments. Every workgroup then reads the same number of K/V bytes, where a grid of
// fixed-size chunks leaves some slots one whole chunk longer than others. A segment of
// unit u is partial slot w - floor(S_u / Qs) of u, S_u being u's first step; qmin bounds
// that slot below nchunk. Both kernels derive T and Qs from the same context lengths, so
// they agree on the slots. (T < 2^31: the launch checks units x steps per unit.)
__device__ __forceinline__ long long decode_total_steps(const DecArgs& a, int lane) {
  long long tot = 0;
  for (int c = 0; c < a.B; c += 64) {
    int s = decode_steps(a, c + lane);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off);
    tot += s;
  }
  return wave_uniform(tot * (a.Hkv * a.nsg));
}
__device__ __forceinline__ long long decode_quota(const DecArgs& a, long long T) {
  return max(max((T + a.nwg - 1) / a.nwg, (long long)a.qmin), 1LL);
}

template <int D, bool PAGED, bool BAL>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecArgs a) {
  constexpr int NCH = D / 8;            // 16-byte chunks per row
  constexpr int VKPL = 64 / NCH;        // keys per V load instruction
  constexpr int VLOADS = kKeysPerStep / VKPL;
  constexpr int QS = D / 32;            // 16x16x32 k-steps over d
  __shared__ __attribute__((aligned(16))) float pl[kKeysPerStep][kHeadsPerPass];

  const int lane = threadIdx.x;
  const int HN = a.Hkv * a.nsg;  // units per request
  int b, kvh, sg, n, w0, c0, c1, k_start, slot;
  // balanced partition: this workgroup's steps [pos, end), the current unit (request b,
  // unit pr of it, sb steps, first step R + pr sb) and the step st within it
  long long pos = 0, end = 0, R = 0, Qs = 1;
  int pr = 0, sb = 0, st = 0;
  if constexpr (!BAL) {
    const int chunk = blockIdx.y;
    const int x = blockIdx.x;  // (b, kvh, head slot group)
    sg = x % a.nsg;
    const int bk = x / a.nsg;
    b = bk / a.Hkv;
    kvh = bk - b * a.Hkv;
    n = min(max(a.ctx[b], 0), a.Lmax);
    w0 = a.window > 0 ? max(n - a.window, 0) : 0;  // first visible key
    // Chunks of 2^cshift keys, counted from the one holding the first visible key (chunk 0
    // of the cache without a window); `chunk` is also the workspace slot.
    c0 = ((w0 >> a.cshift) + chunk) << a.cshift;
    c1 = min(n, c0 + (1 << a.cshift));
    if (c0 >= n || c1 <= w0) return;  // chunk outside the visible keys: nothing to write
    // First step: the 32-key step that holds the first visible key of the chunk, so every
    // step holds at least one visible key; keys of that step before the window are neither
    // loaded (zeros instead) nor counted (score -inf).
    k_start = c0 + ((max(w0, c0) - c0) & ~(kKeysPerStep - 1));
    slot = chunk;
  } else {
    const long long T = decode_total_steps(a, lane);
    Qs = decode_quota(a, T);
    pos = (long long)blockIdx.x * Qs;
    end = min(pos + Qs, T);
    if (pos >= end) return;
    // the request holding step pos: the first whose units end after it
    b = -1;
    for (int c = 0; c < a.B && b < 0; c += 64) {
      const long long sz = (long long)decode_steps(a, c + lane) * HN;
      long long incl = sz;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const long long y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(R + incl > pos);
      if (hit != 0) {
        const int j = (int)__builtin_ctzll(hit);
        b = c + j;
        R += wave_uniform(__shfl(incl - sz, j));
      } else {
        R += wave_uniform(__shfl(incl, 63));
      }
    }
    if (b < 0) return;  // not reached: pos < T
    sb = decode_steps(a, b);
    const long long local = pos - R;
    pr = (int)(local / sb);
    st = (int)(local - (long long)pr * sb);
  }
  for (;;) {
    int seg = 0;
    if constexpr (BAL) {
      seg = (int)min((long long)(sb - st), end - pos);
      kvh = pr / a.nsg;
      sg = pr - kvh * a.nsg;
      n = decode_ctx(a, b);
      w0 = decode_first_key(a, n);
      // the unit's steps start at the one holding w0; keys of it before w0 are masked
      const int s0 = w0 / kKeysPerStep;
      c0 = (s0 + st) * kKeysPerStep;
      k_start = c0;
      c1 = min(n, (s0 + st + seg) * kKeysPerStep);
      slot = (int)((long long)blockIdx.x - (R + (long long)pr * sb) / Qs);
    }
    const int h0 = kvh * a.group + sg * kHeadsPerPass;
    const int nh = min(kHeadsPerPass, a.group - sg * kHeadsPerPass);

    // Rows of the 16 keys from kb0 (a multiple of 16): contiguous cache, or the page that
    // holds them. Paged: this lane holds page numbers first + lane and first + 64 + lane of the
    // chunk (clamped into the pool, so a bad table cannot address outside it).
    // A balanced segment may span more than 128 pages: its page numbers are then reloaded,
    // 128 at a time, before the step that first needs the next ones.
    int pg_lo = 0, pg_hi = 0, first = 0;
    const int npc = BAL ? 128 : max((1 << a.cshift) >> a.page_shift, 1);  // pages held, <= 128
    auto load_pages = [&](int f) {
      first = f;
      pg_lo = pg_hi = 0;
      const int32_t* row = a.table + (size_t)b * a.max_pages;
      if (lane < npc && f + lane < a.max_pages) pg_lo = min(max(row[f + lane], 0), a.num_pages - 1);
      if (64 + lane < npc && f + 64 + lane < a.max_pages) pg_hi = min(max(row[f + 64 + lane], 0), a.num_pages - 1);
    };
    if constexpr (PAGED) load_pages(c0 >> a.page_shift);
    auto rows_at = [&](const __bf16* base, int kb0) -> const __bf16* {
      if constexpr (PAGED) {
        const int cp = (kb0 >> a.page_shift) - first;  // chunk-relative page, uniform
        const int page = cp < 64 ? __builtin_amdgcn_readlane(pg_lo, cp) : __builtin_amdgcn_readlane(pg_hi, cp - 64);
        const int in_page = kb0 & ((1 << a.page_shift) - 1);
        return base + ((size_t)(page * a.Hkv + kvh) * ((size_t)1 << a.page_shift) + in_page) * D;
      } else {
        return base + ((size_t)(b * a.Hkv + kvh) * a.Lmax + kb0) * D;
      }
    };

    // A operand: row r = lane % 16 is head slot r % 4; element t of k-step s is d = 32 s + 8 (lane / 16) + t.
    const int slot_a = (lane & 15) & 3;
    bf16x8 qa[QS];
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (slot_a < nh) u = *reinterpret_cast<const u32x4*>(a.q + (size_t)(b * a.H + h0 + slot_a) * D + 32 * s + 8 * (lane >> 4));
      qa[s] = as_bf16x8(u);
    }

    // K as the B operand: column = key k0 + 16 blk + lane % 16, same d mapping as the A operand.
    // V rows for the VALU product: load i covers key k0 + i * VKPL + lane / NCH, dims 8 * (lane % NCH) .. +8.
    const int vkey = lane / NCH;
    const int vch = lane - vkey * NCH;
    u32x4 kr[2][QS], vr[VLOADS];
    auto load_step = [&](int k0) {
      const __bf16* kb[2] = {rows_at(a.k, k0), rows_at(a.k, k0 + 16)};
      const __bf16* vb[2] = {rows_at(a.v, k0), rows_at(a.v, k0 + 16)};
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int key = k0 + 16 * blk + (lane & 15);
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          u32x4 u = {0u, 0u, 0u, 0u};
          if (key < c1 && key >= w0)
            u = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(kb[blk] + (size_t)(lane & 15) * D + 32 * s + 8 * (lane >> 4)));
          kr[blk][s] = u;
        }
      }
#pragma unroll
      for (int i = 0; i < VLOADS; ++i) {
        const int off = i * VKPL + vkey;  // key offset within the step
        const int key = k0 + off;
        u32x4 u = {0u, 0u, 0u, 0u};
        if (key < c1 && key >= w0)
          u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb[off >> 4] + (size_t)(off & 15) * D + 8 * vch));
        vr[i] = u;
      }
    };

    float m[kHeadsPerPass], lp[kHeadsPerPass], o[kHeadsPerPass][8];
#pragma unroll
    for (int i = 0; i < kHeadsPerPass; ++i) {
      m[i] = kNegInf;
      lp[i] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
    }

    load_step(k_start);
    for (int k0 = k_start; k0 < c1; k0 += kKeysPerStep) {
      // Scores for 32 keys: accumulator element i is head slot i, key k0 + 16 blk + lane % 16.
      f32x4 sc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        sc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < QS; ++s) sc[blk] = mfma_16x16x32(qa[s], as_bf16x8(kr[blk][s]), sc[blk]);
      }
      u32x4 vcur[VLOADS];
#pragma unroll
      for (int i = 0; i < VLOADS; ++i) vcur[i] = vr[i];
      if (k0 + kKeysPerStep < c1) {  // prefetch the next 32 keys
        if constexpr (PAGED && BAL) {
          // loads already issued do not depend on the page numbers any more
          const int nk = k0 + kKeysPerStep;
          if (((nk + kKeysPerStep - 1) >> a.page_shift) - first >= npc) load_pages(nk >> a.page_shift);
        }
        load_step(k0 + kKeysPerStep);
      }

#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int key = k0 + 16 * blk + (lane & 15);
        if (key >= c1 || key < w0) sc[blk] = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
      }

      float p[2][kHeadsPerPass];
#pragma unroll
      for (int i = 0; i < kHeadsPerPass; ++i) {
        float mx = fmaxf(sc[0][i], sc[1][i]);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float m_new = fmaxf(m[i], mx * a.scale_log2);  // finite: every step has a visible key
        const float alpha = exp2_hw(m[i] - m_new);
        p[0][i] = exp2_hw(fmaf(sc[0][i], a.scale_log2, -m_new));
        p[1][i] = exp2_hw(fmaf(sc[1][i], a.scale_log2, -m_new));
        lp[i] = lp[i] * alpha + p[0][i] + p[1][i];
        m[i] = m_new;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
      }

      __syncthreads();  // the previous step's reads of pl are complete
      if (lane < 16) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          *reinterpret_cast<f32x4*>(&pl[16 * blk + lane][0]) = f32x4{p[blk][0], p[blk][1], p[blk][2], p[blk][3]};
      }
      __syncthreads();

#pragma unroll
      for (int i = 0; i < VLOADS; ++i) {
        const f32x4 pp = *reinterpret_cast<const f32x4*>(&pl[i * VKPL + vkey][0]);
        float vf[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vf[2 * j] = bf16_bits_lo(vcur[i][j]);
          vf[2 * j + 1] = bf16_bits_hi(vcur[i][j]);
        }
#pragma unroll
        for (int hs = 0; hs < kHeadsPerPass; ++hs)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[hs][e] = fmaf(pp[hs], vf[e], o[hs][e]);
      }
    }

    // Reduce the partial sums: o over the lanes holding the same dims, l over the 16 key lanes.
#pragma unroll
    for (int hs = 0; hs < kHeadsPerPass; ++hs) {
#pragma unroll
      for (int off = NCH; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hs][e] += __shfl_xor(o[hs][e], off);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) lp[hs] += __shfl_xor(lp[hs], off);
    }
    if (lane < NCH) {
#pragma unroll
      for (int hs = 0; hs < kHeadsPerPass; ++hs) {
        if (hs < nh) {
          float* dst = a.ws_o + ((size_t)(b * a.H + h0 + hs) * a.nchunk + slot) * D + 8 * lane;
          *reinterpret_cast<f32x4*>(dst) = f32x4{o[hs][0], o[hs][1], o[hs][2], o[hs][3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[hs][4], o[hs][5], o[hs][6], o[hs][7]};
          if (lane == 0) {
            float* ml = a.ws_ml + ((size_t)(b * a.H + h0 + hs) * a.nchunk + slot) * 2;
            ml[0] = m[hs];
            ml[1] = lp[hs];
          }
        }
      }
    }
    if constexpr (!BAL) {
      break;
    } else {
      // next segment: the rest of this unit, else the next unit, else the next request
      // with keys
      pos += seg;
      if (pos >= end) break;
      st += seg;
      if (st == sb) {
        st = 0;
        if (++pr == HN) {
          pr = 0;
          R += (long long)sb * HN;
          do ++b; while (b < a.B && decode_steps(a, b) == 0);
          if (b >= a.B) break;  // not reached: pos < T
          sb = decode_steps(a, b);
        }
      }
    }
  }
}

// Merge the chunk states of one (request, head): M = max m_c, L = sum 2^(m_c - M) l_c,
// O = sum 2^(m_c - M) o_c / L, LSE = ln(2) (M + log2 L). One wave per (request, head).
template <int D, bool BAL>
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecArgs a) {
  constexpr int PER = D / 64;  // dims per lane
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int n = min(max(a.ctx[b], 0), a.Lmax);
  int nc;
  if constexpr (!BAL) {
    // Slots 0 .. nc - 1 hold the chunks from the one with the first visible key to the last.
    const int w0 = a.window > 0 ? max(n - a.window, 0) : 0;
    nc = ((n + (1 << a.cshift) - 1) >> a.cshift) - (w0 >> a.cshift);
  } else {
    // Slots 0 .. nc - 1 hold the segments of this head's unit, in key order: one per
    // workgroup its steps [S, S + sb) meet.
    const long long T = decode_total_steps(a, lane);
    const long long Qs = decode_quota(a, T);
    long long before = 0;  // steps of the requests before b, per unit
    for (int c = 0; c < b; c += 64) {
      int s = c + lane < b ? decode_steps(a, c + lane) : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off);
      before += s;
    }
    const int h = bh - b * a.H, kvh = h / a.group;
    const int pr = kvh * a.nsg + (h - kvh * a.group) / kHeadsPerPass;
    const int sb = decode_steps(a, b);
    const long long S = before * (a.Hkv * a.nsg) + (long long)pr * sb;
    nc = sb == 0 ? 0 : (int)((S + sb - 1) / Qs - S / Qs + 1);
  }
  const float* ml = a.ws_ml + (size_t)bh * a.nchunk * 2;
  const float* wo = a.ws_o + (size_t)bh * a.nchunk * D;

  float M = kNegInf;
  for (int c = lane; c < nc; c += 64) M = fmaxf(M, ml[2 * c]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));

  float L = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float wgt = exp2_hw(ml[2 * c] - M);
    L += wgt * ml[2 * c + 1];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(wgt, wo[(size_t)c * D + PER * lane + e], acc[e]);
  }
  const bool ok = nc > 0 && L > 0.f;
  const float inv = ok ? 1.f / L : 0.f;
  __bf16* op = a.o + (size_t)bh * D + PER * lane;
#pragma unroll
  for (int e = 0; e < PER; ++e) op[e] = (__bf16)(ok ? acc[e] * inv : 0.f);
  if (lane == 0) a.lse[bh] = ok ? (M + __log2f(L)) * kLn2 : kNegInf;
}

template <int D, bool PAGED>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  DecArgs a;
  a.q = static_cast<const __bf16*>(p.q);
  a.k = static_cast<const __bf16*>(p.k);
  a.v = static_cast<const __bf16*>(p.v);
  a.o = static_cast<__bf16*>(p.o);
  a.lse = p.lse;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.Lmax = p.Lmax;
  a.group = p.H / p.Hkv;
  a.nsg = (a.group + kHeadsPerPass - 1) / kHeadsPerPass;
  a.nchunk = decode_num_chunks(p.Lmax);
  // Chunk size: kDecodeChunk keys, or less when a sliding window leaves so few chunks per
  // request that the grid would not fill the GPU (at least kDecodeTargetWG workgroups, as long
  // as the window's chunks still fit the workspace's slots).
  const long long nx = (long long)p.B * p.Hkv * a.nsg;
  int ny = a.nchunk;
  a.cshift = kDecodeChunkShift;
  if (p.window > 0) {
    for (int s = kDecodeChunkShift; s >= kDecodeMinChunkShift; --s) {
      const long long cs = 1LL << s;
      const long long span = (p.window + cs - 1) / cs + 1, cap = (p.Lmax + cs - 1) / cs;
      const long long nys = span < cap ? span : cap;
      if (nys > a.nchunk) break;
      a.cshift = s;
      ny = (int)nys;
      if (nx * nys >= kDecodeTargetWG) break;
    }
  }
  a.scale_log2 = p.scale * kLog2e;
  a.ctx = p.ctx_lens;
  a.window = p.window;
  a.table = p.table;
  a.page_shift = 0;
  while (PAGED && (1 << a.page_shift) < p.page_size) ++a.page_shift;
  a.max_pages = p.max_pages;
  a.num_pages = p.num_pages;
  a.ws_o = p.ws_o;
  a.ws_ml = p.ws_ml;
  // Balanced partition: qmin steps per workgroup keep a unit's segments, at most
  // ceil((smax - 1) / Qs) + 1 of them, within its nchunk slots; smax bounds a unit's steps
  // (a window of W keys meets at most ceil(W / 32) + 1 of them).
  long long smax = (p.Lmax + kKeysPerStep - 1) / kKeysPerStep;
  const long long wsteps = ((long long)p.window + kKeysPerStep - 1) / kKeysPerStep + 1;
  if (p.window > 0 && wsteps < smax) smax = wsteps;
  // Windows shorter than a chunk keep the chunk grid, whose chunks shorten to fill the GPU:
  // at a 1024-key window the balanced runs (288 keys) were 6% slower; at 2048 and more
  // keys they were 10-12% faster.
  const bool bal = a.nchunk >= 2 && nx * smax < 0x7fffffffLL && (p.window == 0 || p.window >= kDecodeChunk);
  a.nwg = kBalancedWG;
  a.qmin = bal ? (int)((smax - 1 + a.nchunk - 2) / (a.nchunk - 1)) : 1;  // bal: nchunk >= 2
  void* args[] = {&a};
  hipError_t e = hipSuccess;
  const long long nbh = (long long)p.B * p.H;
  if (nbh > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (bal) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_split_kernel<D, PAGED, true>), dim3(kBalancedWG),
                        dim3(64), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_combine_kernel<D, true>), dim3((unsigned)nbh),
                           dim3(64), args, 0, stream);
  }
  if (ny > 0) {
    if (nx > 0x7fffffffLL || ny > 65535) return hipErrorInvalidConfiguration;
    e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_split_kernel<D, PAGED, false>), dim3((unsigned)nx, ny),
                        dim3(64), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_combine_kernel<D, false>), dim3((unsigned)nbh),
                         dim3(64), args, 0, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.table != nullptr) return p.d == 64 ? launch_d<64, true>(p, stream) : launch_d<128, true>(p, stream);
  return p.d == 64 ? launch_d<64, false>(p, stream) : launch_d<128, false>(p, stream);
}

// The decode workspace of fa_decode_noalloc: a fixed device array, one copy per GPU, held for
// the life of the process. Its name is only a host-side handle; the kernels get its device
// address, looked up once per device (with that device current) and kept.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fa
