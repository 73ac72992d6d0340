/*
 * fa.h — C ABI of libfa: exact scaled-dot-product attention on AMD MI355X (gfx950).
 *
 * What every entry point computes. For one (batch b, query head h):
 *
 *     O = softmax((Q K^T + M) * scale) V,   LSE_i = ln sum_j exp(((Q K^T + M) * scale)_ij)
 *
 * following "FlashAttention 与长上下文：先分清三张账" (charles2530.github.io),
 * section "标准 attention 的问题不只在 FLOPs" (the equation for O, with M a causal or
 * padding mask), and the same page's section "FlashAttention 的关键是 online softmax"
 * (running max / sum / unnormalised output per query row, O = o / l at the end, and
 * the small per-row statistics kept for a backward pass, emitted here as LSE).
 * The tensors use the [batch, heads, n, d] layout of "2.1 FlashAttention-2 的核心思想"
 * (aiknowledge.cn) §2.1.1. M takes only the values 0 and -inf:
 *   - causal: key j is visible to query i iff j <= i + (Lk - Lq) (queries are the
 *     newest positions; with Lq == Lk this is the usual lower triangle);
 *   - padding: with per-sequence lengths n_b, keys j >= n_b are hidden and query
 *     rows i >= n_b are padding, for which O = 0 and LSE = -inf are written.
 * A query row that sees no key gets O = 0 and LSE = -inf (never NaN).
 * Query head h reads KV head h / (H / Hkv) (grouped-query attention; contiguous groups).
 *
 * Conventions shared by every entry point:
 *   - Pointers to tensors are DEVICE pointers (HIP device memory) owned by the caller;
 *     the library never allocates, frees or synchronises on a call.
 *   - Tensors are dense, row-major, with d innermost; every tensor pointer must be
 *     16-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *     call returns at once. Errors in arguments are detected on the host before
 *     anything is enqueued, so a failing call writes nothing. Faults during execution
 *     surface at the caller's next synchronisation.
 *   - Device-resident lengths (seqlens, ctx_lens) cannot be checked without a
 *     synchronisation; the kernels clamp each to [0, capacity].
 *   - Head dimensions 64 and 128 are supported; any other d returns
 *     FA_ERR_UNSUPPORTED (never a slower fallback path).
 *   - Calls are reentrant; the library has no global mutable state, except the fixed
 *     workspace of fa_decode_noalloc (see there).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID = 1,     /* a null/misaligned pointer, a negative size, H % Hkv != 0, ... */
  FA_ERR_UNSUPPORTED = 2, /* valid request this library does not implement (e.g. d = 96) */
  FA_ERR_HIP = 3,         /* the HIP runtime refused the launch */
  FA_ERR_TOO_LARGE = 4    /* fa_decode_noalloc: the call needs more than its fixed workspace */
} fa_status;

/*
 * fa_fwd — prefill / self-attention forward, bf16 in, bf16 out, fp32 accumulation.
 *
 *   q   : bf16 [B, H,   Lq, d]     k, v : bf16 [B, Hkv, Lk, d]
 *   o   : bf16 [B, H,   Lq, d]     lse  : fp32 [B, H, Lq] (natural log)
 *   scale  : multiplies Q K^T (usually 1/sqrt(d)); must be finite and > 0.
 *   causal : 0 or 1 (bottom-right aligned, see above).
 *   seqlens: NULL, or device int32 [B] of per-sequence valid lengths; allowed only
 *            when Lq == Lk (one length covers both query rows and keys).
 *   B, H, Lq == 0 is a valid empty call (nothing is enqueued). Lk == 0 writes O = 0 and
 *   LSE = -inf. Requirements: B, H, Hkv, Lq, Lk >= 0, Hkv >= 1, H % Hkv == 0.
 * The score and probability matrices are never written to memory; the call needs no
 * workspace.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Hkv, int Lq, int Lk, int d, float scale, int causal,
                 const int32_t* seqlens, void* stream);

/*
 * fa_fwd_sliding_window — fa_fwd with the causal mask cut to a sliding window:
 * "FlashAttention 与长上下文：先分清三张账", in its section on prefill and decode,
 * lists the sliding window among the methods that trim the context. Read here as
 * the causal band of width `window`: key j is visible to query i iff
 *     i + (Lk - Lq) - window < j <= i + (Lk - Lq)
 * (and j < n_b with seqlens), so each query sees at most the `window` newest keys,
 * its own position included. window >= 1 (else FA_ERR_INVALID); the mask is always
 * causal. Key tiles wholly before a query tile's band are never read. Everything else
 * (arguments, layouts, ownership, errors) is as for fa_fwd with causal = 1.
 */
fa_status fa_fwd_sliding_window(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Hkv, int Lq, int Lk, int d, float scale, int window,
                                const int32_t* seqlens, void* stream);

/*
 * fa_fwd_fp8 — prefill forward on FP8 operands (d = 128 only; other d: FA_ERR_UNSUPPORTED).
 * The low-precision step of FlashAttention-3 ("FlashAttention 与长上下文：先分清三张账",
 * section on FlashAttention-2/3), whose scaling the pages leave open. The scheme read here:
 *   q : E4M3 codes [B, H, Lq, 128]    k, v : E4M3 codes [B, Hkv, Lk, 128]  (OCP E4M3FN bytes)
 *   q_descale : device fp32 [B, H]; k_descale, v_descale : device fp32 [B, Hkv];
 *               the attended values are decode(code) * descale of their (batch, head).
 *   o : bf16 [B, H, Lq, 128]          lse : fp32 [B, H, Lq] (natural log)
 * Scores come from the FP8 matrix cores (exact products, fp32 sums). Each row keeps an
 * integer base-2 reference m >= every score seen; probabilities relative to it, times 2^8,
 * enter the P V product rounded to E4M3 (nearest even) while the row sum l adds them
 * unrounded; O = descale_v * (sum_j E4M3(2^8 p_j) v_j) / (2^8 l). The result does not depend
 * on the tiling. causal, seqlens as for fa_fwd; window = 0 for none, or a sliding window
 * W >= 1 (needs causal = 1) as in fa_fwd_sliding_window. The call needs no workspace.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                     const float* v_descale, void* o, float* lse, int B, int H, int Hkv, int Lq, int Lk, int d,
                     float scale, int causal, int window, const int32_t* seqlens, void* stream);

/*
 * fa_fwd_f32 — the same contract with fp32 q, k, v and fp32 o. The kernel rounds
 * q, k, v to bf16 (round-to-nearest-even) as it loads them and multiplies them on the
 * bf16 matrix cores with fp32 accumulation; O and LSE are produced in fp32.
 */
fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int B, int H, int Hkv, int Lq, int Lk, int d, float scale, int causal,
                     const int32_t* seqlens, void* stream);

/*
 * fa_decode_workspace_bytes — bytes of device workspace fa_decode needs for a cache of
 * capacity Lmax (the split partials: one (max, sum, d-vector) of fp32 per query head and
 * 2048-key chunk, i.e. B * H * ceil(Lmax / 2048) * (d + 2) * 4 bytes). Returns 0 for
 * invalid sizes.
 */
size_t fa_decode_workspace_bytes(int B, int H, int Lmax, int d);

/*
 * fa_decode — one new query token per request against a long KV cache (Lq = 1).
 *
 *   q        : bf16 [B, H, d]             k_cache, v_cache : bf16 [B, Hkv, Lmax, d]
 *   o        : bf16 [B, H, d]             lse              : fp32 [B, H]
 *   ctx_lens : device int32 [B]; request b attends to cache positions 0 .. ctx_lens[b]-1
 *              (all of them: the new token is the newest position).
 *   workspace: device memory of at least fa_decode_workspace_bytes(B, H, Lmax, d) bytes,
 *              16-byte aligned, owned by the caller; its contents are scratch.
 * The keys are split into ranges; one kernel computes each range's partial (max, sum,
 * unnormalised output) and a second merges the partials of a row with the two-state merge
 * rule of "2.1 FlashAttention-2 的核心思想" §2.1.3 into O and LSE. With Lmax > 2048 the
 * ranges balance the whole call's keys over the GPU (equal runs of 32-key steps per
 * workgroup, from the device-side lengths; the split depends on Lmax as well as on the
 * lengths), otherwise they are 2048-key chunks; the split changes the result only by the
 * rounding of the merge.
 * Requirements: B, H >= 0 (0 = empty call), Hkv >= 1, H % Hkv == 0, Lmax >= 0.
 */
fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                    int B, int H, int Hkv, int Lmax, int d, float scale, const int32_t* ctx_lens,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc — fa_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. It takes no
 * workspace argument and calls no allocating routine (no hipMalloc / hipFree): the split
 * partials go to a fixed device array inside the library, one per GPU, of
 * FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES (32 MiB), held by each GPU the library runs on until
 * the process ends. Its device address is looked up once per device, on that device's first
 * call. Everything else (arguments, layouts, results, errors) is as for fa_decode; the
 * results are bit for bit those of fa_decode with a caller workspace.
 *   - A call whose fa_decode_workspace_bytes(B, H, Lmax, d) exceeds the fixed size returns
 *     FA_ERR_TOO_LARGE and enqueues nothing (the 64-request, 32k-context workload of
 *     32 query heads needs 16.25 MiB).
 *   - Every call on a GPU shares that GPU's array, which keeps the last call's partials.
 *     Nothing in it needs to start at zero: a call writes every partial it later reads.
 *   - Calls that may run at the same time on one GPU (on different streams, or from
 *     different threads without ordering) race on the array and give wrong results; order
 *     them (one stream, or events between streams).
 */
#define FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)32 << 20)
fa_status fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                            int B, int H, int Hkv, int Lmax, int d, float scale, const int32_t* ctx_lens,
                            void* stream);

/*
 * fa_decode_sliding_window — fa_decode with a sliding window (reading as for
 * fa_fwd_sliding_window): request b attends to cache positions
 * max(0, ctx_lens[b] - window) .. ctx_lens[b] - 1 only. Keys before that range are
 * neither read nor merged. A window of 2048 keys or more (with Lmax > 2048) takes the
 * balanced ranges of fa_decode, counted from each request's first visible key. A shorter
 * window takes 2048-key chunks counted from the one holding the window's first key,
 * shortened (down to 512 keys) when they would be too few to fill the GPU. The split
 * changes the result only by the rounding of the merge. window >= 1, else FA_ERR_INVALID;
 * the workspace is the same as fa_decode's.
 */
fa_status fa_decode_sliding_window(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                   int B, int H, int Hkv, int Lmax, int d, float scale, const int32_t* ctx_lens,
                                   int window, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_paged — fa_decode against a paged KV cache. "FlashAttention 与长上下文：先分清
 * 三张账" names PagedAttention's paged KV allocation (section on prefill and decode) without
 * a layout; the one read here:
 *   k_pages, v_pages : bf16 [num_pages, Hkv, page_size, d]  (a page holds page_size
 *                      consecutive positions of one sequence, for every KV head)
 *   block_table      : device int32 [B, max_pages]; position j of request b is row
 *                      j % page_size of page block_table[b][j / page_size]
 *   ctx_lens         : device int32 [B], clamped to [0, max_pages * page_size]
 *   window           : 0 for none, else a sliding window as in fa_decode_sliding_window
 *   workspace        : fa_decode_workspace_bytes(B, H, max_pages * page_size, d) bytes
 * page_size must be a power of two; sizes below 16 return FA_ERR_UNSUPPORTED (a 16-key
 * half step of the kernel must lie in one page). Table entries are device data and are not
 * checked on the host: the kernel clamps each to [0, num_pages - 1], so a bad table gives
 * wrong numbers but never an access outside the pools. Entries past a request's context are
 * not read. The keys are split as for fa_decode (or fa_decode_sliding_window) on a cache of
 * capacity max_pages * page_size, so paged and contiguous calls of equal capacity give
 * identical results. q, o, lse, scale and errors as for fa_decode.
 */
fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse,
                          int B, int H, int Hkv, int d, float scale, int page_size, int num_pages,
                          const int32_t* block_table, int max_pages, const int32_t* ctx_lens, int window,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_workspace_bytes — bytes of device workspace fa_bwd needs: two fp32 per query row
 * (the row's LSE in base 2 and D = rowsum(dO * O)), i.e. B * H * Lq * 8. Returns 0 for
 * invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Lq);

/*
 * fa_bwd — gradients of fa_fwd with respect to q, k and v, given the upstream gradient dout
 * of o. "FlashAttention 与长上下文：先分清三张账", section "FlashAttention 的关键是 online
 * softmax": the backward pass keeps only the forward's per-row statistic and recomputes the
 * score tiles instead of storing them. With P = softmax(scale Q K^T + M) (M as in fa_fwd):
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),  dQ = scale dS K,  dK = scale dS^T Q,
 * with dK and dV of a KV head summed over its query heads (GQA).
 *
 *   q, o, dout, dq : bf16 [B, H, Lq, d]      k, v, dk, dv : bf16 [B, Hkv, Lk, d]
 *   lse            : fp32 [B, H, Lq], the natural-log LSE fa_fwd returned for this o
 *   o              : the fa_fwd output for these inputs (used only through rowsum(dO * O))
 *   causal, scale, seqlens: exactly as passed to fa_fwd.
 *   workspace      : device memory of at least fa_bwd_workspace_bytes(B, H, Lq) bytes,
 *                    16-byte aligned, owned by the caller; its contents are scratch.
 * dq, dk, dv are overwritten (not accumulated into). Padding rows and keys outside a
 * sequence get zero gradients; they are never read. dout and o must be finite on the rows
 * inside each sequence. Accumulation is fp32; results are rounded to bf16 (RNE).
 * Requirements and errors as for fa_fwd, plus the workspace size.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int H, int Hkv, int Lq, int Lk, int d, float scale, int causal,
                 const int32_t* seqlens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_sliding_window — gradients of fa_fwd_sliding_window (the same window, o and lse
 * from that call); otherwise as fa_bwd with causal = 1. window >= 1, else FA_ERR_INVALID.
 */
fa_status fa_bwd_sliding_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Lq,
                                int Lk, int d, float scale, int window, const int32_t* seqlens, void* workspace,
                                size_t workspace_bytes, void* stream);

/* fa_status_string — a static, human-readable name for a status code. */
const char* fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
