// fa_api.cpp — the extern "C" boundary of libfa: argument validation and dispatch.
//
// Every check here runs on the host before anything is enqueued, so a call that fails
// validation writes nothing and touches no device state. Unsupported but well-formed
// requests (a head dimension other than 64 or 128) return FA_ERR_UNSUPPORTED rather than
// taking a slower path: an attention call that silently falls back is the failure mode
// "2.1 FlashAttention-2 的核心思想" §2.1.7 and §2.1.11 warn about.
#include "fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A tensor pointer must be non-null and 16-byte aligned unless the tensor is empty.
bool tensor_ok(const void* p, long long numel) {
  if (numel == 0) return true;
  return p != nullptr && aligned16(p);
}

bool supported_d(int d) { return d == 64 || d == 128; }

bool aligned4(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

fa_status validate_fwd(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int H,
                       int Hkv, int Lq, int Lk, int d, float scale, int causal, const int32_t* seqlens) {
  if (B < 0 || H < 0 || Hkv < 1 || Lq < 0 || Lk < 0 || d < 1) return FA_ERR_INVALID;
  if (H % Hkv != 0) return FA_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (seqlens != nullptr && (Lq != Lk || (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)) return FA_ERR_INVALID;
  const long long nq = (long long)B * H * Lq * d;
  const long long nkv = (long long)B * Hkv * Lk * d;
  if (!tensor_ok(q, nq) || !tensor_ok(o, nq) || !tensor_ok(k, nkv) || !tensor_ok(v, nkv)) return FA_ERR_INVALID;
  if (!tensor_ok(lse, (long long)B * H * Lq)) return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Everything of a decode call but its workspace.
fa_status validate_decode_args(const void* q, const void* kc, const void* vc, const void* o, const void* lse, int B,
                               int H, int Hkv, int Lmax, int d, float scale, const int32_t* ctx) {
  if (B < 0 || H < 0 || Hkv < 1 || Lmax < 0 || d < 1) return FA_ERR_INVALID;
  if (H % Hkv != 0) return FA_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID;
  const long long nq = (long long)B * H * d;
  const long long nkv = (long long)B * Hkv * Lmax * d;
  if (!tensor_ok(q, nq) || !tensor_ok(o, nq) || !tensor_ok(kc, nkv) || !tensor_ok(vc, nkv)) return FA_ERR_INVALID;
  if (!tensor_ok(lse, (long long)B * H)) return FA_ERR_INVALID;
  if (B > 0 && (ctx == nullptr || (reinterpret_cast<uintptr_t>(ctx) & 3u) != 0)) return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa_status validate_decode(const void* q, const void* kc, const void* vc, const void* o, const void* lse, int B, int H,
                          int Hkv, int Lmax, int d, float scale, const int32_t* ctx, const void* ws, size_t ws_bytes) {
  const fa_status s = validate_decode_args(q, kc, vc, o, lse, B, H, Hkv, Lmax, d, scale, ctx);
  if (s != FA_OK) return s;
  const size_t need = fa_decode_workspace_bytes(B, H, Lmax, d);
  if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return FA_ERR_INVALID;
  return FA_OK;
}

static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES,
              "the fixed decode workspace and its documented size agree");

fa_status validate_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const void* lse, const void* dq, const void* dk, const void* dv, int B, int H, int Hkv, int Lq,
                       int Lk, int d, float scale, int causal, const int32_t* seqlens, const void* ws,
                       size_t ws_bytes) {
  const fa_status s = validate_fwd(q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, seqlens);
  if (s == FA_ERR_INVALID) return s;
  const long long nq = (long long)B * H * Lq * d;
  const long long nkv = (long long)B * Hkv * Lk * d;
  if (!tensor_ok(dout, nq) || !tensor_ok(dq, nq) || !tensor_ok(dk, nkv) || !tensor_ok(dv, nkv)) return FA_ERR_INVALID;
  if (s != FA_OK) return s;
  const size_t need = fa_bwd_workspace_bytes(B, H, Lq);
  if (need > 0 && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return FA_ERR_INVALID;
  return FA_OK;
}

fa_status fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int Lq,
                   int Lk, int d, float scale, int causal, int window, const int32_t* seqlens, void* stream) {
  const fa_status s = validate_fwd(q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, seqlens);
  if (s != FA_OK) return s;
  if (B == 0 || H == 0 || Lq == 0) return FA_OK;
  fa::FwdParams p{q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, window, seqlens};
  return fa::launch_fwd_bf16(p, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Launch of the decode kernels after validation. Paged calls pass the block table and the
// page geometry (Lmax = max_pages * page_size); contiguous ones pass table == nullptr.
fa_status decode_run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                     int Lmax, int d, float scale, const int32_t* ctx_lens, int window, const int32_t* table,
                     int page_size, int max_pages, int num_pages, void* workspace, void* stream) {
  if (B == 0 || H == 0) return FA_OK;
  const size_t nc = (size_t)fa::decode_num_chunks(Lmax);
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + (size_t)B * H * nc * d;
  fa::DecodeParams p{q, k, v, o, lse, B, H, Hkv, Lmax, d, scale, ctx_lens, window, table, page_size, max_pages,
                     num_pages, ws_o, ws_ml};
  return fa::launch_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Hkv, int Lq, int Lk, int d, float scale, int causal,
                   int window, const int32_t* seqlens, void* workspace, size_t workspace_bytes, void* stream) {
  const fa_status s = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Lq, Lk, d, scale, causal, seqlens,
                                   workspace, workspace_bytes);
  if (s != FA_OK) return s;
  if (B == 0) return FA_OK;  // otherwise dK/dV are written even when there are no query rows (then zero)
  fa::BwdParams p{q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Lq, Lk, d, scale, causal, window, seqlens,
                  static_cast<float*>(workspace)};
  return fa::launch_bwd(p, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int Lq,
                 int Lk, int d, float scale, int causal, const int32_t* seqlens, void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, 0, seqlens, stream);
}

fa_status fa_fwd_sliding_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                int Hkv, int Lq, int Lk, int d, float scale, int window, const int32_t* seqlens,
                                void* stream) {
  if (window < 1) return FA_ERR_INVALID;
  return fwd_bf16(q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, 1, window, seqlens, stream);
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                     const float* v_descale, void* o, float* lse, int B, int H, int Hkv, int Lq, int Lk, int d,
                     float scale, int causal, int window, const int32_t* seqlens, void* stream) {
  if (window < 0 || (window > 0 && causal != 1)) return FA_ERR_INVALID;
  // Element counts of the fp8 tensors in bf16 units for the shared check: a row of d bytes is
  // d / 2 bf16 elements, so q, k, v are checked as non-null and 16-byte aligned when not empty.
  fa_status s = validate_fwd(q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, seqlens);
  if (s == FA_ERR_INVALID) return s;
  const bool any = (long long)B * H > 0;
  if (any && (!aligned4(q_descale) || !aligned4(k_descale) || !aligned4(v_descale))) return FA_ERR_INVALID;
  if (s != FA_OK) return s;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || Lq == 0) return FA_OK;
  fa::Fp8FwdParams p{q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, Hkv, Lq, Lk, scale, causal, window,
                     seqlens};
  return fa::launch_fwd_fp8(p, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Hkv,
                     int Lq, int Lk, int d, float scale, int causal, const int32_t* seqlens, void* stream) {
  const fa_status s = validate_fwd(q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, seqlens);
  if (s != FA_OK) return s;
  if (B == 0 || H == 0 || Lq == 0) return FA_OK;
  fa::FwdParams p{q, k, v, o, lse, B, H, Hkv, Lq, Lk, d, scale, causal, 0, seqlens};
  return fa::launch_fwd_f32(p, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_workspace_bytes(int B, int H, int Lmax, int d) {
  if (B < 0 || H < 0 || Lmax < 0 || d < 1) return 0;
  const size_t nc = (size_t)fa::decode_num_chunks(Lmax);
  // Partial outputs [B, H, nc, d] then (max, sum) pairs [B, H, nc, 2], both fp32.
  return (size_t)B * H * nc * ((size_t)d + 2) * sizeof(float);
}

fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int H,
                    int Hkv, int Lmax, int d, float scale, const int32_t* ctx_lens, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const fa_status s = validate_decode(q, k_cache, v_cache, o, lse, B, H, Hkv, Lmax, d, scale, ctx_lens, workspace,
                                      workspace_bytes);
  if (s != FA_OK) return s;
  return decode_run(q, k_cache, v_cache, o, lse, B, H, Hkv, Lmax, d, scale, ctx_lens, 0, nullptr, 0, 0, 0, workspace,
                    stream);
}

fa_status fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B,
                            int H, int Hkv, int Lmax, int d, float scale, const int32_t* ctx_lens, void* stream) {
  // Arguments as fa_decode checks them, then the call's workspace against the fixed one.
  const fa_status s = validate_decode_args(q, k_cache, v_cache, o, lse, B, H, Hkv, Lmax, d, scale, ctx_lens);
  if (s != FA_OK) return s;
  if (fa_decode_workspace_bytes(B, H, Lmax, d) > FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES) return FA_ERR_TOO_LARGE;
  if (B == 0 || H == 0) return FA_OK;
  void* ws = nullptr;
  if (fa::decode_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  return decode_run(q, k_cache, v_cache, o, lse, B, H, Hkv, Lmax, d, scale, ctx_lens, 0, nullptr, 0, 0, 0, ws, stream);
}

fa_status fa_decode_sliding_window(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                   int B, int H, int Hkv, int Lmax, int d, float scale, const int32_t* ctx_lens,
                                   int window, void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 1) return FA_ERR_INVALID;
  const fa_status s = validate_decode(q, k_cache, v_cache, o, lse, B, H, Hkv, Lmax, d, scale, ctx_lens, workspace,
                                      workspace_bytes);
  if (s != FA_OK) return s;
  return decode_run(q, k_cache, v_cache, o, lse, B, H, Hkv, Lmax, d, scale, ctx_lens, window, nullptr, 0, 0, 0,
                    workspace, stream);
}

fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse, int B, int H,
                          int Hkv, int d, float scale, int page_size, int num_pages, const int32_t* block_table,
                          int max_pages, const int32_t* ctx_lens, int window, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (page_size < 1 || (page_size & (page_size - 1)) != 0 || max_pages < 0 || num_pages < 0 || window < 0)
    return FA_ERR_INVALID;
  if ((long long)max_pages * page_size > 0x7fffffffLL) return FA_ERR_INVALID;
  const int Lmax = max_pages * page_size;
  // q, o, lse, ctx_lens, sizes and the workspace as for fa_decode (caches checked below)
  fa_status s = validate_decode(q, nullptr, nullptr, o, lse, B, H, Hkv, 0, d, scale, ctx_lens, workspace,
                                workspace_bytes);
  if (s == FA_ERR_INVALID) return s;
  const size_t need = fa_decode_workspace_bytes(B, H, Lmax, d);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)) return FA_ERR_INVALID;
  const long long npool = (long long)num_pages * Hkv * page_size * d;
  if (!tensor_ok(k_pages, npool) || !tensor_ok(v_pages, npool)) return FA_ERR_INVALID;
  if (B > 0 && (num_pages < 1 || block_table == nullptr || (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0))
    return FA_ERR_INVALID;
  if (s != FA_OK) return s;
  if (page_size < 16) return FA_ERR_UNSUPPORTED;  // a 16-key half step must lie in one page
  return decode_run(q, k_pages, v_pages, o, lse, B, H, Hkv, Lmax, d, scale, ctx_lens, window, block_table,
                    page_size, max_pages, num_pages, workspace, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int Lq) {
  if (B < 0 || H < 0 || Lq < 0) return 0;
  return (size_t)B * H * Lq * 2 * sizeof(float);  // (exp2 offset of the LSE, D = rowsum(dO * O)) per row
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int H, int Hkv, int Lq, int Lk, int d, float scale, int causal,
                 const int32_t* seqlens, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Lq, Lk, d, scale, causal, 0, seqlens, workspace,
                  workspace_bytes, stream);
}

fa_status fa_bwd_sliding_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Lq, int Lk,
                                int d, float scale, int window, const int32_t* seqlens, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (window < 1) return FA_ERR_INVALID;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, Lq, Lk, d, scale, 1, window, seqlens, workspace,
                  workspace_bytes, stream);
}

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID: return "FA_ERR_INVALID";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    case FA_ERR_TOO_LARGE: return "FA_ERR_TOO_LARGE";
  }
  return "FA_ERR_UNKNOWN";
}

}  // extern "C"
