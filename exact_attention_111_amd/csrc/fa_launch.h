// fa_launch.h — host-side launch entry points of the kernels (internal to libfa).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Prefill forward. Arguments are already validated; sizes are non-zero.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Lq, Lk, d;
  float scale;
  int causal;
  int window;  // sliding window W, 0 for none (needs causal)
  const int32_t* seqlens;
};
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);

// Workgroups of a persistent grid of `kernel` (blocks of block_threads) on the current
// device: as many as can be resident at once (compute units x workgroups per unit), rounded
// down to a multiple of 8 (the XCDs workgroups are dealt to in turn), or 0 (no persistent
// grid) when that is not known or under 8. Looked up once per device and kernel.
int persistent_programs(const void* kernel, int block_threads);

// FP8 prefill (d = 128): E4M3 q, k, v with per-(batch, head) fp32 descales, bf16 o.
struct Fp8FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* q_descale;  // [B, H]
  const float* k_descale;  // [B, Hkv]
  const float* v_descale;  // [B, Hkv]
  void* o;
  float* lse;
  int B, H, Hkv, Lq, Lk;
  float scale;
  int causal;
  int window;
  const int32_t* seqlens;
};
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);

// Decode: split kernel over key chunks, then the combine kernel.
constexpr int kDecodeChunk = 2048;  // keys per split partial
// Paged cache: k and v are pools [num_pages, Hkv, page_size, d], table is int32
// [B, max_pages] and Lmax = max_pages * page_size; table == nullptr for a contiguous cache.
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, Lmax, d;
  float scale;
  const int32_t* ctx_lens;
  int window;    // sliding window W, 0 for none
  const int32_t* table;
  int page_size, max_pages, num_pages;
  float* ws_o;   // [B, H, nchunk, d]
  float* ws_ml;  // [B, H, nchunk, 2]
};
inline int decode_num_chunks(int Lmax) { return (Lmax + kDecodeChunk - 1) / kDecodeChunk; }
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// Size of the fixed per-GPU decode workspace of fa_decode_noalloc, and its device address on
// the current device (looked up once per device, then cached).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);

// Backward (bf16): per query row the exp2 offset of the saved LSE and D = rowsum(dO * O),
// then dK/dV per key block and dQ per query block, both recomputing P from Q, K and the LSE.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, H, Hkv, Lq, Lk, d;
  float scale;
  int causal;
  int window;  // sliding window W, 0 for none (needs causal)
  const int32_t* seqlens;
  float* ws;  // [B, H, Lq] x (exp2 offset, D) per query row
};
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

}  // namespace fa
