// fa_device.h — vector types and small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier that orders LDS accesses only: outstanding global loads, including
// direct-to-LDS loads, stay in flight across it (a full __syncthreads() would drain them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resource (gfx9 format: 48-bit base, stride 0, byte size in num_records, and
// the format word used for untyped dword loads). Lanes whose byte offset is at or past
// num_records are out of range: they read no memory.
__device__ __forceinline__ u32x4 raw_buffer_rsrc(const void* base, unsigned num_bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)p);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32)) & 0xffffu;
  r[2] = __builtin_amdgcn_readfirstlane(num_bytes);
  r[3] = 0x00020000u;
  return r;
}

// 16 bytes per lane from a raw buffer straight into LDS (buffer_load_dwordx4 ... lds): lane
// i lands at lds_byte_addr + 16 * i, read from byte voff of the buffer. Out-of-range lanes
// read nothing; their LDS bytes are not relied on. Issued as inline assembly so that the
// compiler does not track it: otherwise it cannot tell which LDS bytes are being written and
// stalls every later LDS read until the load completes. Callers must therefore wait for
// completion themselves (s_waitcnt vmcnt) before the barrier that publishes the data. M0
// carries the LDS base; nothing else in these kernels uses M0.
__device__ __forceinline__ void lds_dma16_buf(u32x4 rsrc, unsigned voff, unsigned lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr))
               : "memory");
}

// Wait until at most N vector-memory loads of this wave are outstanding (they complete in
// issue order). Encoding (gfx9 family): vmcnt in bits [3:0] and [15:14]; expcnt [6:4] and
// lgkmcnt [11:8] left at their maxima, i.e. not waited for.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Race-check build (FA_SERIAL_PIPELINE defined): every direct-to-LDS stage is preceded and
// followed by serial_fence(), which waits for all of this wave's loads and then for the whole
// workgroup. No load is then in flight while anyone computes, and a slot is refilled only
// after every wave is past its earlier reads. The arithmetic is unchanged, so this build must
// give results bit for bit equal to the pipelined one; a missing wait or an early slot reuse
// in the pipelined kernels shows up as a difference. In the product build it is empty.
// Callers must reach it in every wave the same number of times (it contains a barrier).
__device__ __forceinline__ void serial_fence() {
#ifdef FA_SERIAL_PIPELINE
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#endif
}

// A wave-uniform pointer, held in SGPRs (the value must be the same in every lane).
// readfirstlane returns int: each half goes through unsigned before widening, or a low
// word with bit 31 set would be sign-extended over the high word.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)v);
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const T*>((hi << 32) | lo);
}

// A load at a wave-uniform address of memory that no kernel writes while this one runs,
// through the scalar cache (s_load): it waits on the scalar counter, not on the vector memory
// counter that also tracks the tile loads and stores.
__device__ __forceinline__ int load_const(const int* p) {
  return *(const __attribute__((address_space(4))) int*)p;
}

// Both halves of a wave at once: v_permlane32_swap exchanges the upper 32 lanes of its
// first operand with the lower 32 lanes of its second, so swapping a value with itself
// leaves [x_lo, x_lo] and [x_hi, x_hi]: every lane then holds its own value and that of
// lane ^ 32. The second operand passes through an empty asm: handed the same value twice,
// the compiler kept only one of the two results (each lane then saw only the lower half's
// value).
__device__ __forceinline__ void wave_halves(unsigned x, unsigned& lo_half, unsigned& hi_half) {
  unsigned y = x;
  asm volatile("" : "+v"(y));
  const auto sw = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  lo_half = sw[0];
  hi_half = sw[1];
}
__device__ __forceinline__ float max_of_halves(float x) {
  unsigned a, b;
  wave_halves(__builtin_bit_cast(unsigned, x), a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ bool any_of_halves(bool x) {
  unsigned a, b;
  wave_halves((unsigned)x, a, b);
  return (a | b) != 0u;
}

// Byte address of a pointer into LDS.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// Eight consecutive input elements as bf16 bits. bf16 input is copied; fp32 input is
// rounded to bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
template <typename T> struct Load8;
template <> struct Load8<__bf16> {
  static __device__ __forceinline__ u32x4 load(const __bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
};
template <> struct Load8<float> {
  static __device__ __forceinline__ u32x4 load(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    bf16x8 r;
    r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
    r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
    return as_u32x4(r);
  }
};

// Four consecutive output elements from fp32 values (bf16 outputs round to nearest even).
template <typename T> struct Store4;
template <> struct Store4<__bf16> {
  static __device__ __forceinline__ void store(__bf16* p, float a, float b, float c, float d) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 r;
    r[0] = (__bf16)a; r[1] = (__bf16)b; r[2] = (__bf16)c; r[3] = (__bf16)d;
    *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, r);
  }
};
template <> struct Store4<float> {
  static __device__ __forceinline__ void store(float* p, float a, float b, float c, float d) {
    f32x4 r = {a, b, c, d};
    *reinterpret_cast<f32x4*>(p) = r;
  }
};

__device__ __forceinline__ float bf16_bits_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_bits_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

}  // namespace fa
