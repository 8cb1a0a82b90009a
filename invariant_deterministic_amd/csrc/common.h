// common.h -- internal helpers shared by the HIP kernels of libbi.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bi.h"

namespace bi {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 bit patterns in one word (lo in the low half), round
// to nearest, ties to even, NaN returned quiet with its sign: one
// v_cvt_pk_bf16_f32.  Its result equals, for every one of the 2^32 fp32 bit
// patterns (checked exhaustively on gfx950), the format's integer
// definition: add half an output ulp minus one plus the kept lsb, truncate;
// NaN -> (bits >> 16) | 0x40.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Two bf16 in one 32-bit word (low half first) -> fp32.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}
// Workgroup barrier without the release/acquire fence of __syncthreads(): the
// fence would also wait for every outstanding global->LDS load, which would
// drain a prefetch pipeline.  Callers issue the waits their data needs; the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Compute units of the current device (256 on MI355X if the query fails).
inline int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Byte span [lo, hi) touched by a row-major [rows, cols] tensor with stride ld.
struct Span {
  uintptr_t lo, hi;
};
inline Span span_of(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  uintptr_t b = (uintptr_t)p;
  if (rows <= 0 || cols <= 0) return Span{b, b};
  return Span{b, b + (uintptr_t)(((rows - 1) * ld + cols) * elem)};
}
inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace bi
