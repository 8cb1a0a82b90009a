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

// Cache-policy operand of the buffer loads: bit 1 is the non-temporal hint.
constexpr int kCpolNT = 2;

// A 16-row operand of v_mfma_f32_16x16x32_bf16 over 2*NP steps of 32 bf16:
// lane l must hold row l & 15, k = 32t + 8(l >> 4) .. +7 of step t.  Loading
// that layout directly makes each of 16 consecutive lanes touch a different
// row, so every lane becomes a request of its own.  Here the loads fetch
// whole 128-byte lines -- a line of one row is 64 k, two steps, and eight
// consecutive lanes take it: lane 8q + u loads unit u (16 bytes) of row q
// into lo and unit u ^ 4 of row 8 + q into hi -- and one select and one lane
// permute per register then move every unit to the lane the matrix core
// wants it in (the values, hence the products, are unchanged).
//   issue(plo, phi): plo = &row q [8u], phi = &row (8 + q) [8(u ^ 4)], with
//     q = lane >> 3, u = lane & 7; step pair g is read at +64g elements.
//   place(out): out[t] for t < 2*NP in the matrix-core layout; place_pair(g,
//     out): steps 2g, 2g + 1 only.
// ROWS8: only rows 0-7 are needed.  The hi loads are skipped and lo stands in
// for hi, so rows 8-15 of the placed fragments hold other values (their
// products must be discarded); rows 0-7 are exactly as with ROWS8 false.
template <int NP, bool NT, bool ROWS8 = false>
struct LineOperand16 {
  u32x4 lo[NP], hi[ROWS8 ? 1 : NP];
  __device__ __forceinline__ void issue(const uint16_t *plo, const uint16_t *phi) {
#pragma unroll
    for (int g = 0; g < NP; ++g) {
      const u32x4 *a = reinterpret_cast<const u32x4 *>(plo + 64 * g);
      const u32x4 *b = reinterpret_cast<const u32x4 *>(phi + 64 * g);
      lo[g] = NT ? __builtin_nontemporal_load(a) : *a;
      if constexpr (!ROWS8) hi[g] = NT ? __builtin_nontemporal_load(b) : *b;
    }
  }
  // Step 2g, lane r + 16c (r < 8) wants unit c of row r: lo of lane 8r + c;
  // (r >= 8) unit c of row r: hi of lane 8(r-8) + 4 + c.  Step 2g+1 wants unit
  // 4 + c: lo of lane 8r + 4 + c, or hi of lane 8(r-8) + c.  So lanes whose
  // unit slot is below 4 offer lo for step 2g and hi for step 2g+1, the others
  // the reverse, and one permute per register gathers each step.
  // Steps 2g and 2g + 1 -> out[0], out[1].
  __device__ __forceinline__ void place_pair(int g, bf16x8 *out, int lane) const {
    const bool first = (lane & 4) == 0;
    const int r = lane & 15, c = lane >> 4;
    const int src0 = (r < 8 ? 8 * r + c : 8 * (r - 8) + 4 + c) * 4;
    const int src1 = (r < 8 ? 8 * r + 4 + c : 8 * (r - 8) + c) * 4;
    u32x4 t0, t1;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if constexpr (ROWS8) {
        t0[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src0, (int)lo[g][d]);
        t1[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src1, (int)lo[g][d]);
      } else {
        t0[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src0, (int)(first ? lo[g][d] : hi[g][d]));
        t1[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src1, (int)(first ? hi[g][d] : lo[g][d]));
      }
    }
    out[0] = __builtin_bit_cast(bf16x8, t0);
    out[1] = __builtin_bit_cast(bf16x8, t1);
  }
  __device__ __forceinline__ void place(bf16x8 *out, int lane) const {
#pragma unroll
    for (int g = 0; g < NP; ++g) place_pair(g, out + 2 * g, lane);
  }
};

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
