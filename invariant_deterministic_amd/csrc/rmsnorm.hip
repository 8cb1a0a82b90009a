// rmsnorm.hip -- batch-invariant RMSNorm: one workgroup per row, fixed tree.
//
// "Cómo superar la no determinación en la inferencia de LLM", section
// "RMSNorm": the batch-invariant form is data-parallel, each batch row reduced
// by one core with the same strategy at every batch size.  Here one workgroup
// (4 wavefronts of 64 lanes, or one wavefront playing those four) owns one
// row; the order of its sum of squares depends on K alone.  The page's split reduction for very small batches is
// deliberately absent: it is the very change of strategy with batch size that
// breaks invariance.
//
// Memory: the row is read once into registers (K <= 16384 means at most 8
// 16-byte chunks per thread), reduced, scaled and written once: 4*K + (weight)
// bytes per row of HBM traffic, which bounds the kernel at large M.
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;  // 16-byte chunks per thread: K <= 8 * 256 * 8

template <int V>
struct IntC {
  static constexpr int value = V;
};

// x + (x moved across lanes by the DPP control CTRL), all rows and banks on.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x, IntC<CTRL>) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                   0xF, 0xF, false));
}

// NCH: 16-byte chunks a thread may own (1, 2, 4 or 8), picked from K alone so
// that the registers fit the row and nothing about the reduction changes.
// RPW: rows per workgroup, one after another through the same 256 threads;
// every load of all RPW rows (and of the weight) is issued before any
// reduction, so a workgroup keeps RPW rows in flight.  Each row keeps its own
// chunks, sum order and tree, so RPW changes no bit.
template <int NCH, int RPW>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(
    const uint16_t *x, const uint16_t *__restrict__ w, uint16_t *y, int M, int K,
    int64_t ldx, int64_t ldy, float eps) {
  const int t = threadIdx.x;
  const int nchunks = K >> 3;
  const int row0 = blockIdx.x * RPW;

  // One memory round trip for the weight and every row (rows past M, in the
  // last workgroup only, load row M - 1 and store nothing).
  const u32x4 *wr = reinterpret_cast<const u32x4 *>(w);
  u32x4 v[RPW][NCH], wv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = t + i * kThreads;
    if (c < nchunks) wv[i] = wr[c];
  }
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const int row = row0 + q < M ? row0 + q : M - 1;
    const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + (int64_t)row * ldx);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = t + i * kThreads;
      if (c < nchunks) v[q][i] = __builtin_nontemporal_load(xr + c);
    }
  }

  __shared__ float part[RPW][kThreads / 64];
  float ss[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    // Thread-local sum of squares in ascending element order.  Each square of
    // a bf16 value is exact in fp32, so only the additions round.
    ss[q] = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = t + i * kThreads;
      if (c < nchunks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = lo_bf16(v[q][i][j]);
          const float b = hi_bf16(v[q][i][j]);
          ss[q] = ss[q] + a * a;
          ss[q] = ss[q] + b * b;
        }
      }
    }
  }
  // Wavefront: fixed xor butterfly over lane offsets 32, 16, 8, 4, 2, 1, each
  // step own + partner.  Partners add the same two values (in swapped operand
  // order, which is exact-commutative), so after the step of offset d the
  // lanes i and i ^ d hold the same bits.  The two steps that cross 16-lane
  // rows use the LDS permute; the four inside a row are DPP lane moves in the
  // VALU: offset 8 is a rotation of the row by 8 (lane i takes (i - 8) mod 16
  // = i ^ 8); offset 4 a rotation by 4, since (i - 4) mod 16 is i ^ 4 or
  // (i ^ 4) ^ 8, which hold the same value by then; offsets 2 and 1 exact
  // quad permutations.  The rows of a workgroup go through each step
  // together.
#pragma unroll
  for (int off = 32; off >= 16; off >>= 1)
#pragma unroll
    for (int q = 0; q < RPW; ++q) ss[q] = ss[q] + __shfl_xor(ss[q], off, 64);
#pragma unroll
  for (int q = 0; q < RPW; ++q) ss[q] = dpp_add(ss[q], IntC<0x128>{});  // row_ror:8
#pragma unroll
  for (int q = 0; q < RPW; ++q) ss[q] = dpp_add(ss[q], IntC<0x124>{});  // row_ror:4
#pragma unroll
  for (int q = 0; q < RPW; ++q) ss[q] = dpp_add(ss[q], IntC<0x4E>{});   // quad_perm [2,3,0,1]
#pragma unroll
  for (int q = 0; q < RPW; ++q) ss[q] = dpp_add(ss[q], IntC<0xB1>{});   // quad_perm [1,0,3,2]
#pragma unroll
  for (int q = 0; q < RPW; ++q)
    if ((t & 63) == 0) part[q][t >> 6] = ss[q];
  __syncthreads();

#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    if (row0 + q >= M) break;
    const float total = ((part[q][0] + part[q][1]) + part[q][2]) + part[q][3];
    const float r = 1.0f / sqrtf(total / (float)K + eps);
    u32x4 *yr = reinterpret_cast<u32x4 *>(y + (int64_t)(row0 + q) * ldy);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = t + i * kThreads;
      if (c < nchunks) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = (lo_bf16(v[q][i][j]) * r) * lo_bf16(wv[i][j]);
          const float hi = (hi_bf16(v[q][i][j]) * r) * hi_bf16(wv[i][j]);
          o[j] = pack_bf16x2(lo, hi);
        }
        __builtin_nontemporal_store(o, yr + c);
      }
    }
  }
}

// The same rows with one 64-lane wavefront per row (a workgroup of one
// wavefront): lane l plays threads l, l + 64, l + 128 and l + 192 of the
// 256-thread kernel above -- virtual wavefront v = 0..3 -- with the same
// chunks, the same per-thread sums in the same order, the same butterfly per
// virtual wavefront, and ((s0 + s1) + s2) + s3 across them, in registers
// instead of through LDS.  So every row's bits equal the 256-thread kernel's.
// No barrier: each wavefront stores its row as soon as its own loads are
// back, which lets loads and stores of different rows overlap like a copy's.
// RW rows per wavefront, each with its own chunks, sums and tree (rows past
// M, in the last wavefront only, load row M - 1 and store nothing).
template <int NCH, int RW>
__global__ __launch_bounds__(64) void rmsnorm_wave_kernel(
    const uint16_t *x, const uint16_t *__restrict__ w, uint16_t *y, int M, int K, int64_t ldx,
    int64_t ldy, float eps) {
  const int l = threadIdx.x;
  const int nchunks = K >> 3;
  const int row0 = blockIdx.x * RW;
  const u32x4 *wr = reinterpret_cast<const u32x4 *>(w);
  u32x4 v[RW][4][NCH], wv[4][NCH];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    // (with one row per wavefront the grid has exactly M wavefronts; the
    // clamp and the store guard below are left out there: measured, their
    // code alone cost 10 % at M = 2048)
    int row = row0 + rr;
    if constexpr (RW > 1) row = row < M ? row : M - 1;
    const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + (int64_t)row * ldx);
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = l + 64 * q + kThreads * i;  // chunk of virtual thread l + 64 q
        if (c < nchunks) v[rr][q][i] = __builtin_nontemporal_load(xr + c);
      }
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = l + 64 * q + kThreads * i;
      if (c < nchunks) wv[q][i] = wr[c];
    }
  float ss[RW][4];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ss[rr][q] = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = l + 64 * q + kThreads * i;
        if (c < nchunks) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float a = lo_bf16(v[rr][q][i][j]);
            const float b = hi_bf16(v[rr][q][i][j]);
            ss[rr][q] = ss[rr][q] + a * a;
            ss[rr][q] = ss[rr][q] + b * b;
          }
        }
      }
    }
  // the butterfly of the 256-thread kernel, once per virtual wavefront and row
#pragma unroll
  for (int off = 32; off >= 16; off >>= 1)
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int q = 0; q < 4; ++q) ss[rr][q] = ss[rr][q] + __shfl_xor(ss[rr][q], off, 64);
#pragma unroll
  for (int rr = 0; rr < RW; ++rr)
#pragma unroll
    for (int q = 0; q < 4; ++q) ss[rr][q] = dpp_add(ss[rr][q], IntC<0x128>{});  // row_ror:8
#pragma unroll
  for (int rr = 0; rr < RW; ++rr)
#pragma unroll
    for (int q = 0; q < 4; ++q) ss[rr][q] = dpp_add(ss[rr][q], IntC<0x124>{});  // row_ror:4
#pragma unroll
  for (int rr = 0; rr < RW; ++rr)
#pragma unroll
    for (int q = 0; q < 4; ++q) ss[rr][q] = dpp_add(ss[rr][q], IntC<0x4E>{});  // quad_perm [2,3,0,1]
#pragma unroll
  for (int rr = 0; rr < RW; ++rr)
#pragma unroll
    for (int q = 0; q < 4; ++q) ss[rr][q] = dpp_add(ss[rr][q], IntC<0xB1>{});  // quad_perm [1,0,3,2]
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    if constexpr (RW > 1) {
      if (row0 + rr >= M) break;
    }
    const float total = ((ss[rr][0] + ss[rr][1]) + ss[rr][2]) + ss[rr][3];
    const float r = 1.0f / sqrtf(total / (float)K + eps);
    u32x4 *yr = reinterpret_cast<u32x4 *>(y + (int64_t)(row0 + rr) * ldy);
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = l + 64 * q + kThreads * i;
        if (c < nchunks) {
          u32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float lo = (lo_bf16(v[rr][q][i][j]) * r) * lo_bf16(wv[q][i][j]);
            const float hi = (hi_bf16(v[rr][q][i][j]) * r) * hi_bf16(wv[q][i][j]);
            o[j] = pack_bf16x2(lo, hi);
          }
          __builtin_nontemporal_store(o, yr + c);
        }
      }
  }
}

// shape: -1 / -4 = one / four rows per 64-lane wavefront, 1 / 4 = rows per
// 256-thread workgroup
template <int NCH>
void launch_rows(int64_t M, int shape, hipStream_t st, const uint16_t *x, const uint16_t *w,
                 uint16_t *y, int K, int64_t ldx, int64_t ldy, float eps) {
  if constexpr (NCH <= 2) {
    if (shape == -1) {
      hipLaunchKernelGGL((rmsnorm_wave_kernel<NCH, 1>), dim3((unsigned)M), dim3(64), 0, st, x, w,
                         y, (int)M, K, ldx, ldy, eps);
      return;
    }
    if (shape == -4) {
      hipLaunchKernelGGL((rmsnorm_wave_kernel<NCH, 4>), dim3((unsigned)((M + 3) / 4)), dim3(64), 0,
                         st, x, w, y, (int)M, K, ldx, ldy, eps);
      return;
    }
  }
  const dim3 grid((unsigned)((M + shape - 1) / shape)), block(kThreads);
  if (shape == 4)
    hipLaunchKernelGGL((rmsnorm_kernel<NCH, 4>), grid, block, 0, st, x, w, y, (int)M, K, ldx, ldy, eps);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<NCH, 1>), grid, block, 0, st, x, w, y, (int)M, K, ldx, ldy, eps);
}

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" int bi_rmsnorm(const uint16_t *x, const uint16_t *w, uint16_t *y,
                          int64_t M, int64_t K, int64_t ldx, int64_t ldy,
                          float eps, void *stream) {
  if (!w || (M > 0 && (!x || !y))) return BI_ERR_NULL;
  if (M < 0 || K < 8 || K > 8 * kThreads * kMaxChunks || ldx < K || ldy < K ||
      M > 0x7FFFFFFF || !(eps >= 0.0f))
    return BI_ERR_SHAPE;
  if ((K | ldx | ldy) & 7 || !aligned16(x) || !aligned16(w) || !aligned16(y))
    return BI_ERR_ALIGN;
  const Span sx = span_of(x, M, K, ldx, 2), sy = span_of(y, M, K, ldy, 2),
             sw = span_of(w, 1, K, K, 2);
  const bool in_place = (x == y) && (ldx == ldy);
  if ((!in_place && overlap(sx, sy)) || overlap(sw, sy)) return BI_ERR_ALIAS;
  if (M == 0) return BI_OK;
  const int nch = (int)((K / 8 + kThreads - 1) / kThreads);
  // Launch shape from the rows per CU, for K <= 4096 (two chunks a thread);
  // every shape gives the same bits.  The one-wavefront kernels do best when
  // every wavefront of the launch is resident at once, at 6-8 wavefronts per
  // CU.  Measured at K = 4096 (graph-timed, inputs rotated), per 256 CUs:
  //   6-12 rows per CU: one row per wavefront (M = 2048: 6.3 us against 7.2
  //     for the best 256-thread shape; M = 2560: 7.8 against 8.4);
  //   12-16: four rows per 256-thread workgroup (M = 3072: 9.2 us against
  //     10.0 for one row per wavefront; M = 4096: 11.7 against 14.0);
  //   16-32: four rows per wavefront (M = 6144: 17.4 us against 18.9;
  //     M = 8192: 22.0-22.3 against 23.6-24.1 on three boxes; above 32 rows
  //     per CU its wavefronts no longer fit at once and it lost 6-17 %);
  //   elsewhere one row per 256-thread workgroup (below 6 rows per CU one
  //     row per wavefront measured 4-12 % slower).
  // At K <= 2048, one row per wavefront lost below 8 rows per CU (M = 1536:
  // 3.9 against 3.6 us) and gained 4-9 % from 8 to 12; four rows per
  // wavefront is only used at K > 2048, where it was measured.
  int shape = 1;
  if (nch <= 2) {
    const int64_t cus = cu_count();
    if (M >= (nch == 2 ? 6 : 8) * cus && M < 12 * cus) shape = -1;
    else if (M >= 12 * cus && M <= 16 * cus) shape = 4;
    else if (nch == 2 && M > 16 * cus && M <= 32 * cus) shape = -4;
  }
  hipStream_t st = (hipStream_t)stream;
  if (nch <= 1) launch_rows<1>(M, shape, st, x, w, y, (int)K, ldx, ldy, eps);
  else if (nch <= 2) launch_rows<2>(M, shape, st, x, w, y, (int)K, ldx, ldy, eps);
  else if (nch <= 4) launch_rows<4>(M, 1, st, x, w, y, (int)K, ldx, ldy, eps);
  else launch_rows<8>(M, 1, st, x, w, y, (int)K, ldx, ldy, eps);
  return launch_status();
}
