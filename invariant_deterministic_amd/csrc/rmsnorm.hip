// rmsnorm.hip -- batch-invariant RMSNorm: one workgroup per row, fixed tree.
//
// "Cómo superar la no determinación en la inferencia de LLM", section
// "RMSNorm": the batch-invariant form is data-parallel, each batch row reduced
// by one core with the same strategy at every batch size.  Here one workgroup
// (4 wavefronts of 64 lanes) owns one row; the order of its sum of squares
// depends on K alone.  The page's split reduction for very small batches is
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
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    // Thread-local sum of squares in ascending element order.  Each square of
    // a bf16 value is exact in fp32, so only the additions round.
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = t + i * kThreads;
      if (c < nchunks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = lo_bf16(v[q][i][j]);
          const float b = hi_bf16(v[q][i][j]);
          ss = ss + a * a;
          ss = ss + b * b;
        }
      }
    }
    // Wavefront: fixed xor butterfly.  Partners add the same two values (in
    // swapped operand order, which is exact-commutative), so every lane ends
    // with the same bits.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss = ss + __shfl_xor(ss, off, 64);
    if ((t & 63) == 0) part[q][t >> 6] = ss;
  }
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

template <int NCH>
void launch_rows(int64_t M, int rpw, hipStream_t st, const uint16_t *x, const uint16_t *w,
                 uint16_t *y, int K, int64_t ldx, int64_t ldy, float eps) {
  const dim3 grid((unsigned)((M + rpw - 1) / rpw)), block(kThreads);
  if (rpw == 4)
    hipLaunchKernelGGL((rmsnorm_kernel<NCH, 4>), grid, block, 0, st, x, w, y, (int)M, K, ldx, ldy, eps);
  else if (rpw == 2)
    hipLaunchKernelGGL((rmsnorm_kernel<NCH, 2>), grid, block, 0, st, x, w, y, (int)M, K, ldx, ldy, eps);
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
  // Rows per workgroup: up to 4096 rows, enough rows per workgroup for about
  // 1024 workgroups (more rows in flight per CU than one row per workgroup
  // gives; measured at K = 4096: M = 2048: 7.5 -> 7.0 us, M = 4096: 13.8 ->
  // 11.7 us, the copy rate of those bytes); above, one row per workgroup.
  // Only rows with K <= 4096 (two chunks a thread) take more than one.
  int rpw = 1;
  if (nch <= 2 && M <= 4096) rpw = M >= 4096 ? 4 : (M >= 2048 ? 2 : 1);
  hipStream_t st = (hipStream_t)stream;
  if (nch <= 1) launch_rows<1>(M, rpw, st, x, w, y, (int)K, ldx, ldy, eps);
  else if (nch <= 2) launch_rows<2>(M, rpw, st, x, w, y, (int)K, ldx, ldy, eps);
  else if (nch <= 4) launch_rows<4>(M, 1, st, x, w, y, (int)K, ldx, ldy, eps);
  else launch_rows<8>(M, 1, st, x, w, y, (int)K, ldx, ldy, eps);
  return launch_status();
}
