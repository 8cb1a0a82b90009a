// lora_expand.hip -- LoRA expand: y[m][n] = bf16(base[m][n] + scale * sum_r l[m][r] * b[n][r]).
//
// "Reproducible LoRA Inference Through Deterministic Split-K Reduction",
// abstract: LoRA adds low-rank multiplications to a layer; the fp32 shrink
// output l (rank R) is expanded back to the layer width and added to the base
// output.  With R = 16 the reduction is short, so there is no split: every
// output sums its 16 products in ascending r in fp32, scales, adds the base
// and rounds to bf16 once -- the same order at any batch size.
//
// The expand streams base and y (4 bytes an output) and is bound by HBM
// bandwidth; the 16 multiply-adds per output run on the vector ALUs.  A
// 256-thread workgroup owns a 64 x 128 output tile: it stages the tile's 128
// rows of b and 64 rows of l in LDS once, and each thread computes 4 rows x 8
// consecutive columns with 16-byte loads and stores of base and y.
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int kR = 16;
constexpr int TM = 64, TN = 128;

__global__ __launch_bounds__(kThreads) void lora_expand_kernel(
    const float *__restrict__ l, const uint16_t *__restrict__ b, const uint16_t *base,
    uint16_t *y, int M, int N, int64_t ldl, int64_t ldb, int64_t ldbase, int64_t ldy,
    float scale) {
  const int m0 = blockIdx.x * TM, n0 = blockIdx.y * TN;
  __shared__ float bs[TN][kR + 1];  // +1: rows land in different banks
  __shared__ float ls[TM][kR + 1];
  for (int i = threadIdx.x; i < TN * kR; i += kThreads) {
    const int r = i % kR, n = i / kR;
    const int gn = n0 + n < N ? n0 + n : N - 1;
    bs[n][r] = bf16_to_f32(b[(int64_t)gn * ldb + r]);
  }
  for (int i = threadIdx.x; i < TM * kR; i += kThreads) {
    const int r = i % kR, m = i / kR;
    const int gm = m0 + m < M ? m0 + m : M - 1;
    ls[m][r] = l[(int64_t)gm * ldl + r];
  }
  __syncthreads();

  const int tc = threadIdx.x & 15, tr = threadIdx.x >> 4;
  const int nn = n0 + tc * 8;
  if (nn >= N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mm = tr * 4 + i;
    const int m = m0 + mm;
    if (m >= M) break;
    u32x4 bv = {0u, 0u, 0u, 0u};
    if (base) bv = *reinterpret_cast<const u32x4 *>(base + (int64_t)m * ldbase + nn);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        acc0 = acc0 + ls[mm][r] * bs[tc * 8 + 2 * j][r];
        acc1 = acc1 + ls[mm][r] * bs[tc * 8 + 2 * j + 1][r];
      }
      const float v0 = lo_bf16(bv[j]) + scale * acc0;
      const float v1 = hi_bf16(bv[j]) + scale * acc1;
      o[j] = pack_bf16x2(v0, v1);
    }
    *reinterpret_cast<u32x4 *>(y + (int64_t)m * ldy + nn) = o;
  }
}

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" int bi_lora_expand(const float *l, const uint16_t *b, const uint16_t *base, uint16_t *y,
                              int64_t M, int64_t N, int64_t R, int64_t ldl, int64_t ldb,
                              int64_t ldbase, int64_t ldy, float scale, void *stream) {
  if (!b || (M > 0 && (!l || !y))) return BI_ERR_NULL;
  if (R != kR) return BI_ERR_UNSUPPORTED;
  if (M < 0 || N < 8 || M > (1 << 30) || N > (1 << 23) || ldl < R || ldb < R || ldy < N ||
      (base && ldbase < N))
    return BI_ERR_SHAPE;
  if ((N | ldy) & 7 || (base && (ldbase & 7)) || !aligned16(y) || (base && !aligned16(base)) ||
      ((uintptr_t)l & 3) || ((uintptr_t)b & 1))
    return BI_ERR_ALIGN;
  const Span sy = span_of(y, M, N, ldy, 2);
  const bool in_place = base == y && ldbase == ldy;
  if (overlap(sy, span_of(l, M, R, ldl, 4)) || overlap(sy, span_of(b, N, R, ldb, 2)) ||
      (base && !in_place && overlap(sy, span_of(base, M, N, ldbase, 2))))
    return BI_ERR_ALIAS;
  if (M == 0) return BI_OK;
  const dim3 grid((unsigned)((M + TM - 1) / TM), (unsigned)((N + TN - 1) / TN));
  hipLaunchKernelGGL(lora_expand_kernel, grid, dim3(kThreads), 0, (hipStream_t)stream, l, b, base,
                     y, (int)M, (int)N, ldl, ldb, ldbase, ldy, scale);
  return launch_status();
}
