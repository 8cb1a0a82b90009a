// lora_expand.hip -- LoRA expand: y[m][n] = bf16(base[m][n] + scale * sum_r l[m][r] * b[n][r]).
//
// "Reproducible LoRA Inference Through Deterministic Split-K Reduction",
// abstract: LoRA adds low-rank multiplications to a layer; the fp32 shrink
// output l (rank R) is expanded back to the layer width and added to the base
// output.  With R = 16 the reduction is short, so there is no split: every
// output accumulates its 16 products in ascending r with fp32 fused
// multiply-adds (one rounding per step), scales, adds the base and rounds to
// bf16 once -- the same order at any batch size.
//
// The expand streams base and y (4 bytes an output) and is bound by HBM
// bandwidth once its arithmetic is lean (16 fp32 FMAs an output at 16 lanes
// per SIMD cycle is close to the HBM time).  Each wavefront owns 512
// consecutive columns -- 8 per lane, 16 bytes of base and of y -- for a run of
// rows: its lanes hold their 8 columns of b, widened to fp32, in registers for
// the whole run (staged through LDS once per workgroup, whole-line loads),
// each row's 16 values of l arrive through the scalar cache, and the row loop
// keeps two batches of kAhead rows of base loads in flight.
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int kR = 16;
constexpr int kCols = 512;   // columns per wavefront: 64 lanes x 8
constexpr int kAhead = 4;    // rows per batch: two batches (8 rows) of base loads in flight

// grid: x = column slice of 512, y = row group; wavefront w of the workgroup
// takes rows [(blockIdx.y * 4 + w) * rpw, + rpw).  HAS_BASE: base != NULL.
template <bool HAS_BASE>
__global__ __launch_bounds__(kThreads) void lora_expand_kernel(
    const float *__restrict__ l, const uint16_t *__restrict__ b, const uint16_t *base,
    uint16_t *y, int M, int N, int64_t ldl, int64_t ldb, int64_t ldbase, int64_t ldy,
    float scale, int rpw) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice0 = blockIdx.x * kCols;
  const int n0 = slice0 + lane * 8;
  const bool col_ok = n0 < N;  // N is a multiple of 8: a lane's 8 columns are all in or all out
  const int nn = col_ok ? n0 : N - 8;

  // The slice's 512 rows of b (16 KiB, the same for the 4 wavefronts) go to
  // LDS once through whole-line loads: thread t moves 16-byte units t, t +
  // 256, ... of the slice's rows.  The 16 units a lane needs (its 8 rows)
  // form block L = lane; unit c of block L is stored at c ^ (L & 15), so the
  // lanes of one read touch different banks.  Rows past N load row N - 1
  // (unused).
  __shared__ u32x4 bs[kCols * kR / 8];
#pragma unroll
  for (int i = 0; i < kCols * kR / 8 / kThreads; ++i) {
    const int u = threadIdx.x + i * kThreads;
    const int L = u >> 4, c = u & 15;
    const int n = min(slice0 + (u >> 1), N - 1);
    bs[L * 16 + (c ^ (L & 15))] =
        *reinterpret_cast<const u32x4 *>(b + (int64_t)n * ldb + (u & 1) * 8);
  }
  __syncthreads();

  const int m_begin = (blockIdx.y * 4 + wv) * rpw;
  if (m_begin >= M) return;
  const int m_end = min(M, m_begin + rpw);

  // This lane's 8 columns of b, widened to fp32 once (exact) and kept in
  // registers for the whole run of rows: the row loop is then 16 fused
  // multiply-adds an output and nothing else per rank.
  float bf[8][kR];
  const int L = (nn - slice0) >> 3;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 w0 = bs[L * 16 + ((2 * j) ^ (L & 15))];
    const u32x4 w1 = bs[L * 16 + ((2 * j + 1) ^ (L & 15))];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf[j][2 * i] = lo_bf16(w0[i]);
      bf[j][2 * i + 1] = hi_bf16(w0[i]);
      bf[j][8 + 2 * i] = lo_bf16(w1[i]);
      bf[j][8 + 2 * i + 1] = hi_bf16(w1[i]);
    }
  }

  auto row = [&](int m, u32x4 bv) {
    const float *lr = l + (int64_t)m * ldl;  // uniform over the wavefront: scalar loads
    float lv[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) lv[r] = lr[r];
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        acc0 = __builtin_fmaf(lv[r], bf[2 * k][r], acc0);
        acc1 = __builtin_fmaf(lv[r], bf[2 * k + 1][r], acc1);
      }
      const float v0 = lo_bf16(bv[k]) + scale * acc0;
      const float v1 = hi_bf16(bv[k]) + scale * acc1;
      o[k] = pack_bf16x2(v0, v1);
    }
    // streamed out: nothing re-reads y within the launch (measured 12 % faster
    // than cached stores at M = 16384)
    if (col_ok) __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(y + (int64_t)m * ldy + nn));
  };
  auto load_base = [&](int m) -> u32x4 {
    if (!HAS_BASE) return u32x4{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + (int64_t)m * ldbase + nn));
  };

  // Rows in batches of kAhead, software-pipelined over two register sets
  // (no copies between them, so no wait for loads in flight): one batch's
  // loads fly while the other batch computes.  Rows past the run load its
  // last row again (an L2 hit) and are not computed.
  auto load_batch = [&](u32x4 (&v)[kAhead], int m) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i) v[i] = load_base(min(m + i, m_end - 1));
  };
  auto compute_batch = [&](const u32x4 (&v)[kAhead], int m) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i)
      if (m + i < m_end) row(m + i, v[i]);
  };
  u32x4 va[kAhead], vb[kAhead];
  load_batch(va, m_begin);
  for (int m = m_begin; m < m_end; m += 2 * kAhead) {
    load_batch(vb, m + kAhead);
    compute_batch(va, m);
    load_batch(va, m + 2 * kAhead);
    compute_batch(vb, m + kAhead);
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
  if ((N | ldy | ldb) & 7 || (base && (ldbase & 7)) || !aligned16(y) || (base && !aligned16(base)) ||
      ((uintptr_t)l & 3) || !aligned16(b))
    return BI_ERR_ALIGN;
  const Span sy = span_of(y, M, N, ldy, 2);
  const bool in_place = base == y && ldbase == ldy;
  if (overlap(sy, span_of(l, M, R, ldl, 4)) || overlap(sy, span_of(b, N, R, ldb, 2)) ||
      (base && !in_place && overlap(sy, span_of(base, M, N, ldbase, 2))))
    return BI_ERR_ALIAS;
  if (M == 0) return BI_OK;
  // Rows per wavefront: enough wavefronts to fill the chip (about 2048), at
  // least kAhead rows each so the b registers are amortised.
  const int64_t slices = (N + kCols - 1) / kCols;
  int64_t rpw = (M * slices + 2047) / 2048;
  rpw = rpw < kAhead ? kAhead : ((rpw + kAhead - 1) / kAhead) * kAhead;
  const int64_t groups = (M + 4 * rpw - 1) / (4 * rpw);
  const dim3 grid((unsigned)slices, (unsigned)groups);
  if (base)
    hipLaunchKernelGGL(lora_expand_kernel<true>, grid, dim3(kThreads), 0, (hipStream_t)stream, l, b,
                       base, y, (int)M, (int)N, ldl, ldb, ldbase, ldy, scale, (int)rpw);
  else
    hipLaunchKernelGGL(lora_expand_kernel<false>, grid, dim3(kThreads), 0, (hipStream_t)stream, l, b,
                       base, y, (int)M, (int)N, ldl, ldb, ldbase, ldy, scale, (int)rpw);
  return launch_status();
}
