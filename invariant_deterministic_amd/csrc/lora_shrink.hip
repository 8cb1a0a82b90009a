// lora_shrink.hip -- LoRA shrink y[m][r] = sum_k x[m][k] * a[r][k] with split-K:
// deterministic fixed-order combine, unsplit reduction, and the atomic control.
//
// "Reproducible LoRA Inference Through Deterministic Split-K Reduction",
// abstract: split-K brings parallelism to the low-rank shrink; combining its
// partial sums with floating-point atomics makes the FP32 shrink output vary
// between identical runs, while a combine in a fixed order does not, at a small
// latency cost over the atomic version and a speed-up over no split at all.
//
// Reduction order (batch- and run-invariant for every path but the atomic one):
//   chunk s covers k in [s*Kc, (s+1)*Kc), Kc = K / S; inside a chunk, one
//   ascending pass in steps of 32 k, one v_mfma_f32_16x16x32_bf16 per step,
//   fp32 accumulator rounded between steps; then
//   y = (((p_0 + p_1) + p_2) + ...) + p_{S-1} in fp32.
// S == 1 is the unsplit reduction: one pass over all of K.
//
// Three ways to run it, all computing the same partials p_s:
//   fused     (bi_lora_shrink): one kernel.  A workgroup is S wavefronts over
//             one 16-row block; wavefront s computes p_s, the S partials meet in
//             LDS (the on-chip fp32 workspace) and wavefront 0 folds them in
//             order.  No second launch, no atomics, no counters.
//   two-pass  (bi_lora_shrink_two_pass): the split spans workgroups; partials go
//             through the caller's fp32 workspace in HBM and a second kernel
//             folds them in order.  Same bits as fused.
//   atomic    (bi_lora_shrink_atomic): the fused layout, but each wavefront adds
//             its partial into the zeroed output with a floating-point atomic,
//             in arrival order.  The nondeterministic control.
// The shrink reads x once from HBM (2*K bytes a row) and the small a from
// cache, so it is bound by HBM bandwidth.
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerBlock = kRowsPerWave * (kThreads / 64);
constexpr int kR = 16;        // LoRA rank handled by the 16x16x32 instruction
constexpr int kStep = 32;     // k per matrix-core step
constexpr int kGroup = 8;     // steps whose loads are issued together

enum Mode { kStoreOut = 0, kStoreWs = 1, kAtomic = 2 };

// One wavefront: 16 rows x 16 ranks over k in [k0, k0 + steps*32).
// Operand roles: the A operand is the LoRA matrix (16 ranks x 32 k), the B
// operand is x (32 k x 16 rows).  Lane l supplies rank / row (l & 15) and
// k = step*32 + (l >> 4)*8 .. +7 of both operands, so products pair matching
// k.  Output lane l holds row (l & 15), ranks 4*(l >> 4) .. +3.
template <int MODE>
__global__ __launch_bounds__(kThreads) void shrink_partial_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ a, float *__restrict__ out,
    int M, int K, int64_t ldx, int64_t lda, int64_t ldo, int chunk) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int mw = blockIdx.x * kRowsPerBlock + wv * kRowsPerWave;
  if (mw >= M) return;  // every row of this wavefront is past the batch
  const int s = blockIdx.y;
  const int k0 = s * chunk;
  const int steps = chunk / kStep;

  int gm = mw + (lane & 15);
  gm = gm < M ? gm : M - 1;  // rows past M read a copy of the last row, never stored
  const int koff = (lane >> 4) * 8;
  const bf16x8 *xp = reinterpret_cast<const bf16x8 *>(x + (int64_t)gm * ldx + k0 + koff);
  const bf16x8 *ap = reinterpret_cast<const bf16x8 *>(a + (int64_t)(lane & 15) * lda + k0 + koff);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bf16x8 xf[kGroup], af[kGroup];
  // Prefetch group 0, then keep one group of loads in flight ahead of the math.
  const int ngroups = (steps + kGroup - 1) / kGroup;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    if (i < steps) {
      xf[i] = __builtin_nontemporal_load(xp + i * (kStep / 8));
      af[i] = ap[i * (kStep / 8)];
    }
  }
  for (int g = 0; g < ngroups; ++g) {
    bf16x8 xn[kGroup], an[kGroup];
    const int base = (g + 1) * kGroup;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (base + i < steps) {
        xn[i] = __builtin_nontemporal_load(xp + (base + i) * (kStep / 8));
        an[i] = ap[(base + i) * (kStep / 8)];
      }
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (g * kGroup + i < steps) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], xf[i], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      xf[i] = xn[i];
      af[i] = an[i];
    }
  }

  const int m = mw + (lane & 15);
  if (m >= M) return;
  const int r0 = (lane >> 4) * 4;
  if (MODE == kStoreOut) {
    *reinterpret_cast<f32x4 *>(out + (int64_t)m * ldo + r0) = acc;
  } else if (MODE == kStoreWs) {
    *reinterpret_cast<f32x4 *>(out + ((int64_t)s * M + m) * kR + r0) = acc;
  } else {
    float *o = out + (int64_t)m * ldo + r0;
#pragma unroll
    for (int v = 0; v < 4; ++v) unsafeAtomicAdd(o + v, acc[v]);
  }
}

// Fused split-K: blockDim = 64 * S; wavefront s computes p_s of the 16 rows
// [blockIdx.x * 16, +16) over chunk s.  Same operand roles, k mapping and step
// order as shrink_partial_kernel.  MODE: kStoreOut folds through LDS (and, if
// ws != nullptr, also stores each p_s there); kAtomic adds each p_s into y.
template <int S, int MODE>
__global__ __launch_bounds__(64 * S) void shrink_fused_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ a, float *__restrict__ y,
    float *__restrict__ ws, int M, int K, int64_t ldx, int64_t lda, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int s = threadIdx.x >> 6;
  const int m0 = blockIdx.x * kRowsPerWave;
  const int chunk = K / S;
  const int k0 = s * chunk;
  const int steps = chunk / kStep;

  int gm = m0 + (lane & 15);
  gm = gm < M ? gm : M - 1;  // rows past M read a copy of the last row, never stored
  const int koff = (lane >> 4) * 8;
  const bf16x8 *xp = reinterpret_cast<const bf16x8 *>(x + (int64_t)gm * ldx + k0 + koff);
  const bf16x8 *ap = reinterpret_cast<const bf16x8 *>(a + (int64_t)(lane & 15) * lda + k0 + koff);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bf16x8 xf[kGroup], af[kGroup];
  const int ngroups = (steps + kGroup - 1) / kGroup;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    if (i < steps) {
      xf[i] = __builtin_nontemporal_load(xp + i * (kStep / 8));
      af[i] = ap[i * (kStep / 8)];
    }
  }
  for (int g = 0; g < ngroups; ++g) {
    bf16x8 xn[kGroup], an[kGroup];
    const int base = (g + 1) * kGroup;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (base + i < steps) {
        xn[i] = __builtin_nontemporal_load(xp + (base + i) * (kStep / 8));
        an[i] = ap[(base + i) * (kStep / 8)];
      }
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (g * kGroup + i < steps) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], xf[i], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      xf[i] = xn[i];
      af[i] = an[i];
    }
  }

  const int m = m0 + (lane & 15);
  const int r0 = (lane >> 4) * 4;
  if (MODE == kAtomic) {
    if (m < M) {
      float *o = y + (int64_t)m * ldy + r0;
#pragma unroll
      for (int v = 0; v < 4; ++v) unsafeAtomicAdd(o + v, acc[v]);
    }
    return;
  }
  if (S == 1) {
    if (m < M) *reinterpret_cast<f32x4 *>(y + (int64_t)m * ldy + r0) = acc;
    return;
  }
  if (ws != nullptr && m < M) *reinterpret_cast<f32x4 *>(ws + ((int64_t)s * M + m) * kR + r0) = acc;
  __shared__ f32x4 part[S][64];
  part[s][lane] = acc;
  __syncthreads();
  if (s == 0 && m < M) {
    f32x4 t = part[0][lane];
#pragma unroll
    for (int q = 1; q < S; ++q) t = t + part[q][lane];  // element-wise fp32, q ascending
    *reinterpret_cast<f32x4 *>(y + (int64_t)m * ldy + r0) = t;
  }
}

template <int MODE>
void launch_fused(int S, dim3 grid, hipStream_t st, const uint16_t *x, const uint16_t *a, float *y,
                  float *ws, int M, int K, int64_t ldx, int64_t lda, int64_t ldy) {
  switch (S) {
    case 1: hipLaunchKernelGGL((shrink_fused_kernel<1, MODE>), grid, dim3(64), 0, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
    case 2: hipLaunchKernelGGL((shrink_fused_kernel<2, MODE>), grid, dim3(128), 0, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
    case 4: hipLaunchKernelGGL((shrink_fused_kernel<4, MODE>), grid, dim3(256), 0, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
    case 8: hipLaunchKernelGGL((shrink_fused_kernel<8, MODE>), grid, dim3(512), 0, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
    default: hipLaunchKernelGGL((shrink_fused_kernel<16, MODE>), grid, dim3(1024), 0, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
  }
}

// Fixed-order combine: y[m][r] = (((p_0 + p_1) + p_2) + ...) + p_{S-1}.
__global__ __launch_bounds__(kThreads) void shrink_combine_kernel(const float *__restrict__ ws,
                                                                  float *__restrict__ y, int M,
                                                                  int S, int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t n = (int64_t)M * kR;
  if (e >= n) return;
  float acc = ws[e];
  for (int s = 1; s < S; ++s) acc = acc + ws[(int64_t)s * n + e];
  y[(e / kR) * ldy + (e % kR)] = acc;
}

// Zero the [M, R] output before the atomic adds (a kernel rather than a
// memset, so the call stays safe to record in a graph).
__global__ __launch_bounds__(kThreads) void zero_rows_kernel(float *__restrict__ y, int M,
                                                             int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= (int64_t)M * kR) return;
  y[(e / kR) * ldy + (e % kR)] = 0.0f;
}

bool split_ok(int S) { return S == 1 || S == 2 || S == 4 || S == 8 || S == 16; }

int validate(const uint16_t *x, const uint16_t *a, float *y, int64_t M, int64_t K, int64_t R,
             int64_t ldx, int64_t lda, int64_t ldy, int S) {
  if (!a || (M > 0 && (!x || !y))) return BI_ERR_NULL;
  if (R != kR) return BI_ERR_UNSUPPORTED;
  if (!split_ok(S)) return BI_ERR_UNSUPPORTED;
  if (M < 0 || K <= 0 || M > (1 << 30) || K > (1 << 30) || ldx < K || lda < K || ldy < R)
    return BI_ERR_SHAPE;
  if (K % (kStep * S)) return BI_ERR_SHAPE;
  if ((ldx | lda) & 7 || ldy & 3 || !aligned16(x) || !aligned16(a) || !aligned16(y))
    return BI_ERR_ALIGN;
  const Span sy = span_of(y, M, R, ldy, 4);
  if (overlap(sy, span_of(x, M, K, ldx, 2)) || overlap(sy, span_of(a, R, K, lda, 2)))
    return BI_ERR_ALIAS;
  return BI_OK;
}

int validate_ws(const uint16_t *x, const uint16_t *a, float *y, int64_t M, int64_t K, int64_t R,
                int64_t ldx, int64_t lda, int64_t ldy, int S, void *ws, size_t ws_bytes) {
  if (ws_bytes < bi_lora_shrink_workspace_bytes(M, R, S)) return BI_ERR_WORKSPACE;
  if (!aligned16(ws)) return BI_ERR_ALIGN;
  const Span sw{(uintptr_t)ws, (uintptr_t)ws + (uintptr_t)(S * M * R * 4)};
  if (overlap(sw, span_of(y, M, R, ldy, 4)) || overlap(sw, span_of(x, M, K, ldx, 2)) ||
      overlap(sw, span_of(a, R, K, lda, 2)))
    return BI_ERR_ALIAS;
  return BI_OK;
}

dim3 partial_grid(int64_t M, int S) {
  return dim3((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)S);
}

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" size_t bi_lora_shrink_workspace_bytes(int64_t M, int64_t R, int split_k) {
  if (M <= 0 || R <= 0 || split_k <= 1) return 0;
  const size_t b = (size_t)split_k * (size_t)M * (size_t)R * 4u;
  return (b + 255u) & ~(size_t)255u;
}

extern "C" int bi_lora_shrink(const uint16_t *x, const uint16_t *a, float *y, int64_t M, int64_t K,
                              int64_t R, int64_t ldx, int64_t lda, int64_t ldy, int split_k,
                              void *ws, size_t ws_bytes, void *stream) {
  int st = validate(x, a, y, M, K, R, ldx, lda, ldy, split_k);
  if (st != BI_OK) return st;
  if (split_k > 1 && ws != nullptr && (st = validate_ws(x, a, y, M, K, R, ldx, lda, ldy, split_k, ws, ws_bytes)) != BI_OK)
    return st;
  if (M == 0) return BI_OK;
  launch_fused<kStoreOut>(split_k, dim3((unsigned)((M + kRowsPerWave - 1) / kRowsPerWave)),
                          (hipStream_t)stream, x, a, y, split_k > 1 ? static_cast<float *>(ws) : nullptr,
                          (int)M, (int)K, ldx, lda, ldy);
  return launch_status();
}

extern "C" int bi_lora_shrink_two_pass(const uint16_t *x, const uint16_t *a, float *y, int64_t M,
                                       int64_t K, int64_t R, int64_t ldx, int64_t lda, int64_t ldy,
                                       int split_k, void *ws, size_t ws_bytes, void *stream) {
  int st = validate(x, a, y, M, K, R, ldx, lda, ldy, split_k);
  if (st != BI_OK) return st;
  if (split_k > 1) {
    if (!ws && M > 0) return BI_ERR_NULL;
    if ((st = validate_ws(x, a, y, M, K, R, ldx, lda, ldy, split_k, ws, ws_bytes)) != BI_OK) return st;
  }
  if (M == 0) return BI_OK;
  hipStream_t s = (hipStream_t)stream;
  const int chunk = (int)(K / split_k);
  if (split_k == 1) {
    hipLaunchKernelGGL(shrink_partial_kernel<kStoreOut>, partial_grid(M, 1), dim3(kThreads), 0, s,
                       x, a, y, (int)M, (int)K, ldx, lda, ldy, chunk);
    return launch_status();
  }
  float *wsf = static_cast<float *>(ws);
  hipLaunchKernelGGL(shrink_partial_kernel<kStoreWs>, partial_grid(M, split_k), dim3(kThreads), 0,
                     s, x, a, wsf, (int)M, (int)K, ldx, lda, (int64_t)kR, chunk);
  if ((st = launch_status()) != BI_OK) return st;
  const int64_t n = M * kR;
  hipLaunchKernelGGL(shrink_combine_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, wsf, y, (int)M, split_k, ldy);
  return launch_status();
}

extern "C" int bi_lora_shrink_atomic(const uint16_t *x, const uint16_t *a, float *y, int64_t M,
                                     int64_t K, int64_t R, int64_t ldx, int64_t lda, int64_t ldy,
                                     int split_k, void *stream) {
  int st = validate(x, a, y, M, K, R, ldx, lda, ldy, split_k);
  if (st != BI_OK || M == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = M * kR;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, y, (int)M, ldy);
  if ((st = launch_status()) != BI_OK) return st;
  launch_fused<kAtomic>(split_k, dim3((unsigned)((M + kRowsPerWave - 1) / kRowsPerWave)), s, x, a, y,
                        nullptr, (int)M, (int)K, ldx, lda, ldy);
  return launch_status();
}
