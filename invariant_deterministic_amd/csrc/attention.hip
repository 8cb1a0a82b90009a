// attention.hip -- batch-invariant decode attention with a fixed split size.
//
// "Cómo superar la no determinación en la inferencia de LLM", section
// "Attention": attention stays batch-invariant when the work is parallel over
// queries and each query's keys/values are reduced in an order that never
// follows the batch; a split-KV (FlashDecoding) reduction keeps one order by
// fixing the split *size* rather than the number of splits; and the cache and
// the new tokens must not take separate paths -- one K/V layout throughout.
//
// Here one decode query per sequence attends to its own cache, the new token
// already appended (one layout).  The keys of sequence b are cut into chunks
// of C tokens (C fixed by the caller, never by the batch); the number of
// chunks follows the sequence's own length T_b only.
//
// Order of every output o[b][h][:] (G = H / Hkv query heads share key/value
// head h / G):
//   chunk c, token t:  s_t = (sum_{d ascending} q[d] * k_t[d]) * scale   (fp32)
//   chunk c:  m_c = max_t s_t;  p_t = exp(s_t - m_c);
//             l_c = sum_t p_t over lanes j = t mod 64 (t ascending within a
//             lane), then a fixed xor tree over the 64 lanes;
//             a_c[d] = sum_{t ascending} p_t * v_t[d]
//   combine:  M = max_c m_c;  L = sum_{c ascending} exp(m_c - M) * l_c;
//             O[d] = sum_{c ascending} exp(m_c - M) * a_c[d];  o = bf16(O / L).
// Decode attention streams the whole cache, so it is bound by HBM bandwidth:
// 2 * T_b * Hkv * D * 2 bytes of K and V per sequence.
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxG = 8;
constexpr int kMaxC = 512;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_chunk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ lens, float *__restrict__ ws,
    int H, int Hkv, int Tmax, int C, int nc_max, float scale) {
  const int c = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int G = H / Hkv;
  int T = lens[b];
  T = T < 1 ? 1 : (T > Tmax ? Tmax : T);
  const int t0 = c * C;
  if (t0 >= T) return;  // this sequence has fewer chunks (uniform over the block)
  const int n = min(C, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  __shared__ float qs[kMaxG][D];
  __shared__ float ps[kMaxG][kMaxC];
  for (int i = tid; i < G * D; i += kThreads) {
    const int g = i / D, d = i % D;
    qs[g][d] = bf16_to_f32(q[((int64_t)b * H + kh * G + g) * D + d]);
  }
  __syncthreads();

  // Scores: thread tid owns tokens tid, tid + 256, ... of the chunk.
  const int64_t row_stride = (int64_t)Hkv * D;  // elements between tokens
  const uint16_t *kbase = kc + ((int64_t)b * Tmax + t0) * row_stride + (int64_t)kh * D;
  for (int t = tid; t < C; t += kThreads) {
    float s[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) s[g] = 0.0f;
    if (t < n) {
      const u32x4 *kr = reinterpret_cast<const u32x4 *>(kbase + (int64_t)t * row_stride);
      u32x4 kv[D / 8];
#pragma unroll
      for (int i = 0; i < D / 8; ++i) kv[i] = __builtin_nontemporal_load(kr + i);
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float k0 = lo_bf16(kv[i][j]), k1 = hi_bf16(kv[i][j]);
          const int d = i * 8 + j * 2;
#pragma unroll
          for (int g = 0; g < kMaxG; ++g) {
            if (g < G) {
              s[g] = s[g] + qs[g][d] * k0;
              s[g] = s[g] + qs[g][d + 1] * k1;
            }
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kMaxG; ++g)
      if (g < G) ps[g][t] = t < n ? s[g] * scale : -INFINITY;
  }
  __syncthreads();

  // Softmax pieces: wavefront w handles heads w, w + 4.
  float *wsb = ws + (((int64_t)b * H + kh * G) * nc_max + c) * (D + 2);
  for (int g = wv; g < G; g += kThreads / 64) {
    float m = -INFINITY;
    for (int t = lane; t < C; t += 64) m = fmaxf(m, ps[g][t]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float l = 0.0f;
    for (int t = lane; t < C; t += 64) {
      const float e = expf(ps[g][t] - m);  // exp(-inf) = 0 for masked tokens
      ps[g][t] = e;
      l = l + e;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l = l + __shfl_xor(l, off, 64);
    if (lane == 0) {
      float *o = wsb + (int64_t)g * nc_max * (D + 2);
      o[D] = m;
      o[D + 1] = l;
    }
  }
  __syncthreads();

  // Weighted values: pair (g, d) -> sum over tokens in ascending order.
  const uint16_t *vbase = vc + ((int64_t)b * Tmax + t0) * row_stride + (int64_t)kh * D;
  for (int pi = tid; pi < G * D; pi += kThreads) {
    const int g = pi / D, d = pi % D;
    float a = 0.0f;
#pragma unroll 8
    for (int t = 0; t < n; ++t) a = a + ps[g][t] * bf16_to_f32(vbase[(int64_t)t * row_stride + d]);
    wsb[(int64_t)g * nc_max * (D + 2) + d] = a;
  }
}

template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float *__restrict__ ws,
                                                         const int32_t *__restrict__ lens,
                                                         uint16_t *__restrict__ o, int H,
                                                         int Tmax, int C, int nc_max) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  int T = lens[b];
  T = T < 1 ? 1 : (T > Tmax ? Tmax : T);
  const int nc = (T + C - 1) / C;
  const float *p = ws + ((int64_t)b * H + h) * nc_max * (D + 2);
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, p[(int64_t)c * (D + 2) + D]);
  float L = 0.0f, O = 0.0f;
  for (int c = 0; c < nc; ++c) {
    const float f = expf(p[(int64_t)c * (D + 2) + D] - M);
    L = L + f * p[(int64_t)c * (D + 2) + D + 1];
    O = O + f * p[(int64_t)c * (D + 2) + d];
  }
  o[((int64_t)b * H + h) * D + d] = f32_to_bf16_rne(O / L);
}

int64_t nchunks(int64_t Tmax, int C) { return (Tmax + C - 1) / C; }

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" size_t bi_decode_attention_workspace_bytes(int64_t B, int64_t H, int64_t Tmax,
                                                      int64_t D, int split_size) {
  if (B <= 0 || H <= 0 || Tmax <= 0 || D <= 0 || split_size <= 0) return 0;
  const size_t b = (size_t)B * (size_t)H * (size_t)nchunks(Tmax, split_size) * (size_t)(D + 2) * 4u;
  return (b + 255u) & ~(size_t)255u;
}

extern "C" int bi_decode_attention(const uint16_t *q, const uint16_t *k_cache,
                                   const uint16_t *v_cache, const int32_t *lens, uint16_t *o,
                                   int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t Tmax,
                                   int split_size, void *ws, size_t ws_bytes, void *stream) {
  if (B > 0 && (!q || !k_cache || !v_cache || !lens || !o || !ws)) return BI_ERR_NULL;
  if (B < 0 || H <= 0 || Hkv <= 0 || Tmax <= 0 || B > 65535 || H > 65535 || Tmax > (1 << 24))
    return BI_ERR_SHAPE;
  if (D != 64 && D != 128) return BI_ERR_UNSUPPORTED;
  if (H % Hkv || H / Hkv > kMaxG) return BI_ERR_UNSUPPORTED;
  if (split_size != 128 && split_size != 256 && split_size != 512) return BI_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned16(ws) || ((uintptr_t)lens & 3))
    return BI_ERR_ALIGN;
  if (B == 0) return BI_OK;
  if (ws_bytes < bi_decode_attention_workspace_bytes(B, H, Tmax, D, split_size))
    return BI_ERR_WORKSPACE;
  const Span so = span_of(o, B * H, D, D, 2);
  const Span sw{(uintptr_t)ws, (uintptr_t)ws + bi_decode_attention_workspace_bytes(B, H, Tmax, D, split_size)};
  const Span sk = span_of(k_cache, B * Tmax * Hkv, D, D, 2), sv = span_of(v_cache, B * Tmax * Hkv, D, D, 2);
  const Span sq = span_of(q, B * H, D, D, 2);
  if (overlap(so, sq) || overlap(so, sk) || overlap(so, sv) || overlap(so, sw) || overlap(sw, sq) ||
      overlap(sw, sk) || overlap(sw, sv))
    return BI_ERR_ALIAS;
  const int nc = (int)nchunks(Tmax, split_size);
  const float scale = 1.0f / sqrtf((float)D);
  hipStream_t s = (hipStream_t)stream;
  float *wsf = static_cast<float *>(ws);
  const dim3 g1((unsigned)nc, (unsigned)Hkv, (unsigned)B), g2((unsigned)H, (unsigned)B);
  if (D == 64) {
    hipLaunchKernelGGL(attn_chunk_kernel<64>, g1, dim3(kThreads), 0, s, q, k_cache, v_cache, lens,
                       wsf, (int)H, (int)Hkv, (int)Tmax, split_size, nc, scale);
    hipLaunchKernelGGL(attn_combine_kernel<64>, g2, dim3(64), 0, s, wsf, lens, o, (int)H,
                       (int)Tmax, split_size, nc);
  } else {
    hipLaunchKernelGGL(attn_chunk_kernel<128>, g1, dim3(kThreads), 0, s, q, k_cache, v_cache, lens,
                       wsf, (int)H, (int)Hkv, (int)Tmax, split_size, nc, scale);
    hipLaunchKernelGGL(attn_combine_kernel<128>, g2, dim3(128), 0, s, wsf, lens, o, (int)H,
                       (int)Tmax, split_size, nc);
  }
  return launch_status();
}
