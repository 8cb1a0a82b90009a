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
// Decode attention streams the whole cache, so it is bound by HBM bandwidth:
// 2 * T_b * Hkv * D * 2 bytes of K and V per sequence.  Both are read as
// whole 128-byte lines with the non-temporal hint: keys into registers, then
// lane-permuted into the matrix-core layout; values as whole rows straight
// into LDS (16-byte units XOR-swizzled by row, so the transposing reads spread
// over the banks), loaded while the scores are computed.
//
// Order of every output o[b][h][:] (G = H / Hkv query heads share key/value
// head h / G; workgroup = 4 wavefronts):
//   score s_t = (q . k_t by v_mfma_f32_16x16x32_bf16 over d blocks of 32,
//               ascending, fp32 accumulator) * scale
//   chunk c:  m_c = max_t s_t;  p_t = exp(s_t - m_c);
//             l_c = sum_t p_t over lanes j = t mod 64 (t ascending within a
//             lane), then a fixed xor tree over the 64 lanes;
//             a_c[d] = sum over 32-token blocks, ascending, of matrix-core
//             products bf16(p_t) * v_t[d] (v_mfma_f32_16x16x32_bf16, fp32
//             accumulator)
//   combine:  M = max_c m_c;  L = sum_{c ascending} exp(m_c - M) * l_c;
//             O[d] = sum_{c ascending} exp(m_c - M) * a_c[d];  o = bf16(O / L).
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxG = 8;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// D: head size; GM: a power of two >= G; C: the split size.
template <int D, int GM, int C>
__global__ __launch_bounds__(kThreads) void attn_chunk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ lens, float *__restrict__ ws,
    int H, int Hkv, int Tmax, int nc_max, float scale) {
  constexpr int NJ = D / 32;                                   // 32-wide d blocks (scores)
  constexpr int VS = C * D * 2 <= 65536 ? C : 65536 / (D * 2);  // value rows per LDS pass
  constexpr int NPASS = C / VS;
  constexpr int RPI = 1024 / (D * 2);                          // value rows per load instruction
  constexpr int LPR = 64 / RPI;                                // lanes per value row
  constexpr int VI = VS / (RPI * 4);                           // load instructions per wavefront per pass
  constexpr int tpw = C / 4;                                   // score tokens per wavefront
  constexpr int NGRP = tpw / 16;
  constexpr int GB = NGRP < 4 ? NGRP : 4;                      // 16-token groups per load batch
  constexpr int CB = D / 64;                                   // 16-wide d blocks per wavefront (values)
  static_assert(VS % 32 == 0 && VS * NPASS == C && VI >= 1 && CB >= 1 && NGRP % GB == 0, "shape");

  const int c = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int G = H / Hkv;
  int T = lens[b];
  T = T < 1 ? 1 : (T > Tmax ? Tmax : T);
  const int t0 = c * C;
  if (t0 >= T) return;  // this sequence has fewer chunks (uniform over the block)
  const int n = min(C, T - t0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  __shared__ __attribute__((aligned(1024))) uint16_t vs[VS * D];
  // Score rows padded by 16 bytes so that rows of different heads start in
  // different LDS banks.
  __shared__ __attribute__((aligned(16))) float ps[GM][C + 4];
  // Value rows in LDS: 16-byte unit u of row r sits at unit u ^ vswz(r), so
  // the 16 rows one transposing read touches (rows 8q + j, j < 4, and the
  // same + 4) fall on different banks instead of all on the same ones (a row
  // is a whole number of bank widths long).
  constexpr int VU = D / 8;  // 16-byte units of a value row
  const auto vswz = [](int r) { return ((r & 3) | (((r >> 3) & 3) << 2)) & (VU - 1); };

  const int64_t row_stride = (int64_t)Hkv * D;  // elements between tokens
  const uint16_t *kseq = kc + ((int64_t)b * Tmax + t0) * row_stride + (int64_t)kh * D;
  const uint16_t *vseq = vc + ((int64_t)b * Tmax + t0) * row_stride + (int64_t)kh * D;

  // Value rows of pass `pass` -> vs (D per row, units swizzled by vswz),
  // direct to LDS: lane l of an instruction fills unit position l % LPR of LDS
  // row row0 + l / LPR, so it loads the row's unit (l % LPR) ^ vswz(row).
  // Rows at or past n load row n - 1 (in bounds, finite; their weight is 0).
  auto issue_v = [&](int pass) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)vseq, (short)0, (int)(((int64_t)(n - 1) * row_stride + D) * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int row0 = (i * 4 + wv) * RPI;
      const int lrow = row0 + lane / LPR;
      const int t = min(pass * VS + lrow, n - 1);
      const int unit = (lane % LPR) ^ vswz(lrow);
      const int off = (int)(((int64_t)t * row_stride + unit * 8) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(vs + row0 * D), 16, off, 0, 0,
                                               kCpolNT);  // read once
    }
  };

  // Scores on the matrix core: s = q . k as v_mfma_f32_16x16x32_bf16 over d
  // blocks of 32 (ascending), query heads as the A rows (zero past G), 16
  // tokens as the B columns.  Lane l supplies head / token (l & 15) and
  // d = 32j + 8(l >> 4) .. +7 of block j; it receives s for token (l & 15),
  // heads 4(l >> 4) .. +3.
  bf16x8 qa[NJ];
  {
    const int g = lane & 15;
    const uint16_t *qr = q + ((int64_t)b * H + kh * G + (g < G ? g : 0)) * D + (lane >> 4) * 8;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      qa[j] = *reinterpret_cast<const bf16x8 *>(qr + 32 * j);
      if (g >= G) qa[j] = bf16x8{};
    }
  }
  static_assert(NJ % 2 == 0, "keys are fetched as 128-byte lines, two d blocks each");
  const int tok = lane & 15;
  const int q8 = lane >> 3, u8 = lane & 7;
#pragma unroll 1
  for (int gb = 0; gb < NGRP; gb += GB) {
    // Keys as whole 128-byte lines, permuted into the matrix-core layout.
    // Tokens at or past n load token n - 1 (in bounds, finite; masked below).
    LineOperand16<NJ / 2, true> kl[GB];
#pragma unroll
    for (int i = 0; i < GB; ++i) {
      const int t16 = wv * tpw + (gb + i) * 16;
      const int tlo = min(t16 + q8, n - 1), thi = min(t16 + 8 + q8, n - 1);
      kl[i].issue(kseq + (int64_t)tlo * row_stride + u8 * 8,
                  kseq + (int64_t)thi * row_stride + (u8 ^ 4) * 8);
    }
    // The first pass of values loads while the scores are computed.
    if (gb == 0) issue_v(0);
#pragma unroll
    for (int i = 0; i < GB; ++i) {
      bf16x8 kf[NJ];
      kl[i].place(kf, lane);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], kf[j], acc, 0, 0, 0);
      const int t = wv * tpw + (gb + i) * 16 + tok;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int g = 4 * (lane >> 4) + v;
        if (g < G) ps[g][t] = t < n ? acc[v] * scale : -INFINITY;
      }
    }
  }
  // The value loads may still be in flight: wait for the score stores only.
  wait_lgkmcnt0();
  barrier_no_fence();

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

  // Weighted values on the matrix core: O[g][d] += P[g][t] V[t][d] as
  // v_mfma_f32_16x16x32_bf16 over 32-token blocks, ascending, with P rounded
  // to bf16 (nearest even).  Wavefront w owns d columns [64w, 64w + 64) in
  // blocks of 16.  A operand: lane l supplies head (l & 15), tokens
  // 8(l >> 4) .. +7 of the block; B operand: the same tokens of column
  // (l & 15), read from the row-major LDS copy by two transposing reads (each
  // lane of a 16-lane group names 4 consecutive columns of one row; lane j of
  // the group receives column j of rows 4h .. 4h+3 of its 8).
  const int q4 = lane >> 4, jl = lane & 15;
  f32x4 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int pass = 0; pass < NPASS; ++pass) {
    if (pass > 0) {
      barrier_no_fence();  // every wavefront is done reading the previous pass
      issue_v(pass);
    }
    wait_vmcnt<0>();  // this wavefront's value rows have landed ...
    wait_lgkmcnt0();
    barrier_no_fence();  // ... and so have every other wavefront's (and the softmax)
#pragma unroll 2
    for (int ks = 0; ks < VS / 32; ++ks) {
      const int tb = pass * VS + ks * 32 + 8 * q4;  // first token of this lane's 8
      u32x4 pa = {0u, 0u, 0u, 0u};
      if (jl < G) {
        const f32x4 p0 = *reinterpret_cast<const f32x4 *>(&ps[jl][tb]);
        const f32x4 p1 = *reinterpret_cast<const f32x4 *>(&ps[jl][tb + 4]);
        pa[0] = pack_bf16x2(p0[0], p0[1]);
        pa[1] = pack_bf16x2(p0[2], p0[3]);
        pa[2] = pack_bf16x2(p1[0], p1[1]);
        pa[3] = pack_bf16x2(p1[2], p1[3]);
      }
      const bf16x8 A = __builtin_bit_cast(bf16x8, pa);
      const int vrow = ks * 32 + 8 * q4 + (jl >> 2);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int d0 = (wv * CB + cb) * 16 + 4 * (jl & 3);
        const int dlo = (((d0 >> 3) ^ vswz(vrow)) << 3) + (d0 & 7);
        const int dhi = (((d0 >> 3) ^ vswz(vrow + 4)) << 3) + (d0 & 7);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16 *)(vs + vrow * D + dlo));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16 *)(vs + (vrow + 4) * D + dhi));
        const v8i16 bb = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bb),
                                                           oacc[cb], 0, 0, 0);
      }
    }
  }
  // Lane l holds O[g = 4(l >> 4) + v][d = block + (l & 15)].
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int d = (wv * CB + cb) * 16 + jl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int g = 4 * q4 + v;
      if (g < G) wsb[(int64_t)g * nc_max * (D + 2) + d] = oacc[cb][v];
    }
  }
}

// Chunk combine for one (head, sequence); thread d owns output column d.
// The order is that of the header: M = max over chunks (exact), then L and
// O[d] summed over chunks c ascending with weights exp(m_c - M).  The loads
// are batched so the loop costs a memory round trip per kCT chunks, not two
// per chunk: chunk statistics go through LDS, kCT rows of values are loaded
// before they are summed.
constexpr int kCT = 16;
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
  constexpr int S = D + 2;  // floats per chunk record

  // The first tile's loads (its statistics and values) do not depend on M:
  // they go out together with the loads M needs, so the usual case (at most
  // kCT chunks) costs one memory round trip after the length.
  float a[kCT];
#pragma unroll
  for (int i = 0; i < kCT; ++i) a[i] = i < nc ? p[(int64_t)i * S + d] : 0.0f;
  const float m_own = d < nc ? p[(int64_t)d * S + D] : -INFINITY;
  const float l_own = d < nc ? p[(int64_t)d * S + D + 1] : 0.0f;

  // M: every thread takes the max over its chunks, then a max over threads
  // (max is exact, so the grouping does not matter).
  __shared__ float red[D / 64];
  float m = m_own;
  for (int c = d + D; c < nc; c += D) m = fmaxf(m, p[(int64_t)c * S + D]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((d & 63) == 0) red[d >> 6] = m;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < D / 64; ++i) M = fmaxf(M, red[i]);

  __shared__ float fw[kCT], lw[kCT];
  float L = 0.0f, O = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += kCT) {
    const int n = min(kCT, nc - c0);
    __syncthreads();  // the previous tile's fw / lw are consumed
    if (d < n) {
      if (c0 == 0) {
        fw[d] = expf(m_own - M);
        lw[d] = l_own;
      } else {
        fw[d] = expf(p[(int64_t)(c0 + d) * S + D] - M);
        lw[d] = p[(int64_t)(c0 + d) * S + D + 1];
      }
    }
    if (c0 > 0) {
#pragma unroll
      for (int i = 0; i < kCT; ++i) a[i] = i < n ? p[(int64_t)(c0 + i) * S + d] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCT; ++i) {
      if (i < n) {
        L = L + fw[i] * lw[i];
        O = O + fw[i] * a[i];
      }
    }
  }
  o[((int64_t)b * H + h) * D + d] = f32_to_bf16_rne(O / L);
}

int64_t nchunks(int64_t Tmax, int C) { return (Tmax + C - 1) / C; }

template <int V>
struct IntC {
  static constexpr int value = V;
};

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
  if ((int64_t)split_size * Hkv * D * 2 > 0x7FFFFFFF) return BI_ERR_UNSUPPORTED;  // 32-bit offsets
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
  const int G = (int)(H / Hkv);
  auto chunk = [&](auto dc, auto gc) {
    constexpr int DD = decltype(dc)::value, GG = decltype(gc)::value;
    if (split_size == 128)
      hipLaunchKernelGGL((attn_chunk_kernel<DD, GG, 128>), g1, dim3(kThreads), 0, s, q, k_cache,
                         v_cache, lens, wsf, (int)H, (int)Hkv, (int)Tmax, nc, scale);
    else if (split_size == 256)
      hipLaunchKernelGGL((attn_chunk_kernel<DD, GG, 256>), g1, dim3(kThreads), 0, s, q, k_cache,
                         v_cache, lens, wsf, (int)H, (int)Hkv, (int)Tmax, nc, scale);
    else
      hipLaunchKernelGGL((attn_chunk_kernel<DD, GG, 512>), g1, dim3(kThreads), 0, s, q, k_cache,
                         v_cache, lens, wsf, (int)H, (int)Hkv, (int)Tmax, nc, scale);
    hipLaunchKernelGGL(attn_combine_kernel<DD>, g2, dim3(DD), 0, s, wsf, lens, o, (int)H,
                       (int)Tmax, split_size, nc);
  };
  auto by_g = [&](auto dc) {
    if (G == 1) chunk(dc, IntC<1>{});
    else if (G == 2) chunk(dc, IntC<2>{});
    else if (G <= 4) chunk(dc, IntC<4>{});
    else chunk(dc, IntC<8>{});
  };
  if (D == 64) by_g(IntC<64>{});
  else by_g(IntC<128>{});
  return launch_status();
}
