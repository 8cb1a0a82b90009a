// bitdiff.hip -- the invariance check on the device: bitwise comparison of rows.
//
// "God Does Not Play Dice: Enforcing Batch Invariance in Agentic Kernel
// Generation", abstract: batch invariance is validated dynamically as bitwise
// consistency of outputs across batch contexts.  This kernel counts, for each
// pair of rows, the differing bits (popcount of the XOR) and the differing
// elements.  Integer counts are exact whatever the order the threads add them.
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;

// One workgroup per compared row pair.  VEC: the row is read as 16-byte
// vectors (every load of a thread issued before any is used, so a row costs one
// memory round trip); otherwise element by element.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void row_bitdiff_kernel(
    const T *__restrict__ a, int64_t lda, const int64_t *__restrict__ a_rows,
    const T *__restrict__ b, int64_t ldb, const int64_t *__restrict__ b_rows, int64_t ncols,
    unsigned long long *__restrict__ counts) {
  const int64_t r = blockIdx.x;
  const int64_t ra = a_rows ? a_rows[r] : r;
  const int64_t rb = b_rows ? b_rows[r] : r;
  const T *pa = a + ra * lda;
  const T *pb = b + rb * ldb;
  unsigned long long bits = 0, elems = 0;
  if (VEC) {
    constexpr int PER = 16 / sizeof(T);  // elements per 16-byte vector
    const u32x4 *va = reinterpret_cast<const u32x4 *>(pa);
    const u32x4 *vb = reinterpret_cast<const u32x4 *>(pb);
    const int64_t nv = ncols / PER;
    constexpr int U = 4;
    for (int64_t c0 = threadIdx.x; c0 < nv; c0 += (int64_t)kThreads * U) {
      u32x4 xa[U], xb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + (int64_t)u * kThreads;
        if (c < nv) {
          xa[u] = va[c];
          xb[u] = vb[c];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + (int64_t)u * kThreads;
        if (c < nv) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t d = xa[u][j] ^ xb[u][j];
            bits += (unsigned long long)__popc(d);
            if (sizeof(T) == 4) {
              elems += d ? 1ull : 0ull;
            } else {
              elems += (d & 0xFFFFu) ? 1ull : 0ull;
              elems += (d >> 16) ? 1ull : 0ull;
            }
          }
        }
      }
    }
  } else {
    for (int64_t c = threadIdx.x; c < ncols; c += kThreads) {
      const uint32_t d = (uint32_t)(pa[c] ^ pb[c]);
      bits += (unsigned long long)__popc(d);
      elems += d ? 1ull : 0ull;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    bits += __shfl_xor(bits, off, 64);
    elems += __shfl_xor(elems, off, 64);
  }
  __shared__ unsigned long long sb[kThreads / 64], se[kThreads / 64];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sb[wv] = bits;
    se[wv] = elems;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long tb = 0, te = 0;
    for (int i = 0; i < kThreads / 64; ++i) {
      tb += sb[i];
      te += se[i];
    }
    counts[2 * r] = tb;
    counts[2 * r + 1] = te;
  }
}

// Several comparisons in one launch: workgroup r takes row r - start[i] of
// item i, where start[i] <= r < start[i + 1].  The same per-row count as
// row_bitdiff_kernel (every row here takes the 16-byte path: the host
// requires it).  The item table travels by value as a kernel argument.
struct BatchArgs {
  const void *a[BI_BITDIFF_BATCH_MAX];
  const void *b[BI_BITDIFF_BATCH_MAX];
  const int64_t *a_rows[BI_BITDIFF_BATCH_MAX];
  const int64_t *b_rows[BI_BITDIFF_BATCH_MAX];
  unsigned long long *counts[BI_BITDIFF_BATCH_MAX];
  int64_t lda[BI_BITDIFF_BATCH_MAX], ldb[BI_BITDIFF_BATCH_MAX], ncols[BI_BITDIFF_BATCH_MAX];
  int64_t start[BI_BITDIFF_BATCH_MAX + 1];
  int elem_bytes[BI_BITDIFF_BATCH_MAX];
  int n;
};

__global__ __launch_bounds__(kThreads) void row_bitdiff_batch_kernel(const BatchArgs args) {
  const int64_t g = blockIdx.x;
  int i = 0;
  while (i + 1 < args.n && g >= args.start[i + 1]) ++i;  // uniform over the workgroup
  const int64_t r = g - args.start[i];
  const int64_t ra = args.a_rows[i] ? args.a_rows[i][r] : r;
  const int64_t rb = args.b_rows[i] ? args.b_rows[i][r] : r;
  const int eb = args.elem_bytes[i];
  const u32x4 *va = reinterpret_cast<const u32x4 *>(static_cast<const char *>(args.a[i]) + ra * args.lda[i] * eb);
  const u32x4 *vb = reinterpret_cast<const u32x4 *>(static_cast<const char *>(args.b[i]) + rb * args.ldb[i] * eb);
  const int64_t nv = args.ncols[i] * eb / 16;
  unsigned long long bits = 0, elems = 0;
  constexpr int U = 4;
  for (int64_t c0 = threadIdx.x; c0 < nv; c0 += (int64_t)kThreads * U) {
    u32x4 xa[U], xb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + (int64_t)u * kThreads;
      if (c < nv) {
        xa[u] = va[c];
        xb[u] = vb[c];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + (int64_t)u * kThreads;
      if (c < nv) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t d = xa[u][j] ^ xb[u][j];
          bits += (unsigned long long)__popc(d);
          if (eb == 4) {
            elems += d ? 1ull : 0ull;
          } else {
            elems += (d & 0xFFFFu) ? 1ull : 0ull;
            elems += (d >> 16) ? 1ull : 0ull;
          }
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    bits += __shfl_xor(bits, off, 64);
    elems += __shfl_xor(elems, off, 64);
  }
  __shared__ unsigned long long sb[kThreads / 64], se[kThreads / 64];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sb[wv] = bits;
    se[wv] = elems;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long tb = 0, te = 0;
    for (int k = 0; k < kThreads / 64; ++k) {
      tb += sb[k];
      te += se[k];
    }
    args.counts[i][2 * r] = tb;
    args.counts[i][2 * r + 1] = te;
  }
}

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" int bi_row_bitdiff_batch(const bi_bitdiff_item *items, int nitems, void *stream) {
  if (!items) return BI_ERR_NULL;
  if (nitems < 1 || nitems > BI_BITDIFF_BATCH_MAX) return BI_ERR_UNSUPPORTED;
  BatchArgs args{};
  args.n = nitems;
  int64_t total = 0;
  for (int i = 0; i < nitems; ++i) {
    const bi_bitdiff_item &it = items[i];
    if (!it.a || !it.b || !it.counts) return BI_ERR_NULL;
    if (it.elem_bytes != 2 && it.elem_bytes != 4) return BI_ERR_UNSUPPORTED;
    if (it.nrows < 0 || it.ncols <= 0 || it.lda < it.ncols || it.ldb < it.ncols ||
        it.nrows > 0x7FFFFFFF)
      return BI_ERR_SHAPE;
    // every row must start 16-byte aligned and hold whole 16-byte vectors
    if (((uintptr_t)it.a | (uintptr_t)it.b) % 16 || (it.lda * it.elem_bytes) % 16 ||
        (it.ldb * it.elem_bytes) % 16 || (it.ncols * it.elem_bytes) % 16 || ((uintptr_t)it.counts & 7))
      return BI_ERR_ALIGN;
    args.a[i] = it.a;
    args.b[i] = it.b;
    args.a_rows[i] = it.a_rows;
    args.b_rows[i] = it.b_rows;
    args.counts[i] = reinterpret_cast<unsigned long long *>(it.counts);
    args.lda[i] = it.lda;
    args.ldb[i] = it.ldb;
    args.ncols[i] = it.ncols;
    args.elem_bytes[i] = it.elem_bytes;
    args.start[i] = total;
    total += it.nrows;
  }
  args.start[nitems] = total;
  if (total > 0x7FFFFFFF) return BI_ERR_SHAPE;
  if (total == 0) return BI_OK;
  hipLaunchKernelGGL(row_bitdiff_batch_kernel, dim3((unsigned)total), dim3(kThreads), 0,
                     (hipStream_t)stream, args);
  return launch_status();
}

extern "C" int bi_row_bitdiff(const void *a, int64_t lda, const int64_t *a_rows, const void *b,
                              int64_t ldb, const int64_t *b_rows, int64_t nrows, int64_t ncols,
                              int elem_bytes, uint64_t *counts, void *stream) {
  if (!a || !b || !counts) return BI_ERR_NULL;
  if (elem_bytes != 2 && elem_bytes != 4) return BI_ERR_UNSUPPORTED;
  if (nrows < 0 || ncols <= 0 || lda < ncols || ldb < ncols || nrows > 0x7FFFFFFF)
    return BI_ERR_SHAPE;
  if (((uintptr_t)a | (uintptr_t)b) & (uintptr_t)(elem_bytes - 1) || ((uintptr_t)counts & 7))
    return BI_ERR_ALIGN;
  if (nrows == 0) return BI_OK;
  hipStream_t s = (hipStream_t)stream;
  unsigned long long *c = reinterpret_cast<unsigned long long *>(counts);
  // 16-byte vectors when every row starts 16-byte aligned and holds whole vectors
  const bool vec = ((uintptr_t)a % 16 == 0) && ((uintptr_t)b % 16 == 0) &&
                   (lda * elem_bytes) % 16 == 0 && (ldb * elem_bytes) % 16 == 0 &&
                   (ncols * elem_bytes) % 16 == 0;
  const dim3 grid((unsigned)nrows), block(kThreads);
  if (elem_bytes == 2) {
    const uint16_t *pa = (const uint16_t *)a, *pb = (const uint16_t *)b;
    if (vec)
      hipLaunchKernelGGL((row_bitdiff_kernel<uint16_t, true>), grid, block, 0, s, pa, lda, a_rows, pb, ldb, b_rows, ncols, c);
    else
      hipLaunchKernelGGL((row_bitdiff_kernel<uint16_t, false>), grid, block, 0, s, pa, lda, a_rows, pb, ldb, b_rows, ncols, c);
  } else {
    const uint32_t *pa = (const uint32_t *)a, *pb = (const uint32_t *)b;
    if (vec)
      hipLaunchKernelGGL((row_bitdiff_kernel<uint32_t, true>), grid, block, 0, s, pa, lda, a_rows, pb, ldb, b_rows, ncols, c);
    else
      hipLaunchKernelGGL((row_bitdiff_kernel<uint32_t, false>), grid, block, 0, s, pa, lda, a_rows, pb, ldb, b_rows, ncols, c);
  }
  return launch_status();
}
