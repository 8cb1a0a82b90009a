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
//             row blocks (16 rows; 8 for small batches); wavefront s computes
//             p_s, the S partials meet in
//             LDS (the on-chip fp32 workspace) and wavefront 0 folds them in
//             order.  No second launch, no atomics, no counters.
//   two-pass  (bi_lora_shrink_two_pass): the split spans workgroups; partials go
//             through the caller's fp32 workspace in HBM and a second kernel
//             folds them in order.  Same bits as fused.
//   atomic    (bi_lora_shrink_atomic): the fused layout, but each wavefront adds
//             its partial into the zeroed output with a floating-point atomic,
//             in arrival order.  The nondeterministic control.
// The shrink reads x once from HBM (2*K bytes a row) and the small a from
// cache, so it is bound by HBM bandwidth.  Two things decide how close it gets:
// how many requests a byte of x costs, and how often a is fetched again.
//   staged kernel (S = 8, 16, the deterministic split): each wavefront keeps
//     its chunk of a in registers for the whole launch, fetched as whole
//     128-byte lines and moved into the matrix-core layout by lane permutes;
//     x reaches LDS through non-temporal direct-to-LDS loads of whole lines
//     (1 KiB per instruction), two pieces in flight per wavefront, and is read
//     back in the matrix-core layout.  Workgroups are persistent over row
//     blocks, so a is fetched once per workgroup rather than once per row
//     block.
//   streamed kernel (other splits, and the two-pass partials): x and a go
//     straight to registers as whole lines, a group of 8 steps per load
//     batch, up to 3 batches in flight, and are lane-permuted into the
//     matrix-core layout before their steps.
// Every kernel feeds the matrix core the same operands in the same step
// order, so they all produce the same bits.
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerBlock = kRowsPerWave * (kThreads / 64);
constexpr int kR = 16;        // LoRA rank handled by the 16x16x32 instruction
constexpr int kStep = 32;     // k per matrix-core step

enum Mode { kStoreOut = 0, kStoreWs = 1, kAtomic = 2 };

// Operand roles of every kernel here: the A operand is the LoRA matrix
// (16 ranks x 32 k), the B operand is x (32 k x 16 rows).  Lane l supplies
// rank / row (l & 15) and k = step*32 + (l >> 4)*8 .. +7 of both operands, so
// products pair matching k.  Output lane l holds row (l & 15), ranks
// 4*(l >> 4) .. +3.
__device__ __forceinline__ f32x4 mfma_step(bf16x8 a, bf16x8 x, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, x, acc, 0, 0, 0);
}

// Where one lane reads its operands: the matrix-core layout (mx / ma: row
// l & 15, 16-byte unit l >> 4 of each step) for the one-step-at-a-time path,
// and the whole-line layout of LineOperand16 (lo / hi rows of x and a) for
// the streamed path.  Rows of x past M read a copy of the last row, never
// stored.  All point at column k0 of the chunk.
struct ChunkPtrs {
  const bf16x8 *mx, *ma;
  const uint16_t *xlo, *xhi, *alo, *ahi;
};
__device__ __forceinline__ ChunkPtrs chunk_ptrs(const uint16_t *x, const uint16_t *a, int M,
                                                int64_t ldx, int64_t lda, int m0, int k0,
                                                int lane) {
  const auto row = [&](int r) { return (int64_t)(r < M ? r : M - 1); };
  const int q = lane >> 3, u = lane & 7;
  const int koff = (lane >> 4) * 8;
  ChunkPtrs p;
  p.mx = reinterpret_cast<const bf16x8 *>(x + row(m0 + (lane & 15)) * ldx + k0 + koff);
  p.ma = reinterpret_cast<const bf16x8 *>(a + (int64_t)(lane & 15) * lda + k0 + koff);
  p.xlo = x + row(m0 + q) * ldx + k0 + u * 8;
  p.xhi = x + row(m0 + 8 + q) * ldx + k0 + (u ^ 4) * 8;
  p.alo = a + (int64_t)q * lda + k0 + u * 8;
  p.ahi = a + (int64_t)(8 + q) * lda + k0 + (u ^ 4) * 8;
  return p;
}

// Partial of one wavefront over STEPS steps (compile-time count): x and a are
// fetched as whole lines in batches of G steps, DEPTH batches ahead of the
// math (64 registers a batch, so DEPTH is capped by the wavefronts a
// workgroup puts on each SIMD), and lane-permuted into the matrix-core layout
// just before their steps.
template <int STEPS, int MAXDEPTH>
__device__ __forceinline__ f32x4 chunk_streamed(const ChunkPtrs &p, int lane) {
  constexpr int G = STEPS < 8 ? STEPS : 8;
  constexpr int NG = STEPS / G;
  constexpr int DEPTH = NG < MAXDEPTH ? NG : MAXDEPTH;
  static_assert(STEPS % G == 0 && G % 2 == 0, "step count");
  LineOperand16<G / 2, true> xl[DEPTH];
  LineOperand16<G / 2, false> al[DEPTH];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < DEPTH; ++g) {
    xl[g].issue(p.xlo + g * G * kStep, p.xhi + g * G * kStep);
    al[g].issue(p.alo + g * G * kStep, p.ahi + g * G * kStep);
  }
  // Keep the batch together: without this the scheduler trades loads in flight
  // for registers.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int pr = 0; pr < G / 2; ++pr) {
      bf16x8 xf[2], af[2];
      xl[g % DEPTH].place_pair(pr, xf, lane);
      al[g % DEPTH].place_pair(pr, af, lane);
      acc = mfma_step(af[0], xf[0], acc);
      acc = mfma_step(af[1], xf[1], acc);
    }
    if (g + DEPTH < NG) {
      xl[g % DEPTH].issue(p.xlo + (g + DEPTH) * G * kStep, p.xhi + (g + DEPTH) * G * kStep);
      al[g % DEPTH].issue(p.alo + (g + DEPTH) * G * kStep, p.ahi + (g + DEPTH) * G * kStep);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return acc;
}

// Same partial for a step count known only at run time (shapes outside the
// compiled set): one step at a time, straight from the matrix-core layout.
__device__ __forceinline__ f32x4 chunk_plain(const bf16x8 *xp, const bf16x8 *ap, int steps) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < steps; ++t)
    acc = mfma_step(ap[t * (kStep / 8)], __builtin_nontemporal_load(xp + t * (kStep / 8)), acc);
  return acc;
}

template <int STEPS, int MAXDEPTH>
__device__ __forceinline__ f32x4 chunk_partial(const ChunkPtrs &p, int steps, int lane) {
  if constexpr (STEPS > 0) {
    (void)steps;
    return chunk_streamed<STEPS, MAXDEPTH>(p, lane);
  } else {
    return chunk_plain(p.mx, p.ma, steps);
  }
}

// Two-pass partials: grid (row blocks of 64, S); wavefront w of workgroup
// (bx, s) computes p_s of rows bx*64 + w*16 .. +15.  STEPS = 0: run-time count.
template <int STEPS, int MODE>
__global__ __launch_bounds__(kThreads) void shrink_partial_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ a, float *__restrict__ out,
    int M, int64_t ldx, int64_t lda, int64_t ldo, int chunk) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int mw = blockIdx.x * kRowsPerBlock + wv * kRowsPerWave;
  if (mw >= M) return;  // every row of this wavefront is past the batch
  const int s = blockIdx.y;
  const f32x4 acc =
      chunk_partial<STEPS, 3>(chunk_ptrs(x, a, M, ldx, lda, mw, s * chunk, lane), chunk / kStep, lane);
  const int m = mw + (lane & 15);
  if (m >= M) return;
  const int r0 = (lane >> 4) * 4;
  if (MODE == kStoreOut) *reinterpret_cast<f32x4 *>(out + (int64_t)m * ldo + r0) = acc;
  else *reinterpret_cast<f32x4 *>(out + ((int64_t)s * M + m) * kR + r0) = acc;
}

// Stores (or adds) the partial of wavefront s for rows m0 .. m0+15 and, in the
// folding modes, the fold of the S partials through LDS (part holds S x 64
// lanes; the caller places a barrier between the writes and wavefront 0's read).
template <int S, int MODE, int RB = kRowsPerWave>
__device__ __forceinline__ void emit(f32x4 acc, f32x4 (*part)[64], float *y, float *ws, int M,
                                     int64_t ldy, int m0, int s, int lane) {
  // RB < 16: the block has RB rows; lanes of the matrix-core rows past them
  // hold copies and store nothing
  const int m = (lane & 15) < RB ? m0 + (lane & 15) : M;
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
  part[s][lane] = acc;
  wait_lgkmcnt0();
  barrier_no_fence();
  if (s == 0 && m < M) {
    f32x4 t = part[0][lane];
#pragma unroll
    for (int q = 1; q < S; ++q) t = t + part[q][lane];  // element-wise fp32, q ascending
    *reinterpret_cast<f32x4 *>(y + (int64_t)m * ldy + r0) = t;
  }
}

// Streamed fused kernel: blockDim = 64 * S; wavefront s computes p_s of the 16
// rows [blockIdx.x * 16, +16) over chunk s.  STEPS = 0: run-time count.
template <int S, int STEPS, int MODE>
__global__ __launch_bounds__(64 * S) void shrink_fused_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ a, float *__restrict__ y,
    float *__restrict__ ws, int M, int K, int64_t ldx, int64_t lda, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int s = threadIdx.x >> 6;
  const int m0 = blockIdx.x * kRowsPerWave;
  const int chunk = K / S;
  const f32x4 acc = chunk_partial<STEPS, (S >= 16 ? 1 : 3)>(
      chunk_ptrs(x, a, M, ldx, lda, m0, s * chunk, lane), chunk / kStep, lane);
  __shared__ f32x4 part[S][64];
  emit<S, MODE>(acc, part, y, ws, M, ldy, m0, s, lane);
}

// Staged fused kernel, S = 8 or 16 wavefronts, STEPS steps per chunk, row
// blocks of RB = 16 or 8 rows.
//
// A piece is RB rows x PS steps of one wavefront's chunk (PS * 64 bytes a
// row); each wavefront owns a ring of two pieces in LDS.  One direct-to-LDS
// instruction moves 1 KiB = 16/PS whole row segments; lane l of instruction i
// loads row i*(16/PS) + l/U (U = PS*4 sixteen-byte units a row), unit
// (l % U) ^ row, so unit u of row r sits at position u ^ r: a matrix-core read
// (16 rows, one unit each, per 16 lanes) then touches 16 different 16-byte
// bank groups.  With RB = 8 the matrix core's rows 8-15 read rows 0-7 again
// and their results are dropped.  At RB = 16 the LDS of a workgroup is S*16
// KiB of pieces plus two S x 1 KiB fold buffers (144 KiB for S = 8, 160 KiB
// for S = 16): one workgroup per CU.  The pieces of a wavefront run block
// after block over the workgroup's row blocks (blockIdx.x, + gridDim.x, ...);
// while one is read, the next is in flight.
template <int S, int STEPS, int MODE, int RB>
__global__ __launch_bounds__(64 * S, 1) void shrink_staged_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ a, float *__restrict__ y,
    float *__restrict__ ws, int M, int K, int64_t ldx, int64_t lda, int64_t ldy, int nblocks) {
  constexpr int PS = 64 / S;                 // steps per piece: 8 (S = 8) or 4 (S = 16)
  constexpr int NP = STEPS / PS;             // pieces per row block
  constexpr int ROWB = PS * 64;              // bytes of one row in a piece
  constexpr int U = ROWB / 16;               // 16-byte units of one row in a piece
  constexpr int RPI = 1024 / ROWB;           // rows per load instruction
  constexpr int NI = RB / RPI;               // load instructions per piece
  constexpr int PIECE = RB * ROWB;
  static_assert(S * PS == 64 && STEPS % PS == 0 && U >= 16 && NP % 2 == 0, "staged shape");
  static_assert((RB == 16 || RB == 8) && NI >= 1, "rows per block");
  // The two slots are separate LDS objects: the compiler's wait counting can
  // then tell that a read of one slot does not depend on a load into the other.
  __shared__ __attribute__((aligned(1024))) char xs0[S][PIECE];
  __shared__ __attribute__((aligned(1024))) char xs1[S][PIECE];
  __shared__ f32x4 part[2][S][64];

  const int lane = threadIdx.x & 63;
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k0 = s * STEPS * kStep;

  const int nmine = (nblocks - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int npieces = nmine * NP;
  const int64_t xbytes = (int64_t)M * ldx * 2;

  // Piece j of this wavefront -> LDS slot j & 1.
  auto issue = [&](int j) {
    const int m0 = ((int)blockIdx.x + (j / NP) * (int)gridDim.x) * RB;
    const int kp = k0 + (j % NP) * PS * kStep;
    const uint16_t *base = x + (int64_t)m0 * ldx;
    const int64_t left = xbytes - (int64_t)m0 * ldx * 2;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)base, (short)0, (int)(left < 0x7FFFFFFF ? left : 0x7FFFFFFF), 0x00020000);
    char *slot = (j & 1) ? xs1[s] : xs0[s];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + lane / U;
      const int gr = (m0 + row < M ? m0 + row : M - 1) - m0;  // rows past M: copy of the last
      const int off = (int)((gr * ldx + kp + (((lane % U) ^ row) * 8)) * 2);
      // x is read once: non-temporal, so it does not push a out of the cache
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(slot + i * 1024), 16, off, 0, 0,
                                               kCpolNT);
    }
  };

  // The chunk of a first (whole-line loads, mostly cache hits, kept in
  // registers for the whole launch), then the first two pieces of x; a is
  // moved into the matrix-core layout while x is on its way.
  LineOperand16<STEPS / 2, false> al;
  {
    const int q = lane >> 3, u = lane & 7;
    al.issue(a + (int64_t)q * lda + k0 + u * 8, a + (int64_t)(8 + q) * lda + k0 + (u ^ 4) * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  issue(0);
  if (npieces > 1) issue(1);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 af[STEPS];
  al.place(af, lane);
  // Matrix-core steps over piece j (slot j & 1) into acc.  With 8-row blocks
  // the matrix core's rows 8-15 repeat rows 0-7 and are never stored.
  const int r = (lane & 15) % RB;
  auto compute = [&](int j, int p, f32x4 &acc) {
    const char *slot = (j & 1) ? xs1[s] : xs0[s];
    bf16x8 xv[PS];
#pragma unroll
    for (int t = 0; t < PS; ++t) {
      const int u = t * 4 + (lane >> 4);
      xv[t] = *reinterpret_cast<const bf16x8 *>(slot + r * ROWB + ((u ^ r) << 4));
    }
    __builtin_amdgcn_sched_barrier(0);  // all reads of the piece in flight together
#pragma unroll
    for (int t = 0; t < PS; ++t) acc = mfma_step(af[p * PS + t], xv[t], acc);
    wait_lgkmcnt0();  // the slot's reads are done before it is refilled
    __builtin_amdgcn_sched_barrier(0);
  };

  // Every block but the last: each piece has a successor in flight and the
  // piece two ahead exists, so the loop body has no branches (the compiler's
  // wait counting then sees straight-line code).
  int bi = 0;
  for (; bi + 1 < nmine; ++bi) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int j = bi * NP + p;
      wait_vmcnt<NI>();
      compute(j, p, acc);
      issue(j + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int m0 = ((int)blockIdx.x + bi * (int)gridDim.x) * RB;
    emit<S, MODE, RB>(acc, part[bi & 1], y, ws, M, ldy, m0, s, lane);
  }
  {  // last block: pieces npieces - NP .. npieces - 1; the first two are in
     // flight already, each later one is issued two pieces ahead (NP > 2)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int j = bi * NP + p;
      if (p + 1 < NP) wait_vmcnt<NI>();
      else wait_vmcnt<0>();
      compute(j, p, acc);
      if (p + 2 < NP) issue(j + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int m0 = ((int)blockIdx.x + bi * (int)gridDim.x) * RB;
    emit<S, MODE, RB>(acc, part[bi & 1], y, ws, M, ldy, m0, s, lane);
  }
}

// Fused shrink -> expand: a workgroup of kExpWaves wavefronts per 16-row
// block.  Wavefronts 0 .. S-1 compute the shrink partials exactly as the
// streamed fused kernel does (wavefront s: p_s; fold in LDS in s order), so l
// equals bi_lora_shrink's output bit for bit.  l stays in LDS and all
// wavefronts expand the block's 16 rows:
// y[m][n] = bf16(base[m][n] + scale * acc), acc = fma(l[m][r], b[n][r], acc)
// for r ascending -- the arithmetic of bi_lora_expand, so the result equals
// expand(shrink(x)) bit for bit.  Each lane owns 4 consecutive columns (b for
// them widened to fp32 in registers, the 16 rows of base loaded at once); a
// wavefront covers 256 columns per pass, the workgroup kExpWaves * 256.
constexpr int kExpWaves = 8;
template <int S, int STEPS>
__global__ __launch_bounds__(64 * kExpWaves, 1) void shrink_expand_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
    const uint16_t *base, uint16_t *y, float *__restrict__ lout, int M, int K, int N,
    int64_t ldx, int64_t lda, int64_t ldb, int64_t ldbase, int64_t ldy, int64_t ldl, float scale) {
  static_assert(S <= kExpWaves, "split");
  const int lane = threadIdx.x & 63;
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = blockIdx.x * kRowsPerWave;
  __shared__ f32x4 part[S][64];
  __shared__ float ls[kRowsPerWave][kR];
  if (s < S) {
    const int chunk = K / S;
    part[s][lane] = chunk_partial<STEPS, 1>(chunk_ptrs(x, a, M, ldx, lda, m0, s * chunk, lane),
                                            chunk / kStep, lane);
  }
  __syncthreads();
  if (s == 0) {
    f32x4 t = part[0][lane];
#pragma unroll
    for (int q = 1; q < S; ++q) t = t + part[q][lane];  // element-wise fp32, q ascending
    const int row = lane & 15, r0 = (lane >> 4) * 4;
    *reinterpret_cast<f32x4 *>(&ls[row][r0]) = t;
    if (lout != nullptr && m0 + row < M)
      *reinterpret_cast<f32x4 *>(lout + (int64_t)(m0 + row) * ldl + r0) = t;
  }
  __syncthreads();  // l of the block is in LDS

  const int nrows = min(kRowsPerWave, M - m0);
  for (int nt = 0; nt < N; nt += kExpWaves * 256) {
    const int n0 = nt + s * 256 + lane * 4;
    if (n0 >= N) continue;  // N % 8 == 0: a lane's 4 columns are all in or all out
    u32x2 bv[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int m = m0 + (i < nrows ? i : nrows - 1);
      bv[i] = base ? __builtin_nontemporal_load(
                         reinterpret_cast<const u32x2 *>(base + (int64_t)m * ldbase + n0))
                   : u32x2{0u, 0u};
    }
    float bf[4][kR];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 *br = reinterpret_cast<const u32x4 *>(b + (int64_t)(n0 + j) * ldb);
      const u32x4 w0 = br[0], w1 = br[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf[j][2 * i] = lo_bf16(w0[i]);
        bf[j][2 * i + 1] = hi_bf16(w0[i]);
        bf[j][8 + 2 * i] = lo_bf16(w1[i]);
        bf[j][8 + 2 * i + 1] = hi_bf16(w1[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (i >= nrows) continue;
      // one row's l at a time: hoisting every row's reads would need 256 registers
      __builtin_amdgcn_sched_barrier(0);
      float lv[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) lv[r] = ls[i][r];
      u32x2 o;
      float acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = 0.0f;
#pragma unroll
        for (int r = 0; r < kR; ++r) acc[j] = __builtin_fmaf(lv[r], bf[j][r], acc[j]);
      }
      o[0] = pack_bf16x2(lo_bf16(bv[i][0]) + scale * acc[0], hi_bf16(bv[i][0]) + scale * acc[1]);
      o[1] = pack_bf16x2(lo_bf16(bv[i][1]) + scale * acc[2], hi_bf16(bv[i][1]) + scale * acc[3]);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2 *>(y + (int64_t)(m0 + i) * ldy + n0));
    }
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

template <int V>
struct IntC {
  static constexpr int value = V;
};

// Calls f(IntC<steps>) for the compiled step counts, f(IntC<0>) (run-time
// count) otherwise.
template <typename F>
void with_steps(int steps, F &&f) {
  switch (steps) {
    case 8: f(IntC<8>{}); break;
    case 16: f(IntC<16>{}); break;
    case 32: f(IntC<32>{}); break;
    case 64: f(IntC<64>{}); break;
    case 128: f(IntC<128>{}); break;
    default: f(IntC<0>{}); break;
  }
}

template <int S, int STEPS, int MODE>
void launch_streamed(dim3 grid, hipStream_t st, const uint16_t *x, const uint16_t *a, float *y,
                     float *ws, int64_t M, int64_t K, int64_t ldx, int64_t lda, int64_t ldy) {
  hipLaunchKernelGGL((shrink_fused_kernel<S, STEPS, MODE>), grid, dim3(64 * S), 0, st, x, a, y, ws,
                     (int)M, (int)K, ldx, lda, ldy);
}

// Row blocks of 16 rows, one workgroup per CU, persistent over the blocks;
// when 16-row blocks would leave at least half of the CUs idle (M <= 8 rows
// per CU), blocks of 8 rows instead, twice as many workgroups.  Both run the
// same matrix-core steps on every row, so the choice changes no bit
// (measured at K = 4096: M = 64: 5.6 -> 4.7 us, M = 2048: 6.3 -> 5.9 us; at
// M = 4096 the 8-row blocks, two workgroups per CU, were slower).
template <int S, int STEPS, int MODE>
void launch_staged(hipStream_t st, const uint16_t *x, const uint16_t *a, float *y, float *ws,
                   int64_t M, int64_t K, int64_t ldx, int64_t lda, int64_t ldy) {
  const int64_t cus = cu_count();
  if (M <= 8 * cus) {
    const int64_t nblocks = (M + 7) / 8;
    hipLaunchKernelGGL((shrink_staged_kernel<S, STEPS, MODE, 8>), dim3((unsigned)nblocks),
                       dim3(64 * S), 0, st, x, a, y, ws, (int)M, (int)K, ldx, lda, ldy,
                       (int)nblocks);
  } else {
    const int64_t nblocks = (M + kRowsPerWave - 1) / kRowsPerWave;
    const int grid = (int)(nblocks < cus ? nblocks : cus);
    hipLaunchKernelGGL((shrink_staged_kernel<S, STEPS, MODE, 16>), dim3(grid), dim3(64 * S), 0,
                       st, x, a, y, ws, (int)M, (int)K, ldx, lda, ldy, (int)nblocks);
  }
}

// One fused launch: the staged kernel for the deterministic splits (S = 8, 16)
// at 8 or 16 steps a chunk, the streamed kernel otherwise.
template <int MODE>
void launch_fused(int S, hipStream_t st, const uint16_t *x, const uint16_t *a, float *y, float *ws,
                  int64_t M, int64_t K, int64_t ldx, int64_t lda, int64_t ldy) {
  const int steps = (int)(K / S / kStep);
  const int64_t nblocks = (M + kRowsPerWave - 1) / kRowsPerWave;
  // the staged loads address x with 32-bit byte offsets inside a 16-row block
  if (((S == 8 && steps == 16) || (S == 16 && (steps == 8 || steps == 16))) &&
      ldx < (int64_t(1) << 26)) {
    if (S == 8) launch_staged<8, 16, MODE>(st, x, a, y, ws, M, K, ldx, lda, ldy);
    else if (steps == 16) launch_staged<16, 16, MODE>(st, x, a, y, ws, M, K, ldx, lda, ldy);
    else launch_staged<16, 8, MODE>(st, x, a, y, ws, M, K, ldx, lda, ldy);
    return;
  }
  const dim3 grid((unsigned)nblocks);
  with_steps(steps, [&](auto c) {
    constexpr int ST = decltype(c)::value;
    switch (S) {
      case 1: launch_streamed<1, ST, MODE>(grid, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
      case 2: launch_streamed<2, ST, MODE>(grid, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
      case 4: launch_streamed<4, ST, MODE>(grid, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
      case 8: launch_streamed<8, ST, MODE>(grid, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
      default: launch_streamed<16, ST, MODE>(grid, st, x, a, y, ws, M, K, ldx, lda, ldy); break;
    }
  });
}

template <int MODE>
void launch_partial(int S, hipStream_t st, const uint16_t *x, const uint16_t *a, float *out,
                    int64_t M, int64_t K, int64_t ldx, int64_t lda, int64_t ldo) {
  const int chunk = (int)(K / S);
  with_steps(chunk / kStep, [&](auto c) {
    constexpr int ST = decltype(c)::value;
    hipLaunchKernelGGL((shrink_partial_kernel<ST, MODE>), partial_grid(M, S), dim3(kThreads), 0, st,
                       x, a, out, (int)M, ldx, lda, ldo, chunk);
  });
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
  launch_fused<kStoreOut>(split_k, (hipStream_t)stream, x, a, y,
                          split_k > 1 ? static_cast<float *>(ws) : nullptr, M, K, ldx, lda, ldy);
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
  if (split_k == 1) {
    launch_partial<kStoreOut>(1, s, x, a, y, M, K, ldx, lda, ldy);
    return launch_status();
  }
  float *wsf = static_cast<float *>(ws);
  launch_partial<kStoreWs>(split_k, s, x, a, wsf, M, K, ldx, lda, (int64_t)kR);
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
  launch_fused<kAtomic>(split_k, s, x, a, y, nullptr, M, K, ldx, lda, ldy);
  return launch_status();
}

extern "C" int bi_lora_shrink_expand(const uint16_t *x, const uint16_t *a, const uint16_t *b,
                                     const uint16_t *base, uint16_t *y, float *l, int64_t M,
                                     int64_t K, int64_t N, int64_t R, int64_t ldx, int64_t lda,
                                     int64_t ldb, int64_t ldbase, int64_t ldy, int64_t ldl,
                                     float scale, int split_k, void *stream) {
  if (!a || !b || (M > 0 && (!x || !y))) return BI_ERR_NULL;
  if (R != kR || !split_ok(split_k) || split_k > 8) return BI_ERR_UNSUPPORTED;
  if (M < 0 || K <= 0 || M > (1 << 30) || K > (1 << 30) || N < 8 || N > (1 << 23) || ldx < K ||
      lda < K || ldb < R || ldy < N || (base && ldbase < N) || (l && ldl < R))
    return BI_ERR_SHAPE;
  if (K % (kStep * split_k)) return BI_ERR_SHAPE;
  if ((ldx | lda | N | ldy | ldb) & 7 || (base && (ldbase & 7)) || (l && (ldl & 3)) ||
      !aligned16(x) || !aligned16(a) || !aligned16(b) || !aligned16(y) ||
      (base && !aligned16(base)) || (l && !aligned16(l)))
    return BI_ERR_ALIGN;
  const Span sy = span_of(y, M, N, ldy, 2);
  const bool in_place = base == y && ldbase == ldy;
  if (overlap(sy, span_of(x, M, K, ldx, 2)) || overlap(sy, span_of(a, R, K, lda, 2)) ||
      overlap(sy, span_of(b, N, R, ldb, 2)) ||
      (base && !in_place && overlap(sy, span_of(base, M, N, ldbase, 2))))
    return BI_ERR_ALIAS;
  if (l) {
    const Span sl = span_of(l, M, R, ldl, 4);
    if (overlap(sl, sy) || overlap(sl, span_of(x, M, K, ldx, 2)) ||
        overlap(sl, span_of(a, R, K, lda, 2)) || overlap(sl, span_of(b, N, R, ldb, 2)) ||
        (base && overlap(sl, span_of(base, M, N, ldbase, 2))))
      return BI_ERR_ALIAS;
  }
  if (M == 0) return BI_OK;
  const dim3 grid((unsigned)((M + kRowsPerWave - 1) / kRowsPerWave));
  hipStream_t st = (hipStream_t)stream;
  with_steps((int)(K / split_k / kStep), [&](auto c) {
    constexpr int ST = decltype(c)::value;
    auto go = [&](auto sc) {
      constexpr int SS = decltype(sc)::value;
      hipLaunchKernelGGL((shrink_expand_kernel<SS, ST>), grid, dim3(64 * kExpWaves), 0, st, x, a, b, base,
                         y, l, (int)M, (int)K, (int)N, ldx, lda, ldb, ldbase, ldy, ldl, scale);
    };
    switch (split_k) {
      case 1: go(IntC<1>{}); break;
      case 2: go(IntC<2>{}); break;
      case 4: go(IntC<4>{}); break;
      default: go(IntC<8>{}); break;
    }
  });
  return launch_status();
}
