// gemm.hip -- batch-invariant bf16 GEMM for gfx950: y = bf16(x . w^T), fp32 accumulation.
//
// "Cómo superar la no determinación en la inferencia de LLM", section
// "Multiplicación de matrices (matmul)": tile the output in 2-D, process tiles
// data-parallel, and force one kernel configuration for every batch size
// (no split-K chosen for small batches), accepting some lost speed.
//
// Reduction order of every output element (the batch-invariance contract):
// one pass over k = 0, 32, 64, ..., K-32, each step a single
// v_mfma_f32_16x16x32_bf16 whose fp32 accumulator is rounded between steps.
// The order never depends on M, on the tile the element falls in, on the
// position of the element inside its 16x16 matrix-core block, or on the
// tile configuration: every configuration below runs the same instruction
// over the same k steps; configurations differ only in how many outputs one
// workgroup owns.  The configuration is picked from (N, K) alone.
//
// Why 16x16x32 and not 32x32x16 (same peak rate): at full load the card sits
// at its socket power limit, and measured under sustained load the 16x16x32
// form runs the same kernels at a ~10 % higher shader clock for the same
// power, 5-9 % more throughput at M >= 4096.
//
// Data path per workgroup (4 compute wavefronts, 2 x 2 over the tile; the
// 64-k kernels add four wavefronts that only load, and at 256 x 256 run two
// ping-pong groups of four compute wavefronts instead):
//   HBM/L2 --buffer_load_dwordx4 ... lds--> LDS
//          --ds_read_b128--> VGPR fragments --MFMA--> fp32 accumulators
//   epilogue: accumulators -> bf16 (round to nearest even) -> LDS -> whole
//   128-byte line stores.
// Two LDS staging schemes feed the same instruction sequence:
//   * BK = 32 stages (K % 64 == 32): 64-byte LDS rows, a ring of 4 stages;
//   * BK = 64 stages (K % 64 == 0): whole 128-byte lines per row, so every L2
//     request is a full line; one operand in a ring of 3 stages, the other in
//     a ring of 2 (160 KiB of LDS at 256 x 256).
// Each LDS row's 16-byte chunks are XOR-permuted by a function of the row so
// that the 16 rows a quarter-wavefront's fragment read touches spread over all
// LDS banks.  Rows
// beyond M (or N) are loaded as copies of the last valid row and never
// stored, so no row's arithmetic depends on how many rows the batch holds.
#include "common.h"

#include <mutex>

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 32;                 // k per LDS stage (one 32-k matrix-core step)
constexpr int kRowBytes = BK * 2;      // one LDS row: 32 bf16 = four 16-byte chunks
constexpr int kStages = 4;             // LDS ring depth: 3 stages of loads in flight

// Chunk permutation of LDS row r (4 chunks of 16 bytes): chunk c of row r is
// stored at c ^ ((r >> 2) & 3).  A fragment read (16 consecutive rows, one
// chunk each, per quarter-wavefront) then hits each 16-byte bank group of the
// four 256-byte LDS windows those rows span once -- conflict-free.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

template <int BN, int BM>
struct Cfg {
  static constexpr int WN = BN / 2, WM = BM / 2;    // wavefront tile (n x m)
  static constexpr int FN = WN / 16, FM = WM / 16;  // 16x16 blocks per wavefront
  static constexpr int W_BYTES = BN * kRowBytes;    // LDS bytes of a weight stage
  static constexpr int X_BYTES = BM * kRowBytes;    // LDS bytes of an activation stage
  static constexpr int STAGE = W_BYTES + X_BYTES;
  static constexpr int LPS = (BN + BM) / 64;        // load instructions per wavefront per stage
  static_assert(BN % 64 == 0 && BM % 64 == 0, "tile must split over 2x2 wavefronts");
  static_assert(3 * LPS < 64, "vmcnt range");
};

// Map the launch index to a tile.  Workgroups are dispatched round-robin over
// the 8 XCDs (index % 8); each XCD gets a contiguous range of logical tiles,
// walked in groups of kGroupM tile-rows so that tiles running at the same time
// on one XCD share weight and activation panels in that XCD's L2.  The mapping
// changes which workgroup computes a tile, never how the tile is computed.
constexpr int kGroupM = 4;
// Launch index -> logical tile index: each XCD gets a contiguous range of the
// T logical tiles.
__device__ __forceinline__ int xcd_lid(int pid, int T) {
  const int q = T >> 3, r = T & 7;
  const int xcd = pid & 7, local = pid >> 3;
  return xcd * q + (xcd < r ? xcd : r) + local;
}
// Logical tile index -> (tile row, tile column), walking groups of kGroupM
// tile-rows column by column.
__device__ __forceinline__ void group_tile(int lid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = lid / per_group;
  const int first_m = g * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_g = lid - g * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}
__device__ __forceinline__ void tile_of(int pid, int tiles_m, int tiles_n, int &tm, int &tn) {
  group_tile(xcd_lid(pid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// Direct-to-LDS loads of one operand tile through a buffer resource: each lane
// keeps a constant 32-bit byte offset and the stage's k offset travels in the
// scalar offset, so a stage costs no vector address arithmetic.  Wavefront
// wv, instruction i fills LDS rows [i*64 + wv*16, +16): lane l writes 16 bytes
// at row (l >> 2),
// physical chunk (l & 3), which holds logical chunk (l & 3) ^ swz(row).
// Rows past the matrix edge are clamped to its last row (loaded, never stored).
template <int ROWS>
struct LoadPlan {
  static constexpr int N = ROWS / 64;
  __amdgpu_buffer_rsrc_t rsrc;
  // Byte offsets of this lane's 16-byte pieces, relative to the matrix base.
  // The hardware reads offsets and the record count as unsigned 32-bit
  // values; the host accepts operands of fewer than 2^31 elements (2^32 bytes).
  uint32_t off[N];
  __device__ __forceinline__ void init(const uint16_t *g, int rows_total, int row0, int row_limit,
                                       int64_t ld, int K, int wv, int lane) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)g, (short)0, (int)(uint32_t)(((int64_t)(rows_total - 1) * ld + K) * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = i * 64 + wv * 16 + (lane >> 2);
      int gr = row0 + r;
      gr = gr < row_limit ? gr : row_limit - 1;
      off[i] = (uint32_t)(gr * ld + (((lane & 3) ^ swz(r)) << 3)) * 2u;
    }
  }
  __device__ __forceinline__ void issue(char *lds, int k0, int wv) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      lds_void *dst = (lds_void *)(lds + (i * 64 + wv * 16) * kRowBytes);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, (int)off[i], k0 * 2, 0, 0);
    }
  }
};

// Fragment of 16 rows x 32 k for the 16x16x32 instruction: lane l takes row
// (l & 15) and k = 8 (l >> 4) .. +7 of the step -- the same k mapping for both
// operands, so the instruction pairs matching k.  A 32-k LDS row holds one
// step.
__device__ __forceinline__ bf16x8 read_frag(const char *lds, int row, int lane) {
  const int lc = lane >> 4;
  const int off = row * kRowBytes + ((lc ^ swz(row)) << 4);
  return *reinterpret_cast<const bf16x8 *>(lds + off);
}

template <int BN, int BM>
struct Frags {
  bf16x8 a[BN / 32], b[BM / 32];
};

template <int BN, int BM>
__device__ __forceinline__ void read_frags(Frags<BN, BM> &f, const char *lds, int wn, int wm,
                                           int lane) {
  using C = Cfg<BN, BM>;
#pragma unroll
  for (int i = 0; i < C::FN; ++i) f.a[i] = read_frag(lds, wn * C::WN + i * 16 + (lane & 15), lane);
#pragma unroll
  for (int j = 0; j < C::FM; ++j)
    f.b[j] = read_frag(lds + C::W_BYTES, wm * C::WM + j * 16 + (lane & 15), lane);
}

// One 32-k step of a wavefront's blocks: block (i, j) of the wavefront's
// WN x WM sub-tile covers n in [16i, 16i + 16) and m in [16j, 16j + 16).
template <int BN, int BM>
__device__ __forceinline__ void mfma_step(f32x4 (&acc)[BN / 32][BM / 32], const Frags<BN, BM> &f) {
#pragma unroll
  for (int i = 0; i < BN / 32; ++i)
#pragma unroll
    for (int j = 0; j < BM / 32; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

template <int LPS>
__device__ __forceinline__ void wait_stages_after(int n) {
  // wait until at most n stages (issued after the one needed) are in flight
  if (n >= 3) wait_vmcnt<3 * LPS>();
  else if (n == 2) wait_vmcnt<2 * LPS>();
  else if (n == 1) wait_vmcnt<LPS>();
  else wait_vmcnt<0>();
}

// The K loop of one tile: x and w point at the first k of this tile's K range
// and nkb stages of BK follow.  Leaves the tile's fp32 sums in acc.
//
// One 32-k step per stage.  Step kb starts once every wavefront holds stage
// kb's fragments in registers and stage kb + 1 has landed (own waits, then
// the barrier for the other wavefronts' loads); stage kb's slot then takes
// stage kb + kStages, and stage kb + 1's fragments are read into the same
// registers as soon as stage kb's products have taken them.  (This path only
// serves K % 64 == 32; K % 64 == 0 takes the 64-k stages below.)
template <int BN, int BM>
__device__ __forceinline__ void gemm_mainloop(f32x4 (&acc)[BN / 32][BM / 32], char *lds,
                                              const uint16_t *__restrict__ x,
                                              const uint16_t *__restrict__ w, int M, int N,
                                              int nkb, int64_t ldx, int64_t ldw, int m0, int n0,
                                              int wv, int lane, int kspan) {
  using C = Cfg<BN, BM>;
  const int wn = wv >> 1, wm = wv & 1;
  LoadPlan<BN> pw;
  LoadPlan<BM> px;
  pw.init(w, N, n0, N, ldw, kspan, wv, lane);
  px.init(x, M, m0, M, ldx, kspan, wv, lane);

#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x4{};

  // Prologue: stages 0 .. kStages-1 in flight.
#pragma unroll
  for (int s = 0; s < kStages; ++s) {
    if (s < nkb) {
      char *buf = lds + s * C::STAGE;
      pw.issue(buf, s * BK, wv);
      px.issue(buf + C::W_BYTES, s * BK, wv);
    }
  }
  wait_stages_after<C::LPS>(min(kStages - 1, nkb - 1));
  barrier_no_fence();

  Frags<BN, BM> f;
  read_frags<BN, BM>(f, lds, wn, wm, lane);
  // Steady state (stage kb + kStages exists; no branches inside, so the
  // compiler's wait-count tracking sees straight-line code): stages
  // kb+1 .. kb+3 are in flight on entry, two may stay in flight.
  int kb = 0;
  for (; kb + kStages < nkb; ++kb) {
    char *cur = lds + (kb & (kStages - 1)) * C::STAGE;
    const char *nxt = lds + ((kb + 1) & (kStages - 1)) * C::STAGE;
    wait_lgkmcnt0();
    wait_vmcnt<2 * C::LPS>();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
    pw.issue(cur, (kb + kStages) * BK, wv);
    px.issue(cur + C::W_BYTES, (kb + kStages) * BK, wv);
    mfma_step<BN, BM>(acc, f);
    read_frags<BN, BM>(f, nxt, wn, wm, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Drain: every stage issued; after kb + 1, nkb - 2 - kb stages (at most
  // two) may still be in flight.
  for (; kb + 1 < nkb; ++kb) {
    const char *nxt = lds + ((kb + 1) & (kStages - 1)) * C::STAGE;
    wait_lgkmcnt0();
    wait_stages_after<C::LPS>(nkb - 2 - kb);
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
    mfma_step<BN, BM>(acc, f);
    read_frags<BN, BM>(f, nxt, wn, wm, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_lgkmcnt0();
  mfma_step<BN, BM>(acc, f);
}

// Epilogue through LDS, so that every global store writes whole 128-byte
// lines (per-lane 8-byte stores straight from the accumulators would issue
// eight partial-line requests per line and, with every tile finishing at the
// same moment, stall on the L2 request rate).
//
// Accumulator block (i, j) of a wavefront, register v, holds
// n = 16i + 4(lane/16) + v and m = 16j + lane%16 of the wavefront's WN x WM
// sub-tile.  Each wavefront writes its sub-tile, rounded to bf16, to its own
// LDS region `mine` as rows of m (WN bf16 = CH 16-byte chunks, chunk c of row
// m stored at c ^ f(m)), then reads it back 16 bytes per lane, eight lanes per
// 128-byte row segment, and stores those segments.  f spreads the 16 rows of
// one accumulator write over the banks and gives two adjacent rows disjoint
// chunk sets for the reads.  The caller has made the LDS free.
template <int FN, int FM>
__device__ __forceinline__ void store_sub(const f32x4 (&acc)[FN][FM], char *mine, uint16_t *y,
                                          int M, int N, int64_t ldy, int m_org, int n_org,
                                          int lane) {
  constexpr int WN = FN * 16, WM = FM * 16;
  constexpr int CH = WN / 8, ROWB = WN * 2, HB = CH / 2;
  static_assert(CH == 8 || CH == 16, "sub-tile width");
  auto f = [](int m) { return ((m & 1) * HB) | ((m >> 1) & (HB - 1)); };
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int m = j * 16 + (lane & 15);
    char *row = mine + m * ROWB + ((lane >> 4) & 1) * 8;
    const int fm = f(m);
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      uint2 o;
      o.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
      o.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
      *reinterpret_cast<uint2 *>(row + (((i * 2 + (lane >> 5)) ^ fm) << 4)) = o;
    }
  }
  // A wavefront's LDS operations complete in order: its reads below see its
  // writes above.
  constexpr int SEG = CH / 8;  // 128-byte segments per row
#pragma unroll 4
  for (int t = 0; t < WM / 8 * SEG; ++t) {
    const int r = (t / SEG) * 8 + (lane >> 3);
    const int c = (t % SEG) * 8 + (lane & 7);
    const u32x4 v = *reinterpret_cast<const u32x4 *>(mine + r * ROWB + ((c ^ f(r)) << 4));
    const int m = m_org + r, n = n_org + c * 8;
    // non-temporal: nothing in the launch reads y back (0.3-1.6 % faster than
    // plain stores on the 256 x 256 tile at M = 4096-8192)
    if (m < M && n < N) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(y + (int64_t)m * ldy + n));
  }
}

// The 4-wavefront tile: wavefront wv = (wn, wm) owns the (BN/2) x (BM/2)
// sub-tile at (wn, wm) and one LDS region of that size.
template <int BN, int BM>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[BN / 32][BM / 32], char *lds,
                                           uint16_t *y, int M, int N, int64_t ldy, int m0, int n0,
                                           int wn, int wm, int wv, int lane) {
  constexpr int WN = BN / 2, WM = BM / 2;
  store_sub<BN / 32, BM / 32>(acc, lds + wv * (WM * WN * 2), y, M, N, ldy, m0 + wm * WM,
                              n0 + wn * WN, lane);
}

// ---------------------------------------------------------------------------
// Wide-stage variant: BK = 64, so an LDS row is a whole 128-byte line of one
// matrix row and each direct-to-LDS load instruction moves 8 full lines (one
// 128-byte L2 request per line instead of two 64-byte ones).  Two stages fit
// the LDS at 256 x 256; stage kb + 2 is issued once every wavefront has read
// its last fragments of stage kb.  The k order is unchanged: 32-k matrix-core
// steps, ascending (two per stage), so the bits equal the BK = 32 kernel's.
constexpr int BK2 = 64;
constexpr int kRow2 = BK2 * 2;  // 128 bytes: eight 16-byte chunks

// Chunk c of LDS row r is stored at c ^ swz2(r).  A quarter-wavefront's
// fragment read touches 16 consecutive rows at one logical chunk; rows r and
// r + 1 share a 256-byte window, so those 16 rows cover the 16 bank groups
// exactly once.
__device__ __forceinline__ int swz2(int row) { return (row >> 1) & 7; }

template <int BN, int BM>
struct Cfg2 {
  static constexpr int WN = BN / 2, WM = BM / 2;
  static constexpr int FN = WN / 16, FM = WM / 16;  // 16x16 blocks per wavefront
  static constexpr int W_BYTES = BN * kRow2;  // one weight stage
  static constexpr int X_BYTES = BM * kRow2;  // one activation stage
  static constexpr int LW = BN / 32, LX = BM / 32;  // load instructions per wavefront per stage
  static_assert(BN % 64 == 0 && BM % 64 == 0 && LW + 2 * LX < 64, "tile");
};

// Wavefront wv, instruction i fills LDS rows [i*32 + wv*8, +8): lane l writes
// row (l >> 3), physical chunk (l & 7), i.e. logical chunk (l & 7) ^ swz2(row).
template <int ROWS>
struct LoadPlan2 {
  static constexpr int N = ROWS / 32;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[N];  // as in LoadPlan: unsigned 32-bit byte offsets
  __device__ __forceinline__ void init(const uint16_t *g, int rows_total, int row0, int row_limit,
                                       int64_t ld, int K, int wv, int lane) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)g, (short)0, (int)(uint32_t)(((int64_t)(rows_total - 1) * ld + K) * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = i * 32 + wv * 8 + (lane >> 3);
      int gr = row0 + r;
      gr = gr < row_limit ? gr : row_limit - 1;
      off[i] = (uint32_t)(gr * ld + (((lane & 7) ^ swz2(r)) << 3)) * 2u;
    }
  }
  // instructions [i0, i1) of a stage (compile-time bounds after inlining)
  __device__ __forceinline__ void issue(char *lds, int k0, int wv, int i0 = 0, int i1 = N) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i < i0 || i >= i1) continue;
      lds_void *dst = (lds_void *)(lds + (i * 32 + wv * 8) * kRow2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, (int)off[i], k0 * 2, 0, 0);
    }
  }
};

// Fragment of step s (k = 32s .. 32s + 31 of the stage), as read_frag.
__device__ __forceinline__ bf16x8 read_frag2(const char *lds, int row, int s, int lane) {
  const int lc = s * 4 + (lane >> 4);
  return *reinterpret_cast<const bf16x8 *>(lds + row * kRow2 + ((lc ^ swz2(row)) << 4));
}

// Issued in the order the products consume them: a[0] with every b[j] comes
// first, then a[1], a[2], ... -- the first product waits for two reads only.
template <int BN, int BM>
__device__ __forceinline__ void read_frags2(Frags<BN, BM> &f, const char *wl, const char *xl,
                                            int s, int wn, int wm, int lane) {
  using C = Cfg2<BN, BM>;
  f.a[0] = read_frag2(wl, wn * C::WN + (lane & 15), s, lane);
#pragma unroll
  for (int j = 0; j < C::FM; ++j) f.b[j] = read_frag2(xl, wm * C::WM + j * 16 + (lane & 15), s, lane);
#pragma unroll
  for (int i = 1; i < C::FN; ++i) f.a[i] = read_frag2(wl, wn * C::WN + i * 16 + (lane & 15), s, lane);
}

// Scheduling hint: spread the NREAD fragment reads, then the NDMA loads,
// evenly between the NMFMA matrix-core instructions of a step.
template <int NMFMA, int NDMA, int NREAD>
__device__ __forceinline__ void interleave_even() {
  constexpr int NMEM = NDMA + NREAD;
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    const int t0 = i * NMEM / NMFMA, t1 = (i + 1) * NMEM / NMFMA;
#pragma unroll
    for (int t = t0; t < t1; ++t) {
      if (t < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
}

// Step 0 of a stage (the fragments of step 1 are read while it multiplies),
// with the loads of a later stage of the operand that has the ring of 3 when
// LOAD.  Leaves step 1's fragments in f1.
template <int BN, int BM, int ER, bool LOAD>
__device__ __forceinline__ void stage_head2(f32x4 (&acc)[BN / 32][BM / 32], Frags<BN, BM> &f0,
                                            Frags<BN, BM> &f1, const char *wc, const char *xc,
                                            const LoadPlan2<ER> &pe, char *edst, int k0, int wn,
                                            int wm, int wv, int lane) {
  using C = Cfg2<BN, BM>;
  constexpr int LE = ER / 32;
  read_frags2<BN, BM>(f1, wc, xc, 1, wn, wm, lane);
  if (LOAD) pe.issue(edst, k0, wv);
  mfma_step<BN, BM>(acc, f0);
  interleave_even<C::FN * C::FM, LOAD ? LE : 0, C::FN + C::FM>();
  __builtin_amdgcn_sched_barrier(0);
}

// LDS bytes of the 64-k scheme: one operand in a ring of 3 stages, the other
// in a ring of 2 (W3: the weights have the ring of 3).
template <int BN, int BM, bool W3>
constexpr int wide_lds_bytes() {
  return W3 ? 3 * BN * kRow2 + 2 * BM * kRow2 : 2 * BN * kRow2 + 3 * BM * kRow2;
}

// One operand in a ring of 3 stages, the other in a ring of 2.  In stage kb
// the ring-of-3 operand's stage kb + 2 loads during the first step (its slot
// held stage kb - 1); the ring-of-2 operand's stage kb + 2 loads after the
// end-of-stage barrier, once every wavefront has read stage kb.  Activations
// take the ring of 3 in the full-size kernels (W3 = false); the small-M
// split-K partials give it to the weights, whose read dominates there.
template <int BN, int BM, bool W3>
__device__ __forceinline__ void gemm_mainloop2(f32x4 (&acc)[BN / 32][BM / 32], char *lds,
                                               const uint16_t *__restrict__ x,
                                               const uint16_t *__restrict__ w, int M, int N,
                                               int nkb, int64_t ldx, int64_t ldw, int m0, int n0,
                                               int wv, int lane, int kspan) {
  using C = Cfg2<BN, BM>;
  const int wn = wv >> 1, wm = wv & 1;
  LoadPlan2<BN> pw;
  LoadPlan2<BM> px;
  pw.init(w, N, n0, N, ldw, kspan, wv, lane);
  px.init(x, M, m0, M, ldx, kspan, wv, lane);
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x4{};

  constexpr int NW = W3 ? 3 : 2;
  // slots: current, next, free (the free slot only for the ring of 3)
  char *wa = lds, *wb = wa + C::W_BYTES, *wf = wb + C::W_BYTES;
  char *xa = lds + NW * C::W_BYTES, *xb = xa + C::X_BYTES, *xf = xb + C::X_BYTES;
  pw.issue(wa, 0, wv);
  px.issue(xa, 0, wv);
  if (nkb > 1) {
    pw.issue(wb, BK2, wv);
    px.issue(xb, BK2, wv);
    wait_vmcnt<C::LW + C::LX>();
  } else {
    wait_vmcnt<0>();
  }
  barrier_no_fence();

  Frags<BN, BM> f0, f1;
  read_frags2<BN, BM>(f0, wa, xa, 0, wn, wm, lane);
  int kb = 0;
  for (; kb + 2 < nkb; ++kb) {
    const int k2 = (kb + 2) * BK2;
    if constexpr (W3)
      stage_head2<BN, BM, BN, true>(acc, f0, f1, wa, xa, pw, wf, k2, wn, wm, wv, lane);
    else
      stage_head2<BN, BM, BM, true>(acc, f0, f1, wa, xa, px, xf, k2, wn, wm, wv, lane);
    wait_lgkmcnt0();
    // stage kb + 1 has landed; stage kb + 2 of the ring-of-3 operand may fly
    wait_vmcnt<W3 ? C::LW : C::LX>();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
    read_frags2<BN, BM>(f0, wb, xb, 0, wn, wm, lane);
    if constexpr (W3) px.issue(xa, k2, wv);
    else pw.issue(wa, k2, wv);
    mfma_step<BN, BM>(acc, f1);
    interleave_even<C::FN * C::FM, W3 ? C::LX : C::LW, C::FN + C::FM>();
    __builtin_amdgcn_sched_barrier(0);
    char *t;
    if constexpr (W3) {
      t = wa; wa = wb; wb = wf; wf = t;
      t = xa; xa = xb; xb = t;
    } else {
      t = wa; wa = wb; wb = t;
      t = xa; xa = xb; xb = xf; xf = t;
    }
  }
  if (kb + 1 < nkb) {
    stage_head2<BN, BM, BM, false>(acc, f0, f1, wa, xa, px, xf, 0, wn, wm, wv, lane);
    wait_lgkmcnt0();
    wait_vmcnt<0>();
    barrier_no_fence();
    read_frags2<BN, BM>(f0, wb, xb, 0, wn, wm, lane);
    mfma_step<BN, BM>(acc, f1);
    wa = wb;
    xa = xb;
  }
  stage_head2<BN, BM, BM, false>(acc, f0, f1, wa, xa, px, xf, 0, wn, wm, wv, lane);
  mfma_step<BN, BM>(acc, f1);
}

// Role-split form of the 64-k scheme: eight wavefronts, two per SIMD.
// Wavefronts 0-3 compute the 2 x 2 sub-tiles with the fragment reads and
// products of gemm_mainloop2, in the same order, so the bits are the same;
// wavefronts 4-7 only issue the direct-to-LDS loads and wait for them.  The
// two sides pass the same sequence of barriers: B(b) before stage b is read
// (stage b has landed and stage b - 1 is read, so its slots are free), for
// b = 0 .. nkb - 1, and one when the last stage is read.  With the loads out
// of the compute wavefronts' instruction stream, an LDS stage is refilled
// while the other SIMD wavefront multiplies.
//
// Activations sit in a ring of 3 stages, weights in a ring of DW (2 or 3).
// Stage s of an operand with a ring of D goes into slot s % D as soon as
// stage s - D is read (after B(s - D + 1); stages 0 .. D - 1 before B(0)):
// the weights run DW - 1 stages ahead, the activations two.
template <int BN, int BM, int DW>
constexpr int role_lds_bytes() {
  return DW * BN * kRow2 + 3 * BM * kRow2;
}

// Tile (tm, tn): rows tm * BM.., columns tn * BN.., by a workgroup of 512 threads.
template <int BN, int BM, int DW>
__device__ __forceinline__ void role_tile(char *lds, const uint16_t *__restrict__ x,
                                          const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
                                          int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy,
                                          int tm, int tn) {
  using C = Cfg2<BN, BM>;
  const int m0 = tm * BM, n0 = tn * BN;
  constexpr int DX = 3;
  static_assert(DW == 2 || DW == 3, "weight ring");
  // loads that may still fly when stage b >= 1 has landed: those issued after
  // the later of W(b) and X(b), up to B(b) -- X(b + 1) when DW = 2, all of
  // stage b + 1 when DW = 3
  constexpr int WAITC = DW < DX ? C::LX : C::LW + C::LX;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool loader = wave >= 4;
  const int wv = wave & 3;
  const int wn = wv >> 1, wm = wv & 1;
  const int nkb = K / BK2;
  char *const xbase = lds + DW * C::W_BYTES;
  LoadPlan2<BN> pw;
  LoadPlan2<BM> px;
  if (loader) {
    pw.init(w, N, n0, N, ldw, K, wv, lane);
    px.init(x, M, m0, M, ldx, K, wv, lane);
  }
  f32x4 acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x4{};
  if (loader) {
    int sw = 0, sx = 0;  // slots of the next weight and activation stages
    auto issue_w = [&](int s) {
      pw.issue(lds + sw * C::W_BYTES, s * BK2, wv);
      sw = sw + 1 == DW ? 0 : sw + 1;
    };
    auto issue_x = [&](int s) {
      px.issue(xbase + sx * C::X_BYTES, s * BK2, wv);
      sx = sx + 1 == DX ? 0 : sx + 1;
    };
    // every slot starts free: stages 0 .. D - 1 of each operand, in stage order
#pragma unroll
    for (int s = 0; s < DX; ++s) {
      if (s < DW && s < nkb) issue_w(s);
      if (s < nkb) issue_x(s);
    }
    if (nkb >= DX) wait_vmcnt<(DW - 1) * C::LW + (DX - 1) * C::LX>();  // stage 0 has landed
    else wait_vmcnt<0>();
    barrier_no_fence();  // B(0)
    int b = 1;
    for (; b + DX - 1 < nkb; ++b) {
      wait_vmcnt<WAITC>();  // stage b has landed
      barrier_no_fence();   // B(b): stage b - 1 is read
      issue_w(b + DW - 1);
      issue_x(b + DX - 1);
    }
    for (; b < nkb; ++b) {
      if (b + DX - 2 < nkb) wait_vmcnt<WAITC>();
      else wait_vmcnt<0>();
      barrier_no_fence();
      if (b + DW - 1 < nkb) issue_w(b + DW - 1);
    }
    barrier_no_fence();  // the last stage is read
    return;
  }
  // slots of stage b (a) and b + 1 (b), and the ring's third slot (c)
  char *wa = lds, *wb = wa + C::W_BYTES, *wc = DW == 3 ? wb + C::W_BYTES : wa;
  char *xa = xbase, *xb = xa + C::X_BYTES, *xc = xb + C::X_BYTES;
  barrier_no_fence();  // B(0)
  Frags<BN, BM> f0, f1;
  read_frags2<BN, BM>(f0, wa, xa, 0, wn, wm, lane);
  int kb = 0;
  for (; kb + 2 < nkb; ++kb) {
    read_frags2<BN, BM>(f1, wa, xa, 1, wn, wm, lane);
    mfma_step<BN, BM>(acc, f0);
    interleave_even<C::FN * C::FM, 0, C::FN + C::FM>();
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    barrier_no_fence();  // B(kb + 1)
    __builtin_amdgcn_sched_barrier(0);
    read_frags2<BN, BM>(f0, wb, xb, 0, wn, wm, lane);
    mfma_step<BN, BM>(acc, f1);
    interleave_even<C::FN * C::FM, 0, C::FN + C::FM>();
    __builtin_amdgcn_sched_barrier(0);
    char *t = wa; wa = wb;
    if constexpr (DW == 3) { wb = wc; wc = t; }
    else wb = t;
    t = xa; xa = xb; xb = xc; xc = t;
  }
  if (kb + 1 < nkb) {
    read_frags2<BN, BM>(f1, wa, xa, 1, wn, wm, lane);
    mfma_step<BN, BM>(acc, f0);
    wait_lgkmcnt0();
    barrier_no_fence();
    read_frags2<BN, BM>(f0, wb, xb, 0, wn, wm, lane);
    mfma_step<BN, BM>(acc, f1);
    wa = wb;
    xa = xb;
  }
  read_frags2<BN, BM>(f1, wa, xa, 1, wn, wm, lane);
  mfma_step<BN, BM>(acc, f0);
  mfma_step<BN, BM>(acc, f1);
  barrier_no_fence();  // the last stage is read
  store_tile<BN, BM>(acc, lds, y, M, N, ldy, m0, n0, wn, wm, wv, lane);
}

template <int BN, int BM, int DW>
__global__ __launch_bounds__(2 * kThreads, 1) void gemm_split_role_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[role_lds_bytes<BN, BM, DW>()];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  role_tile<BN, BM, DW>(lds, x, w, y, M, N, K, ldx, ldw, ldy, tm, tn);
}

// The same tile bounded to 128 registers per lane, so that two workgroups
// share a CU when their LDS fits twice (the 128 x 64 tile: 72 KiB).
template <int BN, int BM, int DW>
__global__ __launch_bounds__(2 * kThreads, 4) void gemm_split_role_pair_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[role_lds_bytes<BN, BM, DW>()];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  role_tile<BN, BM, DW>(lds, x, w, y, M, N, K, ldx, ldw, ldy, tm, tn);
}

template <int BN, int BM>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n) {
  using C = Cfg<BN, BM>;
  __shared__ __attribute__((aligned(1024))) char lds[kStages * C::STAGE];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wv >> 1, wm = wv & 1;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int n0 = tn * BN, m0 = tm * BM;

  f32x4 acc[C::FN][C::FM];
  gemm_mainloop<BN, BM>(acc, lds, x, w, M, N, K / BK, ldx, ldw, m0, n0, wv, lane, K);
  barrier_no_fence();  // every wavefront is done reading the stages
  store_tile<BN, BM>(acc, lds, y, M, N, ldy, m0, n0, wn, wm, wv, lane);
}

// Split-K partial tile: blockIdx.y = chunk s covers k in [s*kc, (s+1)*kc).
// The same K loop as gemm_kernel over that range; the fp32 sums go to
// ws[s][m][n] (row stride N), four consecutive n per 16-byte store.
// WIDE: 64-k stages (kc % 64 == 0), else 32-k stages.
template <int BN, int BM, bool WIDE>
__global__ __launch_bounds__(kThreads, 1) void gemm_partial_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, float *__restrict__ ws,
    int M, int N, int kc, int64_t ldx, int64_t ldw, int tiles_m, int tiles_n) {
  using C = Cfg<BN, BM>;
  constexpr int LDS_BYTES = WIDE ? wide_lds_bytes<BN, BM, true>() : kStages * C::STAGE;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wv >> 1, wm = wv & 1;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int n0 = tn * BN, m0 = tm * BM;
  const int s = blockIdx.y;

  f32x4 acc[C::FN][C::FM];
  if constexpr (WIDE)
    gemm_mainloop2<BN, BM, true>(acc, lds, x + (int64_t)s * kc, w + (int64_t)s * kc, M, N,
                                 kc / BK2, ldx, ldw, m0, n0, wv, lane, kc);
  else
    gemm_mainloop<BN, BM>(acc, lds, x + (int64_t)s * kc, w + (int64_t)s * kc, M, N, kc / BK, ldx,
                          ldw, m0, n0, wv, lane, kc);

  // block (i, j), lane l: n = 16i + 4(l/16) .. +3, m = 16j + l%16 (N % 8 == 0,
  // so n < N covers all four)
  float *part = ws + (int64_t)s * M * N;
#pragma unroll
  for (int j = 0; j < C::FM; ++j) {
    const int m = m0 + wm * C::WM + j * 16 + (lane & 15);
    if (m >= M) continue;
    float *prow = part + (int64_t)m * N;
#pragma unroll
    for (int i = 0; i < C::FN; ++i) {
      const int n = n0 + wn * C::WN + i * 16 + (lane >> 4) * 4;
      if (n < N) *reinterpret_cast<f32x4 *>(prow + n) = acc[i][j];
    }
  }
}

// Fixed-order split-K combine: y[m][n] = bf16(((p_0 + p_1) + ...) + p_{S-1}),
// four outputs per thread.  All loads of a group of up to kCombineGroup
// partials are issued before its adds, which still run in s order, so the
// fold costs one memory round trip per group (one in all the splits used
// here); the skinny batches this path serves give the kernel few threads, so
// its time is that latency.
constexpr int kCombineGroup = 32;
__global__ __launch_bounds__(kThreads) void gemm_splitk_combine_kernel(
    const float *__restrict__ ws, uint16_t *__restrict__ y, int M, int N, int S, int64_t ldy) {
  const int64_t e = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  const int64_t total = (int64_t)M * N;
  if (e >= total) return;
  const int64_t m = e / N, n = e % N;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kCombineGroup) {
    f32x4 p[kCombineGroup];
    const float *q = ws + (int64_t)s0 * total + e;
#pragma unroll
    for (int i = 0; i < kCombineGroup; ++i, q += total)
      if (s0 + i < S) p[i] = *reinterpret_cast<const f32x4 *>(q);
#pragma unroll
    for (int i = 0; i < kCombineGroup; ++i)
      if (s0 + i < S) a = (s0 + i == 0) ? p[i] : a + p[i];  // the fold starts from p_0 itself
  }
  u32x2 o;
  o[0] = pack_bf16x2(a[0], a[1]);
  o[1] = pack_bf16x2(a[2], a[3]);
  *reinterpret_cast<u32x2 *>(y + m * ldy + n) = o;
}

// Split-K in one launch for batches of at most 16 rows.  A workgroup owns 16
// output columns and every chunk of K; wavefront wv takes chunks wv, wv + nw,
// ... one after another.  Each chunk is the same ascending run of 32-k
// matrix-core steps from zero as in gemm_partial_kernel (the weight and
// activation rows fetched as whole 128-byte lines and moved into the
// matrix-core layout in registers), so every partial p_s has the same bits.
// p_s goes to the workspace, as there, and to LDS; once every chunk is in, one
// wavefront folds ((p_0 + p_1) + ...) + p_{S-1} in fp32 and rounds once, as
// gemm_splitk_combine_kernel does.  At these sizes the separate fold's launch
// and the round trip of the partials through memory cost about as much as the
// weight stream itself.
constexpr int kFusedMaxM = 16;
constexpr int kFusedGroupK = 128;  // k per fetch group: two line pairs, four 32-k steps
constexpr int kFusedMaxWaves = 16;
constexpr int kFusedMaxChunks = 64 / kFusedMaxWaves;  // per wavefront (split_k <= 64)

template <bool ROWS8, bool COLS8>
__device__ __forceinline__ void fused_group(const LineOperand16<2, true, COLS8> &wl,
                                            const LineOperand16<2, false, ROWS8> &xl, f32x4 &acc,
                                            bool first, int lane) {
  bf16x8 fw[4], fx[4];
  wl.place(fw, lane);
  xl.place(fx, lane);
  if (first) acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[t], fx[t], acc, 0, 0, 0);
}

// (x and w are not __restrict__: the compiler may then move their loads
// across the empty asm statement that keeps them ahead of the products.)
// ROWS8 (M <= 8): only the first 8 rows of x are fetched; the products of
// fragment rows 8-15 are then meaningless and, as always for rows >= M, never
// stored or folded.  COLS8: the same on the weight side -- a workgroup owns 8
// columns, only those weight rows are fetched, and the block's columns 8-15
// are discarded (twice the workgroups for narrow outputs).
template <bool ROWS8, bool COLS8>
__global__ __launch_bounds__(64 * kFusedMaxWaves) void gemm_splitk_fused_kernel(
    const uint16_t *x, const uint16_t *w, float *__restrict__ ws,
    uint16_t *__restrict__ y, int M, int N, int S, int kc, int64_t ldx, int64_t ldw, int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) float part[];  // [S][16 m][16 n]
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;  // <= S
  constexpr int NB = COLS8 ? 8 : 16;  // output columns of the workgroup
  const int n0 = blockIdx.x * NB;
  // Line loads (LineOperand16): lane 8q + u fetches unit u of row q and unit
  // u ^ 4 of row 8 + q.  Rows past the matrix edge repeat its last row; their
  // results are never stored.
  const int q = lane >> 3, u = lane & 7;
  const uint16_t *wlo = w + (int64_t)min(n0 + q, N - 1) * ldw + 8 * u;
  const uint16_t *whi = w + (int64_t)min(n0 + 8 + q, N - 1) * ldw + 8 * (u ^ 4);
  const uint16_t *xlo = x + (int64_t)min(q, M - 1) * ldx + 8 * u;
  const uint16_t *xhi = x + (int64_t)min(8 + q, M - 1) * ldx + 8 * (u ^ 4);
  const int gpc = kc / kFusedGroupK;            // fetch groups per chunk
  const int nch = (S - 1 - wv) / nw + 1;        // chunks of this wavefront (at most 4)
  const int G = nch * gpc;                      // its fetch groups
  auto k_of = [&](int g) {
    return (int64_t)(wv + (g / gpc) * nw) * kc + (int64_t)(g % gpc) * kFusedGroupK;
  };
  LineOperand16<2, true, COLS8> wa, wb;
  LineOperand16<2, false, ROWS8> xa, xb;
  auto issue = [&](LineOperand16<2, true, COLS8> &wl, LineOperand16<2, false, ROWS8> &xl, int g) {
    const int64_t k = k_of(g);
    wl.issue(wlo + k, whi + k);
    xl.issue(xlo + k, xhi + k);
    // keep these loads ahead of the products that follow them in the source:
    // left alone, the compiler sinks them below and loses the overlap
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // The chunk partials stay in registers until every load has been issued:
  // a store inside the loop would make the compiler wait for every load.
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f}, ps[kFusedMaxChunks] = {};
  auto consume = [&](const LineOperand16<2, true, COLS8> &wl, const LineOperand16<2, false, ROWS8> &xl,
                     int g) {
    fused_group(wl, xl, acc, g % gpc == 0, lane);
    const int ci = g / gpc;
#pragma unroll
    for (int i = 0; i < kFusedMaxChunks; ++i)
      if (i == ci) ps[i] = acc;
  };
  // Two groups in flight: one loads while the other multiplies.  The loop
  // body has no branch around a load, so the waits count exactly.
  issue(wa, xa, 0);
  int g = 0;
  for (; g + 2 < G; g += 2) {
    issue(wb, xb, g + 1);
    consume(wa, xa, g);
    issue(wa, xa, g + 2);
    consume(wb, xb, g + 1);
  }
  if (g + 1 < G) {
    issue(wb, xb, g + 1);
    consume(wa, xa, g);
    consume(wb, xb, g + 1);
  } else {
    consume(wa, xa, g);
  }
  // every chunk's partial, to LDS and to the workspace.  Block layout:
  // register v of lane l is n = 4 (l >> 4) + v, m = l & 15.
  {
    const int m = lane & 15, c = lane >> 4;
#pragma unroll
    for (int i = 0; i < kFusedMaxChunks; ++i) {
      if (i >= nch) break;
      const int s = wv + i * nw;
      *reinterpret_cast<f32x4 *>(part + (s * 16 + m) * 16 + 4 * c) = ps[i];
      if (m < M && 4 * c < NB && n0 + 4 * c < N)
        *reinterpret_cast<f32x4 *>(ws + ((int64_t)s * M + m) * N + n0 + 4 * c) = ps[i];
    }
  }
  __syncthreads();
  if (wv != 0) return;
  // lane t: row t / 4, columns 4 (t % 4) .. +3
  const int m = lane >> 2, c = lane & 3;
  if (m >= M || 4 * c >= NB || n0 + 4 * c >= N) return;
  const float *p = part + m * 16 + 4 * c;
  f32x4 a = *reinterpret_cast<const f32x4 *>(p);  // the fold starts from p_0 itself
  for (int s = 1; s < S; ++s) a = a + *reinterpret_cast<const f32x4 *>(p + s * 256);
  u32x2 o;
  o[0] = pack_bf16x2(a[0], a[1]);
  o[1] = pack_bf16x2(a[2], a[3]);
  *reinterpret_cast<u32x2 *>(y + (int64_t)m * ldy + n0 + 4 * c) = o;
}

// ---------------------------------------------------------------------------
// Ping-pong variant of the 64-k kernel: 8 wavefronts, two per SIMD (the
// dispatcher places wave w on SIMD w & 3; only the overlap described below,
// never a result, depends on that placement), in two groups g = w >> 2.
// SIMD q owns quadrant (q >> 1, q & 1) of the tile, QN x QM; wave (q, g) owns
// half g of it along m, QN x QM/2.  A stage is one phase of fragment reads and one phase of
// matrix-core steps per wave; the groups run these phases in opposition --
// while group 0 reads stage j's fragments, group 1 multiplies stage j - 1, and
// the other way round -- separated by workgroup barriers (group 1 starts one
// barrier late and group 0 ends one barrier later), so each SIMD's matrix core
// always has one wave's products to run while the other wave waits on LDS.
// Group 0 loads the activations (a ring of 2 stages, the next stage issued
// one stage ahead), group 1 the weights (a ring of 3, two stages ahead): with
// few rows the weights are the stream that matters, and the ring of 3 gives
// their loads three phases to land instead of two.
// Every accumulator still receives its 32-k steps in ascending order from one
// wave, so the bits equal the 4-wave kernels'.
//
// Stage timing (B(i): the i-th barrier; phases between them):
//   group 0 reads stage j in (B(2j), B(2j+1)), multiplies it in (B(2j+1), B(2j+2));
//   group 1 reads stage j in (B(2j+1), B(2j+2)), multiplies it in (B(2j+2), B(2j+3)).
//   Stage j's slots are free after B(2j+2).  Group 0 issues activation stage
//   j+1 while reading stage j (slot of j-1) and waits for it before B(2j+2);
//   group 1 issues weight stage j+2 while reading stage j (slot of j-1) and
//   waits for stage j+1 before B(2j+2).
template <int BN, int BM>
constexpr int pp_lds_bytes() {
  return 2 * BM * kRow2 + 3 * BN * kRow2;
}

// Tile (tm, tn): rows tm * BM.., columns tn * BN.., by a workgroup of 512 threads.
template <int BN, int BM>
__device__ __forceinline__ void pp_tile(char *lds, const uint16_t *__restrict__ x,
                                        const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
                                        int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy,
                                        int tm, int tn) {
  const int m0 = tm * BM, n0 = tn * BN;
  constexpr int QN = BN / 2, QM = BM / 2, WM = QM / 2;
  constexpr int FN = QN / 16, FM = WM / 16;  // 16x16 blocks per wave
  constexpr int WB = BN * kRow2, XB = BM * kRow2;
  constexpr int LW = BN / 32, LX = BM / 32;
  static_assert(pp_lds_bytes<BN, BM>() <= 160 * 1024, "LDS");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = wave & 3, g = wave >> 2;
  const int nw = (q >> 1) * QN, mw = (q & 1) * QM + g * WM;
  const int nkb = K / BK2;
  char *const xs0 = lds, *const xs1 = lds + XB;                          // ring of 2
  char *const ws0 = lds + 2 * XB, *const ws1 = ws0 + WB, *const ws2 = ws1 + WB;  // ring of 3
  static_assert(BN == BM, "one load plan per group");
  LoadPlan2<BN> pl;  // group 0: rows of x; group 1: rows of w
  if (g == 0) pl.init(x, M, m0, M, ldx, K, q, lane);
  else pl.init(w, N, n0, N, ldw, K, q, lane);
  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{};

  if (g == 0) {
    pl.issue(xs0, 0, q);
    if (nkb > 1) {
      pl.issue(xs1, BK2, q);
      wait_vmcnt<LX>();
    } else {
      wait_vmcnt<0>();
    }
  } else {
    pl.issue(ws0, 0, q);
    if (nkb > 1) pl.issue(ws1, BK2, q);
    if (nkb > 2) pl.issue(ws2, 2 * BK2, q);
    if (nkb > 2) wait_vmcnt<2 * LW>();
    else if (nkb > 1) wait_vmcnt<LW>();
    else wait_vmcnt<0>();
  }
  barrier_no_fence();
  if (g == 1) barrier_no_fence();

  bf16x8 fa[2][FN], fb[2][FM];
  for (int j = 0; j < nkb; ++j) {
    const char *xc = (j & 1) ? xs1 : xs0;
    const int js = j % 3;
    const char *wc = js == 0 ? ws0 : (js == 1 ? ws1 : ws2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < FN; ++i) fa[st][i] = read_frag2(wc, nw + i * 16 + (lane & 15), st, lane);
#pragma unroll
      for (int jj = 0; jj < FM; ++jj) fb[st][jj] = read_frag2(xc, mw + jj * 16 + (lane & 15), st, lane);
    }
    if (g == 0) {
      if (j >= 1 && j + 1 < nkb) pl.issue((j & 1) ? xs0 : xs1, (j + 1) * BK2, q);
    } else {
      if (j >= 1 && j + 2 < nkb) {
        const int ns = (j + 2) % 3;
        pl.issue(ns == 0 ? ws0 : (ns == 1 ? ws1 : ws2), (j + 2) * BK2, q);
      }
    }
    wait_lgkmcnt0();
    if (g == 1) {
      if (j + 2 < nkb) wait_vmcnt<LW>();
      else wait_vmcnt<0>();
    }
    __builtin_amdgcn_sched_barrier(0);
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int jj = 0; jj < FM; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[st][i], fb[st][jj], acc[i][jj], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (g == 0) wait_vmcnt<0>();
    barrier_no_fence();
  }
  if (g == 0) barrier_no_fence();
  // every stage read is done and no load is in flight: the LDS is free for the
  // epilogue, one QN x WM region per wave
  store_sub<FN, FM>(acc, lds + wave * (WM * QN * 2), y, M, N, ldy, m0 + mw, n0 + nw, lane);
}

template <int BN, int BM>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[pp_lds_bytes<BN, BM>()];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  pp_tile<BN, BM>(lds, x, w, y, M, N, K, ldx, ldw, ldy, tm, tn);
}

// 256 x 256 tiles with the last, at most half full wave of each XCD cut in
// two.  The workgroups of XCD x (launch index % 8) take that XCD's range of
// logical tiles as tile_of does; its full waves run as 256 x 256 tiles
// (pp_tile), and when its remaining tiles would leave at least half of its
// CUs idle, each of them runs as two 256 x 128 tiles (role_tile), which fill
// the XCD.  Each output element still receives the same 32-k steps in
// ascending order from one wavefront, so the bits equal every other
// configuration's; only the number of outputs a workgroup owns changes.
constexpr int kCusPerXcd = 32;  // MI355X: 256 CUs in 8 XCDs
// Of c tiles on one XCD, how many run as halves.
__host__ __device__ inline int mixed_tail(int c) {
  const int t = c % kCusPerXcd;
  return t <= kCusPerXcd / 2 ? t : 0;
}
// Workgroups per XCD slot of the launch (the launch has 8 times as many).
__host__ __device__ inline int mixed_slots(int T) {
  const int q = T >> 3, r = T & 7;
  const int c0 = q + (r > 0 ? 1 : 0), c1 = q;  // tiles of XCD 0 and of XCD 7
  const int n0 = c0 + mixed_tail(c0), n1 = c1 + mixed_tail(c1);
  return n0 > n1 ? n0 : n1;
}

__global__ __launch_bounds__(512, 1) void gemm_mixed_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n) {
  constexpr int PP = pp_lds_bytes<256, 256>(), RS = role_lds_bytes<256, 128, 2>();
  __shared__ __attribute__((aligned(1024))) char lds[PP > RS ? PP : RS];
  const int T = tiles_m * tiles_n;
  const int q = T >> 3, r = T & 7;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int c = q + (xcd < r ? 1 : 0);
  const int first = xcd * q + (xcd < r ? xcd : r);  // the XCD's first logical tile, as xcd_lid
  const int tail = mixed_tail(c), full = c - tail;
  int tm, tn;
  if (local < full) {
    group_tile(first + local, tiles_m, tiles_n, tm, tn);
    pp_tile<256, 256>(lds, x, w, y, M, N, K, ldx, ldw, ldy, tm, tn);
    return;
  }
  const int h = local - full;
  if (h >= 2 * tail) return;  // slots past this XCD's share
  group_tile(first + full + (h >> 1), tiles_m, tiles_n, tm, tn);
  const int th = 2 * tm + (h & 1);  // the half as a 256 x 128 tile row
  if (th * 128 >= M) return;        // a half wholly past the last row
  role_tile<256, 128, 2>(lds, x, w, y, M, N, K, ldx, ldw, ldy, th, tn);
}

typedef void (*GemmKernel)(const uint16_t *, const uint16_t *, uint16_t *, int, int, int, int64_t,
                           int64_t, int64_t, int, int);
struct CfgEntry {
  int bn, bm;
  GemmKernel kernel;  // BK = 32 stages, any K % 32 == 0 (256 threads)
  GemmKernel wide;    // BK = 64 stages, used when K % 64 == 0 (same k order, same bits)
  int wide_threads;   // workgroup size of `wide`
  bool mixed;         // `wide` is gemm_mixed_kernel: its own workgroup count
};

// Every 64-k kernel runs 8 wavefronts.  At 256 x 256 they are two ping-pong
// groups of four (the 4-wavefront form measured 15-20 % slower: its 256
// accumulators per wavefront fill every AGPR, and the compiler then copies
// them between register files inside the K loop).  The smaller tiles split
// the roles: four compute, four load (4-13 % faster than four wavefronts
// doing both, 8-9 % at 256 x 128).  At 128 x 128 the weights take a ring of 3
// too (96 KiB, one workgroup per CU): 11-20 % faster at M <= 4096 than the
// ring of 2 with two workgroups per CU, 8 % slower at M = 8192.
// The 128 x 64 tile runs two workgroups per CU (72 KiB of LDS, 92 registers);
// only bi_gemm_fill picks it, where 128 x 128 tiles would leave at least half
// of the CUs idle: on N = 1024, K = 4096 it measured 434 / 795 TFLOP/s at
// M = 1024 / 2048 against 353 / 701 for 128 x 128, and 868 against 1110 at
// M = 4096.
// The last configuration is the mixed 256 x 256 / 256 x 128 launch: only
// bi_gemm_fill picks it (the split follows M), and with K % 64 == 32 it runs
// as configuration 0.
const CfgEntry kConfigs[] = {
    {256, 256, gemm_kernel<256, 256>, gemm_pp_kernel<256, 256>, 512, false},
    {256, 128, gemm_kernel<256, 128>, gemm_split_role_kernel<256, 128, 2>, 2 * kThreads, false},
    {128, 128, gemm_kernel<128, 128>, gemm_split_role_kernel<128, 128, 3>, 2 * kThreads, false},
    {128, 256, gemm_kernel<128, 256>, gemm_split_role_kernel<128, 256, 2>, 2 * kThreads, false},
    {128, 64, gemm_kernel<128, 64>, gemm_split_role_pair_kernel<128, 64, 3>, 2 * kThreads, false},
    {256, 256, gemm_kernel<256, 256>, gemm_mixed_kernel, 512, true},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

// Split-K path: one tile shape for every (N, K) and M, sized for decode-like
// batches (one 64-row tile covers M <= 64).
constexpr int kSplitBN = 128, kSplitBM = 64;

int splitk_for(int64_t N, int64_t K) {
  const int64_t tiles_n = (N + kSplitBN - 1) / kSplitBN;
  int S = 1;
  // smallest power of two that gives >= 256 workgroups at M <= 64, keeping
  // at least 8 32-k steps per chunk (shorter chunks leave the one-launch
  // kernel a single fetch group per chunk: at N = 1024, K = 4096 a split of 16
  // measured 6-10 % faster than 32 at M = 1-33)
  while (tiles_n * S < 256 && K % (2 * S * BK) == 0 && K / (2 * S) >= 8 * BK && S < 64) S *= 2;
  return S;
}

int config_for(int64_t N, int64_t K) {
  (void)K;
  return N >= 4096 ? 0 : 2;
}

// Tile for bi_gemm_fill: the configuration with the smallest estimated time,
// (waves of tiles over the CUs) x (relative time of one tile).  The tile
// costs are measured ones, relative to 256 x 256: a 256 x 128 tile takes
// ~0.68 of it, a 128 x 256 tile ~0.67, a 128 x 128 tile ~0.34 and a 128 x 64
// tile ~0.23 (a wave is one tile per CU).  So three waves of either half-size
// tile do not replace two of the big tile (measured 1-9 % slower), and the
// 128 x 64 tile wins only where it fills the chip in one wave and 128 x 128
// tiles fill at most half of it.  The mixed launch costs each XCD its full
// waves of 256 x 256 tiles plus, if it cuts a tail, one wave of 256 x 128
// tiles; it is taken only for 64-k stages on a chip of 8 x kCusPerXcd CUs.
// Ties keep the earlier configuration.
int fill_config_for(int64_t M, int64_t N, int64_t K) {
  static const double kTileCost[kNumConfigs] = {1.0, 0.68, 0.34, 0.67, 0.23, 1.0};
  const int64_t cus = cu_count();
  int best = 0;
  double best_t = 0.0;
  for (int c = 0; c < kNumConfigs; ++c) {
    const int64_t tiles = ((M + kConfigs[c].bm - 1) / kConfigs[c].bm) *
                          ((N + kConfigs[c].bn - 1) / kConfigs[c].bn);
    double t = (double)((tiles + cus - 1) / cus) * kTileCost[c];
    // the 128 x 64 tile's cost holds for one wave only: with two tiles per CU
    // each runs slower (Up at M = 512, 3.5 waves: 98 us against 75 us for one
    // wave of 256 x 256 tiles)
    if (kConfigs[c].bm == 64 && tiles > cus) continue;
    if (kConfigs[c].mixed) {
      if (K % BK2 || cus != 8 * kCusPerXcd || tiles > 0x7FFFFFFF) continue;
      const int64_t q = tiles >> 3, r = tiles & 7;
      t = 0.0;
      for (int64_t cx : {q + (r > 0 ? 1 : 0), q}) {
        const int tail = mixed_tail((int)cx);
        const double tx = (double)((cx - tail + kCusPerXcd - 1) / kCusPerXcd) * kTileCost[c] +
                          (tail ? kTileCost[1] : 0.0);
        t = tx > t ? tx : t;
      }
    }
    if (c == 0 || t < best_t - 1e-9) {
      best = c;
      best_t = t;
    }
  }
  return best;
}

int validate(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t N, int64_t K,
             int64_t ldx, int64_t ldw, int64_t ldy) {
  if (!w || (M > 0 && (!x || !y))) return BI_ERR_NULL;
  if (M < 0 || N < 8 || K < BK || ldx < K || ldw < K || ldy < N || M > (1 << 30) ||
      N > (1 << 30) || K > (1 << 30))
    return BI_ERR_SHAPE;
  if (K % BK) return BI_ERR_SHAPE;
  // the loads address each operand with 32-bit element offsets
  if ((M > 0 && (M - 1) * ldx + K >= (int64_t(1) << 31)) || (N - 1) * ldw + K >= (int64_t(1) << 31))
    return BI_ERR_SHAPE;
  if ((N | ldx | ldw | ldy) & 7 || !aligned16(x) || !aligned16(w) || !aligned16(y))
    return BI_ERR_ALIGN;
  const Span sy = span_of(y, M, N, ldy, 2);
  if (overlap(sy, span_of(x, M, K, ldx, 2)) || overlap(sy, span_of(w, N, K, ldw, 2)))
    return BI_ERR_ALIAS;
  return BI_OK;
}

// Everything a launch of configuration cfg depends on.  M enters only the
// number of tile rows (how many workgroups run), never the kernel, its tile or
// its K stage -- except in the mixed configuration, which bi_gemm never uses.
struct Plan {
  int cfg, bm, bn, kstage, threads;
  int64_t tiles_m, tiles_n, groups;
  GemmKernel kern;
};
Plan plan_for(int cfg, int64_t M, int64_t N, int64_t K) {
  const CfgEntry &c = kConfigs[cfg];
  const bool wide = c.wide && K % BK2 == 0;
  const int64_t tm = (M + c.bm - 1) / c.bm, tn = (N + c.bn - 1) / c.bn;
  int64_t groups = tm * tn;
  if (wide && c.mixed && groups <= 0x7FFFFFFF) groups = 8 * (int64_t)mixed_slots((int)groups);
  return Plan{cfg, c.bm, c.bn, wide ? BK2 : BK, wide ? c.wide_threads : kThreads, tm, tn, groups,
              wide ? c.wide : c.kernel};
}

int launch(int cfg, const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t N,
           int64_t K, int64_t ldx, int64_t ldw, int64_t ldy, void *stream) {
  const Plan p = plan_for(cfg, M, N, K);
  if (p.tiles_m * p.tiles_n > 0x7FFFFFFF || p.groups > 0x7FFFFFFF) return BI_ERR_SHAPE;
  hipLaunchKernelGGL(p.kern, dim3((unsigned)p.groups), dim3(p.threads), 0,
                     (hipStream_t)stream, x, w, y, (int)M, (int)N, (int)K, ldx, ldw, ldy,
                     (int)p.tiles_m, (int)p.tiles_n);
  return launch_status();
}

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" int bi_gemm_config_id(int64_t N, int64_t K) {
  if (N < 8 || (N & 7) || K < BK || K % BK) return -1;
  return config_for(N, K);
}

extern "C" int bi_gemm(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t N,
                       int64_t K, int64_t ldx, int64_t ldw, int64_t ldy, void *stream) {
  const int st = validate(x, w, y, M, N, K, ldx, ldw, ldy);
  if (st != BI_OK || M == 0) return st;
  return launch(config_for(N, K), x, w, y, M, N, K, ldx, ldw, ldy, stream);
}

extern "C" int bi_gemm_launch_plan(int64_t M, int64_t N, int64_t K, int64_t *plan) {
  if (!plan) return BI_ERR_NULL;
  const int cfg = bi_gemm_config_id(N, K);
  if (M < 0 || cfg < 0) return BI_ERR_SHAPE;
  // the same function bi_gemm's launch() builds its launch from
  const Plan p = plan_for(cfg, M, N, K);
  int64_t kid = -1;
  for (int c = 0; c < kNumConfigs && kid < 0; ++c) {  // the first entry holding the kernel
    if (p.kern == kConfigs[c].kernel) kid = 2 * c;
    else if (p.kern == kConfigs[c].wide) kid = 2 * c + 1;
  }
  plan[0] = p.cfg;
  plan[1] = kid;
  plan[2] = p.bm;
  plan[3] = p.bn;
  plan[4] = p.kstage;
  plan[5] = p.threads;
  plan[6] = M == 0 ? 0 : p.groups;
  return BI_OK;
}

extern "C" int bi_gemm_num_configs(void) { return kNumConfigs; }

extern "C" int bi_gemm_fill_config_id(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 8 || (N & 7) || K < BK || K % BK) return -1;
  return fill_config_for(M, N, K);
}

extern "C" int bi_gemm_fill(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M,
                            int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                            void *stream) {
  const int st = validate(x, w, y, M, N, K, ldx, ldw, ldy);
  if (st != BI_OK || M == 0) return st;
  return launch(fill_config_for(M, N, K), x, w, y, M, N, K, ldx, ldw, ldy, stream);
}

extern "C" int bi_gemm_with_config(int config, const uint16_t *x, const uint16_t *w, uint16_t *y,
                                   int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw,
                                   int64_t ldy, void *stream) {
  if (config < 0 || config >= kNumConfigs) return BI_ERR_UNSUPPORTED;
  const int st = validate(x, w, y, M, N, K, ldx, ldw, ldy);
  if (st != BI_OK || M == 0) return st;
  return launch(config, x, w, y, M, N, K, ldx, ldw, ldy, stream);
}

extern "C" int bi_gemm_splitk_for(int64_t N, int64_t K) {
  if (N < 8 || (N & 7) || K < BK || K % BK) return -1;
  return splitk_for(N, K);
}

extern "C" size_t bi_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int split_k) {
  if (M <= 0 || N <= 0 || split_k <= 0) return 0;
  const size_t b = (size_t)split_k * (size_t)M * (size_t)N * 4u;
  return (b + 255u) & ~(size_t)255u;
}

namespace bi {
namespace {

// Checks of bi_gemm_splitk's operands other than the workspace.
int splitk_validate(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t N,
                    int64_t K, int64_t ldx, int64_t ldw, int64_t ldy, int split_k) {
  const int st = validate(x, w, y, M, N, K, ldx, ldw, ldy);
  if (st != BI_OK) return st;
  if (split_k < 1 || split_k > 64) return BI_ERR_UNSUPPORTED;
  if (K % ((int64_t)split_k * BK)) return BI_ERR_SHAPE;
  if (M > 0 && ((M + kSplitBM - 1) / kSplitBM) * ((N + kSplitBN - 1) / kSplitBN) > 0x7FFFFFFF)
    return BI_ERR_SHAPE;
  return BI_OK;
}

// The partial kernel over (tiles, split_k), then the fixed-order fold; wsf
// holds split_k * M * N floats.  Batches of at most 16 rows (chunks a multiple
// of 128 k) take the one-launch kernel instead: same partials, same fold.
int splitk_launch(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t N,
                  int64_t K, int64_t ldx, int64_t ldw, int64_t ldy, int split_k, float *wsf,
                  void *stream) {
  const int64_t tiles_m = (M + kSplitBM - 1) / kSplitBM, tiles_n = (N + kSplitBN - 1) / kSplitBN;
  hipStream_t s = (hipStream_t)stream;
  const int kc = (int)(K / split_k);
  if (M <= kFusedMaxM && kc % kFusedGroupK == 0) {
    // 8-column workgroups when 16-column ones would leave at least half of the
    // CUs idle (every workgroup also fetches the activations, so splitting
    // further costs more than it gains: at N = 4096 8-column workgroups
    // measured 15-26 % slower, at N = 1024 3-7 % faster)
    const bool cols8 = 2 * ((N + 15) / 16) <= (int64_t)cu_count();
    // One wavefront per chunk, except with more than 8 rows in 16-column
    // workgroups: there each wavefront takes two chunks (at M = 16 measured
    // 5 % faster on 4096 x 4096 and 9 % on 4096 x 14336).  Which wavefront
    // computes a chunk changes no bit.
    int nw = split_k < kFusedMaxWaves ? split_k : kFusedMaxWaves;
    if (M > 8 && !cols8) nw = split_k / 2 < 1 ? 1 : (split_k / 2 < kFusedMaxWaves ? split_k / 2 : kFusedMaxWaves);
    const dim3 grid((unsigned)(cols8 ? (N + 7) / 8 : (N + 15) / 16)), block(64 * nw);
    const size_t lds = (size_t)split_k * 16 * 16 * sizeof(float);
#define BI_FUSED(R8, C8)                                                                            \
  hipLaunchKernelGGL((gemm_splitk_fused_kernel<R8, C8>), grid, block, lds, s, x, w, wsf, y, (int)M, \
                     (int)N, split_k, kc, ldx, ldw, ldy)
    if (M <= 8) {
      if (cols8) BI_FUSED(true, true);
      else BI_FUSED(true, false);
    } else {
      if (cols8) BI_FUSED(false, true);
      else BI_FUSED(false, false);
    }
#undef BI_FUSED
    return launch_status();
  }
  // 64-column partial tiles when 128-column ones would leave at least half of
  // the CUs idle (N = 1024 at M <= 64: 256 workgroups instead of 128).  Every
  // partial is the same ascending run of 32-k steps whatever the tile, so the
  // bits do not change.
  const bool narrow = 2 * tiles_m * tiles_n * split_k <= (int64_t)cu_count();
  constexpr int kNarrowBN = kSplitBN / 2;
  const int64_t pt_n = narrow ? (N + kNarrowBN - 1) / kNarrowBN : tiles_n;  // partial tile columns
#define BI_PARTIAL(BN, WIDE)                                                                       \
  hipLaunchKernelGGL((gemm_partial_kernel<BN, kSplitBM, WIDE>),                                    \
                     dim3((unsigned)(tiles_m * pt_n), (unsigned)split_k), dim3(kThreads), 0, s, x, \
                     w, wsf, (int)M, (int)N, kc, ldx, ldw, (int)tiles_m, (int)pt_n)
  if (kc % BK2 == 0) {
    if (narrow) BI_PARTIAL(kNarrowBN, true);
    else BI_PARTIAL(kSplitBN, true);
  } else {
    if (narrow) BI_PARTIAL(kNarrowBN, false);
    else BI_PARTIAL(kSplitBN, false);
  }
#undef BI_PARTIAL
  int st = launch_status();
  if (st != BI_OK) return st;
  const int64_t groups = (M * N / 4 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(gemm_splitk_combine_kernel, dim3((unsigned)groups), dim3(kThreads), 0, s, wsf,
                     y, (int)M, (int)N, split_k, ldy);
  return launch_status();
}

// Scratch of the allocation-free split-K entry point: a static device array
// (each GPU the library runs on holds its own copy until the process ends).
// In host code its name is only a stand-in; the device address comes from
// hipGetSymbolAddress, looked up once per device and kept here.
static __device__ __align__(256) unsigned char scratch[BI_GEMM_SPLITK_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream).
int scratch_ptr(void *stream, void **out) {
  int dev = 0;
  if (stream != nullptr) {
    if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return BI_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return BI_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return BI_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return BI_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return BI_ERR_HIP;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return BI_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return BI_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BI_OK;
}

}  // namespace
}  // namespace bi

extern "C" int bi_gemm_splitk(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M,
                              int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                              int split_k, void *ws, size_t ws_bytes, void *stream) {
  const int st = splitk_validate(x, w, y, M, N, K, ldx, ldw, ldy, split_k);
  if (st != BI_OK || M == 0) return st;
  if (!ws) return BI_ERR_NULL;
  if (ws_bytes < bi_gemm_splitk_workspace_bytes(M, N, split_k)) return BI_ERR_WORKSPACE;
  if (!aligned16(ws)) return BI_ERR_ALIGN;
  const Span sw{(uintptr_t)ws, (uintptr_t)ws + (uintptr_t)(split_k * M * N * 4)};
  if (overlap(sw, span_of(y, M, N, ldy, 2)) || overlap(sw, span_of(x, M, K, ldx, 2)) ||
      overlap(sw, span_of(w, N, K, ldw, 2)))
    return BI_ERR_ALIAS;
  return splitk_launch(x, w, y, M, N, K, ldx, ldw, ldy, split_k, static_cast<float *>(ws), stream);
}

extern "C" int bi_gemm_splitk_noalloc(const uint16_t *x, const uint16_t *w, uint16_t *y,
                                      int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw,
                                      int64_t ldy, int split_k, void *stream) {
  const int st = splitk_validate(x, w, y, M, N, K, ldx, ldw, ldy, split_k);
  if (st != BI_OK || M == 0) return st;
  if (bi_gemm_splitk_workspace_bytes(M, N, split_k) > (size_t)BI_GEMM_SPLITK_SCRATCH_BYTES)
    return BI_ERR_WORKSPACE;
  void *p = nullptr;
  const int sp = scratch_ptr(stream, &p);
  if (sp != BI_OK) return sp;
  // every partial the fold reads is written first by the same call: nothing
  // in the scratch has to start at zero
  return splitk_launch(x, w, y, M, N, K, ldx, ldw, ldy, split_k, static_cast<float *>(p), stream);
}

extern "C" int bi_gemm_mswitch_control(const uint16_t *x, const uint16_t *w, uint16_t *y,
                                       int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw,
                                       int64_t ldy, void *ws, size_t ws_bytes, void *stream) {
  // CONTROL ONLY: the configuration switch batch-invariant kernels forbid --
  // split-K when the batch is small, one pass otherwise.
  if (M > 0 && M <= kSplitBM) {
    const int S = bi_gemm_splitk_for(N, K);
    if (S < 1) return BI_ERR_SHAPE;
    return bi_gemm_splitk(x, w, y, M, N, K, ldx, ldw, ldy, S, ws, ws_bytes, stream);
  }
  return bi_gemm(x, w, y, M, N, K, ldx, ldw, ldy, stream);
}
