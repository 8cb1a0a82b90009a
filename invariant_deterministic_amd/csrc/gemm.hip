// gemm.hip -- batch-invariant bf16 GEMM for gfx950: y = bf16(x . w^T), fp32 accumulation.
//
// "Cómo superar la no determinación en la inferencia de LLM", section
// "Multiplicación de matrices (matmul)": tile the output in 2-D, process tiles
// data-parallel, and force one kernel configuration for every batch size
// (no split-K chosen for small batches), accepting some lost speed.
//
// Reduction order of every output element (the batch-invariance contract):
// one pass over k = 0, 16, 32, ..., K-16, each step a single
// v_mfma_f32_32x32x16_bf16 whose fp32 accumulator is rounded between steps.
// The order never depends on M, on the tile the element falls in, on the
// position of the element inside its 32x32 matrix-core block, or on the
// tile configuration: every configuration below runs the same instruction
// over the same k steps; configurations differ only in how many outputs one
// workgroup owns.  The configuration is picked from (N, K) alone.
//
// Data path per workgroup (4 wavefronts, 2 x 2 over the tile):
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
// that the 32 rows a fragment read touches spread over all LDS banks.  Rows
// beyond M (or N) are loaded as copies of the last valid row and never
// stored, so no row's arithmetic depends on how many rows the batch holds.
#include "common.h"

namespace bi {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 32;                 // k per LDS stage (two 16-k matrix-core steps)
constexpr int kRowBytes = BK * 2;      // one LDS row: 32 bf16 = four 16-byte chunks
constexpr int kStages = 4;             // LDS ring depth: 3 stages of loads in flight

// Chunk permutation of LDS row r (4 chunks of 16 bytes): chunk c of row r is
// stored at c ^ ((r >> 2) & 3).  A fragment read (32 rows, one chunk each, per
// half-wavefront) then hits each 16-byte bank group of every 256-byte LDS
// window once per 16 lanes -- conflict-free; measured on gfx950 with four
// wavefronts reading concurrently, where the plain layout costs 2x.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

template <int BN, int BM>
struct Cfg {
  static constexpr int WN = BN / 2, WM = BM / 2;    // wavefront tile (n x m)
  static constexpr int FN = WN / 32, FM = WM / 32;  // 32x32 blocks per wavefront
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

// Fragment of 32 rows x 16 k for the 32x32x16 instruction: lane l takes row
// (l & 31) and k = ks*16 + (l >> 5)*8 .. +7 -- the same k mapping for both
// operands, so the instruction pairs matching k.
__device__ __forceinline__ bf16x8 read_frag(const char *lds, int row, int ks, int lane) {
  const int lc = ks * 2 + (lane >> 5);
  const int off = row * kRowBytes + ((lc ^ swz(row)) << 4);
  return *reinterpret_cast<const bf16x8 *>(lds + off);
}

template <int BN, int BM>
struct Frags {
  bf16x8 a[BN / 64], b[BM / 64];
};

template <int BN, int BM>
__device__ __forceinline__ void read_frags(Frags<BN, BM> &f, const char *lds, int ks, int wn, int wm,
                                           int lane) {
  using C = Cfg<BN, BM>;
#pragma unroll
  for (int i = 0; i < C::FN; ++i) f.a[i] = read_frag(lds, wn * C::WN + i * 32 + (lane & 31), ks, lane);
#pragma unroll
  for (int j = 0; j < C::FM; ++j)
    f.b[j] = read_frag(lds + C::W_BYTES, wm * C::WM + j * 32 + (lane & 31), ks, lane);
}

template <int BN, int BM>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[BN / 64][BM / 64], const Frags<BN, BM> &f) {
#pragma unroll
  for (int i = 0; i < BN / 64; ++i)
#pragma unroll
    for (int j = 0; j < BM / 64; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Scheduling hint for the second half of a steady-state stage: alternate the
// matrix-core instructions with the stage's global->LDS loads, then with the
// next stage's fragment reads, so the memory instructions issue while the
// matrix core is busy instead of in a block in front of it.
template <int NMFMA, int NDMA, int NREAD>
__device__ __forceinline__ void interleave() {
  constexpr int NMEM = NDMA + NREAD;
  constexpr int PER = (NMEM + NMFMA - 1) / NMFMA;  // memory instructions per MFMA slot
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // 1 MFMA
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int t = i * PER + j;
      if (t < NDMA) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // global->LDS
      else if (t < NMEM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
  }
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
template <int BN, int BM>
__device__ __forceinline__ void gemm_mainloop(f32x16 (&acc)[BN / 64][BM / 64], char *lds,
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
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};

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

  Frags<BN, BM> f0, f1;
  read_frags<BN, BM>(f0, lds, 0, wn, wm, lane);
  // Steady state (no branches inside, so the compiler's wait-count tracking
  // sees straight-line code): stage kb computes while kb+1..kb+3 are in
  // flight; at mid-stage, once every wavefront has its last fragments of
  // `cur`, the barrier frees `cur` for stage kb+4.
  int kb = 0;
  for (; kb + kStages < nkb; ++kb) {
    char *cur = lds + (kb & (kStages - 1)) * C::STAGE;
    char *nxt = lds + ((kb + 1) & (kStages - 1)) * C::STAGE;
    read_frags<BN, BM>(f1, cur, 1, wn, wm, lane);
    mfma_step<BN, BM>(acc, f0);
    interleave<C::FN * C::FM, 0, C::FN + C::FM>();
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    wait_vmcnt<2 * C::LPS>();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
    pw.issue(cur, (kb + kStages) * BK, wv);
    px.issue(cur + C::W_BYTES, (kb + kStages) * BK, wv);
    read_frags<BN, BM>(f0, nxt, 0, wn, wm, lane);
    mfma_step<BN, BM>(acc, f1);
    interleave<C::FN * C::FM, C::LPS, C::FN + C::FM>();
    __builtin_amdgcn_sched_barrier(0);
  }
  // Drain: no more stages to issue.
  for (; kb + 1 < nkb; ++kb) {
    char *cur = lds + (kb & (kStages - 1)) * C::STAGE;
    char *nxt = lds + ((kb + 1) & (kStages - 1)) * C::STAGE;
    read_frags<BN, BM>(f1, cur, 1, wn, wm, lane);
    mfma_step<BN, BM>(acc, f0);
    wait_lgkmcnt0();
    wait_stages_after<C::LPS>(nkb - 2 - kb);
    barrier_no_fence();
    read_frags<BN, BM>(f0, nxt, 0, wn, wm, lane);
    mfma_step<BN, BM>(acc, f1);
  }
  {
    const char *cur = lds + (kb & (kStages - 1)) * C::STAGE;
    read_frags<BN, BM>(f1, cur, 1, wn, wm, lane);
    mfma_step<BN, BM>(acc, f0);
    mfma_step<BN, BM>(acc, f1);
  }

}

// Epilogue through LDS, so that every global store writes whole 128-byte
// lines (per-lane 8-byte stores straight from the accumulators would issue
// eight partial-line requests per line and, with every tile finishing at the
// same moment, stall on the L2 request rate).
//
// Accumulator block (i, j) of a wavefront, register v, holds
// n = 32i + 8(v/4) + 4(lane/32) + v%4 and m = 32j + lane%32 of the
// wavefront's WN x WM sub-tile.  Each wavefront writes its sub-tile, rounded
// to bf16, to its own LDS region as rows of m (WN bf16 = CH 16-byte chunks,
// chunk c of row m stored at c ^ f(m)), then reads it back 16 bytes per lane,
// eight lanes per 128-byte row segment, and stores those segments.  f spreads
// the 32 rows of one accumulator write over the banks and gives two adjacent
// rows disjoint chunk sets for the reads.  The caller has made the LDS free.
template <int BN, int BM>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[BN / 64][BM / 64], char *lds,
                                           uint16_t *y, int M, int N, int64_t ldy, int m0, int n0,
                                           int wn, int wm, int wv, int lane) {
  constexpr int WN = BN / 2, WM = BM / 2;
  constexpr int CH = WN / 8;          // 16-byte chunks per LDS row
  constexpr int ROWB = WN * 2;        // bytes per LDS row
  constexpr int HB = CH / 2;
  static_assert(CH == 8 || CH == 16, "sub-tile width");
  char *mine = lds + wv * (WM * ROWB);
  auto f = [](int m) { return ((m & 1) * HB) | ((m >> 1) & (HB - 1)); };
#pragma unroll
  for (int j = 0; j < BM / 64; ++j) {
    const int m = j * 32 + (lane & 31);
    char *row = mine + m * ROWB + (lane >> 5) * 8;
    const int fm = f(m);
#pragma unroll
    for (int i = 0; i < BN / 64; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 o;
        o.x = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
        o.y = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
        *reinterpret_cast<uint2 *>(row + (((i * 4 + q) ^ fm) << 4)) = o;
      }
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
    const int m = m0 + wm * WM + r, n = n0 + wn * WN + c * 8;
    if (m < M && n < N) *reinterpret_cast<u32x4 *>(y + (int64_t)m * ldy + n) = v;
  }
}

// ---------------------------------------------------------------------------
// Wide-stage variant: BK = 64, so an LDS row is a whole 128-byte line of one
// matrix row and each direct-to-LDS load instruction moves 8 full lines (one
// 128-byte L2 request per line instead of two 64-byte ones).  Two stages fit
// the LDS at 256 x 256; stage kb + 2 is issued once every wavefront has read
// its last fragments of stage kb.  The k order is unchanged: 16-k matrix-core
// steps, ascending, so the bits equal the BK = 32 kernel's.
constexpr int BK2 = 64;
constexpr int kRow2 = BK2 * 2;  // 128 bytes: eight 16-byte chunks

// Chunk c of LDS row r is stored at c ^ swz2(r).  A fragment read touches 32
// consecutive rows at one logical chunk; rows r and r + 1 share a 256-byte
// window, so 16 consecutive rows cover the 16 bank groups exactly once.
__device__ __forceinline__ int swz2(int row) { return (row >> 1) & 7; }

template <int BN, int BM>
struct Cfg2 {
  static constexpr int WN = BN / 2, WM = BM / 2;
  static constexpr int FN = WN / 32, FM = WM / 32;
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

__device__ __forceinline__ bf16x8 read_frag2(const char *lds, int row, int ks, int lane) {
  const int lc = ks * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8 *>(lds + row * kRow2 + ((lc ^ swz2(row)) << 4));
}

// Issued in the order the products consume them: a[0] with every b[j] comes
// first, then a[1], a[2], ... -- the first product waits for two reads only.
template <int BN, int BM>
__device__ __forceinline__ void read_frags2(Frags<BN, BM> &f, const char *wl, const char *xl,
                                            int ks, int wn, int wm, int lane) {
  using C = Cfg2<BN, BM>;
  f.a[0] = read_frag2(wl, wn * C::WN + (lane & 31), ks, lane);
#pragma unroll
  for (int j = 0; j < C::FM; ++j) f.b[j] = read_frag2(xl, wm * C::WM + j * 32 + (lane & 31), ks, lane);
#pragma unroll
  for (int i = 1; i < C::FN; ++i) f.a[i] = read_frag2(wl, wn * C::WN + i * 32 + (lane & 31), ks, lane);
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

// Steps 0..2 of a stage (fragments of steps 1..3 are read while the previous
// step multiplies), with the loads of a later stage of the operand that has
// the ring of 3 spread over steps 0 and 1 when LOAD.  Leaves step 3's
// fragments in f1.
template <int BN, int BM, int ER, bool LOAD>
__device__ __forceinline__ void stage_head2(f32x16 (&acc)[BN / 64][BM / 64], Frags<BN, BM> &f0,
                                            Frags<BN, BM> &f1, const char *wc, const char *xc,
                                            const LoadPlan2<ER> &pe, char *edst, int k0, int wn,
                                            int wm, int wv, int lane) {
  using C = Cfg2<BN, BM>;
  constexpr int LE = ER / 32, H = LE / 2;
  read_frags2<BN, BM>(f1, wc, xc, 1, wn, wm, lane);
  if (LOAD) pe.issue(edst, k0, wv, 0, H);
  mfma_step<BN, BM>(acc, f0);
  interleave_even<C::FN * C::FM, LOAD ? H : 0, C::FN + C::FM>();
  __builtin_amdgcn_sched_barrier(0);
  read_frags2<BN, BM>(f0, wc, xc, 2, wn, wm, lane);
  if (LOAD) pe.issue(edst, k0, wv, H, LE);
  mfma_step<BN, BM>(acc, f1);
  interleave_even<C::FN * C::FM, LOAD ? LE - H : 0, C::FN + C::FM>();
  __builtin_amdgcn_sched_barrier(0);
  read_frags2<BN, BM>(f1, wc, xc, 3, wn, wm, lane);
  mfma_step<BN, BM>(acc, f0);
  interleave_even<C::FN * C::FM, 0, C::FN + C::FM>();
  __builtin_amdgcn_sched_barrier(0);
}

// LDS bytes of the 64-k scheme: one operand in a ring of 3 stages, the other
// in a ring of 2 (W3: the weights have the ring of 3).
template <int BN, int BM, bool W3>
constexpr int wide_lds_bytes() {
  return W3 ? 3 * BN * kRow2 + 2 * BM * kRow2 : 2 * BN * kRow2 + 3 * BM * kRow2;
}

// One operand in a ring of 3 stages, the other in a ring of 2.  In stage kb
// the ring-of-3 operand's stage kb + 2 loads during the first steps (its slot
// held stage kb - 1); the ring-of-2 operand's stage kb + 2 loads after the
// end-of-stage barrier, once every wavefront has read stage kb.  Activations
// take the ring of 3 in the full-size kernels (W3 = false); the small-M
// split-K partials give it to the weights, whose read dominates there.
template <int BN, int BM, bool W3>
__device__ __forceinline__ void gemm_mainloop2(f32x16 (&acc)[BN / 64][BM / 64], char *lds,
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
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};

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

// One BN x BM output tile with 64-k stages, at rows m0.., columns n0...
template <int BN, int BM>
__device__ __forceinline__ void wide_tile(char *lds, const uint16_t *__restrict__ x,
                                          const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
                                          int M, int N, int K, int64_t ldx, int64_t ldw,
                                          int64_t ldy, int m0, int n0) {
  using C = Cfg2<BN, BM>;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wv >> 1, wm = wv & 1;
  f32x16 acc[C::FN][C::FM];
  gemm_mainloop2<BN, BM, false>(acc, lds, x, w, M, N, K / BK2, ldx, ldw, m0, n0, wv, lane, K);
  barrier_no_fence();  // every wavefront is done reading the stages
  store_tile<BN, BM>(acc, lds, y, M, N, ldy, m0, n0, wn, wm, wv, lane);
}

template <int BN, int BM>
__global__ __launch_bounds__(kThreads, 1) void gemm_wide_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[wide_lds_bytes<BN, BM, false>()];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  wide_tile<BN, BM>(lds, x, w, y, M, N, K, ldx, ldw, ldy, tm * BM, tn * BN);
}

// 256 x 256 tiles whose last, partly filled wave is split in two along M: the
// first nfull launch indices take whole tiles (logical tiles 0 .. nfull-1),
// the rest take 256 x 128 halves of the remaining logical tiles, two launch
// indices per tile.  Both shapes run the same matrix-core steps in the same
// order, so no output's bits depend on which kind of workgroup computed it.
__global__ __launch_bounds__(kThreads, 1) void gemm_mixed_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n,
    int nfull) {
  __shared__ __attribute__((aligned(1024))) char lds[wide_lds_bytes<256, 256, false>()];
  const int pid = blockIdx.x;
  int tm, tn;
  if (pid < nfull) {
    group_tile(xcd_lid(pid, nfull), tiles_m, tiles_n, tm, tn);
    wide_tile<256, 256>(lds, x, w, y, M, N, K, ldx, ldw, ldy, tm * 256, tn * 256);
  } else {
    const int q = pid - nfull;
    group_tile(nfull + (q >> 1), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * 256 + (q & 1) * 128;
    if (m0 >= M) return;  // the empty lower half of the last tile row
    wide_tile<256, 128>(lds, x, w, y, M, N, K, ldx, ldw, ldy, m0, tn * 256);
  }
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

  f32x16 acc[C::FN][C::FM];
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

  f32x16 acc[C::FN][C::FM];
  if constexpr (WIDE)
    gemm_mainloop2<BN, BM, true>(acc, lds, x + (int64_t)s * kc, w + (int64_t)s * kc, M, N,
                                 kc / BK2, ldx, ldw, m0, n0, wv, lane, kc);
  else
    gemm_mainloop<BN, BM>(acc, lds, x + (int64_t)s * kc, w + (int64_t)s * kc, M, N, kc / BK, ldx,
                          ldw, m0, n0, wv, lane, kc);

  float *part = ws + (int64_t)s * M * N;
#pragma unroll
  for (int j = 0; j < C::FM; ++j) {
    const int m = m0 + wm * C::WM + j * 32 + (lane & 31);
    if (m >= M) continue;
    float *prow = part + (int64_t)m * N;
#pragma unroll
    for (int i = 0; i < C::FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * C::WN + i * 32 + q * 8 + (lane >> 5) * 4;
        if (n < N) {
          f32x4 o = {acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                     acc[i][j][q * 4 + 3]};
          *reinterpret_cast<f32x4 *>(prow + n) = o;
        }
      }
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

typedef void (*GemmKernel)(const uint16_t *, const uint16_t *, uint16_t *, int, int, int, int64_t,
                           int64_t, int64_t, int, int);
struct CfgEntry {
  int bn, bm;
  GemmKernel kernel;  // BK = 32 stages, any K % 32 == 0
  GemmKernel wide;    // BK = 64 stages, used when K % 64 == 0 (same k order, same bits)
};

const CfgEntry kConfigs[] = {
    {256, 256, gemm_kernel<256, 256>, gemm_wide_kernel<256, 256>},
    {256, 128, gemm_kernel<256, 128>, gemm_wide_kernel<256, 128>},
    {128, 128, gemm_kernel<128, 128>, gemm_wide_kernel<128, 128>},
    {128, 256, gemm_kernel<128, 256>, gemm_wide_kernel<128, 256>},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

// Split-K path: one tile shape for every (N, K) and M, sized for decode-like
// batches (one 64-row tile covers M <= 64).
constexpr int kSplitBN = 128, kSplitBM = 64;

int splitk_for(int64_t N, int64_t K) {
  const int64_t tiles_n = (N + kSplitBN - 1) / kSplitBN;
  int S = 1;
  // smallest power of two that gives >= 256 workgroups at M <= 64, keeping
  // at least 4 stages of K per chunk
  while (tiles_n * S < 256 && K % (2 * S * BK) == 0 && K / (2 * S) >= 4 * BK && S < 64) S *= 2;
  return S;
}

int config_for(int64_t N, int64_t K) {
  (void)K;
  return N >= 4096 ? 0 : 2;
}

// Tile for bi_gemm_fill: the configuration with the smallest estimated time,
// (waves of tiles over the CUs) x (relative time of one tile).  The tile
// costs are measured ones, relative to 256 x 256: a 256 x 128 or 128 x 256
// tile takes ~0.6 of it, a 128 x 128 tile ~0.34.  Ties keep the larger tile.
// kMixed: 256 x 256 tiles with the last wave split into 256 x 128 halves
// (gemm_mixed_kernel); only for 64-k stages.
constexpr int kMixed = kNumConfigs;
int fill_config_for(int64_t M, int64_t N, int64_t K) {
  static const double kTileCost[kNumConfigs] = {1.0, 0.6, 0.34, 0.58};
  const int64_t cus = cu_count();
  int best = 0;
  double best_t = 0.0;
  for (int c = 0; c < kNumConfigs; ++c) {
    const int64_t tiles = ((M + kConfigs[c].bm - 1) / kConfigs[c].bm) *
                          ((N + kConfigs[c].bn - 1) / kConfigs[c].bn);
    const double t = (double)((tiles + cus - 1) / cus) * kTileCost[c];
    if (c == 0 || t < best_t - 1e-9) {
      best = c;
      best_t = t;
    }
  }
  // The mixed launch, when the 256 x 256 tiles leave a last wave at most half
  // full after one or two whole waves: whole waves of tiles, then one wave of
  // halves.  After three or more whole waves it measured within a few percent
  // of the plain launch either way (a partly filled last wave runs at a
  // higher clock under the power limit), so it is not used there.
  const int64_t T = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t r = T % cus;
  if (K % BK2 == 0 && T > cus && T < 3 * cus && r > 0 && 2 * r <= cus) {
    const double t = (double)(T / cus) + kTileCost[1];
    if (t < best_t - 1e-9) best = kMixed;
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

int launch(int cfg, const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M, int64_t N,
           int64_t K, int64_t ldx, int64_t ldw, int64_t ldy, void *stream) {
  const CfgEntry &c = kConfigs[cfg];
  const int64_t tiles_m = (M + c.bm - 1) / c.bm, tiles_n = (N + c.bn - 1) / c.bn;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return BI_ERR_SHAPE;
  const GemmKernel kern = (c.wide && K % BK2 == 0) ? c.wide : c.kernel;
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0,
                     (hipStream_t)stream, x, w, y, (int)M, (int)N, (int)K, ldx, ldw, ldy,
                     (int)tiles_m, (int)tiles_n);
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
  const int cfg = fill_config_for(M, N, K);
  if (cfg != kMixed) return launch(cfg, x, w, y, M, N, K, ldx, ldw, ldy, stream);
  const int64_t tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256, T = tiles_m * tiles_n;
  const int64_t nfull = T - T % cu_count();
  const int64_t grid = nfull + 2 * (T - nfull);
  if (grid > 0x7FFFFFFF) return BI_ERR_SHAPE;
  hipLaunchKernelGGL(gemm_mixed_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, x, w, y, (int)M, (int)N, (int)K, ldx, ldw, ldy,
                     (int)tiles_m, (int)tiles_n, (int)nfull);
  return launch_status();
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

extern "C" int bi_gemm_splitk(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t M,
                              int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                              int split_k, void *ws, size_t ws_bytes, void *stream) {
  int st = validate(x, w, y, M, N, K, ldx, ldw, ldy);
  if (st != BI_OK) return st;
  if (split_k < 1 || split_k > 64) return BI_ERR_UNSUPPORTED;
  if (K % ((int64_t)split_k * BK)) return BI_ERR_SHAPE;
  if (M == 0) return BI_OK;
  if (!ws) return BI_ERR_NULL;
  if (ws_bytes < bi_gemm_splitk_workspace_bytes(M, N, split_k)) return BI_ERR_WORKSPACE;
  if (!aligned16(ws)) return BI_ERR_ALIGN;
  const Span sw{(uintptr_t)ws, (uintptr_t)ws + (uintptr_t)(split_k * M * N * 4)};
  if (overlap(sw, span_of(y, M, N, ldy, 2)) || overlap(sw, span_of(x, M, K, ldx, 2)) ||
      overlap(sw, span_of(w, N, K, ldw, 2)))
    return BI_ERR_ALIAS;
  const int64_t tiles_m = (M + kSplitBM - 1) / kSplitBM, tiles_n = (N + kSplitBN - 1) / kSplitBN;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return BI_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  float *wsf = static_cast<float *>(ws);
  const int kc = (int)(K / split_k);
  if (kc % BK2 == 0)
    hipLaunchKernelGGL((gemm_partial_kernel<kSplitBN, kSplitBM, true>),
                       dim3((unsigned)(tiles_m * tiles_n), (unsigned)split_k), dim3(kThreads), 0, s,
                       x, w, wsf, (int)M, (int)N, kc, ldx, ldw, (int)tiles_m, (int)tiles_n);
  else
    hipLaunchKernelGGL((gemm_partial_kernel<kSplitBN, kSplitBM, false>),
                       dim3((unsigned)(tiles_m * tiles_n), (unsigned)split_k), dim3(kThreads), 0, s,
                       x, w, wsf, (int)M, (int)N, kc, ldx, ldw, (int)tiles_m, (int)tiles_n);
  if ((st = launch_status()) != BI_OK) return st;
  const int64_t groups = (M * N / 4 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(gemm_splitk_combine_kernel, dim3((unsigned)groups), dim3(kThreads), 0, s, wsf,
                     y, (int)M, (int)N, split_k, ldy);
  return launch_status();
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
