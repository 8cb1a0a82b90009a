/*
 * bi.h -- C ABI of libbi.so: batch-invariant reduction kernels for MI355X (gfx950).
 *
 * What "batch-invariant" means here.  Serving systems batch requests
 * dynamically, so one request meets different batch partners from run to run;
 * a kernel whose reduction order follows the batch shape then changes an
 * unchanged request's numbers ("God Does Not Play Dice: Enforcing Batch
 * Invariance in Agentic Kernel Generation", abstract; "Cómo superar la no
 * determinación en la inferencia de LLM", section "La verdadera causa clave").
 * Every entry point below except bi_lora_shrink_atomic fixes the floating-point
 * reduction order of each output row from (N, K, R, split_k, eps) and the build
 * alone.  An output row is therefore a pure function of its own input row and
 * the weights: it is bitwise the same whatever the batch size M, the row's
 * position in the batch, the other rows, the stream or the run.
 *
 * Conventions shared by every entry point
 *   - bf16 values cross the ABI as raw 16-bit patterns (uint16_t); fp32 as float.
 *   - All tensors are row-major with an explicit row stride (ld*, in elements).
 *     Weights are stored K-contiguous: the GEMM weight W as [N, K] (one output
 *     column per row) and the LoRA down-projection A as [R, K].
 *   - Pointers to tensors are DEVICE pointers (hipMalloc / torch), owned by the
 *     caller.  The library never allocates, frees or synchronises.  Its only
 *     mutable global state belongs to bi_gemm_splitk_noalloc (a static device
 *     scratch array per GPU and a lock-guarded cache of its address); every
 *     other call is thread-safe without restriction.
 *   - stream is a hipStream_t passed as void*; NULL means the default stream.
 *     Every call is asynchronous on that stream.
 *   - Return value: a bi_status.  Arguments are validated before anything is
 *     launched; on any error nothing is launched and no output is touched.
 *     M == 0 is valid and launches nothing; the [M, *] tensors (x, y and the
 *     workspace) may then be NULL, as an empty tensor's data pointer can be.  After a launch, a HIP launch error
 *     is reported as BI_ERR_HIP.  No exception crosses the ABI; nothing aborts.
 *   - Alignment: every tensor base pointer must be 16-byte aligned; bf16 row
 *     strides (and the contiguous dimension where stated) are multiples of 8
 *     elements, fp32 row strides multiples of 4.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BI_ABI_VERSION 1

typedef enum bi_status {
    BI_OK = 0,
    BI_ERR_NULL = 1,        /* a required pointer is NULL                         */
    BI_ERR_SHAPE = 2,       /* a size or stride is out of range or not supported  */
    BI_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned, or ld/K % 8 != 0 */
    BI_ERR_WORKSPACE = 4,   /* split-K workspace missing or too small             */
    BI_ERR_ALIAS = 5,       /* an output overlaps an input or another output      */
    BI_ERR_HIP = 6,         /* the HIP runtime reported an error at launch        */
    BI_ERR_UNSUPPORTED = 7  /* valid request the library does not implement      */
} bi_status;

/* BI_ABI_VERSION of the loaded library. */
int bi_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *bi_status_str(int status);

/*
 * bi_rmsnorm -- y[i][k] = bf16( x[i][k] * r_i * w[k] ),
 *               r_i = 1 / sqrt( (sum_k x[i][k]^2) / K + eps ), all in fp32.
 *
 * Defined by: "Cómo superar la no determinación en la inferencia de LLM",
 * section "RMSNorm": data-parallel over the batch, each row reduced by one
 * core, with a strategy that never changes with the batch size.  (The page's
 * split reduction for tiny batches gives up invariance and is not offered.)
 *
 *   x   [M, K] bf16, row stride ldx      (input)
 *   w   [K]    bf16                      (weight)
 *   y   [M, K] bf16, row stride ldy      (output; may equal x when ldx == ldy)
 *   M >= 0 rows; 8 <= K <= 16384, K % 8 == 0; eps >= 0.
 * Reduction order of row i: one workgroup of 4 wavefronts; thread t owns the
 * 8-element chunks t, t+256, t+512, ... and sums their squares in ascending
 * element order; each wavefront combines its 64 lanes by a fixed xor
 * butterfly (offsets 32, 16, 8, 4, 2, 1); the 4 wavefront sums are added as
 * ((s0 + s1) + s2) + s3.  The tree depends on K only.  Output rounding is
 * round-to-nearest-even.
 */
int bi_rmsnorm(const uint16_t *x, const uint16_t *w, uint16_t *y,
               int64_t M, int64_t K, int64_t ldx, int64_t ldy, float eps,
               void *stream);

/*
 * bi_gemm -- y[i][j] = bf16( sum_k x[i][k] * w[j][k] ), fp32 accumulation.
 *
 * Defined by: "Cómo superar la no determinación en la inferencia de LLM",
 * section "Multiplicación de matrices (matmul)": 2-D output tiles processed
 * data-parallel, one kernel configuration forced for every batch size, and no
 * split of the K reduction.
 *
 *   x   [M, K] bf16, row stride ldx (activations)
 *   w   [N, K] bf16, row stride ldw (weight, K-contiguous)
 *   y   [M, N] bf16, row stride ldy (output; must not overlap x or w)
 *   M >= 0; N >= 8, N % 8 == 0; K >= 32, K % 32 == 0; x and w each span
 *   fewer than 2^31 elements ((rows - 1) * ld + K).
 * Reduction order of every output: one ascending pass over K in steps of 32
 * (one bf16 16x16x32 matrix-core instruction per step, fp32 accumulator
 * rounded between steps); no split-K, no stream-K.  The tile configuration is
 * bi_gemm_config_id(N, K): it never reads M.  Output rounding is
 * round-to-nearest-even.
 */
int bi_gemm(const uint16_t *x, const uint16_t *w, uint16_t *y,
            int64_t M, int64_t N, int64_t K,
            int64_t ldx, int64_t ldw, int64_t ldy, void *stream);

/*
 * bi_gemm_config_id -- the tile configuration bi_gemm uses for (N, K), or -1
 * if (N, K) is not supported.  It takes no M on purpose: the configuration,
 * and with it every output's reduction order, cannot depend on the batch size.
 *
 * Defined by: "Cómo superar la no determinación en la inferencia de LLM",
 * section "Multiplicación de matrices (matmul)": one kernel configuration
 * forced for every batch size.
 */
int bi_gemm_config_id(int64_t N, int64_t K);

/*
 * bi_gemm_launch_plan -- what bi_gemm(M, N, K) would launch, without launching
 * anything: a static check that the batch size reaches nothing but the number
 * of workgroups.
 *
 * Defined by: "God Does Not Play Dice: Enforcing Batch Invariance in Agentic
 * Kernel Generation", abstract (a static, contract-guided check of what a
 * kernel's reduction depends on, beside the dynamic bitwise one), and "Cómo
 * superar la no determinación en la inferencia de LLM", section
 * "Multiplicación de matrices (matmul)" (one configuration for every batch
 * size).
 *
 *   plan   host int64_t[7], written on BI_OK:
 *          [0] configuration (= bi_gemm_config_id(N, K)),
 *          [1] kernel id (which compiled kernel runs),
 *          [2] tile rows (of M), [3] tile columns (of N),
 *          [4] k per LDS stage (32 or 64; the 32-k matrix-core steps are the
 *              same either way), [5] threads per workgroup,
 *          [6] workgroups = ceil(M / tile rows) * ceil(N / tile columns)
 *              (0 when M == 0).
 *   Entries [0]..[5] depend on (N, K) only.  bi_gemm builds its launch from
 *   the same host function.
 * Returns BI_ERR_NULL for a NULL plan, BI_ERR_SHAPE when M < 0 or (N, K) is
 * not supported (see bi_gemm_config_id); touches no device.
 */
int bi_gemm_launch_plan(int64_t M, int64_t N, int64_t K, int64_t *plan);

/*
 * bi_gemm_num_configs / bi_gemm_with_config -- tuning and verification hooks.
 * bi_gemm_with_config runs bi_gemm with tile configuration `config`
 * (0 <= config < bi_gemm_num_configs()) instead of bi_gemm_config_id(N, K).
 * Every configuration runs the same reduction order, so all of them return the
 * same bits; this entry point exists to demonstrate exactly that and to time
 * the alternatives.  Configurations 0-4 are single tiles (256 x 256,
 * 256 x 128, 128 x 128, 128 x 256, 128 x 64 outputs of w rows x x rows per
 * workgroup);
 * the last one is a mixed launch of 256 x 256 tiles whose last wave on each
 * XCD, when it is at most half full, runs as 256 x 128 halves (with K % 64 ==
 * 32 it runs as configuration 0).  Same arguments and errors as bi_gemm, plus
 * BI_ERR_UNSUPPORTED for an unknown config.
 */
int bi_gemm_num_configs(void);
int bi_gemm_with_config(int config, const uint16_t *x, const uint16_t *w, uint16_t *y,
                        int64_t M, int64_t N, int64_t K,
                        int64_t ldx, int64_t ldw, int64_t ldy, void *stream);

/*
 * bi_gemm_fill -- bi_gemm with the tile configuration picked per call from
 * (M, N, K) to fill the chip, and the same bits as bi_gemm for every input.
 *
 * Defined by: "Cómo superar la no determinación en la inferencia de LLM",
 * section "Multiplicación de matrices (matmul)": the page forces one kernel
 * configuration because, in the kernels it describes, a different
 * configuration reduces in a different order.  Here every configuration runs
 * the same matrix-core instruction over the same ascending k steps (see
 * bi_gemm_with_config), so the configuration can follow M without any output
 * bit following it: row i is still bitwise identical alone or in any batch.
 * The configuration is the one with the smallest estimated time: waves of
 * tiles over the compute units times a measured per-tile cost (for the mixed
 * launch, each XCD's full waves plus one wave of half tiles).  bi_gemm keeps
 * the single (N, K)-keyed configuration.
 *
 * Arguments, layout, ownership and errors as bi_gemm.
 */
int bi_gemm_fill(const uint16_t *x, const uint16_t *w, uint16_t *y,
                 int64_t M, int64_t N, int64_t K,
                 int64_t ldx, int64_t ldw, int64_t ldy, void *stream);

/* bi_gemm_fill_config_id -- the configuration bi_gemm_fill uses for (M, N, K)
 * on the current device, or -1 if the shape is not supported (M >= 1). */
int bi_gemm_fill_config_id(int64_t M, int64_t N, int64_t K);

/*
 * bi_gemm_splitk -- the same product with the K reduction split into split_k
 * equal contiguous chunks, for batches too small to fill the chip with tiles.
 *
 * Defined by: "Cómo superar la no determinación en la inferencia de LLM",
 * section "Multiplicación de matrices (matmul)": small batches need split-K
 * for parallelism, and that breaks batch invariance when the split follows
 * the batch size; keeping the split fixed keeps one reduction order.  The
 * split here is the caller's fixed choice per layer (bi_gemm_splitk_for(N, K)
 * gives one from (N, K) alone) and must not be chosen from M.
 *
 *   Same x, w, y, sizes and strides as bi_gemm; 1 <= split_k <= 64 and
 *   K % (32 * split_k) == 0.
 *   ws, ws_bytes: device fp32 workspace of at least
 *       bi_gemm_splitk_workspace_bytes(M, N, split_k) bytes; on return it holds
 *       the partial sums p_s[m][n] at ws[(s * M + m) * N + n].
 * Reduction order of every output: chunk s covers k in [s*K/S, (s+1)*K/S),
 * one ascending pass in 32-k steps (the bi_gemm main loop over that range);
 * then bf16( (((p_0 + p_1) + p_2) + ...) + p_{S-1} ) in fp32, rounded to nearest
 * even once.  split_k == 1 gives bi_gemm's bits.
 * Launches: M <= 16 with K / split_k a multiple of 128 runs one kernel (each
 * workgroup owns 16 columns, or 8 for narrow outputs, and every chunk, and
 * folds in LDS); other sizes
 * run the partial kernel and then the fold.  Both write the same partials to
 * ws and return the same bits, so a row's result does not depend on which
 * one its batch took.
 */
int bi_gemm_splitk(const uint16_t *x, const uint16_t *w, uint16_t *y,
                   int64_t M, int64_t N, int64_t K,
                   int64_t ldx, int64_t ldw, int64_t ldy, int split_k,
                   void *ws, size_t ws_bytes, void *stream);

/* bi_gemm_splitk_workspace_bytes -- split_k * M * N * 4, rounded up to 256. */
size_t bi_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int split_k);

/* Size of the static scratch array behind bi_gemm_splitk_noalloc: 16 MiB per
 * GPU, enough for M <= 64 at every Llama-3-8B and -70B projection with its
 * bi_gemm_splitk_for split. */
#define BI_GEMM_SPLITK_SCRATCH_BYTES (16u << 20)

/*
 * bi_gemm_splitk_noalloc -- bi_gemm_splitk for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * device allocation): the same kernels, the same bits, but the fp32 partials
 * go to a static device array of BI_GEMM_SPLITK_SCRATCH_BYTES bytes inside the
 * library instead of a caller's workspace.  The caller still passes x, w and
 * y; the call allocates and frees nothing.
 *
 *   Arguments, layout and errors as bi_gemm_splitk without ws / ws_bytes.
 *   BI_ERR_WORKSPACE when bi_gemm_splitk_workspace_bytes(M, N, split_k) >
 *   BI_GEMM_SPLITK_SCRATCH_BYTES (nothing is launched).
 *   The scratch belongs to the GPU of `stream` (the current device for NULL);
 *   its address is looked up once per GPU, on the first call there.  Every
 *   call on one GPU shares that GPU's array and nothing in it needs to start
 *   at zero (each call writes every partial it folds), but calls that overlap
 *   in time on one GPU -- concurrent streams, or host threads -- race on it
 *   and must be serialised by the caller.  Unlike bi_gemm_splitk, the
 *   partials are not returned.
 */
int bi_gemm_splitk_noalloc(const uint16_t *x, const uint16_t *w, uint16_t *y,
                           int64_t M, int64_t N, int64_t K,
                           int64_t ldx, int64_t ldw, int64_t ldy, int split_k, void *stream);

/* bi_gemm_splitk_for -- a split factor for (N, K) that fills the chip at M <= 64
 * (a power of two, at least 8 32-k steps per chunk), or -1 if (N, K) is not
 * supported.  No M parameter, for the same reason as bi_gemm_config_id. */
int bi_gemm_splitk_for(int64_t N, int64_t K);

/*
 * bi_gemm_mswitch_control -- CONTROL ONLY, NOT batch-invariant.  Picks the
 * reduction from the batch size, the way a library tuned per shape does:
 * bi_gemm_splitk(split_k = bi_gemm_splitk_for(N, K)) when 1 <= M <= 64, bi_gemm
 * otherwise.  A row therefore gets different bits alone than inside a large
 * batch.  This is the configuration switch of "Cómo superar la no
 * determinación en la inferencia de LLM" (section "Multiplicación de matrices
 * (matmul)") and the shape-driven source of drift named in the forum thread
 * "You think you are measuring intelligence..." (second comment), kept to show
 * that variation beside the atomic control.  ws as for bi_gemm_splitk (needed
 * when M <= 64).
 */
int bi_gemm_mswitch_control(const uint16_t *x, const uint16_t *w, uint16_t *y,
                            int64_t M, int64_t N, int64_t K,
                            int64_t ldx, int64_t ldw, int64_t ldy,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * bi_lora_shrink_workspace_bytes -- bytes of workspace bi_lora_shrink needs:
 * split_k * M * R * 4 (fp32 partials), rounded up to 256; 0 when split_k == 1.
 */
size_t bi_lora_shrink_workspace_bytes(int64_t M, int64_t R, int split_k);

/*
 * bi_lora_shrink -- LoRA shrink y[m][r] = sum_k x[m][k] * a[r][k], fp32 output,
 * with a deterministic split-K.
 *
 * Defined by: "Reproducible LoRA Inference Through Deterministic Split-K
 * Reduction", abstract: split-K adds parallelism to the low-rank shrink, and
 * combining the partials in a fixed order instead of with floating-point
 * atomics removes the run-to-run variation.
 *
 *   x   [M, K] bf16, row stride ldx     (activations)
 *   a   [R, K] bf16, row stride lda     (LoRA down-projection, K-contiguous)
 *   y   [M, R] fp32, row stride ldy     (output; ldy >= R, ldy % 4 == 0)
 *   R == 16; split_k in {1, 2, 4, 8, 16}; K % (32 * split_k) == 0.
 *   ws, ws_bytes: optional.  One kernel computes the split_k partials of each
 *       16-row block in split_k wavefronts of one workgroup and combines them
 *       through LDS.  If ws is not NULL (and split_k > 1) it must hold
 *       bi_lora_shrink_workspace_bytes(M, R, split_k) bytes and receives the
 *       partials p_s[m][r] at ws[(s * M + m) * R + r] (fp32) as well.
 * Reduction order: chunk s covers k in [s*K/S, (s+1)*K/S); inside a chunk one
 * ascending pass in steps of 32 (one bf16 16x16x32 matrix-core instruction per
 * step); then y = (((p_0 + p_1) + p_2) + ...) + p_{S-1} in fp32.
 * split_k == 1 is the unsplit reduction (one pass over all of K).
 */
int bi_lora_shrink(const uint16_t *x, const uint16_t *a, float *y,
                   int64_t M, int64_t K, int64_t R,
                   int64_t ldx, int64_t lda, int64_t ldy, int split_k,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * bi_lora_shrink_two_pass -- the same result, bit for bit, with the split
 * spread over workgroups: the partials go through the caller's fp32 workspace
 * in HBM (ws, required when split_k > 1, layout as above) and a second kernel
 * combines them in the same fixed order.  Kept to measure that design against
 * the single-kernel one.  Same arguments and errors as bi_lora_shrink.
 */
int bi_lora_shrink_two_pass(const uint16_t *x, const uint16_t *a, float *y,
                            int64_t M, int64_t K, int64_t R,
                            int64_t ldx, int64_t lda, int64_t ldy, int split_k,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * bi_lora_shrink_atomic -- CONTROL ONLY, NOT deterministic.  The same partial
 * sums as bi_lora_shrink, but y is first zeroed (by a fill kernel on the same
 * stream) and each partial is then added into y with a floating-point atomic
 * add, in whatever order the wavefronts arrive.  This is the nondeterministic
 * combine that "Reproducible LoRA Inference Through Deterministic Split-K
 * Reduction" (abstract) measures against; it exists to show that variation.
 * Same arguments as bi_lora_shrink, without a workspace.
 */
int bi_lora_shrink_atomic(const uint16_t *x, const uint16_t *a, float *y,
                          int64_t M, int64_t K, int64_t R,
                          int64_t ldx, int64_t lda, int64_t ldy, int split_k,
                          void *stream);

/*
 * bi_decode_attention -- batch-invariant decode attention with a fixed split
 * size: o[b][h] = sum_t softmax_t(q[b][h] . k[b][t][h/G] / sqrt(D)) v[b][t][h/G].
 *
 * Defined by: "Cómo superar la no determinación en la inferencia de LLM",
 * section "Attention": parallel over queries, each query's keys/values reduced
 * in one order; a split-KV reduction fixes the split *size*, not the number of
 * splits; cache and new tokens share one key/value layout.
 *
 *   q        [B, H, D] bf16, contiguous (one decode query per sequence)
 *   k_cache, v_cache  [B, Tmax, Hkv, D] bf16, contiguous; the new token's key
 *            and value are already written at position lens[b] - 1.
 *   lens     [B] int32 on the device: tokens of sequence b, in [1, Tmax]
 *            (values outside are clamped into that range).
 *   o        [B, H, D] bf16 output.
 *   D in {64, 128}; H % Hkv == 0 and H / Hkv <= 8 (grouped-query heads);
 *   split_size (tokens per chunk) in {128, 256, 512}: a constant of the
 *   deployment, never derived from the batch.  split_size * Hkv * D * 2 must
 *   stay below 2^31 (BI_ERR_UNSUPPORTED otherwise).
 *   ws, ws_bytes: fp32 workspace of bi_decode_attention_workspace_bytes(B, H,
 *   Tmax, D, split_size) bytes (per-chunk max, sum and weighted values).
 * Order of every output: per chunk of split_size tokens, each score a
 * matrix-core dot product over d blocks of 32 in ascending order; max, exp and a sum in a
 * fixed lane/xor order; the weights rounded to bf16 and the weighted values
 * summed by matrix-core products over 32-token blocks in ascending order;
 * chunks folded with c ascending (see attention.hip).  The result for sequence b depends on its own
 * q, cache and length only.
 */
int bi_decode_attention(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                        const int32_t *lens, uint16_t *o,
                        int64_t B, int64_t H, int64_t Hkv, int64_t D, int64_t Tmax,
                        int split_size, void *ws, size_t ws_bytes, void *stream);

/* bi_decode_attention_workspace_bytes -- B * H * ceil(Tmax / split_size) *
 * (D + 2) * 4, rounded up to 256. */
size_t bi_decode_attention_workspace_bytes(int64_t B, int64_t H, int64_t Tmax, int64_t D,
                                           int split_size);

/*
 * bi_lora_shrink_expand -- the LoRA pair in one launch:
 *   l = shrink(x, a) as bi_lora_shrink with split_k (fixed-order fold), then
 *   y = bf16( base + scale * l . b^T ) as bi_lora_expand.
 *
 * Defined by: "Reproducible LoRA Inference Through Deterministic Split-K
 * Reduction", abstract: the two low-rank LoRA multiplications, the shrink with
 * a deterministic split-K whose fp32 output feeds the expand.
 *
 *   x [M, K], a [R, K], b [N, R], base [M, N] (or NULL), y [M, N]: as for
 *   bi_lora_shrink and bi_lora_expand (same strides, alignment and aliasing
 *   rules; base may equal y when ldbase == ldy).
 *   l     optional fp32 [M, R] output (row stride ldl, 16-byte aligned,
 *         ldl % 4 == 0) receiving the shrink result; NULL to skip it.
 *   split_k in {1, 2, 4, 8} (BI_ERR_UNSUPPORTED otherwise); K % (32 *
 *   split_k) == 0.
 * Order: exactly that of bi_lora_shrink followed by bi_lora_expand, so y (and
 * l) equal the two-call result bit for bit; l never leaves the chip.
 */
int bi_lora_shrink_expand(const uint16_t *x, const uint16_t *a, const uint16_t *b,
                          const uint16_t *base, uint16_t *y, float *l,
                          int64_t M, int64_t K, int64_t N, int64_t R,
                          int64_t ldx, int64_t lda, int64_t ldb, int64_t ldbase, int64_t ldy,
                          int64_t ldl, float scale, int split_k, void *stream);

/*
 * bi_lora_expand -- LoRA expand: y[m][n] = bf16( base[m][n] + scale * sum_r l[m][r] * b[n][r] ).
 *
 * Defined by: "Reproducible LoRA Inference Through Deterministic Split-K
 * Reduction", abstract: the low-rank LoRA multiplications; the fp32 shrink
 * output feeds this one.
 *
 *   l     [M, R] fp32, row stride ldl (the shrink output)
 *   b     [N, R] bf16, row stride ldb (LoRA up-projection, R-contiguous)
 *   base  [M, N] bf16, row stride ldbase, or NULL (then 0); may equal y when
 *         ldbase == ldy (in-place add)
 *   y     [M, N] bf16, row stride ldy
 *   R == 16; N >= 8, N % 8 == 0, N <= 2^23; ldy, ldbase, ldb % 8 == 0;
 *   y, base and b 16-byte aligned, l 4-byte aligned (else BI_ERR_ALIGN).
 * Order of every output: acc = fma(l[m][r], b[n][r], acc) in fp32 for r
 * ascending from acc = 0, then base + scale * acc in fp32, rounded to nearest
 * even once.
 */
int bi_lora_expand(const float *l, const uint16_t *b, const uint16_t *base, uint16_t *y,
                   int64_t M, int64_t N, int64_t R,
                   int64_t ldl, int64_t ldb, int64_t ldbase, int64_t ldy, float scale,
                   void *stream);

/*
 * bi_row_bitdiff -- bitwise comparison of rows, the invariance check.
 *
 * Defined by: "God Does Not Play Dice: Enforcing Batch Invariance in Agentic
 * Kernel Generation", abstract: dynamic validation that outputs are bitwise
 * consistent across batch contexts.
 *
 * For r in [0, nrows): compares row a_rows[r] of a with row b_rows[r] of b,
 * ncols elements of elem_bytes (2 or 4) each, as raw bits, and writes
 *   counts[2r]   = number of differing bits (popcount of the XORs)
 *   counts[2r+1] = number of differing elements.
 *   a, b      device pointers, row strides lda, ldb (elements)
 *   a_rows, b_rows  device int64 row indices, or NULL for 0..nrows-1.  The
 *                   indices are trusted: each must address a row inside its
 *                   buffer.
 *   counts    device uint64 [nrows][2], fully overwritten.
 * Integer counts: exact and independent of thread order.
 */
int bi_row_bitdiff(const void *a, int64_t lda, const int64_t *a_rows,
                   const void *b, int64_t ldb, const int64_t *b_rows,
                   int64_t nrows, int64_t ncols, int elem_bytes,
                   uint64_t *counts, void *stream);

/*
 * bi_row_bitdiff_batch -- up to BI_BITDIFF_BATCH_MAX comparisons of
 * bi_row_bitdiff in one launch (a step's outputs checked together).
 *
 * Defined by: the same passage as bi_row_bitdiff ("God Does Not Play Dice:
 * Enforcing Batch Invariance in Agentic Kernel Generation", abstract).
 *
 *   items   HOST array of nitems descriptors (read during the call only); each
 *           has bi_row_bitdiff's arguments and meaning, its counts written as
 *           there.  1 <= nitems <= BI_BITDIFF_BATCH_MAX (else
 *           BI_ERR_UNSUPPORTED).
 * Every row must start 16-byte aligned and hold a whole number of 16-byte
 * vectors (a, b 16-byte aligned; lda, ldb and ncols times elem_bytes
 * multiples of 16), else BI_ERR_ALIGN.  Any invalid item rejects the whole
 * call before anything is launched.  Same counts as one bi_row_bitdiff call
 * per item.
 */
#define BI_BITDIFF_BATCH_MAX 16
typedef struct bi_bitdiff_item {
    const void *a;
    int64_t lda;
    const int64_t *a_rows;
    const void *b;
    int64_t ldb;
    const int64_t *b_rows;
    int64_t nrows;
    int64_t ncols;
    int64_t elem_bytes;
    uint64_t *counts;
} bi_bitdiff_item;

int bi_row_bitdiff_batch(const bi_bitdiff_item *items, int nitems, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
