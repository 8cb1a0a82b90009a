/*
 * oracle.c -- the plain, slow CPU oracle for the batch-invariant reduction path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is not part of the product.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark may load
 * it.  It shares no code, header, table or helper with the HIP kernels, and it
 * includes nothing from the package.
 *
 * Everything here is the mathematical definition written out with plain loops:
 *
 *   GEMM and LoRA shrink  y[i][j] = sum_k x[i][k] * w[j][k]
 *       The pages state this op only as the matrix multiplication that a
 *       batch-invariant kernel must reproduce ("Defeating Nondeterminism in LLM
 *       Inference", Spanish summary, section "Multiplicación de matrices
 *       (matmul)"; "Reproducible LoRA Inference Through Deterministic Split-K
 *       Reduction", abstract: the low-rank shrink with an FP32 output).  The sum
 *       is taken in fp64 in ascending k.  Every bf16 x bf16 product has at most
 *       16 significant bits, so it is exact in fp64; the only error is the fp64
 *       summation, at most (K-1) * 2^-53 * sum_k |x*w|.
 *
 *   RMSNorm  y[i][k] = x[i][k] * w[k] / sqrt(mean_k x[i][k]^2 + eps)
 *       Same summary, section "RMSNorm", gives only the per-row parallel
 *       strategy; the formula is the standard one (mean over K, eps inside the
 *       root, no centring, no bias).  Computed in fp64, unrounded.
 *
 *   Fixed-order combine  out = (((p0 + p1) + p2) + ...) + p_{S-1}
 *       The LoRA abstract says only that the deterministic split-K combines its
 *       partials in a fixed order instead of with floating-point atomics.  The
 *       order used by the product is the left fold over s = 0..S-1 in fp32;
 *       this is that definition, in fp32, because its point is the exact bits.
 *
 *   Decode attention  o[b][h] = sum_t softmax_t(q.k_t / sqrt(D)) v_t
 *       Same summary, section "Attention": one query token per sequence
 *       attends to every cached key/value of its own sequence (the new token
 *       already appended to the cache, one layout for both).  Query head h
 *       reads key/value head h / (H / Hkv).  Scores, softmax and the weighted
 *       sum in fp64, unrounded; exp from libm.
 *
 *   LoRA expand  y[m][n] = base[m][n] + scale * sum_r l[m][r] * b[n][r]
 *       The other low-rank multiplication of a LoRA layer ("Reproducible LoRA
 *       Inference Through Deterministic Split-K Reduction", abstract, speaks of
 *       low-rank LoRA multiplications; the shrink output l feeds it).  fp64,
 *       unrounded; base may be absent (then 0).
 *
 *   Bit differences  popcount(a XOR b), and the count of differing elements.
 *       The check that "God Does Not Play Dice: Enforcing Batch Invariance in
 *       Agentic Kernel Generation" (abstract) asks for: bitwise consistency of
 *       outputs across batch contexts.
 *
 *   bf16 decode and round-to-nearest-even, from the format's definition
 *       (1 sign bit, 8 exponent bits with bias 127, 7 fraction bits).
 *
 * Threads: the row loops may run under OpenMP.  Rows are independent and every
 * row's arithmetic is the same in any thread, so the thread count never changes
 * a result.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- bf16 ---- */

/* Exact value of one bf16 bit pattern, from the format's fields. */
static double bf16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 7) & 0xFF;
    int frac = h & 0x7F;
    double mag;
    if (expo == 0xFF) {
        mag = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        mag = ldexp((double)frac, -126 - 7);          /* subnormal: 0.f * 2^-126 */
    } else {
        mag = ldexp((double)(128 + frac), expo - 127 - 7); /* 1.f * 2^(e-127) */
    }
    return sign ? -mag : mag;
}

void oracle_bf16_decode(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_value(in[i]);
}

/* Round one double to the nearest bf16, ties to even, directly from its value. */
static uint16_t bf16_round(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    /* Largest finite bf16 is (2 - 2^-7) * 2^127; values at or above the midpoint
     * between it and 2^128 round to infinity. */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127))
        return sign | 0x7F80;
    if (a < ldexp(1.0, -126)) {
        /* Subnormal range: the quantum is 2^-133.  rint() rounds half to even
         * under the default rounding mode. */
        double q = rint(ldexp(a, 133));
        /* q == 128 means it rounded up to the smallest normal 2^-126, whose
         * encoding is exponent 1, fraction 0 -- the same bits as 128. */
        return sign | (uint16_t)q;
    }
    int e;
    (void)frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1) */
    int ub = e - 1;                   /* unbiased exponent: a in [2^ub, 2^(ub+1)) */
    double q = rint(ldexp(a, 7 - ub)); /* significand in units of 2^(ub-7): [128, 256] */
    if (q == 256.0) {                 /* rounded up into the next binade */
        q = 128.0;
        ub += 1;
        if (ub > 127)
            return sign | 0x7F80;
    }
    uint16_t biased = (uint16_t)(ub + 127);
    return sign | (uint16_t)(biased << 7) | (uint16_t)((int)q - 128);
}

void oracle_bf16_round(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_round(in[i]);
}

/* ---------------------------------------------------------------- GEMM ---- */

/* y[i*ldy + j] = sum_{k ascending} x[i*ldx + k] * w[j*ldw + k], in fp64.
 * x is [M, K] with row stride ldx; w is [N, K] with row stride ldw (the weight is
 * stored K-contiguous, one output column per row). */
void oracle_gemm(const uint16_t *x, int64_t ldx, const uint16_t *w, int64_t ldw,
                 double *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                 int threads)
{
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += bf16_value(x[i * ldx + k]) * bf16_value(w[j * ldw + k]);
            y[i * ldy + j] = acc;
        }
    }
    (void)threads;
}

/* ------------------------------------------------------------- RMSNorm ---- */

/* y[i][k] = x[i][k] * w[k] / sqrt(sum_k x[i][k]^2 / K + eps), in fp64. */
void oracle_rmsnorm(const uint16_t *x, int64_t ldx, const uint16_t *w,
                    double *y, int64_t ldy, int64_t M, int64_t K, double eps,
                    int threads)
{
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(threads)
#endif
    for (int64_t i = 0; i < M; ++i) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = bf16_value(x[i * ldx + k]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            y[i * ldy + k] = bf16_value(x[i * ldx + k]) * r * bf16_value(w[k]);
    }
    (void)threads;
}

/* ------------------------------------------------- fixed-order combine ---- */

/* out[e] = (((p[0][e] + p[1][e]) + p[2][e]) + ...) + p[S-1][e], each add in fp32.
 * p is [S][n] contiguous. */
void oracle_combine_f32(const float *p, int64_t S, int64_t n, float *out)
{
    for (int64_t e = 0; e < n; ++e) {
        volatile float acc = p[e];     /* volatile: one fp32 rounding per add */
        for (int64_t s = 1; s < S; ++s)
            acc = acc + p[s * n + e];
        out[e] = acc;
    }
}

/* ---------------------------------------------------- decode attention ---- */

/* q [B][H][D], k and v [B][Tmax][Hkv][D] (bf16), lens[b] valid tokens of
 * sequence b; o [B][H][D] in fp64. */
void oracle_decode_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const int32_t *lens, double *o, int64_t B, int64_t H,
                             int64_t Hkv, int64_t D, int64_t Tmax, int threads)
{
    const int64_t G = H / Hkv;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads) collapse(2)
#endif
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t kh = h / G;
            const int64_t T = lens[b];
            const double scale = 1.0 / sqrt((double)D);
            double mx = -INFINITY;
            for (int64_t t = 0; t < T; ++t) {
                double s = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    s += bf16_value(q[(b * H + h) * D + d]) *
                         bf16_value(k[((b * Tmax + t) * Hkv + kh) * D + d]);
                s *= scale;
                if (s > mx)
                    mx = s;
            }
            double l = 0.0;
            for (int64_t d = 0; d < D; ++d)
                o[(b * H + h) * D + d] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                double s = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    s += bf16_value(q[(b * H + h) * D + d]) *
                         bf16_value(k[((b * Tmax + t) * Hkv + kh) * D + d]);
                const double p = exp(s * scale - mx);
                l += p;
                for (int64_t d = 0; d < D; ++d)
                    o[(b * H + h) * D + d] += p * bf16_value(v[((b * Tmax + t) * Hkv + kh) * D + d]);
            }
            for (int64_t d = 0; d < D; ++d)
                o[(b * H + h) * D + d] /= l;
        }
    }
    (void)threads;
}

/* --------------------------------------------------------- LoRA expand ---- */

/* l [M][R] fp32, b [N][R] bf16, base [M][N] bf16 or NULL; y [M][N] fp64. */
void oracle_lora_expand(const float *l, const uint16_t *b, const uint16_t *base, double *y,
                        int64_t M, int64_t N, int64_t R, double scale)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t r = 0; r < R; ++r)
                acc += (double)l[m * R + r] * bf16_value(b[n * R + r]);
            y[m * N + n] = (base ? bf16_value(base[m * N + n]) : 0.0) + scale * acc;
        }
    }
}

/* ------------------------------------------------------- bit differences ---- */

static int popcount_u32(uint32_t v)
{
    int c = 0;
    while (v) {
        c += (int)(v & 1u);
        v >>= 1;
    }
    return c;
}

/* out[0] = number of differing bits, out[1] = number of differing elements,
 * between a and b, n elements of elem_bytes (2 or 4) each. */
void oracle_bitdiff(const void *a, const void *b, int64_t n, int elem_bytes,
                    uint64_t *out)
{
    uint64_t bits = 0, elems = 0;
    for (int64_t i = 0; i < n; ++i) {
        uint32_t va = 0, vb = 0;
        memcpy(&va, (const char *)a + i * elem_bytes, (size_t)elem_bytes);
        memcpy(&vb, (const char *)b + i * elem_bytes, (size_t)elem_bytes);
        int c = popcount_u32(va ^ vb);
        bits += (uint64_t)c;
        elems += c ? 1u : 0u;
    }
    out[0] = bits;
    out[1] = elems;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
