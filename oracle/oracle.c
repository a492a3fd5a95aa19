/*
 * oracle.c -- CPU oracle for the fused dual RMSNorm + per-1x128 FP8 group
 * quantisation of an MLA decode step, and for the block-scaled FP8 GEMM that
 * consumes its (q_fp8, scale) pair.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never links, imports or calls it,
 * and this file shares no code, header, table or constant generator with it.
 *
 * Plain, slow and meant to be checked by eye: every value is carried in fp64
 * unless a step of the method fixes another precision (the stored scale is an
 * fp32 number, the outputs are bf16 / e4m3fn codes).  No blocking, fusion or
 * reordering beyond the definitions below.  The row loops and the GEMM column
 * loop carry an OpenMP pragma; it changes nothing in the arithmetic of a row
 * or of an output element.
 *
 * Sources (web pages; cited by title and section):
 *  [PR53540]  GitHub page "[ROCm][Perf] Fuse SWA q/kv RMSNorm and q FP8 group
 *             quant for DeepSeek-V4 #53540" (vllm-project/vllm), section
 *             "Purpose".
 *  [D53540]   PRHub digest of vLLM PR #53540, sections "功能与动机"
 *             (motivation), "实现拆解" (implementation breakdown) and the
 *             source excerpt of _fused_mla_dual_rms_norm_group_quant_impl.
 *  [D56433]   PRHub report of vLLM PR #56433 "Fix AITER preshuffled FP8
 *             block-scale kernel", "实现拆解" items 2 and 4.
 *  [D27289]   PRHub digest of SGLang PR #27289 (fp8 scale transpose copy),
 *             "功能与动机", "实现拆解" item 2 (fused_rms_fp8_group_quant with
 *             transpose_scale) and the aiter_w8a8_block_fp8_linear excerpt
 *             (its branch B: aiter_per1x128_quant of a bf16 input).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes of the repository):
 *  - FP8 is OCP e4m3fn: bias 7, largest finite 448 (0x7E), 0x7F/0xFF NaN,
 *    no infinities, subnormals down to 2^-9.
 *  - RMSNorm: y = x * gamma / sqrt(mean(x^2) + eps), gamma a plain multiplier.
 *  - The group scale is the dequantisation multiplier s = amax/448, stored as
 *    an fp32 number, floored at 1e-12f; codes = RNE_e4m3(clamp(y/s, +-448)).
 *  - kv_out = bf16 round-to-nearest-even of the exact normalised value.
 *  - Column-major ("transposed") scales: the [M, G] logical array stored as
 *    its transpose, element (m, g) at offset g*M + m, leading dimension M.
 *  - GEMM: out[m,n] = sum_kb As[m,kb]*Bs[n/128,kb]*sum_{k in kb} a*w, with
 *    As in the layout the caller states and Bs row-major [N/128, K/128].
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 128
#define ORACLE_E4M3_MAX 448.0
#define ORACLE_SCALE_FLOOR 1e-12f

/* ---------------------------------------------------------------------------
 * bf16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits.
 * ------------------------------------------------------------------------- */

/* Exact value of a bf16 bit pattern: the top half of the fp32 with the same
 * sign, exponent and mantissa bits. */
double oracle_bf16_decode(uint16_t bits)
{
    int sign = bits >> 15;
    int e = (bits >> 7) & 0xFF;
    int f = bits & 0x7F;
    double v;
    if (e == 0xFF)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -133);            /* subnormal: f * 2^-126 * 2^-7 */
    else
        v = ldexp((double)(128 + f), e - 134); /* (1 + f/128) * 2^(e-127) */
    return sign ? -v : v;
}

/* Round an fp64 value straight to the nearest bf16 (ties to even mantissa),
 * with a single rounding (never via fp32).  Overflow gives +-inf. */
uint16_t oracle_bf16_encode(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int e2;
    frexp(a, &e2);                  /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                 /* a in [2^E, 2^(E+1)) */
    /* spacing of bf16 values around a: 2^(E-7) for normals, 2^-133 below 2^-126 */
    int qexp = (E < -126) ? -133 : E - 7;
    double r = nearbyint(ldexp(a, -qexp)); /* RNE under the default mode */
    /* normals: bits = ((E+127) << 7) + (r - 128); r == 256 carries into the
     * exponent.  subnormals: bits = r; r == 128 is the smallest normal. */
    long bits = (E < -126) ? (long)r : ((long)(E + 127) << 7) + ((long)r - 128);
    if (bits >= 0x7F80)
        return sign | 0x7F80;
    return (uint16_t)(sign | bits);
}

/* ---------------------------------------------------------------------------
 * e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, exponent
 * field 15 with mantissa 7 is NaN, everything else finite (max 448).
 * ------------------------------------------------------------------------- */

double oracle_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int f = code & 0x7;
    double v;
    if (e == 0xF && f == 0x7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);              /* f/8 * 2^-6 */
    else
        v = ldexp((double)(8 + f), e - 10);    /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* Nearest e4m3fn code, ties to even mantissa, saturating at +-448 (0x7E /
 * 0xFE).  NaN input gives 0x7F.  -0.0 gives 0x80. */
uint8_t oracle_e4m3_encode(double v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= ORACLE_E4M3_MAX)
        return sign | 0x7E;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;                             /* a in [2^E, 2^(E+1)) */
    int qexp = (E < -6) ? -9 : E - 3;           /* spacing of codes around a */
    double r = nearbyint(ldexp(a, -qexp));
    int bits = (E < -6) ? (int)r : ((E + 7) << 3) + ((int)r - 8);
    /* a < 448 keeps bits <= 0x7E (ties at 464 cannot occur below 448) */
    return (uint8_t)(sign | bits);
}

/* fp32 round-to-nearest of an fp64 value (the C conversion rounds to nearest
 * even in the default mode). */
static float to_f32(double v) { return (float)v; }

/* ---------------------------------------------------------------------------
 * Fused dual RMSNorm + per-1x128 FP8 group quantisation.
 *
 * [PR53540] "Purpose": one kernel RMSNorms both latents with fp32
 * accumulation and quantises the q latent per 1x128 with fp32 scales; the
 * quantisation reads the fp32 normalised values directly (one rounding), kv
 * stays bf16.  [D53540] impl excerpt: outputs are q_out [M, Nq] fp8, q_scale
 * [M, Nq/group] fp32, kv_normed with kv's shape, all freshly allocated
 * (contiguous); q and kv may be strided split views with unit inner stride.
 * [D56433] item 4 / [D27289]: transpose_scale selects the column-major scale
 * layout, the bytes of x_scale.transpose(-1,-2).contiguous().
 *
 * Oracle arithmetic: everything in fp64 from the exactly decoded bf16 inputs,
 * i.e. the exact mathematical value up to fp64 rounding (far below the fp32
 * accumulation the pages describe).
 *
 * sequential != 0 gives the pre-fusion semantics instead ([PR53540]
 * "Purpose", the three-launch pipeline): the normalised q is first rounded to
 * bf16, then group-quantised.
 *
 * out_ratio (nullable): y/s before clamping and rounding, fp64, [M, Nq]; the
 * value whose rounding decides each code.
 * out_y (nullable): the normalised q value y (after the optional bf16 step).
 * ------------------------------------------------------------------------- */
void oracle_dual_rmsnorm_group_quant(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale, int sequential,
    uint8_t *out_q, float *out_scale, uint16_t *out_kv,
    double *out_ratio, double *out_y)
{
    const int64_t G = Nq / ORACLE_GROUP;

#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xq = q + m * q_row_stride;
        const uint16_t *xk = kv + m * kv_row_stride;

        /* mean of squares and reciprocal RMS, per latent */
        double ssq_q = 0.0, ssq_k = 0.0;
        for (int64_t i = 0; i < Nq; ++i) {
            double x = oracle_bf16_decode(xq[i]);
            ssq_q += x * x;
        }
        for (int64_t i = 0; i < Nkv; ++i) {
            double x = oracle_bf16_decode(xk[i]);
            ssq_k += x * x;
        }
        double rstd_q = 1.0 / sqrt(ssq_q / (double)Nq + (double)eps);
        double rstd_k = 1.0 / sqrt(ssq_k / (double)Nkv + (double)eps);

        /* kv: normalise, scale by gamma, round once to bf16 */
        for (int64_t i = 0; i < Nkv; ++i) {
            double y = oracle_bf16_decode(xk[i]) * rstd_k * oracle_bf16_decode(gamma_kv[i]);
            out_kv[m * Nkv + i] = oracle_bf16_encode(y);
        }

        /* q: per group of 128 consecutive columns */
        for (int64_t g = 0; g < G; ++g) {
            double y[ORACLE_GROUP];
            double amax = 0.0;
            for (int j = 0; j < ORACLE_GROUP; ++j) {
                int64_t i = g * ORACLE_GROUP + j;
                y[j] = oracle_bf16_decode(xq[i]) * rstd_q * oracle_bf16_decode(gamma_q[i]);
                if (sequential)
                    y[j] = oracle_bf16_decode(oracle_bf16_encode(y[j]));
                if (fabs(y[j]) > amax)
                    amax = fabs(y[j]);
            }
            /* dequantisation multiplier, stored in fp32, floored */
            float s = to_f32(amax / ORACLE_E4M3_MAX);
            if (s < ORACLE_SCALE_FLOOR)
                s = ORACLE_SCALE_FLOOR;

            int64_t scale_at = transpose_scale ? g * M + m : m * G + g;
            out_scale[scale_at] = s;

            for (int j = 0; j < ORACLE_GROUP; ++j) {
                int64_t i = g * ORACLE_GROUP + j;
                double ratio = y[j] / (double)s;
                if (out_ratio)
                    out_ratio[m * Nq + i] = ratio;
                if (out_y)
                    out_y[m * Nq + i] = y[j];
                double c = ratio;
                if (c > ORACLE_E4M3_MAX)
                    c = ORACLE_E4M3_MAX;
                if (c < -ORACLE_E4M3_MAX)
                    c = -ORACLE_E4M3_MAX;
                out_q[m * Nq + i] = oracle_e4m3_encode(c);
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * One row of per-1x128 group quantisation of exact values y[0..N): for each
 * group g of 128 consecutive columns, s = max(fp32(max|y| / 448), 1e-12f)
 * and code = e4m3(clamp(y / s, +-448)); the scale goes to element (m, g) of
 * the [M, G] scale array in the requested layout.
 * ------------------------------------------------------------------------- */
static void quantise_row(const double *y, int64_t m, int64_t M, int64_t N, int transpose_scale,
                         uint8_t *out_q, float *out_scale, double *out_ratio)
{
    const int64_t G = N / ORACLE_GROUP;
    for (int64_t g = 0; g < G; ++g) {
        double amax = 0.0;
        for (int j = 0; j < ORACLE_GROUP; ++j)
            if (fabs(y[g * ORACLE_GROUP + j]) > amax)
                amax = fabs(y[g * ORACLE_GROUP + j]);
        float s = to_f32(amax / ORACLE_E4M3_MAX);
        if (s < ORACLE_SCALE_FLOOR)
            s = ORACLE_SCALE_FLOOR;
        out_scale[transpose_scale ? g * M + m : m * G + g] = s;
        for (int j = 0; j < ORACLE_GROUP; ++j) {
            int64_t i = g * ORACLE_GROUP + j;
            double ratio = y[i] / (double)s;
            if (out_ratio)
                out_ratio[m * N + i] = ratio;
            double c = ratio;
            if (c > ORACLE_E4M3_MAX)
                c = ORACLE_E4M3_MAX;
            if (c < -ORACLE_E4M3_MAX)
                c = -ORACLE_E4M3_MAX;
            out_q[m * N + i] = oracle_e4m3_encode(c);
        }
    }
}

/* Per-1x128 dynamic FP8 quantisation of a bf16 activation [M, N] with no
 * normalisation: [D27289] aiter_w8a8_block_fp8_linear excerpt, branch B
 * (aiter_per1x128_quant with transpose_scale); [PR53540] "Purpose", step 2
 * of the pipeline the fused kernel replaces.  y = x exactly. */
void oracle_group_quant(const uint16_t *x, int64_t row_stride, int64_t M, int64_t N,
                        int transpose_scale, uint8_t *out_q, float *out_scale, double *out_ratio)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *y = (double *)malloc(sizeof(double) * (size_t)N);
        for (int64_t i = 0; i < N; ++i)
            y[i] = oracle_bf16_decode(x[m * row_stride + i]);
        quantise_row(y, m, M, N, transpose_scale, out_q, out_scale, out_ratio);
        free(y);
    }
}

/* Single-input RMSNorm + per-1x128 FP8 group quantisation: [D27289]
 * "实现拆解" item 2 (fused_rms_fp8_group_quant with transpose_scale).
 * y = x * gamma / sqrt(mean(x^2) + eps), exact (fp64), quantised as above. */
void oracle_rmsnorm_group_quant(const uint16_t *x, int64_t row_stride, const uint16_t *gamma,
                                float eps, int64_t M, int64_t N, int transpose_scale,
                                uint8_t *out_q, float *out_scale, double *out_ratio)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * row_stride;
        double ssq = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            double v = oracle_bf16_decode(xr[i]);
            ssq += v * v;
        }
        double rstd = 1.0 / sqrt(ssq / (double)N + (double)eps);
        double *y = (double *)malloc(sizeof(double) * (size_t)N);
        for (int64_t i = 0; i < N; ++i)
            y[i] = oracle_bf16_decode(xr[i]) * rstd * oracle_bf16_decode(gamma[i]);
        quantise_row(y, m, M, N, transpose_scale, out_q, out_scale, out_ratio);
        free(y);
    }
}

/* ---------------------------------------------------------------------------
 * Block-scaled FP8 GEMM on the pre-quantised activation.
 *
 * [D53540] excerpt of apply_pre_quantized_block_scaled_mm: the linear's
 * block-scaled GEMM is called as (A = x_fp8, B = weight, As = x_scale,
 * Bs = weight_scale or weight_scale_inv), the weight scale used as given.
 * [D27289] excerpt of aiter_w8a8_block_fp8_linear: weight [N, K], output
 * [M, N] in bf16 for a pre-quantised input.  [D56433] item 2: a GEMM reads As
 * either row-major or column-major, and both have the same logical shape.
 *
 * out[m, n] = sum over K-blocks kb of  As[m, kb] * Bs[n/128, kb]
 *             * sum_{k in kb} dec(a[m, k]) * dec(w[n, k])
 * The inner block sums are exact in fp64 (e4m3 products carry <= 8
 * significant bits); the result is returned in fp64, unrounded.
 * ------------------------------------------------------------------------- */
void oracle_block_scaled_fp8_gemm(
    const uint8_t *a, const float *a_scale, int a_scale_transposed,
    const uint8_t *w, const float *w_scale,
    double *out, int64_t M, int64_t N, int64_t K)
{
    const int64_t KB = K / ORACLE_GROUP;

#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const int64_t nb = n / ORACLE_GROUP;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t kb = 0; kb < KB; ++kb) {
                double block = 0.0;
                for (int64_t k = kb * ORACLE_GROUP; k < (kb + 1) * ORACLE_GROUP; ++k)
                    block += oracle_e4m3_decode(a[m * K + k]) * oracle_e4m3_decode(w[n * K + k]);
                double as = a_scale_transposed ? a_scale[kb * M + m] : a_scale[m * KB + kb];
                double bs = w_scale[nb * KB + kb];
                acc += as * bs * block;
            }
            out[m * N + n] = acc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Power-of-two (e8m0) scales.
 *
 * [D56433] "风险与影响" item 3 (weight block scales stored as
 * float8_e8m0fnu) and the PRHub digest of vLLM PR #56560 (the native gfx950
 * MXFP8 GEMM, scales as e8m0 exponents, K in blocks of 128): an e8m0 scale
 * is a bare exponent byte E with value 2^(E - 127) (E = 255: NaN).  The pages
 * give no rule for picking a power-of-two scale for a group; the reading
 * taken: the smallest power of two not below the group's fp32-path scale
 * before rounding, s = 2^ceil(log2(max(amax / 448, 1e-12))), so that
 * |y| / s <= 448 (no clamping) and y / s is exact (a power-of-two scaling),
 * leaving the e4m3 rounding as the only rounding.
 * ------------------------------------------------------------------------- */
double oracle_e8m0_decode(uint8_t e)
{
    if (e == 0xFF)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* exponent e of the smallest power of two >= v (v > 0, finite) */
static int pow2_ceil_exponent(double v)
{
    int E;
    double f = frexp(v, &E); /* v = f * 2^E, f in [0.5, 1) */
    return f == 0.5 ? E - 1 : E;
}

/* Dual RMSNorm + per-1x128 group quantisation with e8m0 scales: the
 * normalised values y (and kv) exactly as oracle_dual_rmsnorm_group_quant
 * computes them (fused semantics), then per group e = ceil(log2(max(amax /
 * 448, 1e-12))), scale byte e + 127 in the requested layout, code =
 * e4m3(y * 2^-e).  out_ratio (nullable): y * 2^-e. */
void oracle_dual_rmsnorm_group_quant_e8m0(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q, uint8_t *out_scale, uint16_t *out_kv,
    double *out_ratio)
{
    const int64_t G = Nq / ORACLE_GROUP;
    double *y = (double *)malloc(sizeof(double) * (size_t)(M * Nq));
    uint8_t *tmp_q = (uint8_t *)malloc((size_t)(M * Nq));
    float *tmp_s = (float *)malloc(sizeof(float) * (size_t)(M * G));
    oracle_dual_rmsnorm_group_quant(q, q_row_stride, kv, kv_row_stride, gamma_q, gamma_kv, eps, M, Nq, Nkv,
                                    transpose_scale, 0, tmp_q, tmp_s, out_kv, NULL, y);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g) {
            const double *yg = y + m * Nq + g * ORACLE_GROUP;
            double amax = 0.0;
            for (int j = 0; j < ORACLE_GROUP; ++j)
                if (fabs(yg[j]) > amax)
                    amax = fabs(yg[j]);
            double t = amax / ORACLE_E4M3_MAX;
            if (t < (double)ORACLE_SCALE_FLOOR)
                t = (double)ORACLE_SCALE_FLOOR;
            int e = pow2_ceil_exponent(t);
            out_scale[transpose_scale ? g * M + m : m * G + g] = (uint8_t)(e + 127);
            for (int j = 0; j < ORACLE_GROUP; ++j) {
                int64_t i = m * Nq + g * ORACLE_GROUP + j;
                double ratio = ldexp(yg[j], -e);
                if (out_ratio)
                    out_ratio[i] = ratio;
                double c = ratio;
                if (c > ORACLE_E4M3_MAX)
                    c = ORACLE_E4M3_MAX;
                if (c < -ORACLE_E4M3_MAX)
                    c = -ORACLE_E4M3_MAX;
                out_q[i] = oracle_e4m3_encode(c);
            }
        }
    free(y);
    free(tmp_q);
    free(tmp_s);
}

/* ---------------------------------------------------------------------------
 * Load-time weight relayout (the tiled byte order of the library's GEMMs).
 *
 * [D56433] "实现拆解" items 1-3: a block-scale GEMM may ask for its weight to
 * be relaid out once at load time; the relayout is a permutation (not an
 * involution).  The pages do not define a layout for this hardware; the
 * contract checked here is the library's own, the order in which the
 * matrix-core instruction consumes a 16-row x 128-byte weight tile: the
 * [N, K] weight as N/16 x K/128 tiles of 2048 bytes, tile (s, kb) at
 * (s * K/128 + kb) * 2048, and inside a tile byte h*1024 + 16*L + b
 * (h < 2, lane L < 64, b < 16) holding w[16 s + L % 16][128 kb + 32 (L / 16)
 * + 16 h + b].  Written as plain loops over the destination, and its inverse
 * as loops over the source.
 * ------------------------------------------------------------------------- */
void oracle_tile_weight(const uint8_t *w, int64_t N, int64_t K, uint8_t *out)
{
    const int64_t KB = K / ORACLE_GROUP;
    for (int64_t s = 0; s < N / 16; ++s)
        for (int64_t kb = 0; kb < KB; ++kb)
            for (int h = 0; h < 2; ++h)
                for (int L = 0; L < 64; ++L)
                    for (int b = 0; b < 16; ++b) {
                        int64_t row = 16 * s + L % 16;
                        int64_t col = ORACLE_GROUP * kb + 32 * (L / 16) + 16 * h + b;
                        out[(s * KB + kb) * 2048 + h * 1024 + 16 * L + b] = w[row * K + col];
                    }
}

void oracle_untile_weight(const uint8_t *tiled, int64_t N, int64_t K, uint8_t *w)
{
    const int64_t KB = K / ORACLE_GROUP;
    for (int64_t row = 0; row < N; ++row)
        for (int64_t col = 0; col < K; ++col) {
            int64_t s = row / 16, rho = row % 16;
            int64_t kb = col / ORACLE_GROUP, c = col % ORACLE_GROUP;
            int64_t q = c / 32, h = (c % 32) / 16, b = c % 16;
            int64_t L = 16 * q + rho;
            w[row * K + col] = tiled[(s * KB + kb) * 2048 + h * 1024 + 16 * L + b];
        }
}

/* Number of threads the parallel loops above use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
