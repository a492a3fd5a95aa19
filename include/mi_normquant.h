/*
 * mi_normquant.h -- C ABI of the MI355X (gfx950) library for the MLA decode
 * hot path: fused dual RMSNorm + per-1x128 FP8 group quantisation of the q
 * and kv latents, and the block-scaled FP8 GEMM that consumes the quantised
 * q.
 *
 * Conventions shared by every entry point
 *  - Every array argument is a DEVICE pointer owned by the caller.  The
 *    library allocates nothing, keeps no state between calls, never
 *    synchronises, and enqueues its work on `stream` (0 = the null stream).
 *  - bf16 values are passed as uint16_t bit patterns, FP8 values as uint8_t
 *    OCP e4m3fn codes (bias 7, largest finite 448 = 0x7E, 0x7F/0xFF NaN, no
 *    infinities), scales as IEEE fp32.
 *  - All checks run on the host before anything is enqueued; a non-MI_OK
 *    status means nothing was enqueued (MI_ERR_HIP: the launch itself
 *    failed).  M == 0 is a valid no-op.
 *  - Inputs and outputs must not overlap (not checked).
 *  - Two calls that write the same outputs must be ordered by the caller
 *    (same stream or events); the kernels use no atomics, so repeated calls
 *    on the same inputs give bit-identical outputs.
 *
 * Sources (web pages; title and section):
 *  [PR53540] GitHub, vllm-project/vllm pull request #53540 "[ROCm][Perf]
 *            Fuse SWA q/kv RMSNorm and q FP8 group quant for DeepSeek-V4",
 *            section "Purpose".
 *  [D53540]  PRHub digest of the same PR: "实现拆解" (implementation
 *            breakdown) and the source excerpts of
 *            _fused_mla_dual_rms_norm_group_quant_impl and
 *            apply_pre_quantized_block_scaled_mm.
 *  [D56433]  PRHub report of vLLM PR #56433 "[ROCm][Bugfix] Fix AITER
 *            preshuffled FP8 block-scale kernel", "实现拆解" items 2 and 4.
 *  [D27289]  PRHub digest of SGLang PR #27289, "功能与动机" (motivation) and
 *            the aiter_w8a8_block_fp8_linear excerpt.
 */
#ifndef MI_NORMQUANT_H
#define MI_NORMQUANT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MI_OK = 0,
    MI_ERR_NULL = 1,    /* a required pointer is NULL */
    MI_ERR_SHAPE = 2,   /* a size is negative, not a multiple of 128 where one
                           is required, or above a documented limit */
    MI_ERR_STRIDE = 3,  /* a row stride is smaller than the row width */
    MI_ERR_ALIGN = 4,   /* a GEMM operand is not 16-byte aligned */
    MI_ERR_HIP = 5,     /* the HIP launch reported an error */
    MI_ERR_ALIAS = 6,   /* an output is the same buffer as an input */
    MI_ERR_LAYOUT = 7   /* unknown layout value */
} mi_status;

/* Quantisation group: one fp32 scale per 1 x 128 consecutive q elements. */
#define MI_GROUP 128
/* Largest supported widths of the fused norm-quant (one row per wavefront). */
#define MI_MAX_NQ 4096
#define MI_MAX_NKV 2048
/* Largest row width of the single-input quantisations below. */
#define MI_MAX_N_SINGLE 8192

/*
 * mi_fused_dual_rmsnorm_group_quant
 *
 * [PR53540] "Purpose" and [D53540] step 1: in one kernel launch, RMSNorm the
 * q latent and the kv latent of each row with fp32 accumulation, quantise
 * the normalised q per 1x128 group to FP8 with one fp32 scale per group
 * straight from the fp32 values (a single rounding), and write kv as bf16.
 * [D56433] item 4 and [D27289]: the scale layout is chosen by
 * `transpose_scale` so that a consumer reading column-major scales needs no
 * transpose copy.
 *
 * Per row m (x = q row, gamma = gamma_q; likewise for kv):
 *   rstd   = 1 / sqrt(sum_i x_i^2 / Nq + eps)            (fp32 accumulation)
 *   y_i    = x_i * rstd * gamma_i                         (fp32)
 *   s_g    = max(max_{i in g} |y_i| / 448, 1e-12)         (fp32)
 *   code_i = e4m3fn_rne(clamp(y_i / s_g, -448, 448))
 *   kv_out = bf16_rne(x * rstd_kv * gamma_kv)
 * s_g is the dequantisation multiplier: y_i ~= dec(code_i) * s_g.
 *
 * q, q_row_stride   [M, Nq] bf16, row m at q + m*q_row_stride (elements),
 *                   inner stride 1; q_row_stride >= Nq.  May be a column
 *                   slice of a wider fused projection buffer.
 * kv, kv_row_stride [M, Nkv] bf16, same rules; kv_row_stride >= Nkv.
 * gamma_q, gamma_kv [Nq], [Nkv] bf16 RMSNorm weights.
 * eps               added to the mean of squares (same value for q and kv).
 * M, Nq, Nkv        rows and widths: Nq % 128 == 0, 128 <= Nq <= MI_MAX_NQ,
 *                   1 <= Nkv <= MI_MAX_NKV, M >= 0.
 * transpose_scale   0: out_scale[m*G + g]; 1: out_scale[g*M + m], G = Nq/128
 *                   (the [M, G] array stored column-major, leading dim M).
 * out_q_fp8         [M, Nq] e4m3fn codes, contiguous.
 * out_scale         M*G fp32 values in the layout above.
 * out_kv            [M, Nkv] bf16, contiguous (whatever kv_row_stride is).
 * Rows, strides and base addresses need no particular alignment; 16-byte
 * aligned rows take the vector path.
 */
mi_status mi_fused_dual_rmsnorm_group_quant(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q_fp8, float *out_scale, uint16_t *out_kv,
    hipStream_t stream);

/*
 * mi_rmsnorm_group_quant
 *
 * [D27289] "实现拆解" item 2: the single-input form of the fused operation,
 * RMSNorm of one activation followed by the per-1x128 FP8 group quantisation
 * of the normalised values, with the scale layout chosen by
 * `transpose_scale`.  Per row m, with the formulas of
 * mi_fused_dual_rmsnorm_group_quant's q path:
 *   rstd   = 1 / sqrt(sum_i x_i^2 / N + eps)              (fp32 accumulation)
 *   y_i    = x_i * rstd * gamma_i
 *   s_g    = max(max_{i in g} |y_i| / 448, 1e-12)
 *   code_i = e4m3fn_rne(clamp(y_i / s_g, -448, 448))
 * The q outputs of mi_fused_dual_rmsnorm_group_quant for the same q rows are
 * bit-identical to this call's.
 *
 * x, x_row_stride  [M, N] bf16, row m at x + m*x_row_stride (elements),
 *                  x_row_stride >= N; no alignment required.
 * gamma            [N] bf16 RMSNorm weight.
 * eps              added to the mean of squares.
 * M, N             M >= 0; N % 128 == 0, 128 <= N <= MI_MAX_N_SINGLE.
 * transpose_scale  0: out_scale[m*G + g]; 1: out_scale[g*M + m], G = N/128.
 * out_fp8          [M, N] e4m3fn codes, contiguous.
 * out_scale        M*G fp32 values in the layout above.
 */
mi_status mi_rmsnorm_group_quant(
    const uint16_t *x, int64_t x_row_stride, const uint16_t *gamma,
    float eps, int64_t M, int64_t N, int transpose_scale,
    uint8_t *out_fp8, float *out_scale,
    hipStream_t stream);

/*
 * mi_group_quant_1x128
 *
 * [D27289] aiter_w8a8_block_fp8_linear excerpt, branch B: the dynamic
 * per-1x128 FP8 quantisation of a bf16 activation (aiter_per1x128_quant
 * with transpose_scale) that the block-scaled GEMM consumes; [PR53540]
 * "Purpose": the second step of the unfused pipeline (quantising the bf16
 * RMSNorm output).  No normalisation: per row m and group g,
 *   s_g    = max(fp32(max_{i in g} |x_i| / 448), 1e-12)
 *   code_i = e4m3fn_rne(clamp(x_i / s_g, -448, 448))
 * Both are correctly rounded: the scale is one IEEE division, and each code
 * is the single RNE rounding of the exact quotient (ties, which bf16 inputs
 * hit often, included), so results are reproducible bit for bit by any
 * exact implementation.
 *
 * x, x_row_stride, M, N, transpose_scale, out_fp8, out_scale: as in
 * mi_rmsnorm_group_quant.
 */
mi_status mi_group_quant_1x128(
    const uint16_t *x, int64_t x_row_stride,
    int64_t M, int64_t N, int transpose_scale,
    uint8_t *out_fp8, float *out_scale,
    hipStream_t stream);

/*
 * mi_block_scaled_fp8_gemm
 *
 * [D53540] excerpt of apply_pre_quantized_block_scaled_mm: the linear's
 * block-scaled GEMM is driven directly by the pre-quantised activation and
 * its per-1x128 scales (A = x_fp8, B = weight, As = x_scale, Bs = the weight
 * block scale, used as given), skipping a second quantisation of the input.
 * [D27289] aiter_w8a8_block_fp8_linear excerpt: weight [N, K], bf16 output
 * [M, N].  [D56433] item 2: a GEMM may read As column-major; row-major and
 * column-major As have the same logical shape, so the layout is an explicit
 * argument here, never inferred.
 *
 *   out[m, n] = bf16_rne( sum_{kb < K/128} As[m, kb] * Bs[n/128, kb]
 *                         * sum_{k in block kb} dec(a[m, k]) * dec(w[n, k]) )
 *   accumulated in fp32 on the matrix cores.
 *
 * a_fp8              [M, K] e4m3fn codes, contiguous, 16-byte aligned.
 * a_scale            M*K/128 fp32: a_scale_transposed == 0 -> As[m*(K/128)
 *                    + kb]; == 1 -> As[kb*M + m].
 * w_fp8              [N, K] e4m3fn codes, row-major, 16-byte aligned.
 * w_scale            [N/128, K/128] fp32, row-major.
 * out_bf16           [M, N] bf16, contiguous, 16-byte aligned.
 * M, N, K            M >= 0, N % 128 == 0, K % 128 == 0, N > 0, K > 0.
 */
mi_status mi_block_scaled_fp8_gemm(
    const uint8_t *a_fp8, const float *a_scale, int a_scale_transposed,
    const uint8_t *w_fp8, const float *w_scale,
    uint16_t *out_bf16,
    int64_t M, int64_t N, int64_t K,
    hipStream_t stream);

/*
 * mi_block_scaled_fp8_gemm_pair
 *
 * [PR53540] "Purpose": the attention wq_b and the indexer wq_b both consume
 * the same pre-quantised (q_fp8, scale) pair.  This computes both consumers
 * in one call: out1 = the block-scaled GEMM of the pair with (w1, w1_scale),
 * out2 = the same with (w2, w2_scale), each exactly as
 * mi_block_scaled_fp8_gemm defines it (bit-identical results).  One launch
 * streams both weights and stages the shared activations once per compute
 * unit, for decode batches (M <= 64, K / 128 in {4, 8, 12, 16}) and for
 * narrow pairs of up to 256 rows (N1 + N2 <= 64 x the compute units:
 * tensor-parallel shards; K / 128 = 12); other shapes are run as two launches
 * of mi_block_scaled_fp8_gemm on the same stream.
 *
 * a_fp8, a_scale, a_scale_transposed, M, K: as in mi_block_scaled_fp8_gemm.
 * w1_fp8, w1_scale, out1_bf16, N1: first consumer ([N1, K], [N1/128, K/128],
 *                    [M, N1]); w2_fp8, w2_scale, out2_bf16, N2: second.
 * N1 % 128 == 0, N2 % 128 == 0, N1 > 0, N2 > 0; the same alignment rules.
 * The two outputs must not overlap each other or any input.
 */
mi_status mi_block_scaled_fp8_gemm_pair(
    const uint8_t *a_fp8, const float *a_scale, int a_scale_transposed,
    const uint8_t *w1_fp8, const float *w1_scale, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const float *w2_scale, uint16_t *out2_bf16, int64_t N2,
    int64_t M, int64_t K,
    hipStream_t stream);

/*
 * Weight layouts and capabilities (load-time weight relayout).
 *
 * [D56433] "实现拆解" items 1-3: a block-scale GEMM kernel that wants its
 * weight relaid out at load time declares it with a capability flag, the
 * relayout is done once at load time, and code that reads a weight directly
 * keeps the plain layout; the relayout is a permutation, not an involution,
 * so applying it twice corrupts the weight ("功能与动机").  Here the layout
 * is an explicit argument of every GEMM call (as the As order is), the
 * relayout is out of place and invertible, and a caller learns from
 * mi_gemm_capabilities / mi_preferred_weight_layout whether to relayout.
 *
 * MI_WEIGHT_TILED: the [N, K] e4m3fn weight as N/16 x K/128 tiles of
 * 2048 bytes, tile (s, kb) at byte (s * (K/128) + kb) * 2048 (the tiles of
 * one 16-row subtile are contiguous); inside a tile, byte
 * h * 1024 + 16 * L + b (h < 2, L < 64, b < 16) holds
 * w[16 s + L % 16][128 kb + 32 (L / 16) + 16 h + b]: the tile in the order
 * the 16x16x128 matrix instruction takes it (lane L = 16 q + r holds row r,
 * bytes 32 q .. 32 q + 31), so each half of a wave's load of its fragments
 * is 1 KB of contiguous bytes, into registers or into LDS.  The block scales
 * (w_scale) are not relaid out.
 */
typedef enum {
    MI_WEIGHT_ROW_MAJOR = 0,
    MI_WEIGHT_TILED = 1
} mi_weight_layout;

#define MI_CAP_AS_ROW_MAJOR 1u   /* GEMMs read row-major activation scales */
#define MI_CAP_AS_COL_MAJOR 2u   /* ... and column-major ones */
#define MI_CAP_WEIGHT_TILED 4u   /* GEMMs read MI_WEIGHT_TILED weights */
#define MI_CAP_SCALE_E8M0 8u     /* e8m0 (power-of-two) scale entry points */

/* The capability flags of this library's GEMMs (a constant bit set). */
unsigned mi_gemm_capabilities(void);

/*
 * mi_preferred_weight_layout: the layout to store an [N, K] weight in at
 * load time for the GEMMs of this library (N % 128 == 0, K % 128 == 0), or
 * -1 for an invalid shape.  A weight that other code reads directly must
 * stay MI_WEIGHT_ROW_MAJOR whatever this returns; both layouts give
 * bit-identical GEMM results.
 */
int mi_preferred_weight_layout(int64_t N, int64_t K);

/*
 * mi_relayout_weight: out-of-place permutation of an [N, K] e4m3fn weight
 * between the two layouts: from_layout -> to_layout (MI_WEIGHT_ROW_MAJOR ->
 * MI_WEIGHT_TILED, or back; equal layouts copy).  src and dst are device
 * buffers of N*K bytes, 16-byte aligned, not overlapping (src == dst is
 * rejected with MI_ERR_ALIAS).  N % 16 == 0 (GEMM weights: N % 128), K % 128
 * == 0.  Enqueued on `stream`.
 */
mi_status mi_relayout_weight(const uint8_t *src, int from_layout, uint8_t *dst, int to_layout,
                             int64_t N, int64_t K, hipStream_t stream);

/*
 * mi_block_scaled_fp8_gemm_ex / mi_block_scaled_fp8_gemm_pair_ex: as
 * mi_block_scaled_fp8_gemm / mi_block_scaled_fp8_gemm_pair (which read
 * MI_WEIGHT_ROW_MAJOR weights) with the weight layout as an argument (one
 * layout for both weights of a pair).  Results are bit-identical for both
 * layouts.  A weight passed with the wrong layout value is not detected: the
 * result is wrong.
 */
mi_status mi_block_scaled_fp8_gemm_ex(
    const uint8_t *a_fp8, const float *a_scale, int a_scale_transposed,
    const uint8_t *w_fp8, int w_layout, const float *w_scale,
    uint16_t *out_bf16,
    int64_t M, int64_t N, int64_t K,
    hipStream_t stream);

mi_status mi_block_scaled_fp8_gemm_pair_ex(
    const uint8_t *a_fp8, const float *a_scale, int a_scale_transposed, int w_layout,
    const uint8_t *w1_fp8, const float *w1_scale, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const float *w2_scale, uint16_t *out2_bf16, int64_t N2,
    int64_t M, int64_t K,
    hipStream_t stream);

/*
 * mi_fused_normquant_gemm_pair
 *
 * The whole decode-step hot path in one call: mi_fused_dual_rmsnorm_group_quant
 * ([PR53540] "Purpose") followed by mi_block_scaled_fp8_gemm_pair_ex over its
 * outputs ([D53540]: apply_pre_quantized_block_scaled_mm consumes the
 * (q_fp8, scale) pair as produced, K = Nq, As in the layout transpose_scale
 * chose).  All five outputs are bit-identical to those two calls'.
 *
 * For decode batches (M <= 16 rows of the MLA latent shape: Nq = 1536,
 * Nkv = 512, every row slice 16-byte aligned) over wide weights (N1 + N2 >=
 * 24576) the work is one kernel launch, whose blocks each quantise the rows
 * they consume while their first weight loads are in flight (no hand-over
 * between blocks); other shapes run as the two calls, which are faster
 * there (mi_fused_normquant_gemm_pair_launches tells which).
 *
 * Arguments as mi_fused_dual_rmsnorm_group_quant (q ... out_kv; out_q_fp8
 * 16-byte aligned) and mi_block_scaled_fp8_gemm_pair_ex (w_layout ...
 * out2_bf16, N2; N1, N2 % 128 == 0).  Errors: as those two calls.
 */
mi_status mi_fused_normquant_gemm_pair(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q_fp8, float *out_scale, uint16_t *out_kv,
    int w_layout,
    const uint8_t *w1_fp8, const float *w1_scale, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const float *w2_scale, uint16_t *out2_bf16, int64_t N2,
    hipStream_t stream);

/*
 * mi_fused_normquant_gemm_pair_launches
 *
 * Kernel launches mi_fused_normquant_gemm_pair makes for these sizes on the
 * current device when every operand meets the alignment above: 1 (one
 * launch), else the norm-quant's one plus the pair's (one up to 64 rows with
 * K / 128 in {4, 8, 12, 16}, and from 65 to 256 rows for N1 + N2 <= 64 x
 * the compute units with K / 128 = 12; else two); 0 for M == 0; -1 for sizes
 * the call rejects.  Host only; enqueues nothing.
 */
int mi_fused_normquant_gemm_pair_launches(int64_t M, int64_t Nq, int64_t Nkv, int64_t N1, int64_t N2);

/*
 * e8m0 (power-of-two) scales
 *
 * [D56433] "风险与影响" item 3: weight block scales stored as e8m0
 * (float8_e8m0fnu) exponents; the PRHub digest of vLLM PR #56560: the native
 * gfx950 MXFP8 GEMM, whose scales are e8m0 exponents applied by the matrix
 * cores.  An e8m0 scale is a byte E with value 2^(E - 127) (255 is NaN).
 * The pages give no rule for choosing a group's power-of-two scale; here it
 * is the smallest power of two not below the fp32 scale before rounding:
 *   e      = ceil(log2(max(max_{i in g} |y_i| / 448, 1e-12))), E = e + 127
 *   code_i = e4m3fn_rne(y_i * 2^-e)          (|y_i| * 2^-e <= 448)
 * so y_i * 2^-e is exact and the e4m3 rounding is the only one; a group's
 * largest code lies in [224, 448].  The GEMM then needs no fp32 scale
 * arithmetic: the matrix core applies 2^(Ea-127) and 2^(Eb-127) to the
 * operands of each 128-deep K-block and accumulates the whole K in place.
 */

/*
 * mi_fused_dual_rmsnorm_group_quant_e8m0: mi_fused_dual_rmsnorm_group_quant
 * with e8m0 scales (out_scale_e8m0: M*G exponent bytes in the layout chosen by
 * transpose_scale).  kv is identical to the fp32-scale call.  In fp32 the
 * group maximum times rstd / 448 is within a few ulps of its exact value;
 * when that value is that close to a power of two, the exponent may be one
 * higher or lower than the exact rule gives.
 */
mi_status mi_fused_dual_rmsnorm_group_quant_e8m0(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q_fp8, uint8_t *out_scale_e8m0, uint16_t *out_kv,
    hipStream_t stream);

/*
 * mi_block_scaled_fp8_gemm_e8m0 / mi_block_scaled_fp8_gemm_pair_e8m0: the
 * block-scaled GEMM (single / both consumers) with e8m0 scales:
 *   out[m, n] = bf16_rne( sum_kb 2^(As[m,kb]-127) * 2^(Bs[n/128,kb]-127)
 *                         * sum_{k in kb} dec(a[m,k]) * dec(w[n,k]) )
 * a_scale_e8m0: M*K/128 bytes, [M, K/128] row-major (a_scale_transposed 0)
 * or [K/128, M] (1); w*_scale_e8m0: [N/128, K/128] bytes row-major; both
 * 4-byte aligned.  Other arguments as mi_block_scaled_fp8_gemm_ex /
 * mi_block_scaled_fp8_gemm_pair_ex.
 */
mi_status mi_block_scaled_fp8_gemm_e8m0(
    const uint8_t *a_fp8, const uint8_t *a_scale_e8m0, int a_scale_transposed,
    const uint8_t *w_fp8, int w_layout, const uint8_t *w_scale_e8m0,
    uint16_t *out_bf16,
    int64_t M, int64_t N, int64_t K,
    hipStream_t stream);

mi_status mi_block_scaled_fp8_gemm_pair_e8m0(
    const uint8_t *a_fp8, const uint8_t *a_scale_e8m0, int a_scale_transposed, int w_layout,
    const uint8_t *w1_fp8, const uint8_t *w1_scale_e8m0, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const uint8_t *w2_scale_e8m0, uint16_t *out2_bf16, int64_t N2,
    int64_t M, int64_t K,
    hipStream_t stream);

/*
 * mi_fused_normquant_gemm_pair_e8m0: mi_fused_normquant_gemm_pair with e8m0
 * scales on both sides: the step of mi_fused_dual_rmsnorm_group_quant_e8m0
 * followed by mi_block_scaled_fp8_gemm_pair_e8m0 over its outputs (the
 * exponent bytes written to out_scale_e8m0 are the GEMM's As).  All five
 * outputs are bit-identical to those two calls', and the launch count is
 * the one mi_fused_normquant_gemm_pair_launches gives.  out_scale_e8m0 and
 * w*_scale_e8m0 4-byte aligned; other arguments and errors as
 * mi_fused_normquant_gemm_pair.
 */
mi_status mi_fused_normquant_gemm_pair_e8m0(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q_fp8, uint8_t *out_scale_e8m0, uint16_t *out_kv,
    int w_layout,
    const uint8_t *w1_fp8, const uint8_t *w1_scale_e8m0, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const uint8_t *w2_scale_e8m0, uint16_t *out2_bf16, int64_t N2,
    hipStream_t stream);

/*
 * mi_init
 *
 * Prepares the current device for this library's kernels: caches its
 * compute-unit count and raises the dynamic-LDS limit (a per-device
 * function attribute, not a stream operation) of every GEMM kernel that
 * needs more than the default.  Optional for ordinary use: each entry point
 * does the same lazily on its first launch of a kernel on a device.  A
 * caller that captures calls of this library into a HIP graph calls mi_init
 * on that device before the capture begins (or first makes one ordinary call
 * of every entry point and shape it captures), so that no attribute change
 * happens while the stream is capturing.  Enqueues nothing and allocates
 * nothing; safe to call repeatedly and from several host threads (each for
 * its current device).  MI_ERR_HIP if the HIP runtime reports an error (no
 * device, for instance).
 */
mi_status mi_init(void);

/*
 * mi_negotiate_scale_layout
 *
 * [D56433] item 4: the producer writes one scale buffer for several
 * consumers, so they must agree on its major order.  Returns 1 if every
 * consumer wants column-major (transposed) scales, 0 if every one wants
 * row-major, and -1 if they disagree or n <= 0 / the pointer is NULL (the
 * caller then must not share one pre-quantised pair).  Host-only; touches
 * no GPU.
 */
int mi_negotiate_scale_layout(const int *consumer_wants_transposed, int n);

/* Static, human-readable name of a status code (never NULL). */
const char *mi_status_string(mi_status s);

#ifdef __cplusplus
}
#endif

#endif /* MI_NORMQUANT_H */
