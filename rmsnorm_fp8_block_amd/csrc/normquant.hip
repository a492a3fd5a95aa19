// normquant.hip -- fused dual RMSNorm + per-1x128 FP8 group quantisation
// for gfx950.
//
// What is computed follows the GitHub page of vLLM PR #53540 ("[ROCm][Perf]
// Fuse SWA q/kv RMSNorm and q FP8 group quant for DeepSeek-V4"), section
// "Purpose": one launch RMSNorms the q latent and the kv latent with fp32
// accumulation, quantises the normalised q per 1x128 group with an fp32
// scale straight from the fp32 values, and writes kv as bf16.  The scale
// layout flag follows the PRHub report of vLLM PR #56433 (item 4) and the
// PRHub digest of SGLang PR #27289 (scales written column-major directly,
// with no transpose copy afterwards).
//
// Mapping onto CDNA4:
//  - one wave64 per row; each lane owns 8 consecutive elements of every
//    512-element chunk, fetched with one 16-byte load (a 1536 + 512 row is
//    3 + 1 loads per lane), and all loads are issued before any arithmetic;
//  - the row is normalised as z = x * gamma (exact: a product of two bf16
//    values, formed with the packed bf16 dot instruction) times rstd, and
//    the group quantisation uses z * (rstd / s), so the per-element work is
//    a handful of VALU operations (wave64 fp32 VALU ops cost 4 cycles, and
//    at 8192 rows the VALU time is of the same order as the memory time);
//  - a 128-element group is exactly the 16 lanes of one DPP row, so the
//    group amax is a 4-step DPP butterfly and every lane of the row ends up
//    holding its group's scale;
//  - the sums of squares use the packed bf16 dot instruction per lane, then
//    a DPP row butterfly and a combination of the four row totals (fp32
//    throughout); rstd is the hardware reciprocal square root refined by one
//    Newton step;
//  - codes come from the packed fp32 -> e4m3fn convert, kv from the packed
//    fp32 -> bf16 convert;
//  - row-major scales: 4 lanes per chunk store 16 contiguous bytes;
//    column-major scales: element (m, g) lands at g*M + m, and rows are dealt
//    to XCDs in contiguous ranges so that the partial cache lines of
//    neighbouring rows meet in one L2.
#include "normquant_row.h"

namespace mi {

using namespace row;

namespace {

// kQ / kKv: number of 512-element chunks held per lane (compile-time bound);
// the actual widths are a.Nq / a.Nkv.  kVec: every row start, gamma and
// output row is 16-byte aligned and Nkv % 8 == 0.  kRows: consecutive rows
// per wave; all their loads are issued together, gammas once per wave.
// kFull: Nq == 512 * kQ and Nkv == 512 * kKv (no bounds tests).
// kStream: the rows are read, and the outputs written, with non-temporal
// loads and stores (large M: every row is read once; measured slower for a
// handful of rows).
template <int kQ, int kKv, bool kVec, int kRows, bool kFull, bool kNorm, bool kE8m0, bool kStream>
__global__ __launch_bounds__(256) void fused_dual_rmsnorm_group_quant_kernel(NormQuantParams a) {
    constexpr int kKvA = kKv > 0 ? kKv : 1;  // array extents
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar row addressing
    const int waves_per_block = blockDim.x / kWave;
    const int64_t row0 =
        (static_cast<int64_t>(xcd_contiguous_block(blockIdx.x, gridDim.x)) * waves_per_block + wave) * kRows;
    if (row0 >= a.M)
        return;

    // -- all loads first: gammas, then every row's data ------------------------
    uint4 gq_raw[kQ], gk_raw[kKvA];
    if constexpr (kNorm) {
#pragma unroll
        for (int c = 0; c < kQ; ++c)
            gq_raw[c] = load8<kVec, kFull>(a.gamma_q, c * kChunk + lane * 8, a.Nq);
    }
#pragma unroll
    for (int c = 0; c < kKv; ++c)
        gk_raw[c] = load8<kVec, kFull>(a.gamma_kv, c * kChunk + lane * 8, a.Nkv);
    uint4 xq[kRows][kQ], xk[kRows][kKvA];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t m = row0 + r;
        if (m >= a.M)
            break;
        const uint16_t *qrow = a.q + m * a.q_stride;
#pragma unroll
        for (int c = 0; c < kQ; ++c)
            xq[r][c] = load8<kVec, kFull, kStream>(qrow, c * kChunk + lane * 8, a.Nq);
        if constexpr (kKv > 0) {
            const uint16_t *krow = a.kv + m * a.kv_stride;
#pragma unroll
            for (int c = 0; c < kKv; ++c)
                xk[r][c] = load8<kVec, kFull, kStream>(krow, c * kChunk + lane * 8, a.Nkv);
        }
    }
    // gammas prepared once per wave, shared by its rows
    GammaSlice gq[kQ], gk[kKvA];
    if constexpr (kNorm) {
#pragma unroll
        for (int c = 0; c < kQ; ++c)
            gq[c] = prepare_gamma(gq_raw[c]);
    }
#pragma unroll
    for (int c = 0; c < kKv; ++c)
        gk[c] = prepare_gamma(gk_raw[c]);

#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t m = row0 + r;
        if (m >= a.M)
            break;
        process_row<kQ, kKv, kVec, kFull, kNorm, kE8m0, kStream>(a, m, lane, xq[r], xk[r], gq, gk);
    }
}

// Single input, one row split over kSplit waves of a 4-wave block (for few
// rows of many chunks, so that the grid still covers the chip).  Wave part p
// of a row takes chunks p, p + kSplit, ... (at most kC of them).  With the
// norm, each wave reduces its chunks' sums of squares, the kSplit wave sums
// meet in LDS and are added in part order, so every wave of the row
// derives the same rstd.
template <int kC, int kSplit, bool kVec, bool kNorm>
__global__ __launch_bounds__(256) void split_row_group_quant_kernel(NormQuantParams a) {
    constexpr int kRowsPerBlock = 4 / kSplit;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int part = wave % kSplit;
    const int64_t m =
        static_cast<int64_t>(xcd_contiguous_block(blockIdx.x, gridDim.x)) * kRowsPerBlock + wave / kSplit;
    const bool live = m < a.M;  // uniform per wave
    if (!kNorm && !live)
        return;  // no barrier below without the norm
    const int nch = (a.Nq + kChunk - 1) / kChunk;

    uint4 x[kC], graw[kC];
    if (live) {
        const uint16_t *row = a.q + m * a.q_stride;
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            const int col = (part + kSplit * i) * kChunk + lane * 8;
            if constexpr (kNorm)
                graw[i] = load8<kVec>(a.gamma_q, col, a.Nq);
            x[i] = load8<kVec>(row, col, a.Nq);  // zeros past the row
        }
    }
    float rq = 1.0f;
    if constexpr (kNorm) {
        __shared__ float wave_ssq[4];
        float part_ssq[kC];
#pragma unroll
        for (int i = 0; i < kC; ++i)
            part_ssq[i] = live ? sumsq8(x[i]) : 0.0f;
        const float w = wave_sum(fold_sum<kC>(part_ssq));
        if (lane == 0)
            wave_ssq[wave] = w;
        __syncthreads();
        const int first = wave - part;
        float ssq = wave_ssq[first];
#pragma unroll
        for (int j = 1; j < kSplit; ++j)
            ssq += wave_ssq[first + j];
        rq = rstd_from_ssq(ssq, a.inv_nq, a.eps);
    }
    if (!live)
        return;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        const int c = part + kSplit * i;
        if (c >= nch)
            break;  // uniform across the wave
        GammaSlice g;
        if constexpr (kNorm)
            g = prepare_gamma(graw[i]);
        quant_chunk<kVec, false, kNorm>(a, m, lane, c, x[i], g, rq);
    }
}

// rows from which the full-width variants stream their row loads
constexpr int64_t kStreamFromRows = 1024;

template <int kQ, int kKv, bool kVec, int kRows, bool kFull = false, bool kNorm = true, bool kE8m0 = false>
hipError_t launch_variant(const NormQuantParams &p, hipStream_t stream) {
    const int64_t waves = (p.M + kRows - 1) / kRows;
    const int waves_per_block = waves >= 4 ? 4 : static_cast<int>(waves);
    const int64_t blocks = (waves + waves_per_block - 1) / waves_per_block;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    if (kFull && p.M >= kStreamFromRows)
        hipLaunchKernelGGL((fused_dual_rmsnorm_group_quant_kernel<kQ, kKv, kVec, kRows, kFull, kNorm, kE8m0, kFull>),
                           dim3(static_cast<unsigned>(blocks)), dim3(waves_per_block * kWave), 0, stream, p);
    else
        hipLaunchKernelGGL((fused_dual_rmsnorm_group_quant_kernel<kQ, kKv, kVec, kRows, kFull, kNorm, kE8m0, false>),
                           dim3(static_cast<unsigned>(blocks)), dim3(waves_per_block * kWave), 0, stream, p);
    return hipGetLastError();
}

template <int kC, int kSplit, bool kVec, bool kNorm>
hipError_t launch_split(const NormQuantParams &p, hipStream_t stream) {
    constexpr int kRowsPerBlock = 4 / kSplit;
    const int64_t blocks = (p.M + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((split_row_group_quant_kernel<kC, kSplit, kVec, kNorm>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

namespace {

template <bool kE8m0>
hipError_t launch_dual(const NormQuantParams &p, hipStream_t stream) {
    // The vector path needs every 8-element lane slice to be 16-byte aligned.
    // out_q rows are Nq bytes (a multiple of 128) and need 8-byte stores.
    const bool vec = aligned16(p.q) && aligned16(p.kv) && aligned16(p.gamma_q) &&
                     aligned16(p.gamma_kv) && aligned16(p.out_kv) && aligned16(p.out_q) &&
                     (p.q_stride % 8) == 0 && (p.kv_stride % 8) == 0 && (p.Nkv % 8) == 0;
    const int qch = (p.Nq + kChunk - 1) / kChunk;
    const int kch = (p.Nkv + kChunk - 1) / kChunk;
    if (vec && p.Nq == 3 * kChunk && p.Nkv == kChunk)  // the MLA latent shape: 1536 + 512
        return launch_variant<3, 1, true, 1, true, true, kE8m0>(p, stream);
    if (qch <= 8 && kch <= 4)
        return vec ? launch_variant<8, 4, true, 1, false, true, kE8m0>(p, stream)
                   : launch_variant<8, 4, false, 1, false, true, kE8m0>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_normquant(const NormQuantParams &p, hipStream_t stream) { return launch_dual<false>(p, stream); }

hipError_t launch_normquant_e8m0(const NormQuantParams &p, hipStream_t stream) {
    return launch_dual<true>(p, stream);
}

// Below this many rows, one wave per row leaves CUs idle for wide rows.
constexpr int64_t kSplitBelowRows = 2048;

template <bool kNorm>
hipError_t launch_single_kind(const NormQuantParams &p, hipStream_t stream) {
    const bool vec = aligned16(p.q) && (!kNorm || aligned16(p.gamma_q)) && aligned16(p.out_q) &&
                     (p.q_stride % 8) == 0;
    const int qch = (p.Nq + kChunk - 1) / kChunk;
    // few rows of 4 or more chunks: split each row over 2 or 4 waves
    if (p.M < kSplitBelowRows && qch >= 4) {
        if (qch >= 8)
            return vec ? launch_split<4, 4, true, kNorm>(p, stream) : launch_split<4, 4, false, kNorm>(p, stream);
        return vec ? launch_split<4, 2, true, kNorm>(p, stream) : launch_split<4, 2, false, kNorm>(p, stream);
    }
    if (vec && p.Nq == 3 * kChunk)  // 1536: the MLA q latent
        return launch_variant<3, 0, true, 1, true, kNorm>(p, stream);
    if (vec && p.Nq == 14 * kChunk)  // 7168: a DeepSeek hidden row
        return launch_variant<14, 0, true, 1, true, kNorm>(p, stream);
    if (qch <= 16)
        return vec ? launch_variant<16, 0, true, 1, false, kNorm>(p, stream)
                   : launch_variant<16, 0, false, 1, false, kNorm>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_group_quant(const NormQuantParams &p, bool normalize, hipStream_t stream) {
    return normalize ? launch_single_kind<true>(p, stream) : launch_single_kind<false>(p, stream);
}

}  // namespace mi
