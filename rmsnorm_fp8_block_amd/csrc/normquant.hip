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
//    3 + 1 loads per lane, all issued before any arithmetic);
//  - a 128-element group is exactly the 16 lanes of one DPP row, so the
//    group amax is a 4-step DPP butterfly and every lane of the row ends up
//    holding its group's scale;
//  - the sums of squares are pairwise trees in each lane, then a DPP row
//    butterfly and a combination of the four row totals (fp32 throughout);
//  - codes come from the packed fp32 -> e4m3fn convert, kv from the packed
//    fp32 -> bf16 convert;
//  - row-major scales: 4 lanes per chunk store 16 contiguous bytes;
//    column-major scales: element (m, g) lands at g*M + m, and rows are dealt
//    to XCDs in contiguous ranges so that the partial cache lines of
//    neighbouring rows meet in one L2.
#include "device.h"
#include "launch.h"

namespace mi {
namespace {

constexpr int kChunk = 512;     // elements per 16-byte-per-lane wave load
constexpr int kGroup = 128;
constexpr float kE4m3Max = 448.0f;
constexpr float kScaleFloor = 1e-12f;

// 8 consecutive bf16 at p[col, col+8); elements at or beyond n read as zero.
// kVec: p + col is 16-byte aligned whenever col + 8 <= n.
template <bool kVec>
__device__ __forceinline__ uint4 load8(const uint16_t *p, int col, int n) {
    if (kVec && col + 8 <= n)
        return *reinterpret_cast<const uint4 *>(p + col);
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        e[j] = (col + j < n) ? p[col + j] : 0u;
    return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
}

// Pairwise sum of the squares of 8 values.
__device__ __forceinline__ float sumsq8(const float (&x)[8]) {
    const float a = x[0] * x[0] + x[1] * x[1];
    const float b = x[2] * x[2] + x[3] * x[3];
    const float c = x[4] * x[4] + x[5] * x[5];
    const float d = x[6] * x[6] + x[7] * x[7];
    return (a + b) + (c + d);
}

// Pairwise sum of a small fixed-size array.
template <int N>
__device__ __forceinline__ float tree_sum(const float *v) {
    if constexpr (N == 1) {
        return v[0];
    } else {
        constexpr int H = N / 2;
        return tree_sum<H>(v) + tree_sum<N - H>(v + H);
    }
}

// Reciprocal RMS from the fp32 sum of squares.  The division and square root
// are taken in fp64 and rounded once to fp32.
__device__ __forceinline__ float rstd_from_ssq(float ssq, int n, float eps) {
    return static_cast<float>(1.0 / sqrt(static_cast<double>(ssq) / n + static_cast<double>(eps)));
}

// kQ / kKv: number of 512-element chunks held per lane (compile-time bound);
// the actual widths are a.Nq / a.Nkv.  kVec: every row start, gamma and
// output row is 16-byte aligned and Nkv % 8 == 0.
template <int kQ, int kKv, bool kVec>
__global__ __launch_bounds__(256) void fused_dual_rmsnorm_group_quant_kernel(NormQuantParams a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int rows_per_block = blockDim.x / kWave;
    const int64_t m = static_cast<int64_t>(xcd_contiguous_block(blockIdx.x, gridDim.x)) * rows_per_block + wave;
    if (m >= a.M)
        return;

    const uint16_t *qrow = a.q + m * a.q_stride;
    const uint16_t *krow = a.kv + m * a.kv_stride;

    // -- all loads first: row data and gammas --------------------------------
    uint4 xq[kQ], gq[kQ], xk[kKv], gk[kKv];
#pragma unroll
    for (int c = 0; c < kQ; ++c) {
        const int col = c * kChunk + lane * 8;
        xq[c] = load8<kVec>(qrow, col, a.Nq);
        gq[c] = load8<kVec>(a.gamma_q, col, a.Nq);
    }
#pragma unroll
    for (int c = 0; c < kKv; ++c) {
        const int col = c * kChunk + lane * 8;
        xk[c] = load8<kVec>(krow, col, a.Nkv);
        gk[c] = load8<kVec>(a.gamma_kv, col, a.Nkv);
    }

    // -- sums of squares (fp32) and reciprocal RMS -----------------------------
    float part_q[kQ], part_k[kKv];
#pragma unroll
    for (int c = 0; c < kQ; ++c) {
        float x[8];
        unpack8_bf16(xq[c], x);
        part_q[c] = sumsq8(x);
    }
#pragma unroll
    for (int c = 0; c < kKv; ++c) {
        float x[8];
        unpack8_bf16(xk[c], x);
        part_k[c] = sumsq8(x);
    }
    const float ssq_q = wave_sum(tree_sum<kQ>(part_q));
    const float ssq_k = wave_sum(tree_sum<kKv>(part_k));
    const float rq = rstd_from_ssq(ssq_q, a.Nq, a.eps);
    const float rk = rstd_from_ssq(ssq_k, a.Nkv, a.eps);

    // -- kv: normalise, scale, round to bf16 -----------------------------------
    uint16_t *kout = a.out_kv + m * a.Nkv;
#pragma unroll
    for (int c = 0; c < kKv; ++c) {
        const int col = c * kChunk + lane * 8;
        if (col >= a.Nkv)
            continue;
        float x[8], g[8];
        unpack8_bf16(xk[c], x);
        unpack8_bf16(gk[c], g);
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            y[j] = x[j] * rk * g[j];
        const uint4 packed = make_uint4(pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3]),
                                        pack2_bf16(y[4], y[5]), pack2_bf16(y[6], y[7]));
        if (kVec && col + 8 <= a.Nkv) {
            *reinterpret_cast<uint4 *>(kout + col) = packed;
        } else {
            const uint32_t w[4] = {packed.x, packed.y, packed.z, packed.w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (col + j < a.Nkv)
                    kout[col + j] = static_cast<uint16_t>(w[j / 2] >> (16 * (j & 1)));
        }
    }

    // -- q: normalise, group amax, scale, e4m3fn codes -------------------------
    const int G = a.Nq / kGroup;
    uint8_t *qout = a.out_q + m * a.Nq;
#pragma unroll
    for (int c = 0; c < kQ; ++c) {
        const int col = c * kChunk + lane * 8;
        if (c * kChunk >= a.Nq)
            break;  // uniform across the wave
        float x[8], g[8], y[8];
        unpack8_bf16(xq[c], x);
        unpack8_bf16(gq[c], g);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[j] = x[j] * rq * g[j];
            amax = fmaxf(amax, fabsf(y[j]));
        }
        // 16 lanes x 8 elements = one 128-element group
        amax = row16_max(amax);
        const float s = fmaxf(amax / kE4m3Max, kScaleFloor);
        const float inv = 1.0f / s;
        float r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            r[j] = fminf(fmaxf(y[j] * inv, -kE4m3Max), kE4m3Max);
        const uint32_t lo = pack4_e4m3(r[0], r[1], r[2], r[3]);
        const uint32_t hi = pack4_e4m3(r[4], r[5], r[6], r[7]);
        if (col < a.Nq) {  // Nq % 128 == 0: a lane's 8 codes are all in range
            if (kVec) {
                *reinterpret_cast<uint2 *>(qout + col) = make_uint2(lo, hi);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    qout[col + j] = static_cast<uint8_t>((j < 4 ? lo : hi) >> (8 * (j & 3)));
            }
        }

        const int grp = c * (kChunk / kGroup) + lane / 16;
        if ((lane & 15) == 0 && grp < G) {
            const int64_t at = a.transpose_scale ? static_cast<int64_t>(grp) * a.M + m
                                                 : m * G + grp;
            a.out_scale[at] = s;
        }
    }
}

template <int kQ, int kKv, bool kVec>
hipError_t launch_variant(const NormQuantParams &p, hipStream_t stream) {
    const int rows_per_block = p.M >= 4 ? 4 : static_cast<int>(p.M);
    const int64_t blocks = (p.M + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((fused_dual_rmsnorm_group_quant_kernel<kQ, kKv, kVec>),
                       dim3(static_cast<unsigned>(blocks)), dim3(rows_per_block * kWave), 0, stream, p);
    return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_normquant(const NormQuantParams &p, hipStream_t stream) {
    // The vector path needs every 8-element lane slice to be 16-byte aligned.
    // out_q rows are Nq bytes (a multiple of 128) and need 8-byte stores.
    const bool vec = aligned16(p.q) && aligned16(p.kv) && aligned16(p.gamma_q) &&
                     aligned16(p.gamma_kv) && aligned16(p.out_kv) && aligned16(p.out_q) &&
                     (p.q_stride % 8) == 0 && (p.kv_stride % 8) == 0 && (p.Nkv % 8) == 0;
    const int qch = (p.Nq + kChunk - 1) / kChunk;
    const int kch = (p.Nkv + kChunk - 1) / kChunk;
    if (qch == 3 && kch == 1)  // the MLA latent shape: 1536 + 512
        return vec ? launch_variant<3, 1, true>(p, stream) : launch_variant<3, 1, false>(p, stream);
    if (qch <= 8 && kch <= 4)
        return vec ? launch_variant<8, 4, true>(p, stream) : launch_variant<8, 4, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace mi
