// gemm_fp8_bs.hip -- block-scaled FP8 GEMM on the gfx950 matrix cores.
//
// Computes out[m, n] = bf16( sum_kb As[m, kb] * Bs[n/128, kb] *
//                            sum_{k in kb} a[m, k] * w[n, k] )
// for the pre-quantised activation (e4m3fn codes + one fp32 scale per 1x128
// group, row- or column-major) and an e4m3fn weight [N, K] with one fp32
// scale per 128x128 block.  This is the consumer the PRHub digest of vLLM PR
// #53540 describes in its excerpt of apply_pre_quantized_block_scaled_mm
// (A = x_fp8, As = x_scale, Bs = the weight's block scale, used as given),
// with the bf16 output of the aiter_w8a8_block_fp8_linear excerpt in the
// PRHub digest of SGLang PR #27289, and the explicit As major order of the
// PRHub report of vLLM PR #56433 (item 2).
//
// Mapping onto CDNA4:
//  - v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3): one instruction covers one
//    whole 128-deep K-block of a 16 (n) x 16 (m) output tile, so the block's
//    partial sum leaves the matrix core once per K-block and is folded into
//    the fp32 accumulator with As[m, kb] * Bs[nb, kb] (one FMA per value);
//  - the weight is the MFMA "A" operand (rows = n): each lane streams 32
//    contiguous bytes of one weight row per K-block straight from HBM into
//    registers; a weight byte is used by exactly one wave;
//  - the activation is the MFMA "B" operand (columns = m): a block stages
//    its M-tile for 4 K-blocks at a time in LDS, already in fragment order
//    (each lane's 32 bytes split in two 16-byte halves, lane-contiguous, so
//    the ds_read_b128 of a wave hits consecutive banks);
//  - each lane holds outputs (n = 4*(lane/16) + i, m = lane % 16), i < 4, so
//    one lane writes 4 consecutive bf16 (8 bytes) of one output row;
//  - a block is 4 waves = 64 weight rows x up to 64 activation rows; blocks
//    are renumbered so that the M-tiles of one N-tile run on the same XCD
//    and share the weight tile through its L2.
// The K order inside one MFMA is irrelevant to the result as long as both
// operands use the same one; both are loaded with the same lane/byte -> k
// assignment.
#include "device.h"
#include "launch.h"

namespace mi {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBlk = 128;            // K-block = weight scale block = quant group
constexpr int kStageKb = 4;          // K-blocks staged in LDS at a time
constexpr int kWaves = 4;
constexpr int kTileN = 16 * kWaves;  // weight rows per block

__device__ __forceinline__ v8i join(const uint4 &lo, const uint4 &hi) {
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

__device__ __forceinline__ v4f mfma_e4m3_16x16x128(const v8i &a, const v8i &b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // format 0 = e4m3 for both operands; zero scale operands select the
    // unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// kMT: 16-row activation tiles per block (1..4).
template <int kMT>
__global__ __launch_bounds__(256) void block_scaled_fp8_gemm_kernel(GemmParams p) {
    __shared__ uint4 s_act[kStageKb * kMT * 2 * kWave];   // [kb][mt][half][lane]
    __shared__ float s_as[kStageKb][kMT * 16];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t M = p.M, K = p.K;
    const int KB = static_cast<int>(K / kBlk);

    const int mgrid = static_cast<int>((M + kMT * 16 - 1) / (kMT * 16));
    const int b = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const int64_t m0 = static_cast<int64_t>(b % mgrid) * (kMT * 16);
    const int64_t n0 = static_cast<int64_t>(b / mgrid) * kTileN + wave * 16;

    const uint8_t *wrow = p.w + (n0 + (lane & 15)) * K + 32 * (lane >> 4);
    const float *bs_row = p.w_scale + (n0 / kBlk) * KB;

    v4f acc[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t)
        acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (int kb0 = 0; kb0 < KB; kb0 += kStageKb) {
        const int kc = min(kStageKb, KB - kb0);

        // this wave's weight fragments for the stage (issued before the
        // activation staging so the two overlap)
        v8i wf[kStageKb];
#pragma unroll
        for (int j = 0; j < kStageKb; ++j) {
            if (j < kc) {
                const uint4 *src = reinterpret_cast<const uint4 *>(wrow + static_cast<int64_t>(kb0 + j) * kBlk);
                wf[j] = join(src[0], src[1]);
            }
        }

        __syncthreads();  // the previous stage's LDS reads are done
        const int granules = kMT * 16 * kc * 8;  // 16-byte pieces of the tile
        for (int gi = threadIdx.x; gi < granules; gi += blockDim.x) {
            const int r = gi / (kc * 8);
            const int c = gi % (kc * 8);
            const int kb = c >> 3, j = c & 7;
            const int L = (j >> 1) * 16 + (r & 15);
            const int h = j & 1, mt = r >> 4;
            uint4 v = make_uint4(0, 0, 0, 0);
            const int64_t m = m0 + r;
            if (m < M)
                v = *reinterpret_cast<const uint4 *>(p.a + m * K + static_cast<int64_t>(kb0 + kb) * kBlk + j * 16);
            s_act[((kb * kMT + mt) * 2 + h) * kWave + L] = v;
        }
        for (int i = threadIdx.x; i < kMT * 16 * kc; i += blockDim.x) {
            const int r = i % (kMT * 16), kb = i / (kMT * 16);
            const int64_t m = m0 + r;
            float s = 0.0f;
            if (m < M)
                s = p.a_scale_transposed ? p.a_scale[static_cast<int64_t>(kb0 + kb) * M + m]
                                         : p.a_scale[m * KB + kb0 + kb];
            s_as[kb][r] = s;
        }
        __syncthreads();

#pragma unroll
        for (int j = 0; j < kStageKb; ++j) {
            if (j >= kc)
                break;
            const float bs = bs_row[kb0 + j];
#pragma unroll
            for (int t = 0; t < kMT; ++t) {
                const uint4 lo = s_act[((j * kMT + t) * 2 + 0) * kWave + lane];
                const uint4 hi = s_act[((j * kMT + t) * 2 + 1) * kWave + lane];
                const v4f part = mfma_e4m3_16x16x128(wf[j], join(lo, hi));
                const float sc = s_as[j][t * 16 + (lane & 15)] * bs;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[t][i] = fmaf(part[i], sc, acc[t][i]);
            }
        }
    }

    // lane holds out[m0 + 16t + lane%16][n0 + 4*(lane/16) + i]
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
        const int64_t m = m0 + t * 16 + (lane & 15);
        if (m < M) {
            const int64_t n = n0 + 4 * (lane >> 4);
            *reinterpret_cast<uint2 *>(p.out + m * p.N + n) =
                make_uint2(pack2_bf16(acc[t][0], acc[t][1]), pack2_bf16(acc[t][2], acc[t][3]));
        }
    }
}

template <int kMT>
hipError_t launch_mt(const GemmParams &p, hipStream_t stream) {
    const int64_t mgrid = (p.M + kMT * 16 - 1) / (kMT * 16);
    const int64_t blocks = mgrid * (p.N / kTileN);
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((block_scaled_fp8_gemm_kernel<kMT>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kWaves * kWave), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_scaled_gemm(const GemmParams &p, hipStream_t stream) {
    // N % 128 == 0 (validated) so N is a whole number of 64-row tiles.
    if (p.M <= 16)
        return launch_mt<1>(p, stream);
    if (p.M <= 32)
        return launch_mt<2>(p, stream);
    if (p.M <= 48)
        return launch_mt<3>(p, stream);
    return launch_mt<4>(p, stream);
}

}  // namespace mi
