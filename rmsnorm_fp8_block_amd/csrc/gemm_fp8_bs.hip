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
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace mi {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u32 __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------------------
// Weight-streaming variant (M <= 256, K/128 = kKB known at compile time).
// Each wave owns one 16-row weight subtile and loads all kKB K-blocks of it
// with one burst of 16-byte loads (24 KB in flight per wave at K = 1536),
// so the whole weight matrix is read from HBM once, in a single round trip
// spread over every CU.  The activations are processed in chunks of up to
// 64 rows: the block stages a chunk (in fragment order) and its scales in
// LDS with direct global -> LDS loads, then every wave multiplies it with
// the weight fragments it keeps in registers.
//
// Ordering: the first chunk's LDS loads are issued before the weight burst,
// and before the barrier each wave waits only until those have landed
// (loads complete in issue order), so the MFMAs start while the weight
// K-blocks are still arriving.
// ---------------------------------------------------------------------------
constexpr int kStreamMaxWaves = 8;
constexpr int kChunkRows = 64;

// vmcnt-only waits (gfx9 encoding: vmcnt[3:0] + vmcnt[5:4] at bits 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima = no wait)
template <int kVm>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(kVm >= 0 && kVm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int kMT, int kKB>
__device__ __forceinline__ void stage_chunk(const GemmParams &p, int64_t m0, uint4 *s_act, float *s_as,
                                           int wave, int waves, int lane) {
    const int64_t M = p.M, K = p.K;
    // Every block reads the same (small) activation rows.  Each block starts
    // at a different slab so that, at any moment, the CUs ask for different
    // cache lines instead of queueing on the same L2 channel.
    constexpr int kSlabs = kKB * kMT * 2;
    const int rot = static_cast<int>((blockIdx.x * 7u) % kSlabs);
    // Slab i = (kb * kMT + mt) * 2 + h of the fragment layout is 64 lanes x
    // 16 bytes; one global_load_lds_dwordx4 fills it, lane L fetching bytes
    // [kb*128 + 32*(L/16) + 16*h, +16) of activation row m0 + mt*16 + L%16.
    // Rows at or beyond M repeat row M-1: they only feed output columns that
    // are never stored.
    for (int j = wave; j < kSlabs; j += waves) {
        const int i = (j + rot) % kSlabs;
        const int h = i & 1, mt = (i >> 1) % kMT, kb = (i >> 1) / kMT;
        const int64_t r = min<int64_t>(m0 + mt * 16 + (lane & 15), M - 1);
        const uint8_t *src = p.a + r * K + kb * kBlk + 32 * (lane >> 4) + 16 * h;
        __builtin_amdgcn_global_load_lds(src, s_act + i * kWave, 16, 0, 0);
    }
    // activation scales: one 4-byte direct load per K-block, lane = row
    const int krot = static_cast<int>((blockIdx.x * 5u) % kKB);
    for (int j = wave; j < kKB; j += waves) {
        const int kb = (j + krot) % kKB;
        const int64_t r = min<int64_t>(m0 + lane, M - 1);
        const float *src = p.a_scale_transposed ? p.a_scale + static_cast<int64_t>(kb) * M + r
                                                : p.a_scale + r * kKB + kb;
        __builtin_amdgcn_global_load_lds(src, s_as + kb * kWave, 4, 0, 0);
    }
}

// One 64-row chunk: each wave multiplies the staged activations with its
// weight fragments and writes its 16 output columns of the chunk's rows.
template <int kMT, int kKB>
__device__ __forceinline__ void compute_chunk(const GemmParams &p, int64_t m0, int64_t n0, int lane,
                                              const uint4 *s_act, const float *s_as,
                                              const v8i (&wf)[kKB], const float (&bs)[kKB]) {
    v4f acc[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t)
        acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // Pipeline: the MFMAs of K-block kb+1 are issued before the scale FMAs
    // of K-block kb (so the FMAs' wait for the matrix-core results overlaps
    // the next MFMAs), and the activation fragments and scales are read from
    // LDS two K-blocks ahead.  The empty asm statements pin that order: the
    // compiler would otherwise be free to issue every MFMA first and keep all
    // partial results live, which does not fit next to the weight burst.
    auto frag = [&](int kb, int t, uint4 &lo, uint4 &hi, float &as) {
        lo = s_act[((kb * kMT + t) * 2 + 0) * kWave + lane];
        hi = s_act[((kb * kMT + t) * 2 + 1) * kWave + lane];
        as = s_as[kb * kWave + t * 16 + (lane & 15)];
    };
    uint4 lo[kMT], hi[kMT];     // fragments of the next K-block to multiply
    float as_m[kMT];
    v4f part[kMT];              // MFMA results of the K-block being folded
    float sc[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
        uint4 l0, h0;
        float a0;
        frag(0, t, l0, h0, a0);
        part[t] = mfma_e4m3_16x16x128(wf[0], join(l0, h0));
        sc[t] = a0 * bs[0];
    }
    if (kKB > 1) {
#pragma unroll
        for (int t = 0; t < kMT; ++t)
            frag(1, t, lo[t], hi[t], as_m[t]);
    }
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
        v4f next[kMT];
        float nsc[kMT];
        if (kb + 1 < kKB) {
#pragma unroll
            for (int t = 0; t < kMT; ++t) {
                next[t] = mfma_e4m3_16x16x128(wf[kb + 1], join(lo[t], hi[t]));
                nsc[t] = as_m[t] * bs[kb + 1];
            }
            if (kb + 2 < kKB) {
#pragma unroll
                for (int t = 0; t < kMT; ++t)
                    frag(kb + 2, t, lo[t], hi[t], as_m[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < kMT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][i] = fmaf(part[t][i], sc[t], acc[t][i]);
            if (kb + 1 < kKB) {
                part[t] = next[t];
                sc[t] = nsc[t];
            }
            asm volatile("" : "+v"(acc[t]), "+v"(part[t]), "+v"(lo[t].x), "+v"(lo[t].y), "+v"(lo[t].z),
                         "+v"(lo[t].w), "+v"(hi[t].x), "+v"(hi[t].y), "+v"(hi[t].z), "+v"(hi[t].w),
                         "+v"(as_m[t]));
        }
    }
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
        const int64_t m = m0 + t * 16 + (lane & 15);
        if (m < p.M) {
            const int64_t n = n0 + 4 * (lane >> 4);
            *reinterpret_cast<uint2 *>(p.out + m * p.N + n) =
                make_uint2(pack2_bf16(acc[t][0], acc[t][1]), pack2_bf16(acc[t][2], acc[t][3]));
        }
    }
}

template <int kMT, int kKB>
__global__ __launch_bounds__(kStreamMaxWaves * kWave) void block_scaled_fp8_gemm_stream_kernel(
    GemmParams p, int subtiles_per_block) {
    extern __shared__ uint4 s_dyn[];
    uint4 *s_act = s_dyn;                                                   // [kb][mt][half][lane]
    float *s_as = reinterpret_cast<float *>(s_dyn + kKB * kMT * 2 * kWave);  // [kb][64 rows]

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar addressing
    const int waves = blockDim.x / kWave;
    const int64_t M = p.M, K = p.K;
    const int64_t S = p.N / 16;  // 16-row weight subtiles
    const int64_t st = static_cast<int64_t>(blockIdx.x) * subtiles_per_block + wave;
    const bool active = wave < subtiles_per_block && st < S;
    const int64_t n0 = st * 16;

    float bs[kKB];  // the subtile's weight scales (one 128-row block)
    if (active) {
        const float *bs_row = p.w_scale + (n0 / kBlk) * kKB;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
            bs[kb] = bs_row[kb];
    }
    stage_chunk<kMT, kKB>(p, 0, s_act, s_as, wave, waves, lane);
    // The fences keep the program order of the memory operations: scales and
    // staging loads, then the weight burst, then the wait.  Loads complete in
    // issue order, so waiting until only the burst is outstanding means this
    // wave's staging loads have landed in LDS.
    asm volatile("" ::: "memory");
    v8i wf[kKB];
    if (active) {
        const uint8_t *wrow = p.w + (n0 + (lane & 15)) * K + 32 * (lane >> 4);
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const uint4 *src = reinterpret_cast<const uint4 *>(wrow + kb * kBlk);
            wf[kb] = join(src[0], src[1]);
        }
        asm volatile("" ::: "memory");
        wait_vmcnt<2 * kKB>();
    } else {
        wait_vmcnt<0>();
    }
    // A bare barrier: the LDS data is visible once every wave's own staging
    // loads have landed (waited for above).  __syncthreads() would add a
    // release fence that drains the whole weight burst first.
    __builtin_amdgcn_s_barrier();
    if (active)
        compute_chunk<kMT, kKB>(p, 0, n0, lane, s_act, s_as, wf, bs);

    for (int64_t m0 = kChunkRows; m0 < M; m0 += kChunkRows) {
        __syncthreads();  // every wave is done reading the previous chunk
        stage_chunk<kMT, kKB>(p, m0, s_act, s_as, wave, waves, lane);
        wait_vmcnt<0>();
        __syncthreads();
        if (active)
            compute_chunk<kMT, kKB>(p, m0, n0, lane, s_act, s_as, wf, bs);
    }
}

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// ---------------------------------------------------------------------------
// Decode variant (M <= 64, K/128 = kKB known at compile time).
//
// A block of 8 waves covers `subtiles_per_block` 16-row weight subtiles (one
// per wave; the spare waves only help stage).  Phases:
//  1. every thread loads its share of the activation tile (M x K bytes) into
//     registers; then each weight wave starts its ring: the first kRing
//     K-blocks of its subtile (32 bytes of one weight row per lane and
//     K-block);
//  2. the activation tile is written to LDS in fragment order (the compiler
//     waits only for the activation loads: the ring loads were issued after
//     them and loads complete in order), LDS writes are drained and the
//     block meets at a plain s_barrier (no release fence, which would drain
//     the ring too);
//  3. K-block by K-block: MFMAs on the ring slot, scale FMAs, and the slot is
//     refilled with K-block kb + kRing, so each wave computes while its later
//     weight bytes are still arriving;
//  4. the block's output tile goes through LDS and is written as contiguous
//     row segments (2 * 16 * subtiles_per_block bytes per row) instead of
//     32-byte pieces from every wave.
// ---------------------------------------------------------------------------
constexpr int kDecodeWaves = 8;
constexpr int kRing = 6;  // weight K-blocks in flight per wave

template <int kMT, int kKB>
__global__ __launch_bounds__(kDecodeWaves * kWave) void block_scaled_fp8_gemm_decode_kernel(
    GemmParams p, int subtiles_per_block) {
    extern __shared__ uint4 s_dyn[];
    uint4 *s_act = s_dyn;                                                   // [kb][mt][half][lane]
    float *s_as = reinterpret_cast<float *>(s_dyn + kKB * kMT * 2 * kWave);  // [16 kb][64 rows]
    uint16_t *s_out = reinterpret_cast<uint16_t *>(s_as + 2 * kDecodeWaves * kWave);  // [64 rows][cols of block]

    constexpr int kRows = kMT * 16;
    constexpr int kGranules = kRows * kKB * 8;                 // 16-byte pieces of the tile
    constexpr int kPerThread = kGranules / (kDecodeWaves * kWave);
    static_assert(kGranules % (kDecodeWaves * kWave) == 0, "tile must split evenly over the block");
    constexpr int kRingN = kRing < kKB ? kRing : kKB;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar addressing
    const int spb = subtiles_per_block;
    const int64_t M = p.M, K = p.K;
    const int64_t S = p.N / 16;
    const int64_t st = static_cast<int64_t>(blockIdx.x) * spb + wave;
    const bool active = wave < spb && st < S;
    const int64_t n0 = st * 16;

    // The prologue is straight-line code (every load unconditional, indices
    // clamped into range) so that the compiler's wait counts stay exact: a
    // branch around loads makes it drain all outstanding loads where the
    // paths meet.
    // -- 1. activation tile into registers (coalesced: consecutive threads,
    //       consecutive 16-byte pieces of a row; rows at or beyond M repeat
    //       row M-1, they only feed output columns that are never stored),
    //       activation scales, then the weight ring --------------------------
    // (a native vector type: a copy of the HIP uint4 struct from global
    // memory would be kept in scratch)
    v4u32 stage[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int g = threadIdx.x + i * kDecodeWaves * kWave;
        const int64_t r = min<int64_t>(g / (kKB * 8), M - 1);
        const int c = g % (kKB * 8);
        stage[i] = *reinterpret_cast<const v4u32 *>(p.a + r * K + c * 16);
    }
    // wave w stages the scales of K-blocks w and w + 8 (slots past kKB are
    // never read), lane = row
    const int kb0 = wave, kb1 = wave + kDecodeWaves;
    const int64_t ar = min<int64_t>(lane, M - 1);
    const int kb0c = min(kb0, kKB - 1), kb1c = min(kb1, kKB - 1);
    const float *as0p = p.a_scale_transposed ? p.a_scale + static_cast<int64_t>(kb0c) * M + ar : p.a_scale + ar * kKB + kb0c;
    const float *as1p = p.a_scale_transposed ? p.a_scale + static_cast<int64_t>(kb1c) * M + ar : p.a_scale + ar * kKB + kb1c;
    const float as0 = *as0p, as1 = *as1p;
    __builtin_amdgcn_sched_barrier(0);  // ring loads stay behind the staging loads

    // spare waves read their block's last subtile (L2 hits, never used)
    const int64_t st_ld = min<int64_t>(st, min<int64_t>(static_cast<int64_t>(blockIdx.x) * spb + spb, S) - 1);
    const uint8_t *wrow = p.w + (st_ld * 16 + (lane & 15)) * K + 32 * (lane >> 4);
    v8i wf[kRingN];
    float bs[kKB];
#pragma unroll
    for (int kb = 0; kb < kRingN; ++kb) {
        const uint4 *src = reinterpret_cast<const uint4 *>(wrow + kb * kBlk);
        wf[kb] = join(src[0], src[1]);
    }
    const float *bs_row = p.w_scale + (st_ld * 16 / kBlk) * kKB;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
        bs[kb] = bs_row[kb];
    __builtin_amdgcn_sched_barrier(0);  // LDS writes stay behind the ring loads

    // -- 2. activation tile to LDS; drain LDS writes; plain barrier -----------
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int g = threadIdx.x + i * kDecodeWaves * kWave;
        const int r = g / (kKB * 8), c = g % (kKB * 8);
        const int kb = c >> 3, j = c & 7;
        reinterpret_cast<v4u32 *>(s_act)[((kb * kMT + (r >> 4)) * 2 + (j & 1)) * kWave + (j >> 1) * 16 + (r & 15)] =
            stage[i];
    }
    s_as[kb0 * kWave + lane] = as0;
    s_as[kb1 * kWave + lane] = as1;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();

    // -- 3. K-block loop (weight waves only; every wave reaches both barriers)
    const int cols = 16 * spb;  // this block's output columns
    if (active) {
    v4f acc[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t)
        acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    uint4 lo[kMT], hi[kMT];
    float as_m[kMT];
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
        lo[t] = s_act[(t * 2 + 0) * kWave + lane];
        hi[t] = s_act[(t * 2 + 1) * kWave + lane];
        as_m[t] = s_as[t * 16 + (lane & 15)];
    }
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
        v4f part[kMT];
        float sc[kMT];
#pragma unroll
        for (int t = 0; t < kMT; ++t) {
            part[t] = mfma_e4m3_16x16x128(wf[kb % kRingN], join(lo[t], hi[t]));
            sc[t] = as_m[t] * bs[kb];
        }
        if (kb + 1 < kKB) {
#pragma unroll
            for (int t = 0; t < kMT; ++t) {
                lo[t] = s_act[(((kb + 1) * kMT + t) * 2 + 0) * kWave + lane];
                hi[t] = s_act[(((kb + 1) * kMT + t) * 2 + 1) * kWave + lane];
                as_m[t] = s_as[(kb + 1) * kWave + t * 16 + (lane & 15)];
            }
        }
        // refill the slot just consumed with K-block kb + kRing
        if (kb + kRingN < kKB) {
            const uint4 *src = reinterpret_cast<const uint4 *>(wrow + (kb + kRingN) * kBlk);
            wf[kb % kRingN] = join(src[0], src[1]);
        }
#pragma unroll
        for (int t = 0; t < kMT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][i] = fmaf(part[t][i], sc[t], acc[t][i]);
            // see compute_chunk: keeps the FMAs of K-block kb ahead of the
            // MFMAs of K-block kb + 1
            asm volatile("" : "+v"(acc[t]), "+v"(lo[t].x), "+v"(lo[t].y), "+v"(lo[t].z), "+v"(lo[t].w),
                         "+v"(hi[t].x), "+v"(hi[t].y), "+v"(hi[t].z), "+v"(hi[t].w), "+v"(as_m[t]));
        }
    }

    // -- 4. output tile through LDS, contiguous row segments ----------------------
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
        const int m = t * 16 + (lane & 15);
        *reinterpret_cast<uint2 *>(s_out + m * cols + wave * 16 + 4 * (lane >> 4)) =
            make_uint2(pack2_bf16(acc[t][0], acc[t][1]), pack2_bf16(acc[t][2], acc[t][3]));
    }
    }  // active
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();        // every weight wave's tile is in LDS
    const int64_t blk_n0 = static_cast<int64_t>(blockIdx.x) * spb * 16;
    const int pieces_per_row = cols / 8;  // 16-byte pieces
    // only columns of existing subtiles (< N) are read back; those were written
    for (int pi = threadIdx.x; pi < M * pieces_per_row; pi += blockDim.x) {
        const int m = pi / pieces_per_row, part = pi % pieces_per_row;
        if (blk_n0 + part * 8 < p.N)
            *reinterpret_cast<uint4 *>(p.out + m * p.N + blk_n0 + part * 8) =
                *reinterpret_cast<const uint4 *>(s_out + m * cols + part * 8);
    }
}

template <int kMT, int kKB>
hipError_t launch_decode(const GemmParams &p, hipStream_t stream) {
    const int64_t S = p.N / 16;
    const int64_t cus = device_cu_count();
    const int spb = static_cast<int>(std::min<int64_t>(kDecodeWaves, (S + cus - 1) / cus));
    const int64_t blocks = (S + spb - 1) / spb;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const size_t lds = static_cast<size_t>(kKB) * kMT * 2 * kWave * sizeof(uint4) +
                       static_cast<size_t>(2 * kDecodeWaves) * kWave * sizeof(float) +
                       static_cast<size_t>(kChunkRows) * 16 * kDecodeWaves * sizeof(uint16_t);
    auto kern = block_scaled_fp8_gemm_decode_kernel<kMT, kKB>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kDecodeWaves * kWave), lds, stream, p, spb);
    return hipGetLastError();
}

template <int kKB>
hipError_t launch_decode_kb(const GemmParams &p, hipStream_t stream) {
    if (p.M <= 16)
        return launch_decode<1, kKB>(p, stream);
    if (p.M <= 32)
        return launch_decode<2, kKB>(p, stream);
    if (p.M <= 48)
        return launch_decode<3, kKB>(p, stream);
    return launch_decode<4, kKB>(p, stream);
}

template <int kMT, int kKB>
hipError_t launch_stream(const GemmParams &p, hipStream_t stream) {
    // one subtile per wave, at most 8 waves per block, at least one block per CU
    const int64_t S = p.N / 16;
    const int64_t cus = device_cu_count();
    int spb = static_cast<int>(std::min<int64_t>(kStreamMaxWaves, (S + cus - 1) / cus));
    const int64_t blocks = (S + spb - 1) / spb;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const int waves = std::max(4, spb);  // spare waves only help stage the activations
    const size_t lds = static_cast<size_t>(kKB) * kMT * 2 * kWave * sizeof(uint4) +
                       static_cast<size_t>(kKB) * kWave * sizeof(float);
    auto kern = block_scaled_fp8_gemm_stream_kernel<kMT, kKB>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(waves * kWave), lds, stream, p, spb);
    return hipGetLastError();
}

template <int kKB>
hipError_t launch_stream_kb(const GemmParams &p, hipStream_t stream) {
    // m-tiles per 64-row chunk: only the M <= 48 cases stage less than 4
    if (p.M <= 16)
        return launch_stream<1, kKB>(p, stream);
    if (p.M <= 32)
        return launch_stream<2, kKB>(p, stream);
    if (p.M <= 48)
        return launch_stream<3, kKB>(p, stream);
    return launch_stream<4, kKB>(p, stream);
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
    // Decode batches: weight ring per wave, activations resident in LDS.
    if (p.M <= kChunkRows) {
        switch (p.K / kBlk) {
        case 4:
            return launch_decode_kb<4>(p, stream);
        case 8:
            return launch_decode_kb<8>(p, stream);
        case 12:
            return launch_decode_kb<12>(p, stream);
        case 16:
            return launch_decode_kb<16>(p, stream);
        default:
            break;
        }
    }
    // Up to 256 rows: stream the weights once, activations through LDS.
    if (p.M <= 4 * kChunkRows) {
        switch (p.K / kBlk) {
        case 4:
            return launch_stream_kb<4>(p, stream);
        case 8:
            return launch_stream_kb<8>(p, stream);
        case 12:
            return launch_stream_kb<12>(p, stream);
        case 16:
            return launch_stream_kb<16>(p, stream);
        default:
            break;
        }
    }
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
