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
// Mapping onto CDNA4, common to every kernel here:
//  - v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3): one instruction covers one
//    whole 128-deep K-block of a 16 (n) x 16 (m) output tile, so the block's
//    partial sum leaves the matrix core once per K-block and is folded into
//    the fp32 accumulator with As[m, kb] * Bs[nb, kb] (one FMA per value);
//  - the weight is the MFMA "A" operand (rows = n), the activation the "B"
//    operand (columns = m); every weight byte is read from HBM once;
//  - each lane holds outputs (n = 4*(lane/16) + i, m = lane % 16), i < 4.
// The K order inside one MFMA is irrelevant to the result as long as both
// operands use the same one; both are loaded with the same lane/byte -> k
// assignment, so every kernel gives the same bits.
//
// At decode and small-batch sizes the GEMM streams the weight from HBM
// (M <= 256: at most ~380 flop per weight byte); the kernels differ in how
// they keep that stream going:
//  - decode (M <= 32 over weights of more than 4 subtiles per CU): 8 waves
//    per block, each streams its own 16-row weight subtile through a ring of
//    registers while the activation tile sits in LDS;
//  - wide (M <= 256, and both consumers of one activation in one launch):
//    a slab of weight subtiles per block, all M rows, weights / activations
//    / scales streamed through LDS rings by direct global -> LDS loads;
//  - v0 (any other shape): 64-row weight tiles, activations staged through
//    LDS 4 K-blocks at a time, blocks renumbered so the M-tiles of one N-tile
//    share the weight tile through one XCD's L2.
#include <algorithm>
#include <atomic>
#include <vector>

#include "device.h"
#include "launch.h"
#include "normquant_row.h"

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

// Weight fragment of lane L: row L % 16 of a 16-row subtile, chunks 2q and
// 2q + 1 (q = L / 16) of each K-block, as two 16-byte halves.
//  row-major: at row * K + 32 q (halves adjacent), K-blocks 128 bytes apart;
//  tiled: the subtile's K-block tiles are 2 KB apart and hold the fragments
//  in lane order, half h of lane L at h * 1024 + 16 L: each half of a wave's
//  load is 1 KB of contiguous bytes.
struct WeightFrag {
    int64_t lane_off;  // from the subtile's first byte
    int64_t kstride;   // between K-blocks
    int64_t hstride;   // between the two halves
};

__device__ __forceinline__ WeightFrag weight_frag(int lane, int64_t K, int tiled) {
    if (!tiled)
        return {(lane & 15) * K + 32 * (lane >> 4), kBlk, 16};
    return {16 * lane, 16 * kBlk, 1024};
}

__device__ __forceinline__ v8i load_weight_frag(const uint8_t *p, int64_t hstride) {
    return join(*reinterpret_cast<const uint4 *>(p), *reinterpret_cast<const uint4 *>(p + hstride));
}

// e8m0 exponent byte -> its value 2^(e - 127) as fp32 (exact; e = 0 is the
// subnormal 2^-127, e = 255 NaN)
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return e == 0 ? __uint_as_float(0x00400000u) : e == 255 ? __uint_as_float(0x7FC00000u) : __uint_as_float(e << 23);
}

// Block-scaled MFMA with e8m0 scales: acc + sum_k (2^(sa-127) a_k) (2^(sb-127) b_k)
// over one 128-deep K-block, sa / sb in the low byte of each lane's scale
// word (A: the weight, one scale per 16-row subtile and K-block; B: the
// activation, one per row and K-block).
__device__ __forceinline__ v4f mfma_e4m3_16x16x128_scaled(const v8i &a, const v8i &b, const v4f &acc, uint32_t sa,
                                                          uint32_t sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, static_cast<int>(sa), 0,
                                                           static_cast<int>(sb));
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

    const WeightFrag wfrag = weight_frag(lane, K, p.w_tiled);
    const uint8_t *wrow = p.w + n0 * K + wfrag.lane_off;
    const float *bs_row = p.w_scale + (n0 / kBlk) * KB;
    const uint8_t *bs8_row = p.w_scale8 + (n0 / kBlk) * KB;

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
            if (j < kc)
                wf[j] = load_weight_frag(wrow + (kb0 + j) * wfrag.kstride, wfrag.hstride);
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
            if (m < M) {
                const int64_t at = p.a_scale_transposed ? static_cast<int64_t>(kb0 + kb) * M + m : m * KB + kb0 + kb;
                s = p.scale_e8m0 ? e8m0_to_f32(p.a_scale8[at]) : p.a_scale[at];
            }
            s_as[kb][r] = s;
        }
        __syncthreads();

#pragma unroll
        for (int j = 0; j < kStageKb; ++j) {
            if (j >= kc)
                break;
            const float bs = p.scale_e8m0 ? e8m0_to_f32(bs8_row[kb0 + j]) : bs_row[kb0 + j];
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

constexpr int kChunkRows = 64;      // activation rows the decode kernel can hold
constexpr int kDecodeMaxRows = 32;  // batches it is used for (measured crossover)

// Direct global -> LDS load of kBytes per lane (LDS address: the
// wave-uniform base plus lane * kBytes).  The builtin takes its size only as
// a literal constant, and is compiled for the device only: in a template the
// compiler's host pass takes it for a substitution failure and silently
// drops the launch stub of any kernel that reaches it.
// A 1-byte load writes its byte zero-extended to a dword per lane (LDS
// address: base + lane * 4).
template <int kBytes, int kCpol = 0>
__device__ __forceinline__ void load_to_lds(const void *src, void *dst) {
    static_assert(kBytes == 16 || kBytes == 4 || kBytes == 1, "supported loads");
    static_assert(kCpol == 0 || (kBytes == 16 && kCpol == 2), "cache policy: default, or non-temporal 16-byte loads");
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (kBytes == 16 && kCpol == 2)
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);
    else if constexpr (kBytes == 16)
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    else if constexpr (kBytes == 4)
        __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
    else
        __builtin_amdgcn_global_load_lds(src, dst, 1, 0, 0);
#endif
}

// vmcnt-only waits (gfx9 encoding: vmcnt[3:0] + vmcnt[5:4] at bits 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima = no wait)
template <int kVm>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(kVm >= 0 && kVm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// Wide variant (M <= 256, K/128 = kKB known at compile time).
//
// A block of kWaves waves (4: one per SIMD) owns a slab of kNS 16-row weight
// subtiles, of one weight or straddling the two weights of a pair launch,
// and all M activation rows; wave w computes rows [16 kMT w, 16 kMT (w + 1))
// against the whole slab.
// Weights, activations and scales reach LDS through direct global -> LDS
// loads (no registers held for them), each in a ring of K-block stages:
//  - weight stage kb (kNS x 2 KB, shared by all waves, which split its 1 KB
//    slots between them),
//  - activation stage kb (each wave loads its own kMT 16-row tiles),
//  - scales of stage kb (per wave: one As per row, one Bs per subtile).
// The weight ring is deeper than the activation ring: weights come from
// HBM, activations are read by every block and sit in L2.
// Per K-block kb: wait until this wave's loads of stage kb + 1 have landed
// (exact vmcnt count, worked out at compile time from the issue order),
// drain LDS reads, one plain s_barrier (all waves' parts of stage kb + 1 are
// in LDS and every wave has stage kb in registers), then the MFMAs of stage
// kb with the refill of stage kb's slots and the reads of stage kb + 1 into
// the second register set spread between them, one direct load and one
// read step after each MFMA.  The scale FMAs of an MFMA are issued two
// MFMAs later.  With one wave per SIMD a K-block is bound by that wave's
// issue of loads, LDS reads and fold FMAs, which run beside its MFMAs only
// when interleaved with them (measured per K-block at M = 256: 1800 cycles
// with the loads and reads issued as a group before the MFMAs, 1300-1500
// interleaved; the MFMAs alone take 768).
// ---------------------------------------------------------------------------
constexpr int kWideWaves = 4;  // 1 per SIMD

constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// 16-row weight subtile st of the (one or two) consumers: the subtiles of
// p.w come first, then those of p.w2.  All fields uniform when st is.
struct SubTile {
    const uint8_t *w;   // first weight row of the subtile
    const float *ws;    // its row of 128x128 block scales
    const uint8_t *ws8;  // the same row of e8m0 block scales
    uint16_t *out;      // output of its consumer
    int64_t n0;         // its first output column
    int64_t ldo;        // row stride of that output
};

__device__ __forceinline__ SubTile subtile(const GemmParams &p, int64_t st) {
    const int64_t S1 = p.N / 16, KB = p.K / kBlk;
    if (st < S1)
        return {p.w + st * 16 * p.K, p.w_scale + (st * 16 / kBlk) * KB, p.w_scale8 + (st * 16 / kBlk) * KB, p.out,
                st * 16, p.N};
    const int64_t l = st - S1;
    return {p.w2 + l * 16 * p.K, p.w_scale2 + (l * 16 / kBlk) * KB, p.w_scale8_2 + (l * 16 / kBlk) * KB, p.out2,
            l * 16, p.N2};
}

// kE8m0: e8m0 scales, applied by the matrix core (no scale stages in LDS).
template <int kKB, int kNS, int kMT, int kWaves, bool kE8m0 = false>
struct WidePlan {
    static_assert(kNS >= 1 && (kNS <= 3 || kNS % 2 == 0) && kNS <= (kMT == 1 ? 8 : 6),
                  "1-3 subtiles or whole pairs of them; two fragment sets fit the registers");
    static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves");
    static_assert(kMT >= 1 && kMT * kWaves * 16 <= 256, "at most 256 rows");
    static constexpr int kSlot = 1024;                         // 8 rows x 128 bytes
    static constexpr int kWStage = kNS * 2 * kSlot;            // weight bytes per K-block
    static constexpr int kAStage = kWaves * kMT * 2 * kSlot;   // activation bytes per K-block
    // per wave: As (a dword per lane; e8m0: its byte, zero-extended) and,
    // with fp32 scales, Bs
    static constexpr int kSStage = kWaves * (kE8m0 ? 1 : 2) * kWave * 4;
    // Blocks of one 64-row chunk over one to four subtiles (narrow weights:
    // tensor-parallel shards) have 1-4 MFMAs per wave and K-block, so their
    // K loop is paced by the L2 round trip of each activation stage: give
    // them 5 activation stages (74 KB with 6 weight stages at two subtiles,
    // still two blocks per CU; 98 KB at four, chosen only where the grid has
    // a block per CU; measured: TP-8 W_b at M = 256 5.17 -> 4.70 us, TP-4
    // pair at M = 64 5.97 -> 5.48 us, TP-2 pair at M = 32 8.01 -> 6.88 us),
    // the rest 3.
    static constexpr bool kShallowWork = kNS <= 4 && kMT == 1 && kWaves == 4;
    static constexpr int kRA = cmin(kKB, kShallowWork ? 5 : 3);  // activation stages
    // weight stages: as many as the rest of the 160 KB allows, up to 6
    static constexpr int kRW = cmin(kKB, cmin(6, (160 * 1024 - kRA * (kAStage + kSStage)) / kWStage));
    // weight loads per wave per stage; when 2 kNS slots do not split evenly,
    // the extra loads repeat a slot of the same row half (same bytes to the
    // same place: harmless, and every wave then counts the same loads)
    static constexpr int kNW = (2 * kNS + kWaves - 1) / kWaves;
    static constexpr int kNA = 2 * kMT + (kE8m0 ? 1 : 2);      // activation, As and (fp32) Bs loads
    static constexpr int kWOff = 0;
    static constexpr int kAOff = kWOff + kRW * kWStage;
    static constexpr int kSOff = kAOff + kRA * kAStage;
    static constexpr int kLds = kSOff + kRA * kSStage;
    static_assert(kRW >= 2 && kRA >= 2, "a stage is waited for one iteration after it is issued");
    static_assert(kLds <= 160 * 1024, "LDS per CU");

    // Loads a wave has issued after the last load of stage s, at the point
    // where stage s is waited for: after the prologue for s = 0, else in
    // iteration s - 1 before its refill.  Issue order: prologue
    // s = 0, 1, ...: activations(s) if s < kRA, then weights(s) if s < kRW;
    // iteration it, after its barrier: activations(it + kRA), then
    // weights(it + kRW).  Loads complete in order, so a wait for stage s
    // also waits for everything issued before its last load: activations go
    // first so that this never includes a weight stage beyond s (kRW <= kRA + 1)
    // or, with a deeper weight ring, only the weights issued alongside.
    static constexpr int vm_wait(int st) {
        int issued = 0, last_w = -1, last_a = -1;
        for (int s = 0; s < cmax(kRW, kRA); ++s) {
            if (s < kRA && s < kKB) {
                issued += kNA;
                if (s == st) last_a = issued;
            }
            if (s < kRW && s < kKB) {
                issued += kNW;
                if (s == st) last_w = issued;
            }
        }
        for (int it = 0; it + 1 < st; ++it) {
            const int sw = it + kRW, sa = it + kRA;
            if (sa < kKB) {
                issued += kNA;
                if (sa == st) last_a = issued;
            }
            if (sw < kKB) {
                issued += kNW;
                if (sw == st) last_w = issued;
            }
        }
        return issued - cmax(last_w, last_a);
    }
};

__device__ __forceinline__ v8i join4(const v4u32 &lo, const v4u32 &hi) {
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Per-wave state of the wide kernel: load sources, accumulators and the
// MFMA -> FMA pipeline.
template <int kKB, int kNS, int kMT, int kWaves, bool kE8m0>
struct WideWave {
    using P = WidePlan<kKB, kNS, kMT, kWaves, kE8m0>;
    static constexpr int kLag = 2;                // FMAs of MFMA n are issued after MFMA n + kLag
    static constexpr int kRing = kLag + 2;        // partial results in flight
    static constexpr int kSeq = kKB * kNS * kMT;  // MFMAs per wave

    uint8_t *lds;
    int lane, wave;
    const uint8_t *wbase[P::kNW];  // uniform: weight slot sources
    int wslot[P::kNW];             // uniform: their LDS slots
    uint32_t w_off;                // per lane
    uint32_t w_kstride;            // uniform: bytes between K-blocks of a subtile
    const uint8_t *a;
    uint32_t a_off[kMT][2];        // per lane: m-tile j, row half g
    uint32_t frag_lo, frag_hi;     // per lane: LDS offsets of its fragment halves inside a 2 KB tile
    uint32_t wfrag_lo, wfrag_hi;   // the same for weight tiles (tiled weights: lane order)
    static constexpr int kSBytes = kE8m0 ? 1 : 4;  // bytes per As element
    const uint8_t *a_scale;
    int64_t s_stride;  // As bytes between K-blocks
    uint32_t s_off;
    const float *bsrc;  // per lane: block-scale row of subtile lane (lanes >= kNS repeat the last)

    v4f acc[kMT][kNS];
    v4f part[kRing];   // MFMA n -> part[n % kRing]
    float scl[kRing];  // its As * Bs
    // e8m0: weight scale bytes of every K-block, 4 per word, of subtile t
    // (uniform, loaded once)
    uint32_t bsw[kNS][(kKB + 3) / 4];

    __device__ __forceinline__ void issue_w(int s) {
        uint8_t *dst = lds + P::kWOff + (s % P::kRW) * P::kWStage;
#pragma unroll
        for (int i = 0; i < P::kNW; ++i)
            load_to_lds<16, 2>(wbase[i] + s * w_kstride + w_off, dst + wslot[i] * P::kSlot);
    }

    __device__ __forceinline__ void issue_a(int s) {
        uint8_t *dst = lds + P::kAOff + (s % P::kRA) * P::kAStage + wave * kMT * 2 * P::kSlot;
        const uint8_t *src = a + s * kBlk;
#pragma unroll
        for (int j = 0; j < kMT; ++j) {
            load_to_lds<16>(src + a_off[j][0], dst + (2 * j) * P::kSlot);
            load_to_lds<16>(src + a_off[j][1], dst + (2 * j + 1) * P::kSlot);
        }
        uint8_t *sdst = lds + P::kSOff + (s % P::kRA) * P::kSStage + wave * (kE8m0 ? 1 : 2) * kWave * 4;
        const uint8_t *ssrc = a_scale + s * s_stride;
        if constexpr (kE8m0) {
            load_to_lds<1>(ssrc + s_off, sdst);
        } else {
            load_to_lds<4>(ssrc + s_off, sdst);
            load_to_lds<4>(bsrc + s, sdst + kWave * 4);
        }
    }

    // One direct load of iteration kb's refill: the i-th of the order in
    // which issue_a (stage kb + kRA) and then issue_w (stage kb + kRW) issue
    // them, so the wait counts, which depend only on that order, still hold.
    template <int kb, int i>
    __device__ __forceinline__ void load_step() {
        constexpr int sa = kb + P::kRA, sw = kb + P::kRW;
        constexpr int na = sa < kKB ? P::kNA : 0;
        constexpr int nw = sw < kKB ? P::kNW : 0;
        if constexpr (i < na) {
            if constexpr (i < 2 * kMT) {
                uint8_t *dst = lds + P::kAOff + (sa % P::kRA) * P::kAStage + wave * kMT * 2 * P::kSlot;
                load_to_lds<16>(a + sa * kBlk + a_off[i / 2][i % 2], dst + i * P::kSlot);
            } else {
                uint8_t *sdst = lds + P::kSOff + (sa % P::kRA) * P::kSStage + wave * (kE8m0 ? 1 : 2) * kWave * 4;
                const uint8_t *ssrc = a_scale + sa * s_stride;
                if constexpr (kE8m0)
                    load_to_lds<1>(ssrc + s_off, sdst);
                else if constexpr (i == 2 * kMT)
                    load_to_lds<4>(ssrc + s_off, sdst);
                else
                    load_to_lds<4>(bsrc + sa, sdst + kWave * 4);
            }
        } else if constexpr (i < na + nw) {
            constexpr int k = i - na;
            uint8_t *dst = lds + P::kWOff + (sw % P::kRW) * P::kWStage;
            load_to_lds<16, 2>(wbase[k] + sw * w_kstride + w_off, dst + wslot[k] * P::kSlot);
        }
    }

    // One step of read_frags<st>: step i < kMT reads m-tile i's activation
    // fragment and scale, step kMT + t subtile t's weight fragment and scale.
    template <int st, int i>
    __device__ __forceinline__ void read_step() {
        constexpr int b = st & 1;
        if constexpr (i < kMT) {
            const uint8_t *as = lds + P::kAOff + (st % P::kRA) * P::kAStage + wave * kMT * 2 * P::kSlot;
            const float *ss = reinterpret_cast<const float *>(lds + P::kSOff + (st % P::kRA) * P::kSStage) +
                              wave * (kE8m0 ? 1 : 2) * kWave;
            af[b][i] = join4(*reinterpret_cast<const v4u32 *>(as + (2 * i) * P::kSlot + frag_lo),
                             *reinterpret_cast<const v4u32 *>(as + (2 * i) * P::kSlot + frag_hi));
            if constexpr (kE8m0)
                asb[b][i] = reinterpret_cast<const uint32_t *>(ss)[16 * i + (lane & 15)];
            else
                asv[b][i] = ss[16 * i + (lane & 15)];
        } else if constexpr (i < kMT + kNS) {
            constexpr int t = i - kMT;
            const uint8_t *ws = lds + P::kWOff + (st % P::kRW) * P::kWStage;
            wfs[b][t] = join4(*reinterpret_cast<const v4u32 *>(ws + (2 * t) * P::kSlot + wfrag_lo),
                              *reinterpret_cast<const v4u32 *>(ws + (2 * t) * P::kSlot + wfrag_hi));
            if constexpr (!kE8m0) {
                const float *ss = reinterpret_cast<const float *>(lds + P::kSOff + (st % P::kRA) * P::kSStage) +
                                  wave * 2 * kWave;
                bss[b][t] = ss[kWave + t];  // same address in every lane: broadcast read
            }
        }
    }

    // The work issued after MFMA n of K-block kb: loads [n kLPer, (n + 1) kLPer)
    // of the refill, and the read steps of stage kb + 1 whose slot is n (step
    // i after MFMA i when they fit, else spread evenly over the MFMAs).
    static constexpr int kSlots = kNS * kMT;
    static constexpr int kLoads = P::kNA + P::kNW;
    static constexpr int kLPer = (kLoads + kSlots - 1) / kSlots;
    static constexpr int kReads = kMT + kNS;
    static constexpr int read_slot(int i) { return kReads <= kSlots ? i : (i * kSlots) / kReads; }
    static_assert(kLPer * kSlots >= kLoads && read_slot(kReads - 1) < kSlots, "every load and read has a slot");

    template <int kb, int n, int i = 0>
    __device__ __forceinline__ void loads_at() {
        if constexpr (i < kLoads) {
            if constexpr (i / kLPer == n)
                load_step<kb, i>();
            loads_at<kb, n, i + 1>();
        }
    }
    template <int st, int n, int i = 0>
    __device__ __forceinline__ void reads_at() {
        if constexpr (i < kReads) {
            if constexpr (read_slot(i) == n)
                read_step<st, i>();
            reads_at<st, n, i + 1>();
        }
    }

    // The wait counts assume exactly this issue order (activations, then
    // weights, stage by stage); the scheduling barriers keep the compiler
    // from interleaving the groups.
    __device__ __forceinline__ void prologue() {
#pragma unroll
        for (int s = 0; s < cmax(P::kRW, P::kRA); ++s) {
            if (s < P::kRA && s < kKB)
                issue_a(s);
            __builtin_amdgcn_sched_barrier(0);
            if (s < P::kRW && s < kKB)
                issue_w(s);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // fold MFMA n (sequence order: K-block, subtile, m-tile) into its accumulator
    __device__ __forceinline__ void fold(int n) {
        const int j = n % kMT, t = (n / kMT) % kNS, r = n % kRing;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[j][t][i] = fmaf(part[r][i], scl[r], acc[j][t][i]);
    }

    // Fragments of one stage, in registers.  Two sets: the MFMAs of stage
    // kb read set kb % 2 while the LDS reads of stage kb + 1 fill the other,
    // so LDS latency hides behind a whole K-block of matrix-core work.
    v8i af[2][kMT];
    float asv[2][kMT];
    uint32_t asb[2][kMT];  // e8m0: activation scale bytes of this lane's rows
    v8i wfs[2][kNS];
    float bss[2][kNS];

    // Waits until stage st is in LDS for every wave (this wave's loads have
    // landed, every wave has passed the barrier) -- which also means every
    // wave has finished reading stage st - 1 into registers.
    template <int st>
    __device__ __forceinline__ void arrive() {
        wait_vmcnt<P::vm_wait(st)>();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
        __builtin_amdgcn_s_barrier();
    }

    template <int st>
    __device__ __forceinline__ void read_frags() {
        constexpr int b = st & 1;
        const uint8_t *ws = lds + P::kWOff + (st % P::kRW) * P::kWStage;
        const uint8_t *as = lds + P::kAOff + (st % P::kRA) * P::kAStage + wave * kMT * 2 * P::kSlot;
        const float *ss = reinterpret_cast<const float *>(lds + P::kSOff + (st % P::kRA) * P::kSStage) +
                          wave * (kE8m0 ? 1 : 2) * kWave;
#pragma unroll
        for (int j = 0; j < kMT; ++j) {
            af[b][j] = join4(*reinterpret_cast<const v4u32 *>(as + (2 * j) * P::kSlot + frag_lo),
                             *reinterpret_cast<const v4u32 *>(as + (2 * j) * P::kSlot + frag_hi));
            if constexpr (kE8m0)
                asb[b][j] = reinterpret_cast<const uint32_t *>(ss)[16 * j + (lane & 15)];
            else
                asv[b][j] = ss[16 * j + (lane & 15)];
        }
#pragma unroll
        for (int t = 0; t < kNS; ++t) {
            wfs[b][t] = join4(*reinterpret_cast<const v4u32 *>(ws + (2 * t) * P::kSlot + wfrag_lo),
                              *reinterpret_cast<const v4u32 *>(ws + (2 * t) * P::kSlot + wfrag_hi));
            if constexpr (!kE8m0)
                bss[b][t] = ss[kWave + t];  // same address in every lane: broadcast read
        }
    }

    // MFMA n = (t, j) of K-block kb (and, with fp32 scales, the fold of
    // MFMA n - kLag), then the loads and reads of slot n; the scheduling
    // barrier keeps each slot's work where it is.
    template <int kb, int t, int j>
    __device__ __forceinline__ void mfma_step() {
        constexpr int b = kb & 1;
        constexpr int n = (kb * kNS + t) * kMT + j;
        if constexpr (kE8m0) {
            // the scales ride on the MFMA: accumulate the whole K in place
            constexpr int wd = kb / 4, sh = 8 * (kb % 4);
            acc[j][t] = mfma_e4m3_16x16x128_scaled(wfs[b][t], af[b][j], acc[j][t], (bsw[t][wd] >> sh) & 0xFFu,
                                                   asb[b][j]);
        } else {
            part[n % kRing] = mfma_e4m3_16x16x128(wfs[b][t], af[b][j]);
            scl[n % kRing] = asv[b][j] * bss[b][t];
            if constexpr (n >= kLag) {
                fold(n - kLag);
                // the next MFMA reads af[] after this asm, so it stays
                // behind these FMAs (VALU work in the matrix core's shadow)
                v4f &folded = acc[(n - kLag) % kMT][((n - kLag) / kMT) % kNS];
                asm volatile("" : "+v"(af[b][(j + 1) % kMT]), "+v"(folded));
            }
        }
        if constexpr (kb + 1 < kKB) {
            loads_at<kb, t * kMT + j>();
            reads_at<kb + 1, t * kMT + j>();
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j + 1 < kMT)
            mfma_step<kb, t, j + 1>();
        else if constexpr (t + 1 < kNS)
            mfma_step<kb, t + 1, 0>();
    }

    template <int kb>
    __device__ __forceinline__ void kblock() {
        if constexpr (kb + 1 < kKB)
            arrive<kb + 1>();
        __builtin_amdgcn_sched_barrier(0);
        mfma_step<kb, 0, 0>();
        if constexpr (kb + 1 < kKB)
            kblock<kb + 1>();
    }
};

template <int kKB, int kNS, int kMT, int kWaves, bool kE8m0>
__global__ __launch_bounds__(kWaves * kWave) void block_scaled_fp8_gemm_wide_kernel(GemmParams p) {
    using W = WideWave<kKB, kNS, kMT, kWaves, kE8m0>;
    extern __shared__ uint4 s_dyn[];
    W w;
    w.lds = reinterpret_cast<uint8_t *>(s_dyn);
    w.lane = threadIdx.x & (kWave - 1);
    w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: LDS slot bases
    const int lane = w.lane, wave = w.wave;
    const int64_t M = p.M, K = p.K;
    const int64_t S = (p.N + p.N2) / 16;  // subtiles of both consumers
    // block -> (slab, row chunk): a block covers kWaves x 16 kMT rows; when
    // that is fewer than M, the row chunks of one slab get consecutive ids,
    // renumbered onto one XCD so that they share the slab through its L2
    constexpr int kBlockRows = kWaves * 16 * kMT;
    const int nm = static_cast<int>((M + kBlockRows - 1) / kBlockRows);
    const int b = nm > 1 ? xcd_contiguous_block(blockIdx.x, gridDim.x) : static_cast<int>(blockIdx.x);
    const int64_t st0 = static_cast<int64_t>(b / nm) * kNS;
    const int m_base = (b % nm) * kBlockRows + wave * 16 * kMT;

    // LDS tiles.  A 16-row x 128-byte K-block tile of either operand takes
    // 2 KB: rows 8g..8g+7 fill the 1 KB slot g, row r of the slot at 128 r,
    // and its 16-byte chunk c sits at position c ^ f, f = r ^ g.  One direct
    // load fills one slot: lane l fetches row l / 8, chunk (l % 8) ^ f, so
    // each load reads 8 whole cache lines.  The MFMA fragment of lane L is
    // row L % 16, chunks 2 (L / 16) and 2 (L / 16) + 1 (the same K order for
    // both operands); with the XOR the 8 (or 16) lanes that read LDS together
    // hit distinct banks.
    {
        const int rho = lane & 15, g = rho >> 3, r = rho & 7, q = lane >> 4;
        w.frag_lo = static_cast<uint32_t>(g * 1024 + r * 128 + (((2 * q) ^ (r ^ g)) * 16));
        w.frag_hi = static_cast<uint32_t>(g * 1024 + r * 128 + (((2 * q + 1) ^ (r ^ g)) * 16));
    }
    const int lrow = lane >> 3, lchunk = lane & 7;  // this lane's part of one direct load
    // Sources: a uniform base per load plus a 32-bit per-lane offset.
    // Subtiles past the end of W repeat the last one and rows at or beyond M
    // repeat row M - 1: their results are never stored.
    // Weight slot (subtile, row half) = (slot / 2, slot % 2); this wave loads
    // slots (wave + kWaves i) mod 2 kNS, all of row half wave % 2.
    // A tiled weight holds each (subtile, K-block) tile in lane order: its
    // half g is 1 KB of contiguous bytes, copied to slot g as is, and lane L
    // reads its fragment at 16 L of each slot (conflict-free).
    {
        const int g = wave & 1;
        w.w_off = p.w_tiled ? static_cast<uint32_t>(g * 1024 + lane * 16)
                            : static_cast<uint32_t>((8 * g + lrow) * K + 16 * (lchunk ^ lrow ^ g));
        w.w_kstride = p.w_tiled ? 16 * kBlk : kBlk;
        w.wfrag_lo = p.w_tiled ? static_cast<uint32_t>(16 * lane) : w.frag_lo;
        w.wfrag_hi = p.w_tiled ? static_cast<uint32_t>(1024 + 16 * lane) : w.frag_hi;
    }
#pragma unroll
    for (int i = 0; i < W::P::kNW; ++i) {
        const int slot = (wave + kWaves * i) % (2 * kNS);
        w.wslot[i] = slot;
        w.wbase[i] = subtile(p, min<int64_t>(st0 + (slot >> 1), S - 1)).w;
    }
    w.a = p.a;
#pragma unroll
    for (int j = 0; j < kMT; ++j)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int64_t r = min<int64_t>(m_base + 16 * j + 8 * g + lrow, M - 1);
            w.a_off[j][g] = static_cast<uint32_t>(r * K + 16 * (lchunk ^ lrow ^ g));
        }
    // lane l: As of row m_base + l (rows past this wave's or past M repeat)
    const int64_t srow = min<int64_t>(m_base + min(lane, 16 * kMT - 1), M - 1);
    w.a_scale = kE8m0 ? p.a_scale8 : reinterpret_cast<const uint8_t *>(p.a_scale);
    w.s_off = static_cast<uint32_t>(W::kSBytes * (p.a_scale_transposed ? srow : srow * kKB));
    w.s_stride = W::kSBytes * (p.a_scale_transposed ? M : 1);
    // lane t < kNS: the 128x128 block-scale row of subtile t (other lanes
    // repeat the last subtile)
    w.bsrc = subtile(p, min<int64_t>(st0 + min(lane, kNS - 1), S - 1)).ws;

    if constexpr (kE8m0) {
        // the weight scale bytes of every K-block (uniform: scalar loads);
        // the activation scale bytes ride in the scale stages
        constexpr int kWords = (kKB + 3) / 4;
#pragma unroll
        for (int t = 0; t < kNS; ++t) {
            const uint32_t *src =
                reinterpret_cast<const uint32_t *>(subtile(p, min<int64_t>(st0 + t, S - 1)).ws8);
#pragma unroll
            for (int i = 0; i < kWords; ++i)
                w.bsw[t][i] = src[i];
        }
    }
    w.prologue();
#pragma unroll
    for (int j = 0; j < kMT; ++j)
#pragma unroll
        for (int t = 0; t < kNS; ++t)
            w.acc[j][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    w.template arrive<0>();
    w.template read_frags<0>();
    w.template kblock<0>();
    if constexpr (!kE8m0) {
#pragma unroll
        for (int n = W::kSeq - W::kLag; n < W::kSeq; ++n)
            w.fold(n);
    }

    // Output: lane holds out[m_base + 16j + L%16][16 (st0 + t) + 4 (L/16) + i].
    // The wave's tile (16 kMT rows x 16 kNS columns, bf16) goes through LDS
    // so that every row leaves as contiguous 16-byte pieces (8-byte pieces
    // scattered over 16 rows per store make partial cache-line writes), with
    // non-temporal stores (measured: cheaper than plain ones here).
    // The rings are free once every wave has passed this barrier.
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    constexpr int kCols = 16 * kNS;
    static_assert(kWaves * 16 * kMT * kCols * 2 <= W::P::kLds, "output tiles fit in the rings' LDS");
    uint16_t *tile = reinterpret_cast<uint16_t *>(w.lds) + wave * (16 * kMT) * kCols;
#pragma unroll
    for (int j = 0; j < kMT; ++j)
#pragma unroll
        for (int t = 0; t < kNS; ++t)
            *reinterpret_cast<uint2 *>(tile + (16 * j + (lane & 15)) * kCols + 16 * t + 4 * (lane >> 4)) =
                make_uint2(pack2_bf16(w.acc[j][t][0], w.acc[j][t][1]), pack2_bf16(w.acc[j][t][2], w.acc[j][t][3]));
    constexpr int kPieces = 2 * kNS;  // 16-byte pieces per row
    constexpr int kTilePieces = 16 * kMT * kPieces;
#pragma unroll
    for (int i = 0; i < (kTilePieces + kWave - 1) / kWave; ++i) {
        const int pc = lane + i * kWave;
        if (kTilePieces % kWave != 0 && pc >= kTilePieces)
            break;
        const int row = pc / kPieces, col = 8 * (pc % kPieces);
        const int64_t m = m_base + row, st = st0 + col / 16;
        const v4u32 v = *reinterpret_cast<const v4u32 *>(tile + row * kCols + col);
        if (m < M && st < S) {  // streaming store: the output is not read back here
            const SubTile sub = subtile(p, st);
            __builtin_nontemporal_store(v, reinterpret_cast<v4u32 *>(sub.out + m * sub.ldo + sub.n0 + col % 16));
        }
    }
}

// ---------------------------------------------------------------------------
// Stream variant (16 kMT <= 64 rows per block, K/128 = kKB known at compile
// time; more rows are split into chunks of 16 kMT, one block per chunk and
// weight slab, the chunks of one slab on one XCD so the slab is fetched into
// its L2 once).
//
// For decode batches the GEMM is a pure weight stream, and what limits it is
// how the stream is fed, not the matrix cores.  Here the waves of a block
// never wait for each other inside the K loop:
//  - the whole activation tile (all M rows, all K-blocks; 96 KB at M = 64,
//    K = 1536) and its scales are loaded into LDS once, behind one barrier
//    (rows in the 1 KB slot image of the wide kernel);
//  - each wave owns kSW 16-row weight subtiles for all M rows, and streams
//    them through a ring of its own in LDS (kD K-blocks deep) by direct
//    global -> LDS loads, waiting only for its own loads (exact vmcnt
//    counts);
//  - per K-block a wave reads its kSW weight and kMT activation fragments
//    (the next K-block's during this one's matrix-core work), so each
//    weight fragment is read from LDS once.
// (Measured against the same kernel with the weight ring in registers: the
// LDS ring was faster at every batch size.)
// ---------------------------------------------------------------------------
template <int kKB, int kMT, int kSW, int kWaves, int kD, bool kE8m0>
struct StreamPlan {
    static constexpr int kSlot = 1024;
    static constexpr int kASlots = kKB * kMT * 2;                        // activation slots, all K
    static constexpr int kNA = (kASlots + kWaves - 1) / kWaves;          // per wave (spares repeat a slot)
    static constexpr int kNS = (kKB + kWaves - 1) / kWaves;              // As loads per wave (one per K-block)
    static constexpr int kNW = 2 * kSW;                                  // weight loads per wave per K-block
    static constexpr int kDD = kD < kKB ? kD : kKB;                      // ring depth actually used
    static constexpr int kAOff = 0;
    static constexpr int kSOff = kAOff + kASlots * kSlot;
    static constexpr int kWOff = kSOff + kKB * kWave * 4;               // As: a dword per row (e8m0: its byte)
    static constexpr int kWaveRing = kDD * kSW * 2 * kSlot;
    static constexpr int kLds = kWOff + kWaves * kWaveRing;
    static_assert(kLds <= 160 * 1024, "LDS per CU");
    static_assert(kNA + kNS + kDD * kNW <= 63, "outstanding loads per wave fit vmcnt");
    static_assert(16 * kMT * 16 * kSW * 2 <= kWaveRing, "output tile fits the wave's ring");
    // weight loads this wave issued after the last load of stage st, when
    // it waits for st (before the K loop for st = 0, else in iteration
    // st - 1 before that iteration's refill).  Issue order: stage 0,
    // activations and scales, stages 1 .. kDD - 1, then one refill per
    // iteration; stage 0 and the activations are waited for before the
    // barrier, so only weight loads are counted here.
    static constexpr int vm_wait(int st) {
        const int issued = st == 0 ? kDD : (kDD + st - 1 < kKB ? kDD + st - 1 : kKB);
        return (issued - (st + 1)) * kNW;
    }
};

template <int kKB, int kMT, int kSW, int kWaves, int kD, bool kE8m0>
struct StreamWave {
    using P = StreamPlan<kKB, kMT, kSW, kWaves, kD, kE8m0>;
    static constexpr int kLag = 2;
    static constexpr int kRing = kLag + 2;

    uint8_t *lds;
    uint8_t *ring;                 // this wave's weight ring
    int lane;
    const uint8_t *wsrc[kSW];      // uniform: first byte of each owned subtile
    uint32_t w_off[2];             // per lane: its part of the load of slot half g
    uint32_t w_kstride;            // uniform: bytes between K-blocks of a subtile
    uint32_t frag_lo, frag_hi;     // per lane: activation fragment halves in a slot pair
    uint32_t wfrag_lo, wfrag_hi;   // the same for weight slot pairs

    v4f acc[kMT][kSW];
    v4f part[kRing];
    float scl[kRing];
    float bs[kSW][kKB];                  // fp32 weight block scales (uniform)
    uint32_t bsw[kSW][(kKB + 3) / 4];    // e8m0: weight scale bytes (uniform)

    v8i af[2][kMT];
    float asv[2][kMT];
    uint32_t asb[2][kMT];  // e8m0: activation scale bytes of this lane's rows
    v8i wfs[2][kSW];

    __device__ __forceinline__ void issue_w(int s) {
        uint8_t *dst = ring + (s % P::kDD) * kSW * 2 * P::kSlot;
#pragma unroll
        for (int t = 0; t < kSW; ++t)
#pragma unroll
            for (int g = 0; g < 2; ++g)
                load_to_lds<16, 2>(wsrc[t] + s * w_kstride + w_off[g], dst + (2 * t + g) * P::kSlot);
    }

    // activation slots (all K-blocks) and As, split over the waves; slot
    // (kb, j, g) holds rows 16 j + 8 g .. + 7 of K-block kb (rows at or
    // beyond M repeat row M - 1: their results are never stored).
    __device__ __forceinline__ void issue_activations(const GemmParams &p, int wave, int64_t m0) {
        const int lrow = lane >> 3, lchunk = lane & 7;
        const int64_t M = p.M, K = p.K;
#pragma unroll
        for (int i = 0; i < P::kNA; ++i) {
            const int slot = (wave + kWaves * i) % P::kASlots;
            const int kb = slot / (2 * kMT), j = (slot / 2) % kMT, g = slot % 2;
            const int64_t row = min<int64_t>(m0 + 16 * j + 8 * g + lrow, M - 1);
            load_to_lds<16>(p.a + row * K + kb * kBlk + 16 * (lchunk ^ lrow ^ g), lds + P::kAOff + slot * P::kSlot);
        }
        const int64_t row = min<int64_t>(m0 + lane, M - 1);
#pragma unroll
        for (int i = 0; i < P::kNS; ++i) {
            const int kb = (wave + kWaves * i) % kKB;
            const int64_t at = p.a_scale_transposed ? kb * M + row : row * kKB + kb;
            if constexpr (kE8m0)
                load_to_lds<1>(p.a_scale8 + at, lds + P::kSOff + kb * kWave * 4);
            else
                load_to_lds<4>(p.a_scale + at, lds + P::kSOff + kb * kWave * 4);
        }
    }

    __device__ __forceinline__ void fold(int n) {
        const int j = n % kMT, t = (n / kMT) % kSW, r = n % kRing;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[j][t][i] = fmaf(part[r][i], scl[r], acc[j][t][i]);
    }

    template <int st>
    __device__ __forceinline__ void read_frags() {
        constexpr int b = st & 1;
#pragma unroll
        for (int j = 0; j < kMT; ++j) {
            const uint8_t *sl = lds + P::kAOff + (st * kMT + j) * 2 * P::kSlot;
            af[b][j] = join4(*reinterpret_cast<const v4u32 *>(sl + frag_lo),
                             *reinterpret_cast<const v4u32 *>(sl + frag_hi));
            if constexpr (kE8m0)
                asb[b][j] = reinterpret_cast<const uint32_t *>(lds + P::kSOff)[st * kWave + 16 * j + (lane & 15)];
            else
                asv[b][j] = reinterpret_cast<const float *>(lds + P::kSOff)[st * kWave + 16 * j + (lane & 15)];
        }
        const uint8_t *ws = ring + (st % P::kDD) * kSW * 2 * P::kSlot;
#pragma unroll
        for (int t = 0; t < kSW; ++t)
            wfs[b][t] = join4(*reinterpret_cast<const v4u32 *>(ws + 2 * t * P::kSlot + wfrag_lo),
                              *reinterpret_cast<const v4u32 *>(ws + 2 * t * P::kSlot + wfrag_hi));
    }

    template <int kb>
    __device__ __forceinline__ void kblock() {
        if constexpr (kb + 1 < kKB) {
            wait_vmcnt<P::vm_wait(kb + 1)>();     // stage kb + 1 of this wave's ring has landed
            __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's reads of stage kb are done: its slot is free
            if constexpr (kb + P::kDD < kKB)
                issue_w(kb + P::kDD);
            __builtin_amdgcn_sched_barrier(0);
            read_frags<kb + 1>();
        }
        constexpr int b = kb & 1;
        if constexpr (kE8m0) {
            constexpr int wd = kb / 4, sh = 8 * (kb % 4);
#pragma unroll
            for (int t = 0; t < kSW; ++t)
#pragma unroll
                for (int j = 0; j < kMT; ++j)
                    acc[j][t] = mfma_e4m3_16x16x128_scaled(wfs[b][t], af[b][j], acc[j][t], (bsw[t][wd] >> sh) & 0xFFu,
                                                           asb[b][j]);
        } else {
#pragma unroll
            for (int t = 0; t < kSW; ++t) {
#pragma unroll
                for (int j = 0; j < kMT; ++j) {
                    const int n = (kb * kSW + t) * kMT + j;
                    part[n % kRing] = mfma_e4m3_16x16x128(wfs[b][t], af[b][j]);
                    scl[n % kRing] = asv[b][j] * bs[t][kb];
                    if (n >= kLag) {
                        fold(n - kLag);
                        v4f &folded = acc[(n - kLag) % kMT][((n - kLag) / kMT) % kSW];
                        asm volatile("" : "+v"(af[b][(j + 1) % kMT]), "+v"(folded));
                    }
                }
            }
        }
        if constexpr (kb + 1 < kKB)
            kblock<kb + 1>();
    }
    // What issue_w needs for the ring of wave `wave` (owning subtiles st0 ..
    // st0 + kSW - 1): the ring, this lane's offsets, the subtiles' sources.
    // Subtiles past the end repeat the last (never stored).
    __device__ __forceinline__ void setup_ring(const GemmParams &p, int wave, int64_t st0) {
        const int64_t K = p.K;
        const int64_t S = (p.N + p.N2) / 16;
        lane = threadIdx.x & (kWave - 1);
        ring = lds + P::kWOff + wave * P::kWaveRing;
        // weight slot pairs: row-major weights in the activations' image; a
        // tiled weight's halves are copied as they are (lane order)
        const int lrow = lane >> 3, lchunk = lane & 7;
#pragma unroll
        for (int g = 0; g < 2; ++g)
            w_off[g] = p.w_tiled ? static_cast<uint32_t>(g * 1024 + lane * 16)
                                 : static_cast<uint32_t>((8 * g + lrow) * K + 16 * (lchunk ^ lrow ^ g));
        w_kstride = p.w_tiled ? 16 * kBlk : kBlk;
#pragma unroll
        for (int t = 0; t < kSW; ++t)
            wsrc[t] = subtile(p, min<int64_t>(st0 + t, S - 1)).w;
    }

    // Per-lane offsets, the owned subtiles' sources and block scales (scalar
    // loads).  Subtiles past the end repeat the last (never stored).
    __device__ __forceinline__ void setup(const GemmParams &p, int wave, int64_t st0) {
        const int64_t K = p.K;
        const int64_t S = (p.N + p.N2) / 16;
        lane = threadIdx.x & (kWave - 1);
        ring = lds + P::kWOff + wave * P::kWaveRing;
        {
            const int rho = lane & 15, g = rho >> 3, r = rho & 7, q = lane >> 4;
            frag_lo = static_cast<uint32_t>(g * 1024 + r * 128 + (((2 * q) ^ (r ^ g)) * 16));
            frag_hi = static_cast<uint32_t>(g * 1024 + r * 128 + (((2 * q + 1) ^ (r ^ g)) * 16));
        }
        // weight slot pairs: row-major weights in the activations' image; a
        // tiled weight's halves are copied as they are (lane order)
        const int lrow = lane >> 3, lchunk = lane & 7;
#pragma unroll
        for (int g = 0; g < 2; ++g)
            w_off[g] = p.w_tiled ? static_cast<uint32_t>(g * 1024 + lane * 16)
                                 : static_cast<uint32_t>((8 * g + lrow) * K + 16 * (lchunk ^ lrow ^ g));
        w_kstride = p.w_tiled ? 16 * kBlk : kBlk;
        wfrag_lo = p.w_tiled ? static_cast<uint32_t>(16 * lane) : frag_lo;
        wfrag_hi = p.w_tiled ? static_cast<uint32_t>(1024 + 16 * lane) : frag_hi;
#pragma unroll
        for (int t = 0; t < kSW; ++t) {
            const SubTile sub = subtile(p, min<int64_t>(st0 + t, S - 1));
            wsrc[t] = sub.w;
            if constexpr (kE8m0) {
#pragma unroll
                for (int i = 0; i < (kKB + 3) / 4; ++i)
                    bsw[t][i] = reinterpret_cast<const uint32_t *>(sub.ws8)[i];
            } else {
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
                    bs[t][kb] = sub.ws[kb];
            }
        }
    }

    __device__ __forceinline__ void zero_acc() {
#pragma unroll
        for (int j = 0; j < kMT; ++j)
#pragma unroll
            for (int t = 0; t < kSW; ++t)
                acc[j][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // The K loop, entered once every wave's activation loads and this
    // wave's weight stage 0 are in LDS, with at most weight stages
    // 1 .. kDD - 1 of this wave still in flight (vm_wait counts only weight
    // loads issued after the one waited for).
    __device__ __forceinline__ void compute() {
        read_frags<0>();
        kblock<0>();
        if constexpr (!kE8m0) {
#pragma unroll
            for (int n = kKB * kSW * kMT - kLag; n < kKB * kSW * kMT; ++n)
                fold(n);
        }
    }

    // output tile of this wave (16 kMT rows x 16 kSW columns) through its own
    // ring, then 16-byte row pieces
    __device__ __forceinline__ void store_tile(const GemmParams &p, int64_t m0, int64_t st0) {
        const int64_t M = p.M;
        const int64_t S = (p.N + p.N2) / 16;
        wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        constexpr int kCols = 16 * kSW;
        uint16_t *tile = reinterpret_cast<uint16_t *>(ring);
#pragma unroll
        for (int j = 0; j < kMT; ++j)
#pragma unroll
            for (int t = 0; t < kSW; ++t)
                *reinterpret_cast<uint2 *>(tile + (16 * j + (lane & 15)) * kCols + 16 * t + 4 * (lane >> 4)) =
                    make_uint2(pack2_bf16(acc[j][t][0], acc[j][t][1]), pack2_bf16(acc[j][t][2], acc[j][t][3]));
        __builtin_amdgcn_s_waitcnt(0xC07F);
        constexpr int kPieces = 2 * kSW;
        constexpr int kTilePieces = 16 * kMT * kPieces;
#pragma unroll
        for (int i = 0; i < (kTilePieces + kWave - 1) / kWave; ++i) {
            const int pc = lane + i * kWave;
            if (kTilePieces % kWave != 0 && pc >= kTilePieces)
                break;
            const int row = pc / kPieces, col = 8 * (pc % kPieces);
            const int64_t m = m0 + row, st = st0 + col / 16;
            const v4u32 v = *reinterpret_cast<const v4u32 *>(tile + row * kCols + col);
            if (m < M && st < S) {
                // 16-row tiles (decode batches up to 16 rows): plain stores;
                // taller tiles stream their larger output past the caches
                // (measured: plain stores took the M = 1 step 11.2 -> 10.9 us
                // but the M = 64 pair 13.4 -> 14.8 us)
                const SubTile sub = subtile(p, st);
                v4u32 *dst = reinterpret_cast<v4u32 *>(sub.out + m * sub.ldo + sub.n0 + col % 16);
                if constexpr (kMT == 1)
                    *dst = v;
                else
                    __builtin_nontemporal_store(v, dst);
            }
        }
    }
};

template <int kKB, int kMT, int kSW, int kWaves, int kD, bool kE8m0>
__global__ __launch_bounds__(kWaves * kWave) void block_scaled_fp8_gemm_stream_kernel(GemmParams p) {
    using SW = StreamWave<kKB, kMT, kSW, kWaves, kD, kE8m0>;
    using P = typename SW::P;
    extern __shared__ uint4 s_dyn[];
    SW w;
    w.lds = reinterpret_cast<uint8_t *>(s_dyn);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // block -> (weight slab, row chunk); the chunks of a slab get
    // consecutive ids, renumbered onto one XCD
    constexpr int kChunk = 16 * kMT;
    const int nm = static_cast<int>((p.M + kChunk - 1) / kChunk);
    const int b = nm > 1 ? xcd_contiguous_block(blockIdx.x, gridDim.x) : static_cast<int>(blockIdx.x);
    const int64_t m0 = static_cast<int64_t>(b % nm) * kChunk;
    const int64_t st0 = (static_cast<int64_t>(b / nm) * kWaves + wave) * kSW;  // this wave's first subtile
    w.setup(p, wave, st0);
    __builtin_amdgcn_sched_barrier(0);

    // weight stage 0 first (its HBM latency starts at once), then the
    // activation tile and scales (L2), then the rest of the ring
    w.issue_w(0);
    __builtin_amdgcn_sched_barrier(0);
    w.issue_activations(p, wave, m0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 1; s < P::kDD; ++s)
        w.issue_w(s);
    __builtin_amdgcn_sched_barrier(0);
    w.zero_acc();

    // this wave's activation loads and weight stage 0 have landed (only
    // weight stages 1 .. kDD - 1 are younger); then every wave's have
    wait_vmcnt<(P::kDD - 1) * P::kNW>();
    __builtin_amdgcn_s_barrier();
    w.compute();
    w.store_tile(p, m0, st0);
}

// The dynamic-LDS limit is a per-device function attribute.  Every kernel
// instance launched with more than the default registers a function that
// raises it on the current device when the library is loaded (its launcher
// names the instance's DynLds), so that init_dynamic_lds() can raise them all
// before a caller starts capturing launches into a graph; launches also
// raise it lazily, once per device and instance.
using RaiseFn = hipError_t (*)();

std::vector<RaiseFn> &lds_registry() {
    static std::vector<RaiseFn> r;  // filled during the library's static initialisation
    return r;
}

template <auto kKern, int kBytes>
struct DynLds {
    static inline std::atomic<uint64_t> done{0};  // bit d: raised on device d
    static hipError_t raise() {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kKern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                kBytes);
        if (e == hipSuccess && dev >= 0 && dev < 64)
            done.fetch_or(uint64_t{1} << dev, std::memory_order_acq_rel);
        return e;
    }
    static inline const bool registered = (lds_registry().push_back(&raise), true);
    static hipError_t ensure() {
        (void)registered;
        int dev = 0;
        const hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        if (dev >= 0 && dev < 64 && (done.load(std::memory_order_acquire) & (uint64_t{1} << dev)))
            return hipSuccess;
        return raise();
    }
};

int device_cu_count() {
    static std::atomic<int> cached[64] = {};  // per device; calls may come from several host threads
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
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
    const WeightFrag wfrag = weight_frag(lane, K, p.w_tiled);
    const uint8_t *wrow = p.w + st_ld * 16 * K + wfrag.lane_off;
    v8i wf[kRingN];
    float bs[kKB];
#pragma unroll
    for (int kb = 0; kb < kRingN; ++kb)
        wf[kb] = load_weight_frag(wrow + kb * wfrag.kstride, wfrag.hstride);
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
        if (kb + kRingN < kKB)
            wf[kb % kRingN] = load_weight_frag(wrow + (kb + kRingN) * wfrag.kstride, wfrag.hstride);
#pragma unroll
        for (int t = 0; t < kMT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][i] = fmaf(part[t][i], sc[t], acc[t][i]);
            // keeps the FMAs of K-block kb ahead of the
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
        if (blk_n0 + part * 8 < p.N)  // streaming store: the output is not read back here
            __builtin_nontemporal_store(*reinterpret_cast<const v4u32 *>(s_out + m * cols + part * 8),
                                        reinterpret_cast<v4u32 *>(p.out + m * p.N + blk_n0 + part * 8));
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
    constexpr int lds = kKB * kMT * 2 * kWave * static_cast<int>(sizeof(uint4)) +
                        2 * kDecodeWaves * kWave * static_cast<int>(sizeof(float)) +
                        kChunkRows * 16 * kDecodeWaves * static_cast<int>(sizeof(uint16_t));
    constexpr auto kern = block_scaled_fp8_gemm_decode_kernel<kMT, kKB>;
    const hipError_t e = DynLds<kern, lds>::ensure();
    if (e != hipSuccess)
        return e;
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

// ring depth of the stream kernel: as deep as the LDS left after the
// activation tile allows, at most 6 K-blocks
template <int kKB, int kMT, int kSW, int kWaves, bool kE8m0>
constexpr int stream_depth() {
    constexpr int fixed = kKB * kMT * 2 * 1024 + kKB * kWave * 4;
    constexpr int d = (160 * 1024 - fixed) / (kWaves * kSW * 2 * 1024);
    return d < 6 ? d : 6;
}

template <int kKB, int kMT, int kSW, int kWaves, bool kE8m0>
hipError_t launch_stream_scaled(const GemmParams &p, hipStream_t stream) {
    constexpr int kD = stream_depth<kKB, kMT, kSW, kWaves, kE8m0>();
    static_assert(kD >= 2, "at least two ring stages");
    using P = StreamPlan<kKB, kMT, kSW, kWaves, kD, kE8m0>;
    const int64_t per_block = kWaves * kSW;
    const int64_t nm = (p.M + 16 * kMT - 1) / (16 * kMT);
    const int64_t blocks = ((p.N + p.N2) / 16 + per_block - 1) / per_block * nm;
    if (blocks > 0x7FFFFFFF || p.M > 256)
        return hipErrorInvalidValue;
    constexpr auto kern = block_scaled_fp8_gemm_stream_kernel<kKB, kMT, kSW, kWaves, kD, kE8m0>;
    const hipError_t e = DynLds<kern, P::kLds>::ensure();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kWaves * kWave), P::kLds, stream, p);
    return hipGetLastError();
}

template <int kKB, int kMT, int kWaves>
hipError_t launch_stream_w(const GemmParams &p, hipStream_t stream) {
    return p.scale_e8m0 ? launch_stream_scaled<kKB, kMT, 2, kWaves, true>(p, stream)
                        : launch_stream_scaled<kKB, kMT, 2, kWaves, false>(p, stream);
}

template <int kKB>
hipError_t launch_stream_kb(const GemmParams &p, int waves, hipStream_t stream) {
    if (p.M <= 16)
        return waves == 3 ? launch_stream_w<kKB, 1, 3>(p, stream) : launch_stream_w<kKB, 1, 4>(p, stream);
    if (p.M <= 32)
        return waves == 3 ? launch_stream_w<kKB, 2, 3>(p, stream) : launch_stream_w<kKB, 2, 4>(p, stream);
    return waves == 3 ? launch_stream_w<kKB, 4, 3>(p, stream) : launch_stream_w<kKB, 4, 4>(p, stream);
}

// The stream kernel with one 16-row subtile per wave and as many waves per
// block as the CU has subtiles (2 .. 8), for decode batches of up to 16 rows.
template <bool kE8m0>
hipError_t launch_stream_one_per_wave(const GemmParams &p, int waves, hipStream_t stream) {
    switch (waves) {
    case 2:
        return launch_stream_scaled<12, 1, 1, 2, kE8m0>(p, stream);
    case 3:
        return launch_stream_scaled<12, 1, 1, 3, kE8m0>(p, stream);
    case 4:
        return launch_stream_scaled<12, 1, 1, 4, kE8m0>(p, stream);
    case 5:
        return launch_stream_scaled<12, 1, 1, 5, kE8m0>(p, stream);
    case 6:
        return launch_stream_scaled<12, 1, 1, 6, kE8m0>(p, stream);
    case 7:
        return launch_stream_scaled<12, 1, 1, 7, kE8m0>(p, stream);
    default:
        return launch_stream_scaled<12, 1, 1, 8, kE8m0>(p, stream);
    }
}

// The stream kernel, 2 subtiles per wave, where its grid (weight slabs x
// 64-row chunks) covers the CUs: decode batches (M <= 64) over at least 6
// weight subtiles per CU (3 waves per block at 6, else 4), and 64 < M <= 256
// (4 waves) except at three subtiles per CU.  K/128 in {4, 8, 12}.  Returns
// hipErrorNotSupported otherwise.
hipError_t launch_stream(const GemmParams &p, hipStream_t stream) {
    const int64_t S = (p.N + p.N2) / 16, cus = device_cu_count();
    const int64_t per_cu = (S + cus - 1) / cus;
    // Decode batches of up to 16 rows over weights of two to eight 16-row
    // subtiles per CU (4096-32768 weight rows: tensor-parallel shards, W_a,
    // the pair): one subtile per wave, a wave per subtile of the CU, a block
    // per CU.  Measured against the wide kernel (two to five subtiles per
    // CU): the TP4 pair at M = 1 5.4 -> 4.9 us, the TP2 pair 7.5 -> 6.0 us
    // at M = 1 and 7.6 -> 6.4 us at M = 16, TP2 W_a alone 6.7 -> 5.4 us;
    // against two subtiles per wave (six and eight per CU): W_a alone and
    // the pair 2-5 % faster at M = 1 and 16.  At 32 and 64 rows no steady
    // gain; one subtile per CU takes the split-K kernel.
    if (p.M <= 16 && per_cu >= 2 && per_cu <= 8 && p.K / kBlk == 12)
        return p.scale_e8m0 ? launch_stream_one_per_wave<true>(p, static_cast<int>(per_cu), stream)
                            : launch_stream_one_per_wave<false>(p, static_cast<int>(per_cu), stream);
    if (p.M > 256 || (p.M <= 64 && per_cu < 6))
        return hipErrorNotSupported;
    // three subtiles per CU above 64 rows: the wide kernel's six-subtile
    // slabs in two row chunks are faster (TP-2 W_a shard at M = 256 13.6 ->
    // 12.4 us, at M = 128 9.75 -> 8.69 us)
    if (p.M > 64 && per_cu == 3)
        return hipErrorNotSupported;
    if (p.M > 64) {
        // Row chunks re-read their slab's weights (from L2), the wide kernel
        // re-reads every activation row per block: take the stream kernel only
        // where it moves fewer bytes from L2 into LDS, and fills the CUs.
        const int64_t nm = (p.M + 63) / 64, slabs = (S + 7) / 8;
        const int64_t wbytes = S * 16 * p.K;
        const int64_t ns_wide = per_cu <= 2 ? 2 : per_cu <= 4 ? 4 : 6;
        const int64_t wide_bytes = wbytes + (S + ns_wide - 1) / ns_wide * p.M * p.K;
        const int64_t stream_bytes = nm * wbytes + slabs * nm * 64 * p.K;
        if (slabs * nm < cus || stream_bytes >= wide_bytes)
            return hipErrorNotSupported;
    }
    const int waves = p.M <= 64 && per_cu <= 6 ? 3 : 4;
    switch (p.K / kBlk) {
    case 4:
        return launch_stream_kb<4>(p, waves, stream);
    case 8:
        return launch_stream_kb<8>(p, waves, stream);
    case 12:
        return launch_stream_kb<12>(p, waves, stream);
    default:
        return hipErrorNotSupported;
    }
}

// ---------------------------------------------------------------------------
// Decode step in one launch (up to 16 rows of the MLA latent shape: Nq = K =
// 1536, Nkv = 512): the fused dual RMSNorm + 1x128 FP8 group quantisation of
// the rows and both consumer GEMMs of its output.
//
// As two launches, the GEMM's weight stream cannot start before the
// norm-quant kernel has ended, and the norm-quant of a few rows is a memory
// round trip of latency with the chip nearly idle.  Handing the quantised
// rows from the blocks that make them to the blocks that use them inside one
// launch would need a grid-wide barrier, and on this chip every hop of one
// (a device-scope atomic or a poll) is a memory round trip of about a
// microsecond, several of them in a row.  Instead every block of the stream
// kernel quantises all M rows itself, straight into the LDS image the
// stream kernel would have loaded (the rows are L2 hits after the first
// block of an XCD; the VALU work is M rows per block):
//  - wave kWaves of the block (one extra wave) issues the first kDD stages
//    of every compute wave's weight ring, so the weight stream starts at
//    once, and the compute waves' own loads of the rows never queue behind
//    those direct loads in their vmcnt order;
//  - compute wave w quantises rows w, w + kWaves, ... (the norm-quant
//    kernel's arithmetic, so codes and scales are bit-identical) into the
//    activation slots and the scale area; block b also writes row b's
//    outputs (codes, scales, kv) to memory with the norm-quant kernel's own
//    per-row code;
//  - one barrier, then the stream kernel's K loop and output stores
//    unchanged (the compute waves have no direct loads in flight).
// The results are bit-identical to the norm-quant kernel followed by the
// stream kernel.
// ---------------------------------------------------------------------------

// Batches the one-launch step takes: each block quantises every row itself,
// so its VALU and L2 work grows with M; measured, the one launch is ahead of
// the two up to 16 rows (M = 1: 11.0 against 13.5 us, M = 16: 12.7 against
// 14.5 us), even at 32 and behind at 64 (23.4 against 16.7 us).
constexpr int kStepMaxRows = 16;

// Row m of the MLA latent shape (Nq = 1536, Nkv = 512, 16-byte aligned
// slices) to memory: the norm-quant kernel's loads and per-row code.
template <bool kE8m0>
__device__ __forceinline__ void normquant_row_mla(const NormQuantParams &a, int64_t m, int lane) {
    constexpr int kQ = 3;
    uint4 gq_raw[kQ], gk_raw[1], xq[kQ], xk[1];
#pragma unroll
    for (int c = 0; c < kQ; ++c)
        gq_raw[c] = row::load8<true, true>(a.gamma_q, c * row::kChunk + lane * 8, a.Nq);
    gk_raw[0] = row::load8<true, true>(a.gamma_kv, lane * 8, a.Nkv);
    const uint16_t *qrow = a.q + m * a.q_stride;
#pragma unroll
    for (int c = 0; c < kQ; ++c)
        xq[c] = row::load8<true, true>(qrow, c * row::kChunk + lane * 8, a.Nq);
    xk[0] = row::load8<true, true>(a.kv + m * a.kv_stride, lane * 8, a.Nkv);
    row::GammaSlice gq[kQ], gk[1];
#pragma unroll
    for (int c = 0; c < kQ; ++c)
        gq[c] = row::prepare_gamma(gq_raw[c]);
    gk[0] = row::prepare_gamma(gk_raw[0]);
    row::process_row<kQ, 1, true, true, true, kE8m0, false>(a, m, lane, xq, xk, gq, gk);
}

// Rows of q quantised into the stream kernel's LDS image (row r of wave w
// is row w + r * kWaves, all of a wave's row loads issued first): codes of
// row m, K-block kb, 16-byte piece c16 at slot (kb * kMT + m / 16) * 2 +
// (m / 8) % 2, byte 128 (m % 8) + 16 (c16 ^ (m % 8) ^ g) (g: that slot's
// parity); its scale at the scale area + kb * 256 + 4 m (e8m0: the
// exponent byte, zero-extended, as the stream kernel's 1-byte loads leave it).
template <int kMT, int kWaves, int kAOff, int kSOff, bool kE8m0>
struct RowsToLds {
    static constexpr int kQ = 3;  // 512-element chunks of a 1536 row
    static constexpr int kRowsMax = (16 * kMT + kWaves - 1) / kWaves;

    __device__ __forceinline__ static void store(uint8_t *lds, const NormQuantParams &a, int m, int lane,
                                                 const uint4 (&x)[kQ], const row::GammaSlice (&g)[kQ]) {
        const float rq = row::row_rstd<kQ>(x, a.inv_nq, a.eps);
        const int r = m & 7, gp = (m >> 3) & 1, j = m >> 4;
#pragma unroll
        for (int c = 0; c < kQ; ++c) {
            const row::ChunkCodes q = row::quantise_chunk<true, kE8m0>(x[c], g[c], rq);
            const int col = c * row::kChunk + lane * 8;
            const int kb = col / kBlk, c16 = (col % kBlk) / 16, half = (col % 16) / 8;
            const int slot = (kb * kMT + j) * 2 + gp;
            *reinterpret_cast<uint2 *>(lds + kAOff + slot * 1024 + 128 * r + 16 * (c16 ^ r ^ gp) + 8 * half) =
                make_uint2(q.lo, q.hi);
            if ((lane & 15) == 0)
                reinterpret_cast<uint32_t *>(lds + kSOff)[kb * kWave + m] =
                    kE8m0 ? static_cast<uint32_t>(q.e + 127) : __float_as_uint(q.s);
        }
    }

    __device__ __forceinline__ static void run(uint8_t *lds, const NormQuantParams &a, int wave, int lane) {
        uint4 graw[kQ], x[kRowsMax][kQ];
#pragma unroll
        for (int c = 0; c < kQ; ++c)
            graw[c] = row::load8<true, true>(a.gamma_q, c * row::kChunk + lane * 8, a.Nq);
        const int M = static_cast<int>(a.M);
#pragma unroll
        for (int i = 0; i < kRowsMax; ++i) {
            const int m = wave + i * kWaves;
            if (m < M) {
                const uint16_t *qrow = a.q + m * a.q_stride;
#pragma unroll
                for (int c = 0; c < kQ; ++c)
                    x[i][c] = row::load8<true, true>(qrow, c * row::kChunk + lane * 8, a.Nq);
            }
        }
        row::GammaSlice g[kQ];
#pragma unroll
        for (int c = 0; c < kQ; ++c)
            g[c] = row::prepare_gamma(graw[c]);
#pragma unroll
        for (int i = 0; i < kRowsMax; ++i) {
            if (wave + i * kWaves >= M)
                break;  // uniform
            store(lds, a, wave + i * kWaves, lane, x[i], g);
        }
    }
};

template <int kKB, int kMT, int kSW, int kWaves, int kD, bool kE8m0>
__global__ __launch_bounds__((kWaves + 1) * kWave) void normquant_gemm_pair_kernel(NormQuantParams a,
                                                                                   GemmParams p) {
    using SW = StreamWave<kKB, kMT, kSW, kWaves, kD, kE8m0>;
    using P = typename SW::P;
    extern __shared__ uint4 s_dyn[];
    SW w;
    w.lds = reinterpret_cast<uint8_t *>(s_dyn);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    if (wave == kWaves) {
        // the first ring stages of every compute wave; landed before the
        // barrier, so the compute waves start with nothing in flight
#pragma unroll
        for (int cw = 0; cw < kWaves; ++cw) {
            w.setup_ring(p, cw, (static_cast<int64_t>(blockIdx.x) * kWaves + cw) * kSW);
#pragma unroll
            for (int s = 0; s < P::kDD; ++s)
                w.issue_w(s);
        }
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        return;
    }
    const int64_t st0 = (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * kSW;  // one row chunk: m0 = 0
    w.setup(p, wave, st0);
    if (blockIdx.x < a.M && wave == 0)
        normquant_row_mla<kE8m0>(a, blockIdx.x, lane);
    RowsToLds<kMT, kWaves, P::kAOff, P::kSOff, kE8m0>::run(w.lds, a, wave, lane);
    w.zero_acc();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    w.compute();
    w.store_tile(p, 0, st0);
}

template <int kMT, int kWaves, bool kE8m0, int kSW>
hipError_t launch_normquant_gemm_pair_mt(const NormQuantParams &a, const GemmParams &p, hipStream_t stream) {
    constexpr int kKB = 12;
    constexpr int kD = stream_depth<kKB, kMT, kSW, kWaves, kE8m0>();
    using P = StreamPlan<kKB, kMT, kSW, kWaves, kD, kE8m0>;
    const int64_t per_block = kWaves * kSW;
    const int64_t blocks = ((p.N + p.N2) / 16 + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    constexpr auto kern = normquant_gemm_pair_kernel<kKB, kMT, kSW, kWaves, kD, kE8m0>;
    const hipError_t e = DynLds<kern, P::kLds>::ensure();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3((kWaves + 1) * kWave), P::kLds, stream, a, p);
    return hipGetLastError();
}

template <int kKB, int kNS, int kMT, int kWaves, bool kE8m0>
hipError_t launch_wide_scaled(const GemmParams &p, hipStream_t stream) {
    using P = WidePlan<kKB, kNS, kMT, kWaves, kE8m0>;
    const int64_t nm = (p.M + kWaves * 16 * kMT - 1) / (kWaves * 16 * kMT);
    const int64_t blocks = ((p.N + p.N2) / 16 + kNS - 1) / kNS * nm;
    if (blocks > 0x7FFFFFFF || p.M > 256)
        return hipErrorInvalidValue;
    constexpr auto kern = block_scaled_fp8_gemm_wide_kernel<kKB, kNS, kMT, kWaves, kE8m0>;
    const hipError_t e = DynLds<kern, P::kLds>::ensure();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kWaves * kWave), P::kLds, stream, p);
    return hipGetLastError();
}

template <int kKB, int kNS, int kMT, int kWaves>
hipError_t launch_wide(const GemmParams &p, hipStream_t stream) {
    if (p.scale_e8m0)
        return launch_wide_scaled<kKB, kNS, kMT, kWaves, true>(p, stream);
    return launch_wide_scaled<kKB, kNS, kMT, kWaves, false>(p, stream);
}

template <int kKB, int kMT>
hipError_t launch_wide_ns(const GemmParams &p, hipStream_t stream) {
    // subtiles per block: the smallest even count that covers N (+ N2) with
    // one block per CU; beyond 6 per CU (8 with one 16-row tile per wave)
    // the grid simply has more blocks than CUs (registers: two fragment sets).
    // At most one subtile per CU (a TP-8 shard pair, 17-64 rows): one subtile
    // per block, so every CU streams (measured: TP-8 pair at M = 32 5.40 ->
    // 4.64 us, at M = 64 5.55 -> 5.17 us).
    const int64_t per_cu = ((p.N + p.N2) / 16 + device_cu_count() - 1) / device_cu_count();
    if constexpr (kMT == 1) {
        if (per_cu <= 1)
            return launch_wide<kKB, 1, kMT, kWideWaves>(p, stream);
    }
    if (per_cu <= 2)
        return launch_wide<kKB, 2, kMT, kWideWaves>(p, stream);
    // three subtiles per CU (e.g. a TP-2 W_a shard): three per block rather
    // than four, so no CU idles (TP-2 W_a at M = 32 6.80 -> 6.49 us)
    if constexpr (kMT == 1) {
        if (per_cu == 3)
            return launch_wide<kKB, 3, kMT, kWideWaves>(p, stream);
    }
    if (per_cu <= 4)
        return launch_wide<kKB, 4, kMT, kWideWaves>(p, stream);
    if constexpr (kMT == 1) {
        if (per_cu > 6)
            return launch_wide<kKB, 8, kMT, kWideWaves>(p, stream);
    }
    return launch_wide<kKB, 6, kMT, kWideWaves>(p, stream);
}

template <int kKB, int kNS>
hipError_t launch_wide_split(const GemmParams &p, int64_t slabs, hipStream_t stream) {
    // row chunks of 128 if that already gives a block per CU, else of 64
    const int64_t chunks128 = (p.M + 127) / 128;
    if (slabs * chunks128 >= device_cu_count())
        return launch_wide<kKB, kNS, 2, kWideWaves>(p, stream);
    // 64-row chunks of two-subtile slabs, or of three-subtile slabs where
    // two would give more blocks than CUs and three do not (TP-8 W_a at
    // M = 256: 384 blocks, half the CUs holding two, against 256; 7.37 ->
    // 6.18 us)
    const int64_t S = (p.N + p.N2) / 16, nm = (p.M + 63) / 64, cus = device_cu_count();
    if ((S + 1) / 2 * nm > cus && (S + 2) / 3 * nm <= cus)
        return launch_wide<kKB, 3, 1, kWideWaves>(p, stream);
    return launch_wide<kKB, kNS, 1, kWideWaves>(p, stream);
}

template <int kKB>
hipError_t launch_wide_kb(const GemmParams &p, hipStream_t stream) {
    static_assert(kWideWaves == 4, "a block covers 64 kMT rows");
    if (p.M <= 64)
        return launch_wide_ns<kKB, 1>(p, stream);
    // With weight slabs for fewer than half the CUs, split the rows over
    // blocks (each slab is then read once per row chunk, the repeats from
    // L2) rather than leave CUs idle; otherwise one block holds all M rows
    // (measured: splitting a grid that fills more than half the CUs loses).
    const int64_t S = (p.N + p.N2) / 16, cus = device_cu_count();
    // One to two subtiles per CU (a TP-4 / TP-8 shard pair, a TP-4 shard):
    // 64-row chunks of the fewest subtiles per block that still give one
    // block per CU (measured, paired A/B: the TP-8 pair at M = 128 9.78 ->
    // 5.12 us and at M = 256 10.95 -> 6.64 us together with its one launch,
    // the TP-4 W_a shard at M = 256 8.37 -> 8.10 us, 5120 rows at M = 256
    // 9.10 -> 8.11 us).
    if (S >= cus && S < 2 * cus) {
        const int64_t nm = (p.M + 63) / 64;
        if ((S + 1) / 2 * nm <= cus)
            return launch_wide<kKB, 2, 1, kWideWaves>(p, stream);
        if ((S + 2) / 3 * nm <= cus)
            return launch_wide<kKB, 3, 1, kWideWaves>(p, stream);
        if ((S + 3) / 4 * nm <= cus)
            return launch_wide<kKB, 4, 1, kWideWaves>(p, stream);
        if ((S + 5) / 6 * nm <= cus)
            return launch_wide<kKB, 6, 1, kWideWaves>(p, stream);
    }
    const int64_t slabs = (S + 1) / 2;  // at 2 subtiles per block
    if (2 * slabs < cus)
        return launch_wide_split<kKB, 2>(p, slabs, stream);
    // three subtiles per CU: six-subtile slabs in two row chunks, a block
    // per CU
    if ((S + cus - 1) / cus == 3) {
        if (p.M <= 128)
            return launch_wide<kKB, 6, 1, kWideWaves>(p, stream);
        return launch_wide<kKB, 6, 2, kWideWaves>(p, stream);
    }
    // Fewer two-subtile slabs than CUs (at most two subtiles per CU) would
    // leave CUs idle with all M rows per block: three-subtile slabs of half
    // the rows where that fills more of them (a TP-4 W_a shard at M = 256:
    // 256 blocks against 192; 9.77 -> 8.43 us, at M = 128 6.72 -> 6.52 us).
    if (slabs < cus && (S + 2) / 3 * 2 <= cus && (S + 2) / 3 * 2 > slabs) {
        if (p.M <= 128)
            return launch_wide<kKB, 3, 1, kWideWaves>(p, stream);
        return launch_wide<kKB, 3, 2, kWideWaves>(p, stream);
    }
    if (p.M <= 128)
        return launch_wide_ns<kKB, 2>(p, stream);
    return launch_wide_ns<kKB, 4>(p, stream);
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

// ---------------------------------------------------------------------------
// Split-K variant: one 16-row weight subtile per block, for decode batches
// (up to 16 rows) over a narrow weight, such as a tensor-parallel shard of
// a few thousand rows, that gives every CU at most one subtile: there a K
// loop per subtile leaves the memory system idle between its stages.
// The block's kWaves waves take contiguous ranges of kKB / kWaves
// K-blocks; each wave loads its weight fragments, the activation fragments
// of its K-blocks and their scales straight into registers (every load
// issued before the first MFMA: one memory round trip per block), runs
// one MFMA per (m-tile, K-block) and leaves the partial sums with their
// scales As * Bs in LDS.  After one barrier wave j folds m-tile j's
// partials in K-block order, as every kernel here does, so the results are
// bit-identical to theirs.  Activation rows at or beyond M repeat row M - 1
// (their results are never stored).
// ---------------------------------------------------------------------------
namespace {

template <int kKB, int kMT, int kWaves>
__global__ __launch_bounds__(kWaves * kWave) void block_scaled_fp8_gemm_splitk_kernel(GemmParams p) {
    static_assert(kKB % kWaves == 0 && kMT <= kWaves, "K ranges per wave; an m-tile per folding wave");
    constexpr int kPer = kKB / kWaves;
    __shared__ v4f s_part[kMT][kKB][kWave];
    __shared__ float s_scl[kMT][kKB][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t M = p.M, K = p.K;
    const SubTile sub = subtile(p, blockIdx.x);
    const WeightFrag wfr = weight_frag(lane, K, p.w_tiled);
    const int kb0 = wave * kPer;

    // the scales first (their latency then hides under the fragments'),
    // then the weight fragments (HBM), then the activation fragments
    v8i wf[kPer], af[kMT][kPer];
    float as[kMT][kPer], bs[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        bs[i] = sub.ws[kb0 + i];
#pragma unroll
    for (int j = 0; j < kMT; ++j) {
        const int64_t row = min<int64_t>(16 * j + (lane & 15), M - 1);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t kb = kb0 + i;
            as[j][i] = p.a_scale[p.a_scale_transposed ? kb * M + row : row * kKB + kb];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        wf[i] = load_weight_frag(sub.w + wfr.lane_off + (kb0 + i) * wfr.kstride, wfr.hstride);
#pragma unroll
    for (int j = 0; j < kMT; ++j) {
        const int64_t row = min<int64_t>(16 * j + (lane & 15), M - 1);
        const uint8_t *arow = p.a + row * K + 32 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            af[j][i] = load_weight_frag(arow + (kb0 + i) * kBlk, 16);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kMT; ++j)
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            s_part[j][kb0 + i][lane] = mfma_e4m3_16x16x128(wf[i], af[j][i]);
            s_scl[j][kb0 + i][lane] = as[j][i] * bs[i];
        }
    __syncthreads();
    if (wave < kMT) {
        const int j = wave;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const v4f part = s_part[j][kb][lane];
            const float sc = s_scl[j][kb][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = fmaf(part[i], sc, acc[i]);
        }
        const int64_t row = 16 * j + (lane & 15);
        if (row < M)
            *reinterpret_cast<uint2 *>(sub.out + row * sub.ldo + sub.n0 + 4 * (lane >> 4)) =
                make_uint2(pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3]));
    }
}

template <int kMT>
hipError_t launch_splitk_mt(const GemmParams &p, int64_t blocks, hipStream_t stream) {
    hipLaunchKernelGGL((block_scaled_fp8_gemm_splitk_kernel<12, kMT, 4>), dim3(static_cast<unsigned>(blocks)),
                       dim3(4 * kWave), 0, stream, p);
    return hipGetLastError();
}

// The split-K kernel where it applies: fp32 scales, K = 1536, batches of
// up to 16 rows (one m-tile), at most one weight subtile per CU.
// hipErrorNotSupported otherwise.  (Measured on the TP-8 shards: the pair
// at M = 1 4.9 -> 3.8 us, at M = 16 5.0 -> 4.3 us; at 32 rows and more the
// activation fragments, read straight from memory in fragment order, cost
// more than the split saves: M = 32 5.1 -> 5.3 us, M = 64 5.2 -> 7.1 us.)
hipError_t launch_splitk(const GemmParams &p, hipStream_t stream) {
    const int64_t S = (p.N + p.N2) / 16;
    if (p.scale_e8m0 || p.K != 12 * kBlk || p.M < 1 || p.M > 16 || S < 1 || S > device_cu_count())
        return hipErrorNotSupported;
    return launch_splitk_mt<1>(p, S, stream);
}

}  // namespace

hipError_t launch_block_scaled_gemm(const GemmParams &p, hipStream_t stream) {
    // decode batches over narrow weights (a subtile per CU at most): split-K
    {
        const hipError_t e = launch_splitk(p, stream);
        if (e != hipErrorNotSupported)
            return e;
    }
    // decode batches over wide weights: the barrier-free stream kernel
    {
        const hipError_t e = launch_stream(p, stream);
        if (e != hipErrorNotSupported)
            return e;
    }
    // Small decode batches over wide weights (more than 4 subtiles per CU):
    // weight ring per wave, activations resident in LDS.
    // (e8m0 scales: the wide kernel, whose matrix cores apply them)
    if (!p.scale_e8m0 && p.M <= kDecodeMaxRows && p.N / 16 > 4 * static_cast<int64_t>(device_cu_count())) {
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
    // Up to 256 rows: weight slab per block, everything streamed through
    // LDS rings.
    if (p.M <= 4 * kChunkRows) {
        switch (p.K / kBlk) {
        case 4:
            return launch_wide_kb<4>(p, stream);
        case 8:
            return launch_wide_kb<8>(p, stream);
        case 12:
            return launch_wide_kb<12>(p, stream);
        case 16:
            return launch_wide_kb<16>(p, stream);
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

namespace {

// Row-major <-> tiled weight, one thread per 16-byte chunk of the tiled
// image: a wave covers one 1 KB half-tile (lane order), contiguous on the
// tiled side, 4 alternate 16-byte chunks of each of 16 rows of one K-block
// on the row-major side.
__global__ __launch_bounds__(256) void weight_relayout_kernel(const uint8_t *src, uint8_t *dst, int64_t N,
                                                              int64_t K, int to_tiled) {
    const int64_t chunks = N * K / 16;
    const int64_t KB = K / kBlk;
    for (int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; o < chunks;
         o += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        // o = ((st * KB + kb) * 2 + h) * 64 + L: lane L = 16 q + rho holds
        // row rho, chunks 2q (h = 0) and 2q + 1 (h = 1) of the K-block
        const int L = static_cast<int>(o & 63), h = static_cast<int>((o >> 6) & 1);
        const int64_t tile = o >> 7, st = tile / KB, kb = tile % KB;
        const int64_t rm = ((st * 16 + (L & 15)) * K + kb * kBlk) / 16 + 2 * (L >> 4) + h;  // row-major chunk
        const uint4 *s = reinterpret_cast<const uint4 *>(src);
        uint4 *d = reinterpret_cast<uint4 *>(dst);
        if (to_tiled)
            d[o] = s[rm];
        else
            d[rm] = s[o];
    }
}

}  // namespace

hipError_t launch_weight_relayout(const uint8_t *src, uint8_t *dst, int64_t N, int64_t K, bool to_tiled,
                                  hipStream_t stream) {
    const int64_t chunks = N * K / 16;
    const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 65536);
    hipLaunchKernelGGL(weight_relayout_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, src, dst,
                       N, K, to_tiled ? 1 : 0);
    return hipGetLastError();
}

bool normquant_gemm_pair_one_launch(int64_t M, int64_t Nq, int64_t Nkv, int64_t N1, int64_t N2) {
    // the MLA latent shape, a block for every row (block b writes row b's
    // outputs), and the stream kernel's shapes (at least 6 weight subtiles
    // per CU)
    if (Nq != 1536 || Nkv != 512 || M < 1 || M > kStepMaxRows || N1 <= 0 || N2 <= 0)
        return false;
    const int64_t S = (N1 + N2) / 16, cus = device_cu_count();
    const int64_t per_cu = (S + cus - 1) / cus;
    return per_cu >= 6 && M <= S / (per_cu <= 6 ? 6 : 8);  // the grid's blocks (6 or 8 subtiles each)
}

hipError_t launch_normquant_gemm_pair(const NormQuantParams &a, const GemmParams &p, hipStream_t stream) {
    const auto al16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    const bool vec = al16(a.q) && al16(a.kv) && al16(a.gamma_q) && al16(a.gamma_kv) && al16(a.out_kv) &&
                     al16(a.out_q) && (a.q_stride % 8) == 0 && (a.kv_stride % 8) == 0;
    // both in fp32 scales or both in e8m0 (the norm-quant's exponent bytes are the GEMM's As)
    const bool e8m0 = a.out_scale_e8m0 != nullptr;
    if (!vec || e8m0 != (p.scale_e8m0 != 0) || p.K != a.Nq || p.M != a.M ||
        !normquant_gemm_pair_one_launch(a.M, a.Nq, a.Nkv, p.N, p.N2))
        return hipErrorNotSupported;
    const int64_t S = (p.N + p.N2) / 16, cus = device_cu_count();
    const bool three = (S + cus - 1) / cus <= 6;
    static_assert(kStepMaxRows <= 16, "one 16-row chunk per block");
    // one weight subtile per compute wave (six or eight waves: the stream
    // kernel's decode form for these widths; the M = 16 step 11.7 -> 10.9 us
    // against two subtiles per wave, M = 1 unchanged)
    if (e8m0)
        return three ? launch_normquant_gemm_pair_mt<1, 6, true, 1>(a, p, stream)
                     : launch_normquant_gemm_pair_mt<1, 8, true, 1>(a, p, stream);
    return three ? launch_normquant_gemm_pair_mt<1, 6, false, 1>(a, p, stream)
                 : launch_normquant_gemm_pair_mt<1, 8, false, 1>(a, p, stream);
}

hipError_t init_device() {
    device_cu_count();
    for (RaiseFn f : lds_registry()) {
        const hipError_t e = f();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// Both consumers in one launch: decode batches, and above 64 rows
// tensor-parallel shard pairs (at most four subtiles per CU together,
// K / 128 = 12; the full W_a + W_b pair, eight per CU, is 2.0-2.6 us faster
// as two launches).
static bool gemm_pair_one_launch(int64_t M, int64_t K, int64_t N1, int64_t N2) {
    const int64_t kb = K / kBlk;
    if (M <= kChunkRows)
        return kb == 4 || kb == 8 || kb == 12 || kb == 16;
    return M <= 256 && kb == 12 && (N1 + N2) / 16 <= 4 * device_cu_count();
}

int gemm_pair_launches(int64_t M, int64_t K, int64_t N1, int64_t N2) {
    return gemm_pair_one_launch(M, K, N1, N2) ? 1 : 2;
}

hipError_t launch_block_scaled_gemm_pair(const GemmParams &p, hipStream_t stream) {
    // decode batches: one launch over the subtiles of both weights, sharing
    // the activation tile (split-K over narrow weights, the stream kernel
    // where the weights are wide enough, else the wide kernel)
    // shard pairs above 64 rows: one wide launch over the subtiles of both
    // (against two launches: TP-8 pair at M = 128 9.8 -> 5.1 us, TP-4 pair
    // 11.3 -> 7.0 us, TP-2 pair 14.8 -> 10.6 us)
    if (p.M > kChunkRows && gemm_pair_one_launch(p.M, p.K, p.N, p.N2))
        return launch_wide_kb<12>(p, stream);
    if (p.M <= kChunkRows) {
        hipError_t e = launch_splitk(p, stream);
        if (e == hipErrorNotSupported)
            e = launch_stream(p, stream);
        if (e != hipErrorNotSupported)
            return e;
        switch (p.K / kBlk) {
        case 4:
            return launch_wide_kb<4>(p, stream);
        case 8:
            return launch_wide_kb<8>(p, stream);
        case 12:
            return launch_wide_kb<12>(p, stream);
        case 16:
            return launch_wide_kb<16>(p, stream);
        default:
            break;
        }
    }
    GemmParams a = p, b = p;
    a.w2 = nullptr;
    a.w_scale2 = nullptr;
    a.w_scale8_2 = nullptr;
    a.out2 = nullptr;
    a.N2 = 0;
    b.w = p.w2;
    b.w_scale = p.w_scale2;
    b.w_scale8 = p.w_scale8_2;
    b.out = p.out2;
    b.N = p.N2;
    b.w2 = nullptr;
    b.w_scale2 = nullptr;
    b.w_scale8_2 = nullptr;
    b.out2 = nullptr;
    b.N2 = 0;
    const hipError_t e = launch_block_scaled_gemm(a, stream);
    return e != hipSuccess ? e : launch_block_scaled_gemm(b, stream);
}

}  // namespace mi
