// normquant_row.h -- the per-row device code of the fused dual RMSNorm +
// per-1x128 FP8 group quantisation (one wave64 per row): 16-byte row-slice
// loads, sums of squares, the normalisation, group amax, scale and e4m3fn
// codes, kv in bf16.  Used by the norm-quant kernels and by the one-launch
// decode step, which must produce bit-identical outputs.
//
// What is computed follows the GitHub page of vLLM PR #53540 ("[ROCm][Perf]
// Fuse SWA q/kv RMSNorm and q FP8 group quant for DeepSeek-V4"), section
// "Purpose"; the scale layout flag the PRHub report of vLLM PR #56433
// (item 4).
#pragma once

#include "device.h"
#include "launch.h"

namespace mi {
namespace row {

constexpr int kChunk = 512;     // elements per 16-byte-per-lane wave load
constexpr int kGroup = 128;
constexpr float kE4m3Max = 448.0f;
constexpr float kInvE4m3Max = 1.0f / 448.0f;  // rounded to fp32
constexpr float kScaleFloor = 1e-12f;
constexpr int kE8m0MinExponent = -39;  // ceil(log2(1e-12)): the floor as a power of two

typedef unsigned v4u32 __attribute__((ext_vector_type(4)));

// 8 consecutive bf16 at p[col, col+8); elements at or beyond n read as zero.
// kVec: p + col is 16-byte aligned whenever col + 8 <= n.  kFull: the caller
// guarantees col + 8 <= n (no bounds test, a single 16-byte load).
template <bool kVec, bool kFull = false, bool kStream = false>
__device__ __forceinline__ uint4 load8(const uint16_t *p, int col, int n) {
    if (kFull && kStream) {  // read once: streamed past the caches
        const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p + col));
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    if (kFull)
        return *reinterpret_cast<const uint4 *>(p + col);
    if (kVec && col + 8 <= n)
        return *reinterpret_cast<const uint4 *>(p + col);
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        e[j] = (col + j < n) ? p[col + j] : 0u;
    return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
}

// Sum of squares of the 8 bf16 values of a 16-byte slice, with the packed
// bf16 dot product (products exact in fp32, fp32 accumulation).
__device__ __forceinline__ float sumsq8(const uint4 &v) {
    return bf16_dot2(v.x, v.x, bf16_dot2(v.y, v.y, 0.0f)) + bf16_dot2(v.z, v.z, bf16_dot2(v.w, v.w, 0.0f));
}

// A gamma slice prepared for bf16_dot2: word 2i keeps the low bf16 of
// gamma word i (high half zero), word 2i+1 the high bf16 (low half zero).
struct GammaSlice {
    uint32_t w[8];
};

__device__ __forceinline__ GammaSlice prepare_gamma(const uint4 &g) {
    const uint32_t v[4] = {g.x, g.y, g.z, g.w};
    GammaSlice r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.w[2 * i] = v[i] & 0x0000FFFFu;
        r.w[2 * i + 1] = v[i] & 0xFFFF0000u;
    }
    return r;
}

// z = x * gamma for the 8 elements of a slice, exact in fp32.
__device__ __forceinline__ void times_gamma8(const uint4 &x, const GammaSlice &g, float (&z)[8]) {
    const uint32_t v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        z[2 * i] = bf16_dot2(v[i], g.w[2 * i], 0.0f);
        z[2 * i + 1] = bf16_dot2(v[i], g.w[2 * i + 1], 0.0f);
    }
}

// Output stores.  kNt: non-temporal, streamed to memory instead of
// displacing cached lines (large batches: measured faster at 8192 rows, most
// of all with column-major scales); plain for a handful of rows, whose codes
// the GEMM reads next (measured: the M = 64 decode step 0.5 us faster, the
// M = 8192 column-major calls 1.2-1.7 us slower).
typedef unsigned v2u32 __attribute__((ext_vector_type(2)));
template <bool kNt>
__device__ __forceinline__ void store_out(uint16_t *p, const uint4 &v) {
    if constexpr (kNt)
        __builtin_nontemporal_store(v4u32{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u32 *>(p));
    else
        *reinterpret_cast<v4u32 *>(p) = v4u32{v.x, v.y, v.z, v.w};
}
template <bool kNt>
__device__ __forceinline__ void store_out(uint8_t *p, uint32_t lo, uint32_t hi) {
    if constexpr (kNt)
        __builtin_nontemporal_store(v2u32{lo, hi}, reinterpret_cast<v2u32 *>(p));
    else
        *reinterpret_cast<v2u32 *>(p) = v2u32{lo, hi};
}

// Left-to-right sum of the per-chunk partial sums.  Chunks past the row
// width contribute +0.0, which leaves a left fold unchanged, so every kernel
// variant sums a row in the same order and gives the same bits.
template <int N>
__device__ __forceinline__ float fold_sum(const float *v) {
    float s = v[0];
#pragma unroll
    for (int i = 1; i < N; ++i)
        s += v[i];
    return s;
}

// 1 / sqrt(mean of squares + eps) in fp32: hardware reciprocal square root
// refined by one Newton step (exact for powers of four).
__device__ __forceinline__ float rstd_from_ssq(float ssq, float inv_n, float eps) {
    const float x = ssq * inv_n + eps;
    const float r = __builtin_amdgcn_rsqf(x);
    return r * (1.5f - (0.5f * x) * r * r);
}

// x / s rounded to fp32 "to odd" (an inexact quotient takes whichever of its
// two fp32 neighbours has an odd last bit), so that the e4m3 RNE convert of
// the result equals the single RNE rounding of the exact quotient: fp32
// carries more than two bits beyond e4m3's precision, and no e4m3 rounding
// midpoint has an odd last fp32 bit.  q0 = x * (1/s) is within about 1.5
// fp32 ULP; one remainder step (the FMA remainder x - q*s is exact this close
// to the quotient) makes it faithful; the sign of the second remainder says
// on which side of it the exact quotient lies.  The sign is taken from x
// (s > 0): the remainder step turns a -0 quotient into +0.
__device__ __forceinline__ float div_round_to_odd(float x, float s, float inv) {
    const float q0 = x * inv;
    const float q1 = fmaf(fmaf(-q0, s, x), inv, q0);
    const float r1 = fmaf(-q1, s, x);
    uint32_t b = __float_as_uint(q1);
    if (r1 != 0.0f && (b & 1u) == 0u)
        b += ((r1 > 0.0f) == (q1 > 0.0f)) ? 1u : 0xFFFFFFFFu;  // one ULP towards the quotient
    return __builtin_copysignf(__uint_as_float(b), x);
}

// Chunk c (512 elements, 4 groups) of row m: group amax, scale, e4m3fn codes.
// x: this lane's 8 elements; g: their gamma (unused without the norm);
// rq: the row's rstd (1 without the norm).  kE8m0: the scale is rounded up
// to a power of two 2^e (the smallest not below the fp32 scale), stored as
// the exponent byte e + 127, and the codes are z * (rq * 2^-e).
// The 8 codes of one lane's slice of chunk c and its group's scale.
struct ChunkCodes {
    uint32_t lo, hi;  // codes of the 8 elements, first in the lowest byte
    float s;          // the group's fp32 scale (e8m0: 2^e)
    int e;            // e8m0: the scale's exponent
};

// Group amax, scale and e4m3fn codes of one lane's 8 elements of a chunk.
// x: the elements; g: their gamma (unused without the norm); rq: the row's
// rstd (1 without the norm).  kE8m0: the scale is rounded up to a power of
// two 2^e (the smallest not below the fp32 scale) and the codes are
// z * (rq * 2^-e).
template <bool kNorm, bool kE8m0>
__device__ __forceinline__ ChunkCodes quantise_chunk(const uint4 &x, const GammaSlice &g, float rq) {
    float z[8];
    if constexpr (kNorm)
        times_gamma8(x, g, z);
    else
        unpack8_bf16(x, z);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        amax = fmaxf(amax, fabsf(z[j]));
    // 16 lanes x 8 elements = one 128-element group
    amax = row16_max(amax);
    // without the norm, amax is an exact bf16 value and one correctly
    // rounded division gives the scale bit for bit (once per group)
    float s = kNorm ? fmaxf((amax * rq) * kInvE4m3Max, kScaleFloor)
                    : fmaxf(amax / kE4m3Max, kScaleFloor);
    int e = 0;
    if constexpr (kE8m0) {
        // e = ceil(log2(v / 448)), v = amax * rq, read off v's bits exactly
        // (no rounded 1/448): with v = 1.f * 2^E and 448 = 1.75 * 2^8, v / 448
        // lies in (2^(E-9), 2^(E-8)] when 1.f <= 1.75, else in (2^(E-8),
        // 2^(E-7)); then the floor 2^ceil(log2(1e-12)) = 2^-39 (also taking
        // zero and subnormal v)
        const uint32_t vb = __float_as_uint(amax * rq);
        e = static_cast<int>((vb >> 23) & 0xFFu) - 127 - 8 + ((vb & 0x7FFFFFu) > 0x600000u);
        e = e < kE8m0MinExponent ? kE8m0MinExponent : e;
        s = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    }
    const float inv = kE8m0 ? rq * __uint_as_float(static_cast<uint32_t>(127 - e) << 23)
                            : rq * __builtin_amdgcn_rcpf(s);
    float r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        r[j] = __builtin_amdgcn_fmed3f(kNorm || kE8m0 ? z[j] * inv : div_round_to_odd(z[j], s, inv),
                                       -kE4m3Max, kE4m3Max);
    return {pack4_e4m3(r[0], r[1], r[2], r[3]), pack4_e4m3(r[4], r[5], r[6], r[7]), s, e};
}

// Chunk c (512 elements, 4 groups) of row m: codes and scales to memory.
template <bool kVec, bool kFull, bool kNorm, bool kE8m0 = false, bool kNt = true>
__device__ __forceinline__ void quant_chunk(const NormQuantParams &a, int64_t m, int lane, int c,
                                            const uint4 &x, const GammaSlice &g, float rq) {
    const int G = a.Nq / kGroup;
    uint8_t *qout = a.out_q + m * a.Nq;
    const int col = c * kChunk + lane * 8;
    const ChunkCodes q = quantise_chunk<kNorm, kE8m0>(x, g, rq);
    const uint32_t lo = q.lo, hi = q.hi;
    if (kFull || col < a.Nq) {  // Nq % 128 == 0: a lane's 8 codes are all in range
        if (kFull) {
            store_out<kNt>(qout + col, lo, hi);
        } else if (kVec) {
            *reinterpret_cast<uint2 *>(qout + col) = make_uint2(lo, hi);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                qout[col + j] = static_cast<uint8_t>((j < 4 ? lo : hi) >> (8 * (j & 3)));
        }
    }

    const int grp = c * (kChunk / kGroup) + lane / 16;
    if ((lane & 15) == 0 && (kFull || grp < G)) {
        const int64_t at = a.transpose_scale ? static_cast<int64_t>(grp) * a.M + m
                                             : m * G + grp;
        if constexpr (kE8m0)
            a.out_scale_e8m0[at] = static_cast<uint8_t>(q.e + 127);
        else
            a.out_scale[at] = q.s;
    }
}

// Reciprocal RMS of row q (kQ chunks of this lane), the same bits as
// process_row's.
template <int kQ>
__device__ __forceinline__ float row_rstd(const uint4 (&xq)[kQ], float inv_n, float eps) {
    float part[kQ];
#pragma unroll
    for (int c = 0; c < kQ; ++c)
        part[c] = sumsq8(xq[c]);
    return rstd_from_ssq(wave_sum(fold_sum<kQ>(part)), inv_n, eps);
}

// One row.  With z = x * gamma (exact in fp32: a product of two bf16 values)
// and r = rstd, the normalised value is y = z * r; the group scale is
// s = max(max|z| * r / 448, 1e-12) and the quantised value y / s is formed
// as z * (r / s), so the row's rstd is applied once per group instead of
// once per element.  kNorm == false: the per-1x128 quantisation of x itself
// (z = x, r = 1, no gamma); there x and s are exact, and scales and codes
// are the correctly rounded ones.  kKv == 0: no second input.
template <int kQ, int kKv, bool kVec, bool kFull, bool kNorm, bool kE8m0, bool kNt>
__device__ __forceinline__ void process_row(const NormQuantParams &a, int64_t m, int lane,
                                            const uint4 (&xq)[kQ], const uint4 (&xk)[kKv > 0 ? kKv : 1],
                                            const GammaSlice (&gq)[kQ], const GammaSlice (&gk)[kKv > 0 ? kKv : 1]) {
    // -- sums of squares (fp32) and reciprocal RMS -----------------------------
    float rq = 1.0f;
    if constexpr (kNorm)
        rq = row_rstd<kQ>(xq, a.inv_nq, a.eps);

    // -- kv: y = (x * gamma) * rstd, rounded to bf16 ---------------------------
    if constexpr (kKv > 0) {
    float part_k[kKv];
#pragma unroll
    for (int c = 0; c < kKv; ++c)
        part_k[c] = sumsq8(xk[c]);
    const float rk = rstd_from_ssq(wave_sum(fold_sum<kKv>(part_k)), a.inv_nkv, a.eps);
    uint16_t *kout = a.out_kv + m * a.Nkv;
#pragma unroll
    for (int c = 0; c < kKv; ++c) {
        const int col = c * kChunk + lane * 8;
        if (!kFull && col >= a.Nkv)
            continue;
        float y[8];
        times_gamma8(xk[c], gk[c], y);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            y[j] *= rk;
        const uint4 packed = make_uint4(pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3]),
                                        pack2_bf16(y[4], y[5]), pack2_bf16(y[6], y[7]));
        if (kFull) {
            store_out<kNt>(kout + col, packed);
        } else if (kVec && col + 8 <= a.Nkv) {
            *reinterpret_cast<uint4 *>(kout + col) = packed;
        } else {
            const uint32_t w[4] = {packed.x, packed.y, packed.z, packed.w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (col + j < a.Nkv)
                    kout[col + j] = static_cast<uint16_t>(w[j / 2] >> (16 * (j & 1)));
        }
    }
    }  // kKv > 0

    // -- q: group amax, scale, e4m3fn codes -------------------------------------
#pragma unroll
    for (int c = 0; c < kQ; ++c) {
        if (!kFull && c * kChunk >= a.Nq)
            break;  // uniform across the wave
        quant_chunk<kVec, kFull, kNorm, kE8m0, kNt>(a, m, lane, c, xq[c], gq[c], rq);
    }
}

}  // namespace row
}  // namespace mi
