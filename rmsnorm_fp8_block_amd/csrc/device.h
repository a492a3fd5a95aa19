// device.h -- small gfx950 (CDNA4, wave64) device helpers shared by the
// kernels of this library: bf16 unpacking, DPP reductions inside a 16-lane
// row, wave-wide reductions, packed fp32 -> e4m3fn / bf16 conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi {

constexpr int kWave = 64;

// bf16 halves of a 32-bit word -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8_bf16(const uint4 &v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// One DPP move inside a 16-lane row (all lanes read a valid source for the
// controls used here: quad permutes and mirrors).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7 - i inside each 8
constexpr int kRowMirror = 0x140;     // lane i <-> 15 - i inside each 16

// Sum / max over the 16 lanes of a DPP row.  Every lane of the row ends with
// the same bits: each step combines a value with its partner's value, and
// fp32 addition and max are commutative.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<kQuadSwap1>(v);
    v += dpp_mov<kQuadSwap2>(v);
    v += dpp_mov<kRowHalfMirror>(v);
    v += dpp_mov<kRowMirror>(v);
    return v;
}

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_mov<kQuadSwap1>(v));
    v = fmaxf(v, dpp_mov<kQuadSwap2>(v));
    v = fmaxf(v, dpp_mov<kRowHalfMirror>(v));
    v = fmaxf(v, dpp_mov<kRowMirror>(v));
    return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Wave-wide sum, identical in all 64 lanes: row sums by DPP, then the four
// row totals combined as (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    const float r0 = readlane_f(v, 0), r1 = readlane_f(v, 16);
    const float r2 = readlane_f(v, 32), r3 = readlane_f(v, 48);
    return (r0 + r1) + (r2 + r3);
}

// Four fp32 values (already inside [-448, 448]) -> four e4m3fn codes, RNE,
// first value in the lowest byte.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return static_cast<uint32_t>(w);
}

typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef float v2f32 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (RNE, one packed convert), first value in the low half.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    const v2f32 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, v2bf16));
}

// Products of packed bf16 pairs, exact in fp32: dot2(x, g masked to one
// half) = x_lo * g_lo (or x_hi * g_hi) + 0.
__device__ __forceinline__ float bf16_dot2(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf16, x), __builtin_bit_cast(v2bf16, y), acc,
                                          false);
}

// Workgroups are dealt round-robin over the 8 XCDs.  Renumber them so that
// each XCD works on one contiguous range of logical block ids (when the grid
// divides evenly); neighbouring rows / tiles then share an L2.
__device__ __forceinline__ int xcd_contiguous_block(int b, int nblocks) {
    if ((nblocks & 7) != 0)
        return b;
    return (b & 7) * (nblocks >> 3) + (b >> 3);
}

}  // namespace mi
