// ceiling.hip -- data-movement skeletons that give the measured ceilings the
// benchmark reports the kernels against (a separate library,
// libmi_ceiling.so, loaded by the benchmark only; nothing in the hot path
// calls it).  They move exactly the bytes of the real kernels, in the same
// launch shape and with the same load/store widths and cache policies, and
// do no arithmetic, so their time is what this GPU's memory system allows
// for that access pattern at that size.
//
//  - normquant_skeleton: the fused dual norm-quant of the MLA latent shape
//    (q [M, 1536] and kv [M, 512] bf16 rows at a row stride; codes [M, 1536]
//    bytes, 12 fp32 scales per row, kv [M, 512] bf16 out): one wave64 per
//    row, 4 waves per block, rows dealt to XCDs in contiguous ranges, rows
//    read and outputs written non-temporally (the kernel's form from 1024
//    rows on).
//  - weight_stream: a GEMM's weight stream: `blocks` workgroups of 8 waves,
//    each reading its own contiguous slab through an LDS ring by direct
//    global -> LDS loads of 1 KB per wave instruction, never waiting for
//    another wave (the floor of any kernel that reads every weight byte
//    once from HBM into LDS).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int xcd_contiguous(int b, int n) { return (n & 7) ? b : (b & 7) * (n >> 3) + (b >> 3); }

__global__ __launch_bounds__(256) void normquant_skeleton_kernel(const uint16_t *in, int64_t stride, uint8_t *q,
                                                                 float *s, uint16_t *kv, int64_t M) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m = static_cast<int64_t>(xcd_contiguous(blockIdx.x, gridDim.x)) * 4 + wave;
    if (m >= M)
        return;
    const uint16_t *r = in + m * stride;
    v4u x[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        x[c] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(r + c * 512 + lane * 8));
    // codes: 8 bytes per lane and 512-element chunk; kv: 16 bytes per lane;
    // scales: 3 lanes of each 16-lane row (48 bytes per row)
#pragma unroll
    for (int c = 0; c < 3; ++c)
        __builtin_nontemporal_store(v2u{x[c].x ^ x[c].z, x[c].y ^ x[c].w},
                                    reinterpret_cast<v2u *>(q + m * 1536 + c * 512 + lane * 8));
    __builtin_nontemporal_store(x[3], reinterpret_cast<v4u *>(kv + m * 512 + lane * 8));
    if ((lane & 15) < 3 && lane < 48)
        __builtin_nontemporal_store(__uint_as_float(x[0].x), s + m * 12 + (lane >> 4) * 3 + (lane & 15));
}

constexpr int kRing = 8;          // K-block stages in flight per block
constexpr int kStageBytes = 16384;  // 8 waves x 2 KB

__global__ __launch_bounds__(512) void weight_stream_kernel(const uint8_t *w, int64_t slab_bytes, unsigned *sink) {
    extern __shared__ v4u lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t *slab = w + static_cast<int64_t>(blockIdx.x) * slab_bytes;
    char *ring = reinterpret_cast<char *>(lds);
    const int64_t stages = slab_bytes / kStageBytes;
    for (int64_t st = 0; st < stages; ++st) {
        const uint8_t *src = slab + st * kStageBytes + wave * 2048 + lane * 16;
        char *dst = ring + (st % kRing) * kStageBytes + wave * 2048;
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);
        __builtin_amdgcn_global_load_lds(src + 1024, dst + 1024, 16, 0, 2);
        // keep kRing - 1 stages (2 loads each) in flight
        __builtin_amdgcn_s_waitcnt((2 * (kRing - 1)) | (7 << 4) | (15 << 8));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const unsigned v = reinterpret_cast<const unsigned *>(lds)[threadIdx.x];
    if (v == 0x9E3779B9u)  // practically never: keeps the loads observable
        sink[0] = v;
}

}  // namespace

// Both return a hipError_t value (0 = success); arguments are device
// pointers owned by the caller, the launch goes to `stream`.
extern "C" int mi_ceiling_normquant_skeleton(const uint16_t *in, int64_t row_stride, uint8_t *out_q, float *out_scale,
                                            uint16_t *out_kv, int64_t M, hipStream_t stream) {
    if (M <= 0)
        return hipSuccess;
    const int64_t blocks = (M + 3) / 4;
    hipLaunchKernelGGL(normquant_skeleton_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, in,
                       row_stride, out_q, out_scale, out_kv, M);
    return hipGetLastError();
}

// slab_bytes: a multiple of 16 KB; reads blocks * slab_bytes bytes from w
extern "C" int mi_ceiling_weight_stream(const uint8_t *w, int64_t slab_bytes, int64_t blocks, unsigned *sink,
                                        hipStream_t stream) {
    if (slab_bytes <= 0 || slab_bytes % kStageBytes != 0 || blocks <= 0 || blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const size_t lds = static_cast<size_t>(kRing) * kStageBytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(weight_stream_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(weight_stream_kernel, dim3(static_cast<unsigned>(blocks)), dim3(512), lds, stream, w,
                       slab_bytes, sink);
    return hipGetLastError();
}
