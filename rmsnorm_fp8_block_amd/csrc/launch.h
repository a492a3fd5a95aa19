// launch.h -- host-side launchers behind the C ABI (internal).  Arguments
// have been validated by the caller; these only pick a kernel variant and a
// grid and enqueue it.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mi {

struct NormQuantParams {
    const uint16_t *q;
    int64_t q_stride;
    const uint16_t *kv;
    int64_t kv_stride;
    const uint16_t *gamma_q;
    const uint16_t *gamma_kv;
    float eps;
    float inv_nq;   // 1 / Nq and 1 / Nkv, rounded to fp32
    float inv_nkv;
    int64_t M;
    int Nq;
    int Nkv;
    int transpose_scale;
    uint8_t *out_q;
    float *out_scale;
    uint16_t *out_kv;
    // e8m0 mode: power-of-two scales, one exponent byte each, written here
    // (out_scale unused)
    uint8_t *out_scale_e8m0 = nullptr;
};

struct GemmParams {
    const uint8_t *a;
    const float *a_scale;
    int a_scale_transposed;
    const uint8_t *w;
    const float *w_scale;
    uint16_t *out;
    int64_t M;
    int64_t N;
    int64_t K;
    // optional second consumer of the same activations (N2 == 0: none);
    // its 16-row subtiles follow those of w in one subtile index space
    const uint8_t *w2 = nullptr;
    const float *w_scale2 = nullptr;
    uint16_t *out2 = nullptr;
    int64_t N2 = 0;
    // weight byte order of w (and w2): 0 row-major, 1 tiled (see
    // mi_relayout_weight)
    int w_tiled = 0;
    // e8m0 scales: a_scale8 / w_scale8 / w_scale8_2 hold exponent bytes (value
    // 2^(e - 127)) in the layouts of a_scale / w_scale / w_scale2, which are
    // then unused
    int scale_e8m0 = 0;
    const uint8_t *a_scale8 = nullptr;
    const uint8_t *w_scale8 = nullptr;
    const uint8_t *w_scale8_2 = nullptr;
};

hipError_t launch_normquant(const NormQuantParams &p, hipStream_t stream);
// the same with e8m0 scales (p.out_scale_e8m0)
hipError_t launch_normquant_e8m0(const NormQuantParams &p, hipStream_t stream);
// weight [N, K] row-major <-> tiled (to_tiled selects the direction)
hipError_t launch_weight_relayout(const uint8_t *src, uint8_t *dst, int64_t N, int64_t K, bool to_tiled,
                                  hipStream_t stream);
// one input (kv unused): RMSNorm + group quant (normalize) or the group
// quant of q itself (gamma_q, eps unused)
hipError_t launch_group_quant(const NormQuantParams &p, bool normalize, hipStream_t stream);
hipError_t launch_block_scaled_gemm(const GemmParams &p, hipStream_t stream);
// both consumers (p.N2 > 0) in one launch where the shape allows, else two
hipError_t launch_block_scaled_gemm_pair(const GemmParams &p, hipStream_t stream);
// kernel launches launch_block_scaled_gemm_pair makes for M rows, depth K,
// consumers of N1 and N2 rows (on the current device)
int gemm_pair_launches(int64_t M, int64_t K, int64_t N1, int64_t N2);
// the decode step in one launch: the norm-quant of a.M rows and both
// consumer GEMMs of its outputs (p.a / p.a_scale are a.out_q / a.out_scale).
// hipErrorNotSupported where the shapes or alignment do not allow it.
hipError_t launch_normquant_gemm_pair(const NormQuantParams &a, const GemmParams &p, hipStream_t stream);
// on the current device: caches the CU count and raises the dynamic-LDS
// limit of every kernel instance that needs it
hipError_t init_device();
// whether launch_normquant_gemm_pair takes these sizes (alignment aside)
bool normquant_gemm_pair_one_launch(int64_t M, int64_t Nq, int64_t Nkv, int64_t N1, int64_t N2);

}  // namespace mi
