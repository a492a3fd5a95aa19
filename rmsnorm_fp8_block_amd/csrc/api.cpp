// api.cpp -- the C ABI declared in include/mi_normquant.h: argument
// validation on the host, then one kernel launch on the caller's stream.
#include "mi_normquant.h"

#include "launch.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

namespace {

// Shape, pointer and stride checks of the dual norm-quant (MI_OK with
// *empty set for M == 0), and its kernel parameters.
mi_status dual_params(const uint16_t *q, int64_t q_row_stride, const uint16_t *kv, int64_t kv_row_stride,
                      const uint16_t *gamma_q, const uint16_t *gamma_kv, float eps, int64_t M, int64_t Nq,
                      int64_t Nkv, int transpose_scale, uint8_t *out_q_fp8, float *out_scale,
                      uint8_t *out_scale_e8m0, bool e8m0, uint16_t *out_kv, mi::NormQuantParams &p, bool &empty) {
    empty = false;
    if (M < 0 || Nq < MI_GROUP || Nq > MI_MAX_NQ || (Nq % MI_GROUP) != 0 || Nkv < 1 ||
        Nkv > MI_MAX_NKV)
        return MI_ERR_SHAPE;
    if (M == 0) {
        empty = true;
        return MI_OK;
    }
    if (!q || !kv || !gamma_q || !gamma_kv || !out_q_fp8 || !(e8m0 ? out_scale_e8m0 != nullptr : out_scale != nullptr) ||
        !out_kv)
        return MI_ERR_NULL;
    if (q_row_stride < Nq || kv_row_stride < Nkv)
        return MI_ERR_STRIDE;

    p.q = q;
    p.q_stride = q_row_stride;
    p.kv = kv;
    p.kv_stride = kv_row_stride;
    p.gamma_q = gamma_q;
    p.gamma_kv = gamma_kv;
    p.eps = eps;
    p.inv_nq = static_cast<float>(1.0 / static_cast<double>(Nq));
    p.inv_nkv = static_cast<float>(1.0 / static_cast<double>(Nkv));
    p.M = M;
    p.Nq = static_cast<int>(Nq);
    p.Nkv = static_cast<int>(Nkv);
    p.transpose_scale = transpose_scale ? 1 : 0;
    p.out_q = out_q_fp8;
    p.out_scale = out_scale;
    p.out_kv = out_kv;
    p.out_scale_e8m0 = out_scale_e8m0;
    return MI_OK;
}

// e8m0: scales to out_scale_e8m0 (exponent bytes), else to out_scale (fp32)
mi_status dual_normquant(const uint16_t *q, int64_t q_row_stride, const uint16_t *kv, int64_t kv_row_stride,
                         const uint16_t *gamma_q, const uint16_t *gamma_kv, float eps, int64_t M, int64_t Nq,
                         int64_t Nkv, int transpose_scale, uint8_t *out_q_fp8, float *out_scale,
                         uint8_t *out_scale_e8m0, bool e8m0, uint16_t *out_kv, hipStream_t stream) {
    mi::NormQuantParams p;
    bool empty = false;
    const mi_status st = dual_params(q, q_row_stride, kv, kv_row_stride, gamma_q, gamma_kv, eps, M, Nq, Nkv,
                                     transpose_scale, out_q_fp8, out_scale, out_scale_e8m0, e8m0, out_kv, p, empty);
    if (st != MI_OK || empty)
        return st;
    const hipError_t e = e8m0 ? mi::launch_normquant_e8m0(p, stream) : mi::launch_normquant(p, stream);
    return e == hipSuccess ? MI_OK : MI_ERR_HIP;
}

}  // namespace

extern "C" mi_status mi_fused_dual_rmsnorm_group_quant(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q_fp8, float *out_scale, uint16_t *out_kv,
    hipStream_t stream) {
    return dual_normquant(q, q_row_stride, kv, kv_row_stride, gamma_q, gamma_kv, eps, M, Nq, Nkv, transpose_scale,
                          out_q_fp8, out_scale, nullptr, false, out_kv, stream);
}

extern "C" mi_status mi_fused_dual_rmsnorm_group_quant_e8m0(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q_fp8, uint8_t *out_scale_e8m0, uint16_t *out_kv,
    hipStream_t stream) {
    return dual_normquant(q, q_row_stride, kv, kv_row_stride, gamma_q, gamma_kv, eps, M, Nq, Nkv, transpose_scale,
                          out_q_fp8, nullptr, out_scale_e8m0, true, out_kv, stream);
}

namespace {

mi_status single_input_quant(const uint16_t *x, int64_t x_row_stride, const uint16_t *gamma, float eps,
                             int64_t M, int64_t N, int transpose_scale, uint8_t *out_fp8,
                             float *out_scale, bool normalize, hipStream_t stream) {
    if (M < 0 || N < MI_GROUP || N > MI_MAX_N_SINGLE || (N % MI_GROUP) != 0)
        return MI_ERR_SHAPE;
    if (M == 0)
        return MI_OK;
    if (!x || (normalize && !gamma) || !out_fp8 || !out_scale)
        return MI_ERR_NULL;
    if (x_row_stride < N)
        return MI_ERR_STRIDE;

    mi::NormQuantParams p = {};
    p.q = x;
    p.q_stride = x_row_stride;
    p.gamma_q = gamma;
    p.eps = eps;
    p.inv_nq = static_cast<float>(1.0 / static_cast<double>(N));
    p.M = M;
    p.Nq = static_cast<int>(N);
    p.transpose_scale = transpose_scale ? 1 : 0;
    p.out_q = out_fp8;
    p.out_scale = out_scale;
    return mi::launch_group_quant(p, normalize, stream) == hipSuccess ? MI_OK : MI_ERR_HIP;
}

}  // namespace

extern "C" mi_status mi_rmsnorm_group_quant(
    const uint16_t *x, int64_t x_row_stride, const uint16_t *gamma,
    float eps, int64_t M, int64_t N, int transpose_scale,
    uint8_t *out_fp8, float *out_scale,
    hipStream_t stream) {
    return single_input_quant(x, x_row_stride, gamma, eps, M, N, transpose_scale, out_fp8, out_scale, true,
                              stream);
}

extern "C" mi_status mi_group_quant_1x128(
    const uint16_t *x, int64_t x_row_stride,
    int64_t M, int64_t N, int transpose_scale,
    uint8_t *out_fp8, float *out_scale,
    hipStream_t stream) {
    return single_input_quant(x, x_row_stride, nullptr, 0.0f, M, N, transpose_scale, out_fp8, out_scale, false,
                              stream);
}

extern "C" mi_status mi_block_scaled_fp8_gemm_ex(
    const uint8_t *a_fp8, const float *a_scale, int a_scale_transposed,
    const uint8_t *w_fp8, int w_layout, const float *w_scale,
    uint16_t *out_bf16,
    int64_t M, int64_t N, int64_t K,
    hipStream_t stream) {
    if (w_layout != MI_WEIGHT_ROW_MAJOR && w_layout != MI_WEIGHT_TILED)
        return MI_ERR_LAYOUT;
    if (M < 0 || N <= 0 || K <= 0 || (N % MI_GROUP) != 0 || (K % MI_GROUP) != 0)
        return MI_ERR_SHAPE;
    if (M == 0)
        return MI_OK;
    if (!a_fp8 || !a_scale || !w_fp8 || !w_scale || !out_bf16)
        return MI_ERR_NULL;
    if (!aligned16(a_fp8) || !aligned16(w_fp8) || !aligned16(out_bf16) ||
        (reinterpret_cast<uintptr_t>(a_scale) & 3) || (reinterpret_cast<uintptr_t>(w_scale) & 3))
        return MI_ERR_ALIGN;

    mi::GemmParams p;
    p.a = a_fp8;
    p.a_scale = a_scale;
    p.a_scale_transposed = a_scale_transposed ? 1 : 0;
    p.w = w_fp8;
    p.w_scale = w_scale;
    p.out = out_bf16;
    p.M = M;
    p.N = N;
    p.K = K;
    p.w_tiled = w_layout == MI_WEIGHT_TILED ? 1 : 0;
    return mi::launch_block_scaled_gemm(p, stream) == hipSuccess ? MI_OK : MI_ERR_HIP;
}

extern "C" mi_status mi_block_scaled_fp8_gemm(
    const uint8_t *a_fp8, const float *a_scale, int a_scale_transposed,
    const uint8_t *w_fp8, const float *w_scale,
    uint16_t *out_bf16,
    int64_t M, int64_t N, int64_t K,
    hipStream_t stream) {
    return mi_block_scaled_fp8_gemm_ex(a_fp8, a_scale, a_scale_transposed, w_fp8, MI_WEIGHT_ROW_MAJOR, w_scale,
                                       out_bf16, M, N, K, stream);
}

extern "C" mi_status mi_block_scaled_fp8_gemm_pair_ex(
    const uint8_t *a_fp8, const float *a_scale, int a_scale_transposed, int w_layout,
    const uint8_t *w1_fp8, const float *w1_scale, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const float *w2_scale, uint16_t *out2_bf16, int64_t N2,
    int64_t M, int64_t K,
    hipStream_t stream) {
    if (w_layout != MI_WEIGHT_ROW_MAJOR && w_layout != MI_WEIGHT_TILED)
        return MI_ERR_LAYOUT;
    if (M < 0 || N1 <= 0 || N2 <= 0 || K <= 0 || (N1 % MI_GROUP) != 0 || (N2 % MI_GROUP) != 0 ||
        (K % MI_GROUP) != 0)
        return MI_ERR_SHAPE;
    if (M == 0)
        return MI_OK;
    if (!a_fp8 || !a_scale || !w1_fp8 || !w1_scale || !out1_bf16 || !w2_fp8 || !w2_scale || !out2_bf16)
        return MI_ERR_NULL;
    if (!aligned16(a_fp8) || !aligned16(w1_fp8) || !aligned16(out1_bf16) || !aligned16(w2_fp8) ||
        !aligned16(out2_bf16) || (reinterpret_cast<uintptr_t>(a_scale) & 3) ||
        (reinterpret_cast<uintptr_t>(w1_scale) & 3) || (reinterpret_cast<uintptr_t>(w2_scale) & 3))
        return MI_ERR_ALIGN;

    mi::GemmParams p;
    p.a = a_fp8;
    p.a_scale = a_scale;
    p.a_scale_transposed = a_scale_transposed ? 1 : 0;
    p.w = w1_fp8;
    p.w_scale = w1_scale;
    p.out = out1_bf16;
    p.M = M;
    p.N = N1;
    p.K = K;
    p.w2 = w2_fp8;
    p.w_scale2 = w2_scale;
    p.out2 = out2_bf16;
    p.N2 = N2;
    p.w_tiled = w_layout == MI_WEIGHT_TILED ? 1 : 0;
    return mi::launch_block_scaled_gemm_pair(p, stream) == hipSuccess ? MI_OK : MI_ERR_HIP;
}

extern "C" mi_status mi_block_scaled_fp8_gemm_pair(
    const uint8_t *a_fp8, const float *a_scale, int a_scale_transposed,
    const uint8_t *w1_fp8, const float *w1_scale, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const float *w2_scale, uint16_t *out2_bf16, int64_t N2,
    int64_t M, int64_t K,
    hipStream_t stream) {
    return mi_block_scaled_fp8_gemm_pair_ex(a_fp8, a_scale, a_scale_transposed, MI_WEIGHT_ROW_MAJOR, w1_fp8,
                                            w1_scale, out1_bf16, N1, w2_fp8, w2_scale, out2_bf16, N2, M, K, stream);
}

namespace {

// the whole step; e8m0 selects exponent-byte scales on both sides (out_scale_e8m0, w*_scale8),
// else fp32 scales (out_scale, w*_scale)
mi_status fused_step(const uint16_t *q, int64_t q_row_stride, const uint16_t *kv, int64_t kv_row_stride,
                     const uint16_t *gamma_q, const uint16_t *gamma_kv, float eps, int64_t M, int64_t Nq,
                     int64_t Nkv, int transpose_scale, uint8_t *out_q_fp8, float *out_scale,
                     uint8_t *out_scale_e8m0, bool e8m0, uint16_t *out_kv, int w_layout, const uint8_t *w1_fp8,
                     const float *w1_scale, const uint8_t *w1_scale8, uint16_t *out1_bf16, int64_t N1,
                     const uint8_t *w2_fp8, const float *w2_scale, const uint8_t *w2_scale8, uint16_t *out2_bf16,
                     int64_t N2, hipStream_t stream) {
    if (w_layout != MI_WEIGHT_ROW_MAJOR && w_layout != MI_WEIGHT_TILED)
        return MI_ERR_LAYOUT;
    if (N1 <= 0 || N2 <= 0 || (N1 % MI_GROUP) != 0 || (N2 % MI_GROUP) != 0)
        return MI_ERR_SHAPE;
    mi::NormQuantParams a;
    bool empty = false;
    const mi_status st = dual_params(q, q_row_stride, kv, kv_row_stride, gamma_q, gamma_kv, eps, M, Nq, Nkv,
                                     transpose_scale, out_q_fp8, out_scale, out_scale_e8m0, e8m0, out_kv, a, empty);
    if (st != MI_OK || empty)
        return st;
    const void *ws1 = e8m0 ? static_cast<const void *>(w1_scale8) : static_cast<const void *>(w1_scale);
    const void *ws2 = e8m0 ? static_cast<const void *>(w2_scale8) : static_cast<const void *>(w2_scale);
    const void *as = e8m0 ? static_cast<const void *>(out_scale_e8m0) : static_cast<const void *>(out_scale);
    if (!w1_fp8 || !ws1 || !out1_bf16 || !w2_fp8 || !ws2 || !out2_bf16)
        return MI_ERR_NULL;
    if (!aligned16(out_q_fp8) || !aligned16(w1_fp8) || !aligned16(out1_bf16) || !aligned16(w2_fp8) ||
        !aligned16(out2_bf16) || (reinterpret_cast<uintptr_t>(as) & 3) || (reinterpret_cast<uintptr_t>(ws1) & 3) ||
        (reinterpret_cast<uintptr_t>(ws2) & 3))
        return MI_ERR_ALIGN;

    mi::GemmParams p = {};
    p.a = out_q_fp8;
    p.a_scale_transposed = a.transpose_scale;
    p.w = w1_fp8;
    p.out = out1_bf16;
    p.M = M;
    p.N = N1;
    p.K = Nq;
    p.w2 = w2_fp8;
    p.out2 = out2_bf16;
    p.N2 = N2;
    p.w_tiled = w_layout == MI_WEIGHT_TILED ? 1 : 0;
    if (e8m0) {
        p.scale_e8m0 = 1;
        p.a_scale8 = out_scale_e8m0;
        p.w_scale8 = w1_scale8;
        p.w_scale8_2 = w2_scale8;
    } else {
        p.a_scale = out_scale;
        p.w_scale = w1_scale;
        p.w_scale2 = w2_scale;
    }
    hipError_t e = mi::launch_normquant_gemm_pair(a, p, stream);
    if (e == hipErrorNotSupported) {  // two launches
        e = e8m0 ? mi::launch_normquant_e8m0(a, stream) : mi::launch_normquant(a, stream);
        if (e == hipSuccess)
            e = mi::launch_block_scaled_gemm_pair(p, stream);
    }
    return e == hipSuccess ? MI_OK : MI_ERR_HIP;
}

}  // namespace

extern "C" mi_status mi_fused_normquant_gemm_pair(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q_fp8, float *out_scale, uint16_t *out_kv,
    int w_layout,
    const uint8_t *w1_fp8, const float *w1_scale, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const float *w2_scale, uint16_t *out2_bf16, int64_t N2,
    hipStream_t stream) {
    return fused_step(q, q_row_stride, kv, kv_row_stride, gamma_q, gamma_kv, eps, M, Nq, Nkv, transpose_scale,
                      out_q_fp8, out_scale, nullptr, false, out_kv, w_layout, w1_fp8, w1_scale, nullptr, out1_bf16,
                      N1, w2_fp8, w2_scale, nullptr, out2_bf16, N2, stream);
}

extern "C" mi_status mi_fused_normquant_gemm_pair_e8m0(
    const uint16_t *q, int64_t q_row_stride,
    const uint16_t *kv, int64_t kv_row_stride,
    const uint16_t *gamma_q, const uint16_t *gamma_kv,
    float eps, int64_t M, int64_t Nq, int64_t Nkv,
    int transpose_scale,
    uint8_t *out_q_fp8, uint8_t *out_scale_e8m0, uint16_t *out_kv,
    int w_layout,
    const uint8_t *w1_fp8, const uint8_t *w1_scale_e8m0, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const uint8_t *w2_scale_e8m0, uint16_t *out2_bf16, int64_t N2,
    hipStream_t stream) {
    return fused_step(q, q_row_stride, kv, kv_row_stride, gamma_q, gamma_kv, eps, M, Nq, Nkv, transpose_scale,
                      out_q_fp8, nullptr, out_scale_e8m0, true, out_kv, w_layout, w1_fp8, nullptr, w1_scale_e8m0,
                      out1_bf16, N1, w2_fp8, nullptr, w2_scale_e8m0, out2_bf16, N2, stream);
}

extern "C" int mi_fused_normquant_gemm_pair_launches(int64_t M, int64_t Nq, int64_t Nkv, int64_t N1, int64_t N2) {
    if (M < 0 || Nq < MI_GROUP || Nq > MI_MAX_NQ || (Nq % MI_GROUP) != 0 || Nkv < 1 || Nkv > MI_MAX_NKV ||
        N1 <= 0 || N2 <= 0 || (N1 % MI_GROUP) != 0 || (N2 % MI_GROUP) != 0)
        return -1;
    if (M == 0)
        return 0;
    return mi::normquant_gemm_pair_one_launch(M, Nq, Nkv, N1, N2) ? 1 : 1 + mi::gemm_pair_launches(M, Nq, N1, N2);
}

extern "C" mi_status mi_block_scaled_fp8_gemm_e8m0(
    const uint8_t *a_fp8, const uint8_t *a_scale_e8m0, int a_scale_transposed,
    const uint8_t *w_fp8, int w_layout, const uint8_t *w_scale_e8m0,
    uint16_t *out_bf16,
    int64_t M, int64_t N, int64_t K,
    hipStream_t stream) {
    if (w_layout != MI_WEIGHT_ROW_MAJOR && w_layout != MI_WEIGHT_TILED)
        return MI_ERR_LAYOUT;
    if (M < 0 || N <= 0 || K <= 0 || (N % MI_GROUP) != 0 || (K % MI_GROUP) != 0)
        return MI_ERR_SHAPE;
    if (M == 0)
        return MI_OK;
    if (!a_fp8 || !a_scale_e8m0 || !w_fp8 || !w_scale_e8m0 || !out_bf16)
        return MI_ERR_NULL;
    if (!aligned16(a_fp8) || !aligned16(w_fp8) || !aligned16(out_bf16) ||
        (reinterpret_cast<uintptr_t>(a_scale_e8m0) & 3) || (reinterpret_cast<uintptr_t>(w_scale_e8m0) & 3))
        return MI_ERR_ALIGN;
    mi::GemmParams p = {};
    p.a = a_fp8;
    p.a_scale_transposed = a_scale_transposed ? 1 : 0;
    p.w = w_fp8;
    p.out = out_bf16;
    p.M = M;
    p.N = N;
    p.K = K;
    p.w_tiled = w_layout == MI_WEIGHT_TILED ? 1 : 0;
    p.scale_e8m0 = 1;
    p.a_scale8 = a_scale_e8m0;
    p.w_scale8 = w_scale_e8m0;
    return mi::launch_block_scaled_gemm(p, stream) == hipSuccess ? MI_OK : MI_ERR_HIP;
}

extern "C" mi_status mi_block_scaled_fp8_gemm_pair_e8m0(
    const uint8_t *a_fp8, const uint8_t *a_scale_e8m0, int a_scale_transposed, int w_layout,
    const uint8_t *w1_fp8, const uint8_t *w1_scale_e8m0, uint16_t *out1_bf16, int64_t N1,
    const uint8_t *w2_fp8, const uint8_t *w2_scale_e8m0, uint16_t *out2_bf16, int64_t N2,
    int64_t M, int64_t K,
    hipStream_t stream) {
    if (w_layout != MI_WEIGHT_ROW_MAJOR && w_layout != MI_WEIGHT_TILED)
        return MI_ERR_LAYOUT;
    if (M < 0 || N1 <= 0 || N2 <= 0 || K <= 0 || (N1 % MI_GROUP) != 0 || (N2 % MI_GROUP) != 0 ||
        (K % MI_GROUP) != 0)
        return MI_ERR_SHAPE;
    if (M == 0)
        return MI_OK;
    if (!a_fp8 || !a_scale_e8m0 || !w1_fp8 || !w1_scale_e8m0 || !out1_bf16 || !w2_fp8 || !w2_scale_e8m0 ||
        !out2_bf16)
        return MI_ERR_NULL;
    if (!aligned16(a_fp8) || !aligned16(w1_fp8) || !aligned16(out1_bf16) || !aligned16(w2_fp8) ||
        !aligned16(out2_bf16) || (reinterpret_cast<uintptr_t>(a_scale_e8m0) & 3) ||
        (reinterpret_cast<uintptr_t>(w1_scale_e8m0) & 3) || (reinterpret_cast<uintptr_t>(w2_scale_e8m0) & 3))
        return MI_ERR_ALIGN;
    mi::GemmParams p = {};
    p.a = a_fp8;
    p.a_scale_transposed = a_scale_transposed ? 1 : 0;
    p.w = w1_fp8;
    p.out = out1_bf16;
    p.M = M;
    p.N = N1;
    p.K = K;
    p.w2 = w2_fp8;
    p.out2 = out2_bf16;
    p.N2 = N2;
    p.w_tiled = w_layout == MI_WEIGHT_TILED ? 1 : 0;
    p.scale_e8m0 = 1;
    p.a_scale8 = a_scale_e8m0;
    p.w_scale8 = w1_scale_e8m0;
    p.w_scale8_2 = w2_scale_e8m0;
    return mi::launch_block_scaled_gemm_pair(p, stream) == hipSuccess ? MI_OK : MI_ERR_HIP;
}

extern "C" unsigned mi_gemm_capabilities(void) {
    return MI_CAP_AS_ROW_MAJOR | MI_CAP_AS_COL_MAJOR | MI_CAP_WEIGHT_TILED | MI_CAP_SCALE_E8M0;
}

extern "C" int mi_preferred_weight_layout(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || (N % MI_GROUP) != 0 || (K % MI_GROUP) != 0)
        return -1;
    return MI_WEIGHT_TILED;
}

extern "C" mi_status mi_relayout_weight(const uint8_t *src, int from_layout, uint8_t *dst, int to_layout,
                                        int64_t N, int64_t K, hipStream_t stream) {
    const auto known = [](int l) { return l == MI_WEIGHT_ROW_MAJOR || l == MI_WEIGHT_TILED; };
    if (!known(from_layout) || !known(to_layout))
        return MI_ERR_LAYOUT;
    if (N < 0 || K < 0 || (N % 16) != 0 || (K % MI_GROUP) != 0)
        return MI_ERR_SHAPE;
    if (N == 0 || K == 0)
        return MI_OK;
    if (!src || !dst)
        return MI_ERR_NULL;
    if (src == dst)
        return MI_ERR_ALIAS;
    if (!aligned16(src) || !aligned16(dst))
        return MI_ERR_ALIGN;
    if (from_layout == to_layout)
        return hipMemcpyAsync(dst, src, static_cast<size_t>(N * K), hipMemcpyDeviceToDevice, stream) == hipSuccess
                   ? MI_OK
                   : MI_ERR_HIP;
    return mi::launch_weight_relayout(src, dst, N, K, to_layout == MI_WEIGHT_TILED, stream) == hipSuccess
               ? MI_OK
               : MI_ERR_HIP;
}

extern "C" mi_status mi_init(void) { return mi::init_device() == hipSuccess ? MI_OK : MI_ERR_HIP; }

extern "C" int mi_negotiate_scale_layout(const int *consumer_wants_transposed, int n) {
    if (!consumer_wants_transposed || n <= 0)
        return -1;
    const int first = consumer_wants_transposed[0] ? 1 : 0;
    for (int i = 1; i < n; ++i)
        if ((consumer_wants_transposed[i] ? 1 : 0) != first)
            return -1;
    return first;
}

extern "C" const char *mi_status_string(mi_status s) {
    switch (s) {
    case MI_OK:
        return "MI_OK";
    case MI_ERR_NULL:
        return "MI_ERR_NULL: a required pointer is NULL";
    case MI_ERR_SHAPE:
        return "MI_ERR_SHAPE: unsupported size";
    case MI_ERR_STRIDE:
        return "MI_ERR_STRIDE: row stride smaller than the row width";
    case MI_ERR_ALIGN:
        return "MI_ERR_ALIGN: operand not 16-byte aligned";
    case MI_ERR_HIP:
        return "MI_ERR_HIP: kernel launch failed";
    case MI_ERR_ALIAS:
        return "MI_ERR_ALIAS: an output is the same buffer as an input";
    case MI_ERR_LAYOUT:
        return "MI_ERR_LAYOUT: unknown layout value";
    }
    return "unknown mi_status";
}
