"""The fused kernel against the pre-fusion pipeline it replaces, in the
dequantised domain (PRHub digest of vLLM PR #53540, "实现拆解": the fused
RMSNorm + group quant checked against the sequential norm -> bf16 -> quant
path within an error budget of the dequantised values; the GitHub page of
the same PR, "Purpose": the fused kernel quantises straight from the fp32
normalised values, the old pipeline from their bf16 rounding).

The device's fused outputs (codes x scales) are compared with the oracle's
sequential mode (the normalised q rounded to bf16, then the per-1x128
quant) on the decode cases: M = 1 (separate q / kv buffers) and the M = 64
strided batch, both scale layouts.  The pages name the budget but give no
number; the one used here follows from the half-ULP bounds of the two
paths (each dequantised value is within half an e4m3 ULP times its scale
of the value it quantised, and the bf16 rounding of the sequential path
moves y by at most half a bf16 ULP, 2^-8 |y| at worst):
    |deq_fused - deq_sequential| <= ulp_e4m3(|y| / s) * s + 2^-8 |y|
per element, with y the exact normalised value and the larger of the two
paths' ULPs and scales, and every scale within 2^-8 relative of the
sequential one; both with a 2^-10 relative margin for the fused kernel's
fp32 arithmetic.  The worst case is reached (a group maximum half a bf16 ULP
from its rounding), so the budget is tight by construction; the largest use
of it is printed."""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_fp8_block_amd as mi
from rmsnorm_fp8_block_amd import workloads as W

from helpers import bf16_ord, dev_u16_as_bf16, gpu_or_skip, host_bf16_bits

pytestmark = pytest.mark.gpu


def e4m3_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of e4m3fn values at magnitude v: 2^(e-3) in binade [2^e,
    2^(e+1)), 2^-9 below 2^-6 (subnormals)."""
    v = np.maximum(np.abs(v), 2.0 ** -6)
    return 2.0 ** (np.floor(np.log2(v)) - 3)


def device_fused(case, transpose, dev):
    if case.buffer is not None:
        buf = dev_u16_as_bf16(case.buffer, dev)
        q, kv = buf[:, :case.q.shape[1]], buf[:, case.q.shape[1]:]
    else:
        q, kv = dev_u16_as_bf16(case.q, dev), dev_u16_as_bf16(case.kv, dev)
    gq, gk = dev_u16_as_bf16(case.gamma_q, dev), dev_u16_as_bf16(case.gamma_kv, dev)
    codes, scale, kv_out = mi.mi_fused_dual_rmsnorm_group_quant(q, kv, gq, gk, case.eps, transpose)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scale.cpu().numpy().astype(np.float64), host_bf16_bits(kv_out)


@pytest.mark.parametrize("name", ["decode_M1", "strided_M64"])
@pytest.mark.parametrize("transpose", [False, True])
def test_fused_within_budget_of_sequential(name, transpose):
    dev = gpu_or_skip()
    case = W.decode_single() if name == "decode_M1" else W.strided_batch(64)
    M, Nq = case.q.shape
    G = Nq // 128
    codes, s_f, kv_f = device_fused(case, transpose, dev)
    seq = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, case.eps, transpose,
                                          sequential=True)
    exact = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, case.eps, transpose,
                                            want_ratio=True)
    as_mg = (lambda b: b.reshape(G, M).T) if transpose else (lambda b: b.reshape(M, G))
    s_s = as_mg(seq["scale"]).astype(np.float64)
    y = exact["y"]
    rep = lambda s: np.repeat(s, 128, axis=1)
    deq_f = oracle.e4m3_decode_array(codes) * rep(s_f)
    deq_s = oracle.e4m3_decode_array(seq["q"]) * rep(s_s)
    ulp = np.maximum(e4m3_ulp(np.abs(y) / rep(s_f)), e4m3_ulp(np.abs(y) / rep(s_s)))
    budget = ulp * np.maximum(rep(s_f), rep(s_s)) + 2.0 ** -8 * np.abs(y)
    used = np.abs(deq_f - deq_s) / budget
    scale_rel = np.abs(s_f / s_s - 1.0)
    print(f"{name} transpose={transpose}: largest use of the dequantised budget {used.max():.3f}, "
          f"largest scale difference {scale_rel.max():.2e} (budget 2^-8 = {2.0 ** -8:.2e}), "
          f"codes identical to the sequential path {np.mean(codes == seq['q']):.4f}")
    assert used.max() <= 1.0 + 2.0 ** -10, f"dequantised difference over budget by {used.max():.3f}x"
    assert scale_rel.max() <= 2.0 ** -8 * (1.0 + 2.0 ** -10)
    # kv: both pipelines round the normalised kv to bf16 once (the device in
    # fp32: within one bf16 ULP of the exact rounding)
    assert np.abs(bf16_ord(kv_f) - bf16_ord(seq["kv"])).max() <= 1
