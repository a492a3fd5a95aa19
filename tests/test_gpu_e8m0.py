"""GPU parity of the e8m0 (power-of-two) scale mode against the CPU oracle,
through the C ABI: the fused dual RMSNorm + 1x128 quant with e8m0 scales,
and the block-scaled GEMM whose scaled matrix-core instructions apply e8m0
activation and weight scales (PRHub report of vLLM PR #56433, "风险与影响"
item 3: e8m0 weight scales; PRHub digest of vLLM PR #56560: the native
gfx950 MX GEMM with e8m0 scale exponents).

Bar: kv bit-identical to the fp32-scale call; scale bytes equal to the
oracle's except where the oracle's group maximum / 448 lies within a few
fp32 ulps of a power of two (the exponent may then differ by one, the codes
of that group are not compared); elsewhere codes within 1 e4m3 ULP, any
difference next to a rounding midpoint, >= 99.9 % identical.  GEMM: the
same bound as the fp32-scale GEMM against the fp64 oracle on the decoded
scales, both As layouts bit-identical, tiled = row-major bit for bit, the
pair = two single launches bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_fp8_block_amd as mi
from rmsnorm_fp8_block_amd import workloads as W

from helpers import (assert_gemm_close, bf16_to_f64, compare_e8m0, dev_f32, dev_u8, dev_u16_as_bf16, gpu_or_skip,
                     host_bf16_bits, scale_buffer)

pytestmark = pytest.mark.gpu

def run_case(case, transpose, dev):
    if case.buffer is not None:
        buf = dev_u16_as_bf16(case.buffer, dev)
        q, kv = buf[:, :case.q.shape[1]], buf[:, case.q.shape[1]:]
    else:
        q, kv = dev_u16_as_bf16(case.q, dev), dev_u16_as_bf16(case.kv, dev)
    gq, gk = dev_u16_as_bf16(case.gamma_q, dev), dev_u16_as_bf16(case.gamma_kv, dev)
    codes, scale, kvo = mi.mi_fused_dual_rmsnorm_group_quant_e8m0(q, kv, gq, gk, case.eps, transpose)
    _, _, kv32 = mi.mi_fused_dual_rmsnorm_group_quant(q, kv, gq, gk, case.eps, transpose)
    torch.cuda.synchronize()
    assert torch.equal(kvo, kv32), "kv must equal the fp32-scale call's"
    return codes.cpu().numpy(), scale_buffer(scale), scale


WORKLOADS = {
    "decode_M1": lambda: W.decode_single(),
    "strided_M64": lambda: W.strided_batch(64),
    "outliers_M256": lambda: W.outlier_stress(256),
    "prefill_M8192": lambda: W.prefill(8192),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_normquant_e8m0_workloads(name):
    dev = gpu_or_skip()
    case = WORKLOADS[name]()
    M, G = case.M, case.q.shape[1] // 128
    for t in (0, 1):
        codes, sbytes, _ = run_case(case, t, dev)
        ref = oracle.dual_rmsnorm_group_quant_e8m0(case.q, case.kv, case.gamma_q, case.gamma_kv, case.eps, t,
                                                   want_ratio=True)
        exact, ndiff = compare_e8m0(codes, sbytes, ref, M, G, t, f"{name} t{t}")
        print(f"{name} t={t}: codes exact {exact:.6f}, exponent boundary groups {ndiff}")


@pytest.mark.parametrize("M,Nq,Nkv,seed", [(3, 256, 64, 1), (7, 640, 100, 2), (5, 4096, 2048, 3)])
def test_normquant_e8m0_generic_shapes(M, Nq, Nkv, seed):
    dev = gpu_or_skip()
    r = np.random.default_rng(seed)
    q = W.f32_to_bf16_bits(r.standard_normal((M, Nq)).astype(np.float32))
    kv = W.f32_to_bf16_bits(r.standard_normal((M, Nkv)).astype(np.float32))
    gq = W.f32_to_bf16_bits((1 + 0.1 * r.standard_normal(Nq)).astype(np.float32))
    gk = W.f32_to_bf16_bits((1 + 0.1 * r.standard_normal(Nkv)).astype(np.float32))
    case = W.NormQuantCase("adhoc", q, kv, gq, gk)
    for t in (0, 1):
        codes, sbytes, _ = run_case(case, t, dev)
        ref = oracle.dual_rmsnorm_group_quant_e8m0(q, kv, gq, gk, W.EPS, t, want_ratio=True)
        compare_e8m0(codes, sbytes, ref, M, Nq // 128, t, f"M{M} Nq{Nq} t{t}")


def test_normquant_e8m0_exact_powers_of_two():
    """Constant rows, eps = 0: y = sign(c) gamma with each group's largest
    |gamma| = 448 * 2^k, so amax / 448 is exactly 2^k: the device must pick
    exponent k (not k + 1) and reproduce the oracle's codes exactly."""
    dev = gpu_or_skip()
    r = np.random.default_rng(5)
    Nq, Nkv, M = 1536, 512, 4
    g = (r.uniform(-1, 1, Nq) * 0.9).astype(np.float32)
    for grp in range(12):
        k = int(r.integers(-8, 4))
        g[grp * 128:(grp + 1) * 128] *= np.float32(448 * 2.0 ** k)
        g[grp * 128 + int(r.integers(0, 128))] = np.float32(448 * 2.0 ** k)
    gq = W.f32_to_bf16_bits(g)
    one = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    q = np.full((M, Nq), W.f32_to_bf16_bits(np.array([-1.5], np.float32))[0], np.uint16)
    kv = np.full((M, Nkv), one, np.uint16)
    gk = np.full(Nkv, one, np.uint16)
    case = W.NormQuantCase("pow2", q, kv, gq, gk, eps=0.0)
    codes, sbytes, _ = run_case(case, 0, dev)
    ref = oracle.dual_rmsnorm_group_quant_e8m0(q, kv, gq, gk, 0.0, 0, want_ratio=True)
    assert np.array_equal(sbytes, ref["scale"])
    assert np.array_equal(codes, ref["q"])


def e8m0_operands(M, N, K, seed):
    r = np.random.default_rng(seed)
    a = r.integers(0, 256, size=(M, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38
    As = r.integers(117, 128, size=(M, K // 128)).astype(np.uint8)     # 2^-10 .. 1
    Bs = r.integers(112, 128, size=(N // 128, K // 128)).astype(np.uint8)
    return a, As, w, Bs


def gemm_ref(a, As, w, Bs, cols=None, blocks=None):
    asf = oracle.e8m0_decode_array(As).astype(np.float32)
    bsf = oracle.e8m0_decode_array(Bs).astype(np.float32)
    if cols is not None:
        w, bsf = w[cols], bsf[blocks]
    ref = oracle.block_scaled_fp8_gemm(a, asf.reshape(-1), False, w, bsf)
    mag = (np.abs(oracle.e4m3_decode_array(a)) * np.repeat(asf.astype(np.float64), 128, axis=1)) @ \
        (np.abs(oracle.e4m3_decode_array(w)) * np.kron(bsf.astype(np.float64), np.ones((128, 128)))).T
    return ref, mag


# decode-size batches (the wide kernel), 64 < M <= 256 (wide, row split for
# narrow weights), M > 256 and K / 128 = 5 (the generic kernel)
# (two subtiles per CU at M <= 16: the stream kernel with one subtile per wave;
# 200 and 256 rows of 8192 and 12288 weight rows: the stream kernel in 64-row chunks;
# the wide kernel's narrow-weight blocks: one subtile per block at 40 rows of 3072,
# three subtiles per block at 32 rows of 12288, 64-row chunks of three-subtile slabs
# at 256 rows of 3072, three-subtile slabs of half the rows at 200 rows of 6144)
@pytest.mark.parametrize("M,N,K,seed", [(1, 24576, 1536, 1), (16, 8192, 1536, 2), (64, 1024, 512, 3),
                                        (100, 1536, 1536, 4), (256, 6144, 1536, 5), (300, 640, 1536, 6),
                                        (40, 384, 640, 7), (64, 2048, 2048, 8), (1, 6144, 1536, 9),
                                        (16, 6144, 1536, 10), (200, 8192, 1536, 11), (256, 12288, 1536, 12),
                                        (40, 3072, 1536, 13), (32, 12288, 1536, 14), (256, 3072, 1536, 15),
                                        (200, 6144, 1536, 16)])
def test_gemm_e8m0_vs_oracle(M, N, K, seed):
    dev = gpu_or_skip()
    a, As, w, Bs = e8m0_operands(M, N, K, seed)
    nb = N // 128
    blocks = np.unique([0, nb // 2, nb - 1])
    cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    ref, mag = gemm_ref(a, As, w, Bs, cols, blocks)
    da, dw, dbs = dev_u8(a, dev), dev_u8(w, dev), dev_u8(Bs, dev)
    tw = mi.relayout_weight(dw)
    outs = []
    for t in (False, True):
        das = dev_u8(As.T.copy(), dev).T if t else dev_u8(As, dev)
        out = mi.mi_block_scaled_fp8_gemm(da, das, dw, dbs)
        out_t = mi.mi_block_scaled_fp8_gemm(da, das, tw, dbs)
        torch.cuda.synchronize()
        got = bf16_to_f64(out)[:, cols]
        assert_gemm_close(got, ref, f"e8m0 M{M} N{N} K{K} t{t}")
        err = np.abs(got - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * mag), f"M{M} N{N} K{K} t{t}"
        assert np.array_equal(host_bf16_bits(out), host_bf16_bits(out_t)), "tiled must equal row-major"
        outs.append(host_bf16_bits(out))
    assert np.array_equal(outs[0], outs[1]), "row- and column-major As must give identical bits"


@pytest.mark.parametrize("M", [1, 16, 64, 100])
def test_gemm_pair_e8m0_equals_two_gemms(M):
    dev = gpu_or_skip()
    wa = W.block_fp8_weight_e8m0(*W.W_A_SHAPE, W.W_A_SEED)
    wb = W.block_fp8_weight_e8m0(*W.W_B_SHAPE, W.W_B_SEED)
    r = np.random.default_rng(M)
    a = dev_u8(r.integers(0, 0x78, size=(M, 1536), dtype=np.uint8), dev)
    As = dev_u8(r.integers(118, 127, size=(12, M)).astype(np.uint8), dev).T
    dwa, dwb = mi.relayout_weight(dev_u8(wa.codes, dev)), mi.relayout_weight(dev_u8(wb.codes, dev))
    sa, sb = dev_u8(wa.scale, dev), dev_u8(wb.scale, dev)
    o1, o2 = mi.mi_block_scaled_fp8_gemm_pair(a, As, dwa, sa, dwb, sb)
    s1 = mi.mi_block_scaled_fp8_gemm(a, As, dwa, sa)
    s2 = mi.mi_block_scaled_fp8_gemm(a, As, dwb, sb)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(o1), host_bf16_bits(s1))
    assert np.array_equal(host_bf16_bits(o2), host_bf16_bits(s2))


@pytest.mark.parametrize("M", [1, 16])
def test_gemm_pair_e8m0_tp4_shard_equals_two_gemms(M):
    """The TP-4 shard of both weights (W_a rows 18432.., W_b rows 6144..):
    the pair is one launch with two subtiles per CU, the W_b shard alone
    another kernel; the outputs must agree bit for bit."""
    dev = gpu_or_skip()
    wa = W.block_fp8_weight_e8m0(*W.W_A_SHAPE, W.W_A_SEED)
    wb = W.block_fp8_weight_e8m0(*W.W_B_SHAPE, W.W_B_SEED)
    na, nb = W.W_A_SHAPE[0] // 4, W.W_B_SHAPE[0] // 4
    r = np.random.default_rng(40 + M)
    a = dev_u8(r.integers(0, 0x78, size=(M, 1536), dtype=np.uint8), dev)
    As = dev_u8(r.integers(118, 127, size=(12, M)).astype(np.uint8), dev).T
    dwa = mi.relayout_weight(dev_u8(wa.codes[3 * na:], dev))
    dwb = mi.relayout_weight(dev_u8(wb.codes[3 * nb:], dev))
    sa, sb = dev_u8(wa.scale[3 * na // 128:], dev), dev_u8(wb.scale[3 * nb // 128:], dev)
    o1, o2 = mi.mi_block_scaled_fp8_gemm_pair(a, As, dwa, sa, dwb, sb)
    s1 = mi.mi_block_scaled_fp8_gemm(a, As, dwa, sa)
    s2 = mi.mi_block_scaled_fp8_gemm(a, As, dwb, sb)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(o1), host_bf16_bits(s1))
    assert np.array_equal(host_bf16_bits(o2), host_bf16_bits(s2))


@pytest.mark.parametrize("M", [1, 64, 256])
def test_producer_and_two_consumers_e8m0(M):
    """e8m0 norm-quant of the first M rows of a [256, 2048] buffer, both
    consumers with e8m0 weights in one launch (or two at M > 64); the oracle
    chain is the e8m0 oracle quant followed by the fp64 GEMM on decoded
    scales, compared on sampled column blocks."""
    dev = gpu_or_skip()
    case = W.producer_activations(M)
    buf = dev_u16_as_bf16(case.buffer, dev)
    codes, scale, _ = mi.mi_fused_dual_rmsnorm_group_quant_e8m0(
        buf[:, :W.NQ], buf[:, W.NQ:], dev_u16_as_bf16(case.gamma_q, dev), dev_u16_as_bf16(case.gamma_kv, dev),
        W.EPS, True)
    qref = oracle.dual_rmsnorm_group_quant_e8m0(case.q, case.kv, case.gamma_q, case.gamma_kv, W.EPS, True,
                                                want_ratio=True)
    wa = W.block_fp8_weight_e8m0(*W.W_A_SHAPE, W.W_A_SEED)
    wb = W.block_fp8_weight_e8m0(*W.W_B_SHAPE, W.W_B_SEED)
    o1, o2 = mi.mi_block_scaled_fp8_gemm_pair(codes, scale, mi.relayout_weight(dev_u8(wa.codes, dev)),
                                              dev_u8(wa.scale, dev), mi.relayout_weight(dev_u8(wb.codes, dev)),
                                              dev_u8(wb.scale, dev))
    torch.cuda.synchronize()
    compare_e8m0(codes.cpu().numpy(), scale_buffer(scale), qref, M, 12, True, f"producer M{M}")
    # the oracle GEMM on the oracle's own quantised pair
    asf = oracle.e8m0_decode_array(qref["scale"]).astype(np.float32)
    for o, wt, name in ((o1, wa, "W_a"), (o2, wb, "W_b")):
        nb = wt.codes.shape[0] // 128
        blocks = np.unique([0, nb // 3, nb - 1])
        cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
        bsf = oracle.e8m0_decode_array(wt.scale[blocks]).astype(np.float32)
        ref = oracle.block_scaled_fp8_gemm(qref["q"], asf, True, wt.codes[cols], bsf)
        fro, mx = assert_gemm_close(bf16_to_f64(o)[:, cols], ref, f"{name} M{M}")
        print(f"e8m0 chain {name} M={M}: rel fro {fro:.2e} max {mx:.2e}")
