"""GPU parity of the block-scaled FP8 GEMM (MFMA, gfx950) against the CPU
oracle, through the C ABI, and of the producer -> two consumers chain.

The GEMM is the consumer that the PRHub digest of vLLM PR #53540 describes
(apply_pre_quantized_block_scaled_mm: A = x_fp8, As = x_scale, Bs = weight
block scale) with the As major order made explicit (PRHub report of vLLM PR
#56433, item 2: a GEMM reading column-major As silently returns wrong
numbers for M > 1 when handed row-major bytes).  Bar: relative error <= 2e-2
(Frobenius and max-abs, normalised by the oracle); the two As layouts give
bit-identical outputs; repeat runs are bit-identical.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import rmsnorm_fp8_block_amd as mi
from rmsnorm_fp8_block_amd import _binding as B
from rmsnorm_fp8_block_amd import workloads as W

from helpers import (assert_gemm_close, bf16_to_f64, compare_normquant, dev_f32, dev_u8,
                     dev_u16_as_bf16, gemm_error, gpu_or_skip, host_bf16_bits, scale_buffer)

pytestmark = pytest.mark.gpu


def random_operands(M, N, K, seed):
    r = np.random.default_rng(seed)
    a = r.integers(0, 256, size=(M, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38
    As = np.exp2(r.uniform(-10, 0, (M, K // 128))).astype(np.float32)
    Bs = np.exp2(r.uniform(-10, 0, (N // 128, K // 128))).astype(np.float32)
    return a, As, w, Bs


def run_gemm(a, As, w, Bs, transposed, dev):
    M, K = a.shape
    da = dev_u8(a, dev)
    if transposed:
        das = dev_f32(As.T.copy(), dev).T       # [M, KB] view with strides (1, M)
    else:
        das = dev_f32(As, dev)
    out = mi.mi_block_scaled_fp8_gemm(da, das, dev_u8(w, dev), dev_f32(Bs, dev))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M,N,K,seed", [(1, 256, 256, 1), (5, 384, 640, 2), (16, 256, 1536, 3), (3, 1280, 512, 8), (40, 384, 1024, 9), (64, 8192, 2048, 10),
                                        (17, 512, 384, 4), (64, 128, 1536, 5), (100, 640, 896, 6),
                                        (256, 256, 1536, 7)])
def test_gemm_random_vs_oracle(M, N, K, seed):
    dev = gpu_or_skip()
    a, As, w, Bs = random_operands(M, N, K, seed)
    ref = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w, Bs)
    # sum of |a*w| over k with the scales applied: the size the fp32 (and
    # matrix-core internal) accumulation error is relative to
    mag = (np.abs(oracle.e4m3_decode_array(a)) * np.repeat(As.astype(np.float64), 128, axis=1)) @ \
        (np.abs(oracle.e4m3_decode_array(w)) * np.kron(Bs.astype(np.float64), np.ones((128, 128)))).T
    outs = []
    for t in (False, True):
        out = run_gemm(a, As, w, Bs, t, dev)
        fro, mx = assert_gemm_close(bf16_to_f64(out), ref, f"M{M} N{N} K{K} t{t}")
        # element-wise: bf16 output rounding plus accumulation error
        err = np.abs(bf16_to_f64(out) - ref)
        excess = np.maximum(err - 2.0 ** -8 * np.abs(ref), 0) / mag
        print(f"M{M} N{N} K{K} t{t}: fro {fro:.2e} max {mx:.2e} "
              f"max(err/mag) {np.max(err / mag):.3e} max excess/mag {excess.max():.3e}")
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * mag)
        outs.append(host_bf16_bits(out))
    assert np.array_equal(outs[0], outs[1]), "row- and column-major As must give identical bits"
    again = host_bf16_bits(run_gemm(a, As, w, Bs, False, dev))
    assert np.array_equal(again, outs[0])


@pytest.mark.parametrize("M,N,K,seed", [(65, 384, 512, 21), (129, 1280, 1024, 22), (100, 1536, 1536, 23),
                                        (256, 16640, 1536, 24), (72, 32768, 512, 25), (200, 12288, 1536, 26),
                                        (256, 8192, 2048, 27), (256, 24576, 1536, 28), (193, 8192, 1536, 29),
                                        (256, 3072, 1536, 30), (150, 6144, 1536, 31), (100, 3072, 1536, 32)])
def test_gemm_wide_shapes_sampled(M, N, K, seed):
    """64 < M <= 256 at widths that give 2, 4, 6 and 8 weight subtiles per
    block, with a ragged last block (N = 16640: 1040 subtiles in blocks of 6);
    W_b's width at 193 rows (the stream kernel, one row in its last chunk);
    narrow weights split into row chunks: 64-row chunks of three-subtile
    slabs (N = 3072 at 256 rows), three-subtile slabs of half the rows
    (N = 6144 at 150 rows), and two-subtile slabs (N = 3072 at 100 rows).
    The oracle runs on the first, the last and two random 128-column blocks."""
    dev = gpu_or_skip()
    a, As, w, Bs = random_operands(M, N, K, seed)
    nb = N // 128
    r = np.random.default_rng(seed)
    blocks = np.unique(np.concatenate([[0, nb - 1], r.choice(nb, size=min(2, nb), replace=False)]))
    cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    ref = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w[cols], Bs[blocks])
    mag = (np.abs(oracle.e4m3_decode_array(a)) * np.repeat(As.astype(np.float64), 128, axis=1)) @ \
        (np.abs(oracle.e4m3_decode_array(w[cols])) * np.kron(Bs[blocks].astype(np.float64), np.ones((128, 128)))).T
    outs = []
    for t in (False, True):
        out = run_gemm(a, As, w, Bs, t, dev)
        got = bf16_to_f64(out)[:, cols]
        assert_gemm_close(got, ref, f"M{M} N{N} K{K} t{t}")
        err = np.abs(got - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * mag), f"M{M} N{N} K{K} t{t}"
        outs.append(host_bf16_bits(out))
    assert np.array_equal(outs[0], outs[1]), "row- and column-major As must give identical bits"


def test_one_hot_weights_closed_form():
    """W row n = 1.0 at column k_n, Bs = 1: out[m, n] = bf16(dec(a[m, k_n]) *
    As[m, k_n / 128]) exactly."""
    dev = gpu_or_skip()
    M, N, K = 8, 256, 512
    r = np.random.default_rng(11)
    a, As, _, _ = random_operands(M, N, K, 12)
    # scales with 8 significant bits: dec(a) * As is exact in fp32, so the
    # kernel's only rounding is the final bf16 one
    As = W.f32_to_bf16_bits(As).astype(np.uint32) << 16
    As = As.view(np.float32)
    kn = r.integers(0, K, size=N)
    w = np.zeros((N, K), np.uint8)
    w[np.arange(N), kn] = 0x38
    Bs = np.ones((N // 128, K // 128), np.float32)
    out = host_bf16_bits(run_gemm(a, As, w, Bs, False, dev))
    want = oracle.e4m3_decode_array(a)[:, kn] * As[:, kn // 128].astype(np.float64)
    want_bits = np.vectorize(oracle.bf16_encode)(want).astype(np.uint16)
    # a product that is -0 (code 0x80) summed with +0 terms is +0: both zeros
    # are the same value
    zero = lambda b: np.where((b & 0x7FFF) == 0, 0, b)
    bad = np.argwhere(zero(out) != zero(want_bits))
    assert bad.size == 0, [(int(out[i, j]), int(want_bits[i, j]), float(want[i, j])) for i, j in bad[:8]]


def test_row_major_scales_read_as_column_major_are_wrong_for_m_gt_1():
    """The silent failure of a layout mismatch: same logical shape, wrong
    bytes.  At M = 1 both layouts are the same bytes, so it is harmless."""
    dev = gpu_or_skip()
    N, K = 256, 1536
    for M, expect_ok in ((1, True), (16, False)):
        a, As, w, Bs = random_operands(M, N, K, 20 + M)
        ref = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w, Bs)
        da, das = dev_u8(a, dev), dev_f32(As, dev)           # row-major bytes
        dw, dbs = dev_u8(w, dev), dev_f32(Bs, dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        st = mi.lib().mi_block_scaled_fp8_gemm(p(da), p(das), 1, p(dw), p(dbs), p(out), M, N, K,
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == B.MI_OK
        torch.cuda.synchronize()
        fro, _ = gemm_error(bf16_to_f64(out), ref)
        if expect_ok:
            assert fro <= 2e-2
        else:
            assert fro > 0.1, "a layout mismatch must show up as a large error"


WEIGHTS = {}


def weight(name):
    if name not in WEIGHTS:
        (N, K), seed = (W.W_A_SHAPE, W.W_A_SEED) if name == "W_a" else (W.W_B_SHAPE, W.W_B_SEED)
        WEIGHTS[name] = W.block_fp8_weight(N, K, seed)
    return WEIGHTS[name]


def sample_columns(wt, nblocks, seed):
    """A few 128-column blocks of the weight (the oracle is too slow for all
    24576 columns): returns (column indices, codes, scales)."""
    N = wt.codes.shape[0]
    r = np.random.default_rng(seed)
    blocks = np.sort(r.choice(N // 128, size=nblocks, replace=False))
    cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    return cols, wt.codes[cols], wt.scale[blocks]


@pytest.mark.parametrize("M", [1, 16, 64, 256])
@pytest.mark.parametrize("transpose", [0, 1])
def test_producer_and_two_consumers(M, transpose):
    """Fused norm-quant on strided views of the first M rows of a [256, 2048]
    buffer; both consumers (W_a [24576, 1536] and W_b [8192, 1536]) read the
    same (q_fp8, scale) pair in the negotiated layout.  The oracle chain runs
    on the same inputs; GEMM outputs are compared on sampled 128-column
    blocks (all columns for the last-row block check of shape)."""
    dev = gpu_or_skip()
    layout = mi.mi_negotiate_scale_layout([transpose, transpose])
    assert layout is bool(transpose)
    case = W.producer_activations(M)
    buf = dev_u16_as_bf16(case.buffer, dev)
    q, kv = buf[:, :W.NQ], buf[:, W.NQ:]
    codes, scale, kv_out = mi.mi_fused_dual_rmsnorm_group_quant(
        q, kv, dev_u16_as_bf16(case.gamma_q, dev), dev_u16_as_bf16(case.gamma_kv, dev), W.EPS, layout)
    ref = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, W.EPS,
                                          layout, want_ratio=True)
    torch.cuda.synchronize()
    compare_normquant(codes.cpu().numpy(), scale_buffer(scale), host_bf16_bits(kv_out), ref,
                      label=f"producer M{M}")
    for name in ("W_a", "W_b"):
        wt = weight(name)
        out = mi.mi_block_scaled_fp8_gemm(codes, scale, dev_u8(wt.codes, dev), dev_f32(wt.scale, dev))
        torch.cuda.synchronize()
        assert out.shape == (M, wt.codes.shape[0])
        cols, wc, ws = sample_columns(wt, 4, seed=M)
        gref = oracle.block_scaled_fp8_gemm(ref["q"], ref["scale"], layout, wc, ws)
        got = bf16_to_f64(out)[:, cols]
        fro, mx = assert_gemm_close(got, gref, f"{name} M{M} t{transpose}")
        print(f"{name} M={M} transpose={transpose}: rel fro {fro:.2e} max {mx:.2e}")


@pytest.mark.parametrize("M,N1,N2,K,seed", [(1, 24576, 8192, 1536, 31), (16, 24576, 8192, 1536, 32),
                                            (64, 24576, 8192, 1536, 33), (40, 1280, 384, 512, 34),
                                            (64, 3200, 1664, 1024, 35), (100, 1280, 640, 1536, 36),
                                            (256, 2048, 1024, 2048, 37), (7, 384, 128, 896, 38),
                                            (64, 12800, 6400, 1536, 39), (200, 3072, 1024, 1536, 40),
                                            (128, 6144, 2048, 1536, 41), (100, 3200, 2944, 1536, 42),
                                            (256, 12288, 4096, 1536, 43)])
def test_gemm_pair_equals_two_gemms(M, N1, N2, K, seed):
    """The two-consumer entry point returns, bit for bit, what two calls of
    the single GEMM return (fused launch for M <= 64 and K/128 in {4, 8, 12,
    16}, including 6-subtile slabs that straddle the two weights at
    N1 = 12800, and above 64 rows for shard pairs with K/128 = 12: TP-8,
    TP-4 and TP-2 pairs, and three-subtile slabs straddling the two weights
    at N1 = 3200;
    two launches otherwise), and matches the oracle on sampled column blocks
    of both."""
    dev = gpu_or_skip()
    a, As, w1, Bs1 = random_operands(M, N1, K, seed)
    _, _, w2, Bs2 = random_operands(M, N2, K, seed + 100)
    da = dev_u8(a, dev)
    for t in (False, True):
        das = dev_f32(As.T.copy(), dev).T if t else dev_f32(As, dev)
        dw1, dbs1, dw2, dbs2 = dev_u8(w1, dev), dev_f32(Bs1, dev), dev_u8(w2, dev), dev_f32(Bs2, dev)
        o1, o2 = mi.mi_block_scaled_fp8_gemm_pair(da, das, dw1, dbs1, dw2, dbs2)
        s1 = mi.mi_block_scaled_fp8_gemm(da, das, dw1, dbs1)
        s2 = mi.mi_block_scaled_fp8_gemm(da, das, dw2, dbs2)
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16_bits(o1), host_bf16_bits(s1)), f"out1 M{M} t{t}"
        assert np.array_equal(host_bf16_bits(o2), host_bf16_bits(s2)), f"out2 M{M} t{t}"
        for w, Bs, o, name in ((w1, Bs1, o1, "out1"), (w2, Bs2, o2, "out2")):
            nb = w.shape[0] // 128
            blocks = np.unique([0, nb - 1, nb // 2])
            cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
            ref = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w[cols], Bs[blocks])
            assert_gemm_close(bf16_to_f64(o)[:, cols], ref, f"{name} M{M} N{w.shape[0]} t{t}")


def test_gemm_large_batch_generic_kernel_sampled():
    """M = 1024 rows (beyond the decode and wide kernels: the generic one)
    over W_b [8192, 1536], both As layouts bit-identical, sampled columns
    against the oracle."""
    dev = gpu_or_skip()
    M, N, K = 1024, 8192, 1536
    a, As, w, Bs = random_operands(M, N, K, 91)
    r = np.random.default_rng(91)
    blocks = np.unique(np.concatenate([[0, N // 128 - 1], r.choice(N // 128, size=2, replace=False)]))
    cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    ref = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w[cols], Bs[blocks])
    outs = []
    for t in (False, True):
        out = run_gemm(a, As, w, Bs, t, dev)
        assert_gemm_close(bf16_to_f64(out)[:, cols], ref, f"M{M} t{t}")
        outs.append(host_bf16_bits(out))
    assert np.array_equal(outs[0], outs[1])
