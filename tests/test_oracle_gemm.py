"""Pins for the oracle's block-scaled FP8 GEMM.

The GEMM the pages describe (PRHub digest of vLLM PR #53540, excerpt of
apply_pre_quantized_block_scaled_mm; PRHub digest of SGLang PR #27289,
excerpt of aiter_w8a8_block_fp8_linear) multiplies the pre-quantised
activation (fp8 codes + one fp32 scale per 1x128 group) by an fp8 weight
[N, K] with one fp32 scale per 128x128 block and returns [M, N].  Pins:

* with unit scales it is a plain matrix product of the decoded operands
  (numpy matmul over torch-decoded fp8 values, exact in fp64 at these sizes);
* with general scales it equals the product of the dequantised operands,
  built with np.kron / np.repeat and a numpy matmul (a different order of
  operations: scale each element first, then one long sum);
* one-hot weights give a closed form; a single live K-block isolates the
  scale indices; column-major As equals row-major As; scaling one As row by a
  power of two scales one output row exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from rmsnorm_fp8_block_amd import workloads as W


def dec(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def random_codes(shape, rng):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return c


def random_scales(shape, rng):
    return np.exp2(rng.uniform(-12, 0, size=shape)).astype(np.float32)


def test_unit_scales_is_plain_matmul():
    rng = np.random.default_rng(40)
    M, N, K = 5, 256, 384
    a, w = random_codes((M, K), rng), random_codes((N, K), rng)
    out = oracle.block_scaled_fp8_gemm(a, np.ones(M * 3, np.float32), False, w,
                                       np.ones((2, 3), np.float32))
    assert np.array_equal(out, dec(a) @ dec(w).T)


@pytest.mark.parametrize("transposed", [False, True])
def test_general_scales_equal_dequantised_product(transposed):
    rng = np.random.default_rng(41)
    M, N, K = 7, 384, 256           # N/128 = 3 != K/128 = 2: a swapped Bs index fails
    a, w = random_codes((M, K), rng), random_codes((N, K), rng)
    As = random_scales((M, K // 128), rng)
    Bs = random_scales((N // 128, K // 128), rng)
    As_buf = As.T.reshape(-1) if transposed else As.reshape(-1)
    out = oracle.block_scaled_fp8_gemm(a, As_buf, transposed, w, Bs)
    A_deq = dec(a) * np.repeat(As.astype(np.float64), 128, axis=1)
    W_deq = dec(w) * np.kron(Bs.astype(np.float64), np.ones((128, 128)))
    ref = A_deq @ W_deq.T
    # fp64 summation error is relative to sum |a*w|, not to the (cancelling) result
    mag = np.abs(A_deq) @ np.abs(W_deq).T
    assert np.all(np.abs(out - ref) <= 1e-13 * mag)
    # the transposed operand / swapped scale layout would not agree
    assert not np.allclose(out, (dec(a) * np.repeat(As, 128, axis=1)) @ (dec(w)).T, rtol=1e-3)


def test_one_hot_weight_closed_form():
    rng = np.random.default_rng(42)
    M, N, K = 4, 256, 512
    a = random_codes((M, K), rng)
    As = random_scales((M, K // 128), rng)
    kn = rng.integers(0, K, size=N)
    w = np.zeros((N, K), np.uint8)
    w[np.arange(N), kn] = 0x38                       # e4m3 1.0
    out = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w, np.ones((N // 128, K // 128), np.float32))
    want = dec(a)[:, kn] * As[:, kn // 128].astype(np.float64)
    assert np.array_equal(out, want)


def test_single_live_k_block_isolates_scale_indices():
    rng = np.random.default_rng(43)
    M, N, K = 3, 384, 512
    a, w = random_codes((M, K), rng), random_codes((N, K), rng)
    As = random_scales((M, K // 128), rng)
    Bs = random_scales((N // 128, K // 128), rng)
    kb = 2
    a_live = np.zeros_like(a)
    a_live[:, kb * 128:(kb + 1) * 128] = a[:, kb * 128:(kb + 1) * 128]
    out = oracle.block_scaled_fp8_gemm(a_live, As.reshape(-1), False, w, Bs)
    part = dec(a)[:, kb * 128:(kb + 1) * 128] @ dec(w)[:, kb * 128:(kb + 1) * 128].T
    want = part * As[:, kb:kb + 1].astype(np.float64) * np.repeat(Bs[:, kb], 128)[None, :].astype(np.float64)
    assert np.allclose(out, want, rtol=1e-15, atol=0)
    # a swapped Bs index (Bs[kb, nb]) or As column would not agree
    assert not np.allclose(out, part * As[:, 0:1] * np.repeat(Bs[:, 0], 128)[None, :], rtol=1e-6)


def test_column_major_as_equals_row_major_and_row_scaling():
    rng = np.random.default_rng(44)
    M, N, K = 6, 256, 384
    a, w = random_codes((M, K), rng), random_codes((N, K), rng)
    As = random_scales((M, K // 128), rng)
    Bs = random_scales((N // 128, K // 128), rng)
    r = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w, Bs)
    c = oracle.block_scaled_fp8_gemm(a, As.T.reshape(-1), True, w, Bs)
    assert np.array_equal(r, c)
    # row-major bytes read as column-major: right only when M == 1
    bad = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), True, w, Bs)
    assert not np.allclose(bad, r, rtol=1e-3)
    one = oracle.block_scaled_fp8_gemm(a[:1], As[:1].reshape(-1), True, w, Bs)
    assert np.array_equal(one, r[:1])
    As2 = As.copy()
    As2[3] *= np.float32(4.0)
    r2 = oracle.block_scaled_fp8_gemm(a, As2.reshape(-1), False, w, Bs)
    assert np.array_equal(r2[3], 4.0 * r[3])
    assert np.array_equal(np.delete(r2, 3, axis=0), np.delete(r, 3, axis=0))


def test_checkpoint_style_weight_roundtrip():
    """The weight generator's codes times block scales reproduce the drawn
    N(0, 0.02) weights to e4m3 precision (relative error <= 2^-4 per element
    above the subnormal range)."""
    wt = W.block_fp8_weight(256, 384, seed=45)
    deq = dec(wt.codes) * np.kron(wt.scale.astype(np.float64), np.ones((128, 128)))
    ref = np.random.Generator(np.random.PCG64(45)).standard_normal((256, 384), dtype=np.float32) * np.float32(0.02)
    big = np.abs(ref) > 0.01
    assert np.all(np.abs(deq - ref)[big] <= np.abs(ref)[big] * 2.0 ** -4)
