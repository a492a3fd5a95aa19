"""Pins for the oracle's single-input operations: the per-1x128 dynamic FP8
quantisation of a bf16 activation (PRHub digest of SGLang PR #27289, the
aiter_w8a8_block_fp8_linear excerpt, branch B: aiter_per1x128_quant with
transpose_scale; GitHub page of vLLM PR #53540, "Purpose": the per-1x128
quant of the bf16 q-lora), and the single-input RMSNorm + group quant (the
same digest, "实现拆解" item 2: fused_rms_fp8_group_quant with
transpose_scale).

Pinned by closed forms (exact round trips of codes with power-of-two
scales, constant groups, single non-zero elements, all-zero groups),
invariants (scale equivariance, layouts, the half-ULP bound), a recomputation
in exact rational arithmetic with brute-force nearest searches on tiny
inputs, and the pre-fusion pipeline the pages describe: RMSNorm rounded to
bf16, then the per-1x128 quant, equals the dual oracle's sequential mode.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from rmsnorm_fp8_block_amd import workloads as W

from test_oracle_normquant import EPS32, FLOOR, ONE_BF16, bf16, bf16_scalar, nearest_e4m3, nearest_f32


def gq(x, transpose=False, ratio=False):
    return oracle.group_quant(x, transpose, want_ratio=ratio)


# ------------------------------------------------------- per-1x128 quant

def test_codes_round_trip_with_power_of_two_scale():
    """x = dec(c) * 2^k for random codes c with a +-448 code in every group:
    amax = 448 * 2^k, so s = 2^k exactly and every x / s is the code's value:
    the quantiser must return the codes themselves."""
    r = np.random.default_rng(1)
    M, N = 5, 1024
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    codes = r.choice(finite, size=(M, N)).astype(np.uint8)
    codes[:, ::128] = 0x7E
    codes[1, 128] = 0xFE                    # a negative maximum in one group
    k = r.integers(-20, 6, size=(M, 1))
    vals = oracle.e4m3_decode_array(codes) * np.exp2(k)
    x = bf16(vals)                           # exact: e4m3 values x 2^k are bf16 values
    assert np.array_equal(oracle.bf16_decode_array(x), vals)
    out = gq(x)
    zero = lambda c: np.where((c & 0x7F) == 0, 0, c)     # +-0 are both correct
    assert np.array_equal(zero(out["q"]), zero(codes))
    assert np.array_equal(out["scale"].reshape(M, -1), np.broadcast_to(np.exp2(k).astype(np.float32), (M, N // 128)))


@pytest.mark.parametrize("c", [1.0, -3.0, 2.0 ** -30, 1000.0])
def test_constant_group(c):
    """Every element c: s = fp32(|c| / 448) and every code is the largest
    magnitude of c's sign (c / s rounds to 448 within one ULP of s)."""
    x = np.full((2, 256), bf16_scalar(c), np.uint16)
    out = gq(x, ratio=True)
    cv = oracle.bf16_decode(int(x[0, 0]))
    assert np.all(out["scale"] == np.float32(abs(cv) / 448))
    want = nearest_e4m3(Fraction(cv) / Fraction(float(np.float32(abs(cv) / 448))))
    assert want in (0x7E, 0xFE)
    assert np.all(out["q"] == want)


def test_single_nonzero_element_zero_group_and_floor():
    """A lone non-zero v: its code is +-448, the rest 0, s = fp32(|v|/448).
    An all-zero group takes the 1e-12 floor.  A lone value so small that
    |v|/448 < 1e-12 also takes the floor, and then v / 1e-12 rounds to 0."""
    x = np.zeros((4, 384), np.uint16)
    x[0, 5] = bf16_scalar(-2.5)
    x[1, 200] = bf16_scalar(1e-6)
    x[3, 300] = bf16_scalar(1e-20)
    out = gq(x)
    assert out["q"][0, 5] == 0xFE and np.count_nonzero(out["q"][0]) == 1
    assert out["q"][1, 200] == 0x7E and np.count_nonzero(out["q"][1]) == 1
    s = out["scale"].reshape(4, 3)
    assert s[0, 0] == np.float32(2.5 / 448) and s[0, 1] == np.float32(FLOOR)
    assert s[1, 1] == np.float32(oracle.bf16_decode(int(x[1, 200])) / 448)
    assert np.all(s[2] == np.float32(FLOOR)) and not np.any(out["q"][2])
    assert s[3, 2] == np.float32(FLOOR) and not np.any(out["q"][3])


def test_scale_equivariance_and_layouts():
    r = np.random.default_rng(2)
    x = bf16(r.standard_normal((7, 640)).astype(np.float32))
    a = gq(x)
    for k in (-9, 5):
        xk = bf16(oracle.bf16_decode_array(x) * 2.0 ** k)
        b = gq(xk)
        assert np.array_equal(a["q"], b["q"])
        assert np.array_equal(a["scale"] * np.float32(2.0 ** k), b["scale"])
    t = gq(x, transpose=True)
    assert np.array_equal(t["q"], a["q"])
    assert np.array_equal(t["scale"], a["scale"].reshape(7, 5).T.reshape(-1))
    one = gq(x[:1])
    assert np.array_equal(one["scale"], gq(x[:1], transpose=True)["scale"])


def test_half_ulp_bound_and_max_code_on_outliers():
    case = W.outlier_stress(64)
    out = gq(case.q, ratio=True)
    x = oracle.bf16_decode_array(case.q)
    s = np.repeat(out["scale"].reshape(64, -1), 128, axis=1).astype(np.float64)
    deq = oracle.e4m3_decode_array(out["q"]) * s
    r = np.abs(x / s)
    e = np.floor(np.log2(np.maximum(r, 2.0 ** -6)))
    half_ulp = np.where(r < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
    assert np.all(np.abs(x - deq) <= half_ulp * s * (1 + 1e-12))
    live = out["scale"].reshape(64, -1) > FLOOR
    mags = (out["q"] & 0x7F).reshape(64, -1, 128)
    assert np.all(np.any(mags == 0x7E, axis=2)[live])


@pytest.mark.parametrize("seed", [41, 42])
def test_tiny_inputs_vs_exact_brute_force(seed):
    r = np.random.default_rng(seed)
    x32 = r.standard_normal((3, 256)).astype(np.float32)
    x32[0, :128] *= 1e-4
    x32[r.random((3, 256)) < 0.05] *= 60
    x = bf16(x32)
    for transpose in (False, True):
        out = gq(x, transpose)
        for m in range(3):
            for g in range(2):
                vals = [Fraction(oracle.bf16_decode(int(b))) for b in x[m, g * 128:(g + 1) * 128]]
                s = max(nearest_f32(max(abs(v) for v in vals) / 448), FLOOR)
                assert out["scale"][g * 3 + m if transpose else m * 2 + g] == np.float32(s)
                for j, v in enumerate(vals):
                    assert out["q"][m, g * 128 + j] == nearest_e4m3(v / Fraction(s)), (m, g, j)


# ------------------------------------- single-input RMSNorm + group quant

def test_rmsnorm_quant_equals_the_q_path_of_the_dual_op():
    """The q path of the dual operation is this operation on q alone (kv
    only contributes its own, independent normalisation)."""
    case = W.strided_batch(64)
    dual = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, W.EPS, True)
    single = oracle.rmsnorm_group_quant(case.q, case.gamma_q, W.EPS, True)
    assert np.array_equal(single["q"], dual["q"])
    assert np.array_equal(single["scale"], dual["scale"])


def test_rmsnorm_quant_constant_row_with_gamma():
    """x = 1 everywhere, eps = 0: y = gamma, so the codes are those of the
    per-1x128 quant of gamma itself (exact: gamma is bf16)."""
    r = np.random.default_rng(3)
    gamma = bf16(1 + 0.1 * r.standard_normal(512))
    x = np.full((2, 512), ONE_BF16, np.uint16)
    out = oracle.rmsnorm_group_quant(x, gamma, 0.0, False)
    ref = gq(np.broadcast_to(gamma, (2, 512)).copy())
    assert np.array_equal(out["q"], ref["q"]) and np.array_equal(out["scale"], ref["scale"])


def test_pre_fusion_pipeline_norm_to_bf16_then_quant():
    """The pipeline the fused kernel replaces (vLLM PR #53540, "Purpose"):
    RMSNorm to bf16, then the per-1x128 quant of that bf16 tensor.  The dual
    oracle's sequential mode computes exactly this; the per-1x128 quant of
    the bf16-rounded normalised q must agree with it bit for bit."""
    case = W.producer_activations(32)
    seq = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, W.EPS, False,
                                          sequential=True, want_ratio=True)
    fused = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, W.EPS, False,
                                            want_ratio=True)
    y_bf16 = np.vectorize(oracle.bf16_encode, otypes=[np.uint16])(fused["y"])
    two_step = gq(y_bf16)
    assert np.array_equal(two_step["q"], seq["q"])
    assert np.array_equal(two_step["scale"], seq["scale"])
