"""Pins for the oracle's e8m0 (power-of-two) scale mode of the dual
RMSNorm + per-1x128 group quant, and for the e8m0 decode the block-scaled
GEMM uses (PRHub report of vLLM PR #56433, "风险与影响" item 3: e8m0 weight
block scales; PRHub digest of vLLM PR #56560: the native gfx950 MXFP8 GEMM,
e8m0 scale exponents).  The scale rule is a reading (the pages give none):
s = 2^ceil(log2(max(amax / 448, 1e-12))).

Pinned by: the e8m0 decode against torch's float8_e8m0fnu cast for all 256
bytes; the minimality of s (the smallest power of two not below amax/448);
agreement with the fp32-scale oracle wherever amax/448 is itself a power of
two (then both modes pick the same scale and the same codes); scale
equivariance under gamma -> 2^k gamma; the largest code of every live group
lying in [224, 448]; an independent 50-digit recomputation with
brute-force nearest searches on tiny inputs.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from rmsnorm_fp8_block_amd import workloads as W

from test_oracle_normquant import EPS32, FLOOR, ONE_BF16, bf16, bf16_scalar, nearest_bf16, nearest_e4m3


def run(q, kv, gq, gk, eps=EPS32, transpose=False):
    return oracle.dual_rmsnorm_group_quant_e8m0(q, kv, gq, gk, eps, transpose, want_ratio=True)


def test_e8m0_decode_matches_torch_for_every_byte():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_decode_array(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


@pytest.mark.parametrize("make", [lambda: W.strided_batch(64), lambda: W.outlier_stress(64)])
def test_scale_is_the_smallest_power_of_two_not_below_amax_over_448(make):
    case = make()
    e8 = run(case.q, case.kv, case.gamma_q, case.gamma_kv)
    M, G = case.M, W.NQ // 128
    s = oracle.e8m0_decode_array(e8["scale"]).reshape(M, G)
    # amax / 448 from the oracle's exact y: y = ratio * s
    y = e8["ratio"] * np.repeat(s, 128, axis=1)
    t = np.maximum(np.abs(y).reshape(M, G, 128).max(axis=2) / 448, FLOOR)
    assert np.all(s >= t) and np.all(s / 2 < t)
    assert np.all(np.abs(e8["ratio"]) <= 448)
    # kv is the dual operation's
    ref = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, case.eps, False)
    assert np.array_equal(e8["kv"], ref["kv"])


def test_equals_fp32_mode_where_amax_over_448_is_a_power_of_two():
    """Constant row c, eps = 0: y = sign(c) * gamma.  With each group's
    largest |gamma| equal to 448 * 2^k, amax / 448 = 2^k exactly, so the
    fp32-scale mode also stores s = 2^k and both modes give identical codes."""
    r = np.random.default_rng(4)
    Nq, Nkv, M = 384, 64, 3
    g = (r.uniform(-1, 1, Nq) * 0.9).astype(np.float32)
    for grp, k in zip(range(3), (-5, 0, 3)):
        g[grp * 128:(grp + 1) * 128] *= np.float32(448 * 2.0 ** k)
        g[grp * 128 + 7] = np.float32(-448 * 2.0 ** k)       # the group's largest magnitude
    gq = bf16(g)
    q, kv, _, gk = const_rows(-1.5, M, Nq, Nkv)
    e8 = run(q, kv, gq, gk, eps=0.0)
    f32 = oracle.dual_rmsnorm_group_quant(q, kv, gq, gk, 0.0, False)
    assert np.array_equal(oracle.e8m0_decode_array(e8["scale"]), f32["scale"].astype(np.float64))
    assert np.array_equal(e8["q"], f32["q"])


def const_rows(c, M, Nq, Nkv):
    q = np.full((M, Nq), bf16_scalar(c), np.uint16)
    kv = np.full((M, Nkv), bf16_scalar(c), np.uint16)
    return q, kv, np.full(Nq, ONE_BF16, np.uint16), np.full(Nkv, ONE_BF16, np.uint16)


def test_gamma_times_power_of_two_scales_s_and_keeps_codes():
    case = W.strided_batch(16)
    base = run(case.q, case.kv, case.gamma_q, case.gamma_kv)
    for k in (-3, 4):
        gq = bf16(oracle.bf16_decode_array(case.gamma_q) * 2.0 ** k)
        out = run(case.q, case.kv, gq, case.gamma_kv)
        assert np.array_equal(out["q"], base["q"])
        assert np.array_equal(out["scale"].astype(int), base["scale"].astype(int) + k)


def test_largest_code_of_a_live_group_is_between_224_and_448():
    case = W.outlier_stress(128)
    out = run(case.q, case.kv, case.gamma_q, case.gamma_kv, transpose=True)
    M, G = case.M, W.NQ // 128
    mag = np.abs(oracle.e4m3_decode_array(out["q"])).reshape(M, G, 128).max(axis=2)
    s = oracle.e8m0_decode_array(out["scale"]).reshape(G, M).T
    live = s > 2.0 ** -39          # groups above the floor
    # amax / s lies in (224, 448]; rounding to e4m3 keeps the largest code in [224, 448]
    assert np.all((mag[live] >= 224) & (mag[live] <= 448))
    assert np.all(mag[~live] == 0)
    # zero groups (m mod 12) take the floor: 2^ceil(log2(1e-12)) = 2^-39
    assert np.all(s[~live] == 2.0 ** -39)


@pytest.mark.parametrize("seed,Nq,Nkv", [(41, 256, 64), (42, 384, 8)])
def test_tiny_inputs_vs_decimal_brute_force(seed, Nq, Nkv):
    getcontext().prec = 50
    r = np.random.default_rng(seed)
    M = 3
    q32 = r.standard_normal((M, Nq)).astype(np.float32)
    q32[r.random((M, Nq)) < 0.05] *= 40
    q32[1, :128] *= 1e-3
    q, kv = bf16(q32), bf16(r.standard_normal((M, Nkv)).astype(np.float32))
    gq = bf16(1 + 0.1 * r.standard_normal(Nq))
    gk = bf16(1 + 0.1 * r.standard_normal(Nkv))
    for transpose in (False, True):
        out = run(q, kv, gq, gk, transpose=transpose)
        G = Nq // 128
        for m in range(M):
            xq = [Decimal(oracle.bf16_decode(b)) for b in q[m]]
            rq = 1 / (sum(x * x for x in xq) / Nq + Decimal(EPS32)).sqrt()
            xk = [Decimal(oracle.bf16_decode(b)) for b in kv[m]]
            rk = 1 / (sum(x * x for x in xk) / Nkv + Decimal(EPS32)).sqrt()
            for i in range(Nkv):
                assert out["kv"][m, i] == nearest_bf16(Fraction(xk[i] * rk * Decimal(oracle.bf16_decode(gk[i]))))
            for g in range(G):
                ys = [xq[i] * rq * Decimal(oracle.bf16_decode(gq[i])) for i in range(g * 128, (g + 1) * 128)]
                t = max(Fraction(max(abs(v) for v in ys)) / 448, Fraction(FLOOR))
                e = 0
                while Fraction(2) ** e < t:         # smallest power of two >= t, by search
                    e += 1
                while Fraction(2) ** (e - 1) >= t:
                    e -= 1
                at = g * M + m if transpose else m * G + g
                assert int(out["scale"][at]) == e + 127, (m, g)
                for j, y in enumerate(ys):
                    assert out["q"][m, g * 128 + j] == nearest_e4m3(Fraction(y) / Fraction(2) ** e), (m, g, j)
