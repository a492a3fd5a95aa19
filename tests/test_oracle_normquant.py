"""Pins for the oracle's fused dual RMSNorm + per-1x128 FP8 group quant.

What the method computes is stated on the pages only in words (vLLM PR
#53540, "Purpose": RMSNorm of the q and kv latents with fp32 accumulation, q
quantised per 1x128 with fp32 scales straight from the normalised values, kv
kept bf16; PRHub digest of PR #53540, the source excerpt of
_fused_mla_dual_rms_norm_group_quant_impl: output shapes and dtypes; PRHub
report of vLLM PR #56433 and digest of SGLang PR #27289: the column-major
scale layout).  Nothing numeric is printed there, so the oracle is pinned by:

* closed forms (a constant row, a constant row with a non-constant gamma, a
  group with a single non-zero element, an all-zero group, eps placement);
* invariants (unit RMS of the normalised row, independence of q and kv,
  scale equivariance, permutation within a group, amax -> +-448, the half-ULP
  dequantisation bound, layouts, strided views);
* an independent recomputation on tiny inputs in 50-digit decimal arithmetic
  with brute-force nearest-value searches for every rounding.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from rmsnorm_fp8_block_amd import workloads as W

EPS32 = float(np.float32(1e-6))
FLOOR = float(np.float32(1e-12))
ONE_BF16 = 0x3F80


def bf16(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def bf16_scalar(v) -> int:
    return int(W.f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])


def const_rows(c, M, Nq, Nkv, gq=None, gk=None):
    q = np.full((M, Nq), bf16_scalar(c), np.uint16)
    kv = np.full((M, Nkv), bf16_scalar(c), np.uint16)
    gq = np.full(Nq, ONE_BF16, np.uint16) if gq is None else gq
    gk = np.full(Nkv, ONE_BF16, np.uint16) if gk is None else gk
    return q, kv, gq, gk


def run(q, kv, gq, gk, eps=EPS32, transpose=False, sequential=False, ratio=True):
    return oracle.dual_rmsnorm_group_quant(q, kv, gq, gk, eps, transpose, sequential, ratio)


def nearest_f32(fr: Fraction) -> float:
    """Brute force: the fp32 value nearest to ``fr`` (ties to even)."""
    c = np.float32(float(fr))
    cands = {float(c), float(np.nextafter(c, np.float32(np.inf))), float(np.nextafter(c, np.float32(-np.inf)))}
    best = min(cands, key=lambda v: (abs(Fraction(v) - fr),
                                     int(np.float32(v).view(np.uint32)) & 1))
    return best


E4M3_GRID = [(Fraction(oracle.e4m3_decode(c)), c) for c in range(0x7F)]


def nearest_e4m3(fr: Fraction) -> int:
    """Brute force over all finite magnitudes: nearest code, ties to the even
    code, saturating at 448."""
    sign = 0x80 if fr < 0 else 0
    a = abs(fr)
    if a >= 448:
        return sign | 0x7E
    best = min(E4M3_GRID, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return sign | best[1]


def nearest_bf16(fr: Fraction) -> int:
    """Brute force over the bf16 neighbours of the fp32 value nearest ``fr``."""
    f = np.float32(float(fr))
    b0 = int(W.f32_to_bf16_bits(np.array([f]))[0])
    cands = [b for b in (b0 - 1, b0, b0 + 1) if 0 <= b < 0x10000]
    cands = [b for b in cands if (b & 0x8000) == (b0 & 0x8000)] or [b0]
    return min(cands, key=lambda b: (abs(Fraction(oracle.bf16_decode(b)) - fr), b & 1))


# -------------------------------------------------------------- closed forms

@pytest.mark.parametrize("c", [1.0, -2.0, 0.5, 3.0, 2.0 ** -10])
def test_constant_row_closed_form(c):
    """x = c everywhere, gamma = 1: y = c / sqrt(c^2 + eps) in every lane, so
    every code is +-448, s = fp32(|y|/448) and kv = bf16(y)."""
    q, kv, gq, gk = const_rows(c, 2, 256, 64)
    out = run(q, kv, gq, gk)
    getcontext().prec = 60
    cd = Decimal(c)
    y = cd / (cd * cd + Decimal(EPS32)).sqrt()
    s = nearest_f32(Fraction(abs(y)) / 448)
    code = 0x7E if c > 0 else 0xFE
    assert np.all(out["q"] == code)
    assert np.all(out["scale"] == np.float32(s))
    assert np.all(out["kv"] == nearest_bf16(Fraction(y)))
    if c == 1.0:
        # 1/sqrt(1 + 1e-6f) = 0.99999950000037...; bf16 -> 1.0
        assert abs(float(y) - 0.99999950000037) < 1e-13
        assert np.all(out["kv"] == ONE_BF16)


def test_eps_sits_inside_the_square_root():
    """c = 2^-10 has c^2 ~ eps, so the placement of eps shows: only
    c/sqrt(c^2+eps) (not c/(|c|+eps), c/sqrt(c^2)+eps, ...) gives this kv."""
    c = 2.0 ** -10
    q, kv, gq, gk = const_rows(c, 1, 128, 32)
    out = run(q, kv, gq, gk)
    y = c / math.sqrt(c * c + EPS32)          # 0.6985...
    assert 0.69 < y < 0.70
    assert np.all(out["kv"] == nearest_bf16(Fraction(y)))
    for wrong in (c / (abs(c) + EPS32), 1.0 + EPS32, c / math.sqrt(c * c) * 1.0):
        assert nearest_bf16(Fraction(wrong)) != nearest_bf16(Fraction(y))


def test_constant_row_with_gamma_gives_gamma_ratios():
    """x = c, gamma varying: within a group y_i is proportional to gamma_i, so
    the codes are RNE(448 * gamma_i / max|gamma|) independent of c and eps
    (up to the fp32 rounding of s, which moves a ratio by <= 2^-24 relative;
    ratios that close to a rounding midpoint are skipped).  A (1 + gamma)
    multiplier or a row-wide amax would give other codes."""
    gq, _ = W.gammas(256, 64, seed=123)
    for c in (1.0, -0.75):
        q, kv, _, gk = const_rows(c, 1, 256, 64)
        out = run(q, kv, gq, gk)
        g = np.array([Fraction(oracle.bf16_decode(b)) for b in gq])
        checked = 0
        for grp in range(2):
            gg = g[grp * 128:(grp + 1) * 128]
            gmax = max(abs(v) for v in gg)
            for j, gi in enumerate(gg):
                r = 448 * gi / gmax * (1 if c > 0 else -1)
                want = nearest_e4m3(r)
                lo, hi = nearest_e4m3(r * (1 - Fraction(1, 2 ** 23))), nearest_e4m3(r * (1 + Fraction(1, 2 ** 23)))
                if lo != hi:
                    continue
                assert out["q"][0, grp * 128 + j] == want
                checked += 1
        assert checked > 250


def test_single_nonzero_element_per_group():
    Nq = 384
    q = np.zeros((1, Nq), np.uint16)
    vals = [3.0, -0.125, 1e-3]
    for g, v in enumerate(vals):
        q[0, g * 128 + 17 * g + 5] = bf16_scalar(v)
    kv = bf16(np.ones((1, 16)))
    gq = np.full(Nq, ONE_BF16, np.uint16)
    gk = np.full(16, ONE_BF16, np.uint16)
    out = run(q, kv, gq, gk)
    for g, v in enumerate(vals):
        row = out["q"][0, g * 128:(g + 1) * 128]
        pos = 17 * g + 5
        assert row[pos] == (0x7E if v > 0 else 0xFE)
        assert np.all(np.delete(row, pos) == 0)
    assert np.all(out["scale"] > 0)


def test_zero_group_takes_the_scale_floor():
    case = W.outlier_stress(M=24, seed=3)
    out = run(case.q, case.kv, case.gamma_q, case.gamma_kv, transpose=False)
    G = 12
    sc = out["scale"].reshape(24, G)
    for m in range(24):
        g = m % G
        assert sc[m, g] == np.float32(1e-12)
        assert np.all(out["q"][m, g * 128:(g + 1) * 128] == 0)
        others = np.delete(sc[m], g)
        assert np.all(others > np.float32(1e-12))


def test_sequential_mode_rounds_through_bf16():
    """Pre-fusion pipeline: normalise to bf16, then quantise.  For a constant
    row of ones bf16(y) = 1.0 exactly, so s = fp32(1/448) there, while the
    fused path keeps y = 0.9999995 and its scale differs."""
    q, kv, gq, gk = const_rows(1.0, 1, 128, 32)
    seq = run(q, kv, gq, gk, sequential=True)
    fused = run(q, kv, gq, gk)
    assert np.all(seq["scale"] == np.float32(1.0 / 448.0))
    assert np.all(fused["scale"] != np.float32(1.0 / 448.0))
    assert np.all(seq["q"] == 0x7E) and np.all(fused["q"] == 0x7E)
    assert np.array_equal(seq["kv"], fused["kv"])


# ---------------------------------------------------------------- invariants

def test_unit_rms_of_normalised_row():
    """gamma = 1, eps = 0: mean(y^2) over the q row is exactly 1 (fp64)."""
    case = W.strided_batch(M=8, seed=21)
    gq = np.full(W.NQ, ONE_BF16, np.uint16)
    gk = np.full(W.NKV, ONE_BF16, np.uint16)
    out = run(case.q, case.kv, gq, gk, eps=0.0)
    ms = np.mean(out["y"] ** 2, axis=1)
    assert np.allclose(ms, 1.0, rtol=1e-12, atol=0)
    kvv = oracle.bf16_decode_array(out["kv"])
    assert np.allclose(np.mean(kvv ** 2, axis=1), 1.0, rtol=2 ** -7)


def test_q_and_kv_are_normalised_independently():
    case = W.strided_batch(M=4, seed=22)
    base = run(case.q, case.kv, case.gamma_q, case.gamma_kv)
    q2 = W.f32_to_bf16_bits(np.random.default_rng(5).standard_normal(case.q.shape).astype(np.float32) * 30)
    kv2 = W.f32_to_bf16_bits(np.random.default_rng(6).standard_normal(case.kv.shape).astype(np.float32) * 0.01)
    a = run(q2, case.kv, case.gamma_q, case.gamma_kv)
    b = run(case.q, kv2, case.gamma_q, case.gamma_kv)
    assert np.array_equal(a["kv"], base["kv"])
    assert np.array_equal(b["q"], base["q"]) and np.array_equal(b["scale"], base["scale"])
    assert not np.array_equal(a["q"], base["q"]) and not np.array_equal(b["kv"], base["kv"])


def test_scale_equivariance_without_eps():
    case = W.strided_batch(M=4, seed=23)
    q = np.ascontiguousarray(case.q)
    kv = np.ascontiguousarray(case.kv)
    base = run(q, kv, case.gamma_q, case.gamma_kv, eps=0.0)
    for k in (1, -3, 7):
        f = 2.0 ** k
        q2 = W.f32_to_bf16_bits(oracle.bf16_decode_array(q).astype(np.float32) * np.float32(f))
        kv2 = W.f32_to_bf16_bits(oracle.bf16_decode_array(kv).astype(np.float32) * np.float32(f))
        out = run(q2, kv2, case.gamma_q, case.gamma_kv, eps=0.0)
        for key in ("q", "scale", "kv"):
            assert np.array_equal(out[key], base[key]), (k, key)


def test_permutation_within_group_permutes_codes():
    case = W.decode_single(seed=24)
    q = np.ascontiguousarray(case.q).copy()
    gq = case.gamma_q.copy()
    base = run(q, case.kv, gq, case.gamma_kv)
    perm = np.random.default_rng(3).permutation(128)
    g = 5
    sl = slice(g * 128, (g + 1) * 128)
    q2, gq2 = q.copy(), gq.copy()
    q2[0, sl] = q[0, sl][perm]
    gq2[sl] = gq[sl][perm]
    out = run(q2, case.kv, gq2, case.gamma_kv)
    assert np.array_equal(out["scale"], base["scale"])
    assert np.array_equal(out["q"][0, sl], base["q"][0, sl][perm])
    assert np.array_equal(np.delete(out["q"][0], np.arange(sl.start, sl.stop)),
                          np.delete(base["q"][0], np.arange(sl.start, sl.stop)))


def e4m3_half_ulp(r):
    a = np.abs(r)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(e - 3))


@pytest.mark.parametrize("make", [lambda: W.decode_single(), lambda: W.strided_batch(64),
                                  lambda: W.outlier_stress(256), lambda: W.producer_activations(256)])
def test_group_invariants_on_workloads(make):
    case = make()
    out = run(case.q, case.kv, case.gamma_q, case.gamma_kv)
    M = case.M
    codes = out["q"]
    sc = out["scale"].reshape(M, 12)
    # no NaN codes
    assert not np.any((codes & 0x7F) == 0x7F)
    # every group with a non-floor scale holds a +-448 code
    mag = (codes & 0x7F).reshape(M, 12, 128)
    live = sc > np.float32(1e-12)
    assert np.all(np.any(mag == 0x7E, axis=2)[live])
    # dequantisation error <= half an e4m3 ULP (of y/s) times s; above 448
    # the clamp adds at most the excess over 448
    s_full = np.repeat(sc, 128, axis=1).astype(np.float64)
    deq = oracle.e4m3_decode_array(codes) * s_full
    r = out["ratio"]
    bound = (e4m3_half_ulp(np.minimum(np.abs(r), 448.0)) + np.maximum(np.abs(r) - 448.0, 0)) * s_full
    assert np.all(np.abs(out["y"] - deq) <= bound * (1 + 1e-12))
    # the clamp only ever removes a sub-ULP excess (s rounded to fp32)
    assert np.max(np.abs(r)) <= 448.0 * (1 + 2.0 ** -23)


def test_layouts_and_strided_views():
    case = W.strided_batch(M=16, seed=25)
    rowm = run(case.q, case.kv, case.gamma_q, case.gamma_kv, transpose=False)
    colm = run(case.q, case.kv, case.gamma_q, case.gamma_kv, transpose=True)
    # column-major bytes = x_scale.transpose(-1, -2).contiguous()
    assert np.array_equal(colm["scale"], rowm["scale"].reshape(16, 12).T.reshape(-1))
    assert np.array_equal(colm["q"], rowm["q"]) and np.array_equal(colm["kv"], rowm["kv"])
    cont = run(np.ascontiguousarray(case.q), np.ascontiguousarray(case.kv), case.gamma_q, case.gamma_kv)
    for key in ("q", "scale", "kv"):
        assert np.array_equal(cont[key], rowm[key])
    one = W.decode_single()
    a = run(one.q, one.kv, one.gamma_q, one.gamma_kv, transpose=False)
    b = run(one.q, one.kv, one.gamma_q, one.gamma_kv, transpose=True)
    assert np.array_equal(a["scale"], b["scale"])


# ------------------------------------------- independent high-precision check

@pytest.mark.parametrize("seed,Nq,Nkv", [(31, 256, 64), (32, 128, 8), (33, 384, 40)])
def test_tiny_inputs_vs_decimal_brute_force(seed, Nq, Nkv):
    getcontext().prec = 50
    r = np.random.default_rng(seed)
    M = 3
    q32 = r.standard_normal((M, Nq)).astype(np.float32)
    q32[r.random((M, Nq)) < 0.05] *= 40
    q32[1, :128] *= 1e-3
    kv32 = r.standard_normal((M, Nkv)).astype(np.float32)
    q, kv = bf16(q32), bf16(kv32)
    gq = bf16(1 + 0.1 * r.standard_normal(Nq))
    gk = bf16(1 + 0.1 * r.standard_normal(Nkv))
    eps = EPS32
    for transpose in (False, True):
        out = run(q, kv, gq, gk, eps=eps, transpose=transpose)
        G = Nq // 128
        for m in range(M):
            xq = [Decimal(oracle.bf16_decode(b)) for b in q[m]]
            xk = [Decimal(oracle.bf16_decode(b)) for b in kv[m]]
            rq = 1 / (sum(x * x for x in xq) / Nq + Decimal(eps)).sqrt()
            rk = 1 / (sum(x * x for x in xk) / Nkv + Decimal(eps)).sqrt()
            for i in range(Nkv):
                y = xk[i] * rk * Decimal(oracle.bf16_decode(gk[i]))
                assert out["kv"][m, i] == nearest_bf16(Fraction(y)), (m, i)
            for g in range(G):
                ys = [xq[i] * rq * Decimal(oracle.bf16_decode(gq[i])) for i in range(g * 128, (g + 1) * 128)]
                amax = max(abs(v) for v in ys)
                s = max(nearest_f32(Fraction(amax) / 448), FLOOR)
                at = g * M + m if transpose else m * G + g
                assert out["scale"][at] == np.float32(s), (m, g)
                for j, y in enumerate(ys):
                    want = nearest_e4m3(Fraction(y) / Fraction(s))
                    assert out["q"][m, g * 128 + j] == want, (m, g, j)
