"""Pins for the oracle's bf16 and e4m3fn codecs.

The codecs are checked against the format definitions (closed-form values of
particular codes), against torch's CPU casts (library routines, on the inputs
where those casts are single, correctly rounded conversions), exhaustively over
all codes and all midpoints, and against a brute-force nearest-value search.
FP8 is read as OCP e4m3fn (bias 7, max 448, saturating encoder); the pages
name only "FP8" and a 1x128 group (vLLM PR #53540, "Purpose").
"""
import math

import numpy as np
import pytest
import torch

import oracle

ALL_E4M3 = np.arange(256, dtype=np.uint8)


def torch_e4m3_values():
    return torch.from_numpy(ALL_E4M3.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def finite_codes_sorted():
    """(value, code) for every finite non-negative e4m3fn code, ascending."""
    out = []
    for c in range(0x7F):          # 0x00 .. 0x7E; 0x7F is NaN
        out.append((oracle.e4m3_decode(c), c))
    return out


# ---------------------------------------------------------------- e4m3fn ----

def test_e4m3_decode_matches_format_definition():
    assert oracle.e4m3_decode(0x00) == 0.0
    assert math.copysign(1.0, oracle.e4m3_decode(0x80)) == -1.0
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9          # smallest subnormal
    assert oracle.e4m3_decode(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6          # smallest normal
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0x39) == 1.125
    assert oracle.e4m3_decode(0x7E) == 448.0              # largest finite
    assert oracle.e4m3_decode(0xFE) == -448.0
    assert math.isnan(oracle.e4m3_decode(0x7F))
    assert math.isnan(oracle.e4m3_decode(0xFF))


def test_e4m3_decode_all_codes_vs_torch():
    ours = oracle.e4m3_decode_array(ALL_E4M3)
    ref = torch_e4m3_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_roundtrip_every_finite_code():
    for c in range(256):
        v = oracle.e4m3_decode(c)
        if math.isnan(v):
            continue
        assert oracle.e4m3_encode(v) == c, hex(c)


def test_e4m3_midpoints_round_to_even_and_neighbours_to_nearest():
    vals = finite_codes_sorted()
    for (lo, clo), (hi, chi) in zip(vals, vals[1:]):
        mid = (lo + hi) / 2.0                 # exact in fp64
        even = clo if clo % 2 == 0 else chi   # even mantissa == even code
        assert oracle.e4m3_encode(mid) == even, (lo, hi)
        assert oracle.e4m3_encode(-mid) == 0x80 | even
        below = math.nextafter(mid, -math.inf)
        above = math.nextafter(mid, math.inf)
        assert oracle.e4m3_encode(below) == clo
        assert oracle.e4m3_encode(above) == chi


def test_e4m3_saturates_and_handles_specials():
    for v in (448.0, 448.0000001, 463.99, 464.0, 480.0, 1e30, math.inf):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_encode(math.nan) == 0x7F
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00          # tie between 0 and 2^-9 -> even
    assert oracle.e4m3_encode(1.5 * 2.0 ** -10) == 0x01
    assert oracle.e4m3_encode(2.0 ** -30) == 0x00


def test_e4m3_encode_vs_torch_cast_in_range():
    r = np.random.Generator(np.random.PCG64(7))
    # log-uniform magnitudes over the whole e4m3 range, both signs (fp32
    # inputs: torch's cast is then a single RNE rounding)
    mags = np.exp2(r.uniform(-12, math.log2(463.0), 20000)).astype(np.float32)
    x = mags * np.where(r.random(20000) < 0.5, -1, 1).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(ours, ref)


def test_e4m3_encode_vs_brute_force_nearest():
    vals = finite_codes_sorted()
    grid = np.array([v for v, _ in vals])
    codes = [c for _, c in vals]
    r = np.random.Generator(np.random.PCG64(8))
    xs = np.concatenate([r.uniform(0, 448, 3000), np.exp2(r.uniform(-11, 8.8, 3000))])
    for x in xs:
        d = np.abs(grid - x)
        best = np.flatnonzero(d == d.min())
        # ties -> the even code
        pick = [codes[i] for i in best if codes[i] % 2 == 0] or [codes[best[0]]]
        want = min(pick) if x < 448 else 0x7E
        assert oracle.e4m3_encode(float(x)) == want, x


# ------------------------------------------------------------------ bf16 ----

def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.bf16_decode_array(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_roundtrip_all_finite_patterns():
    for b in range(65536):
        v = oracle.bf16_decode(b)
        if math.isnan(v):
            continue
        assert oracle.bf16_encode(v) == b, hex(b)


def test_bf16_encode_vs_torch_for_fp32_inputs():
    r = np.random.Generator(np.random.PCG64(9))
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        np.exp2(r.uniform(-140, 127, 20000)).astype(np.float32),
        # exact bf16 midpoints (fp32 values with the low 16 bits = 0x8000)
        ((r.integers(0x0080, 0x7F00, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_encode(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encode_rounds_fp64_once():
    # 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7; anything above it must
    # round up even if the excess is lost by an intermediate fp32 rounding.
    assert oracle.bf16_encode(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_encode(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert oracle.bf16_encode(1.0 + 3 * 2.0 ** -8) == 0x3F82            # tie -> even
    assert oracle.bf16_encode(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    # subnormals: spacing 2^-133
    assert oracle.bf16_encode(2.0 ** -133) == 0x0001
    assert oracle.bf16_encode(2.0 ** -134) == 0x0000
    assert oracle.bf16_encode(1.5 * 2.0 ** -134) == 0x0001
    assert oracle.bf16_encode(2.0 ** -126) == 0x0080
    # overflow to infinity beyond the largest finite value
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127                               # largest finite
    assert oracle.bf16_encode(big) == 0x7F7F
    assert oracle.bf16_encode((2.0 - 2.0 ** -8) * 2.0 ** 127) == 0x7F80  # tie -> even = inf
    assert oracle.bf16_encode(math.nextafter((2.0 - 2.0 ** -8) * 2.0 ** 127, 0)) == 0x7F7F
