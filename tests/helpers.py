"""Shared helpers for the GPU parity tests: host <-> device transfer of raw
bit patterns and the comparison metrics against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

GROUP = 128

# Tolerances (the targets the build is held to):
#   FP8 codes within 1 e4m3 ULP, >= 99.9 % identical; scales relative error
#   <= 1e-6; kv within 1 bf16 ULP; GEMM relative error <= 2e-2.
CODE_EXACT_FRACTION = 0.999
SCALE_RTOL = 1e-6
GEMM_RTOL = 2e-2
# A code may differ from the oracle's only where the oracle's exact y/s lies
# this close (relative) to an e4m3 rounding midpoint: the kernel works in
# fp32 (a few fp32 ULPs, ~2^-21, of error in y/s), the oracle in fp64.
MIDPOINT_WINDOW = 2.0 ** -18


def gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def dev_u16_as_bf16(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def dev_u8(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def dev_f32(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def scale_buffer(scale: torch.Tensor) -> np.ndarray:
    """The bytes of a [M, G] scale tensor in storage order (row-major or
    column-major as its strides say)."""
    M, G = scale.shape
    if scale.stride() == (1, M) and M > 1:
        return scale.T.contiguous().reshape(-1).cpu().numpy()
    return scale.contiguous().reshape(-1).cpu().numpy()


def e4m3_ord(c: np.ndarray) -> np.ndarray:
    c = np.asarray(c, dtype=np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def bf16_ord(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def e4m3_midpoint_distance(ratio: np.ndarray) -> np.ndarray:
    """Relative distance of |ratio| to the nearest e4m3fn rounding midpoint
    (inf above the largest finite value)."""
    a = np.minimum(np.abs(ratio), 448.0)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    q = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(e - 3))     # code spacing
    mid = (np.floor(a / q) + 0.5) * q
    d = np.abs(a - mid)
    # the midpoint just below the binade start is half the lower spacing away
    lower_mid = np.exp2(e) - 0.25 * q
    d = np.where(a >= 2.0 ** -6, np.minimum(d, np.abs(a - lower_mid)), d)
    return d / np.maximum(a, 2.0 ** -12)


def compare_quant(got_q, got_scale_buf, ref, label="", scale_rtol=SCALE_RTOL):
    """Assert the parity bar on codes and scales; return statistics.

    Codes: within 1 e4m3 ULP everywhere; every differing code must sit where
    the oracle's exact y/s is within MIDPOINT_WINDOW of a rounding midpoint
    (away from a midpoint the code is unique and must match); and, on inputs
    large enough for the fraction to mean something (>= 10^4 codes), at
    least 99.9 % identical.  Scales: relative error <= scale_rtol (0: equal
    bit for bit)."""
    rq = ref["q"]
    assert got_q.shape == rq.shape
    assert not np.any((got_q & 0x7F) == 0x7F), f"{label}: NaN code"
    d = np.abs(e4m3_ord(got_q) - e4m3_ord(rq))
    exact = float((d == 0).mean())
    assert d.max() <= 1, f"{label}: code off by {d.max()} ULP"
    n_mis = int((d != 0).sum())
    if n_mis and "ratio" in ref:
        near = e4m3_midpoint_distance(ref["ratio"])[d != 0]
        assert np.all(near <= MIDPOINT_WINDOW), \
            f"{label}: {int((near > MIDPOINT_WINDOW).sum())} code mismatches away from a midpoint"
    if d.size >= 10_000:
        assert exact >= CODE_EXACT_FRACTION, f"{label}: only {exact:.5f} of codes exact"
    rs = ref["scale"]
    if scale_rtol == 0:
        assert np.array_equal(got_scale_buf, rs), f"{label}: scales not bit-exact"
    rel = np.abs(got_scale_buf.astype(np.float64) / rs.astype(np.float64) - 1.0)
    assert rel.max() <= scale_rtol, f"{label}: scale rel err {rel.max():.3e}"
    return {"code_exact": exact, "code_mismatches": n_mis, "scale_max_rel": float(rel.max())}


def compare_normquant(got_q, got_scale_buf, got_kv, ref, label=""):
    """compare_quant on the q outputs, and kv within 1 bf16 ULP."""
    stats = compare_quant(got_q, got_scale_buf, ref, label)
    dk = np.abs(bf16_ord(got_kv) - bf16_ord(ref["kv"]))
    assert dk.max() <= 1, f"{label}: kv off by {dk.max()} bf16 ULP"
    stats["kv_exact"] = float((dk == 0).mean())
    return stats


def gemm_error(out: np.ndarray, ref: np.ndarray):
    """(relative Frobenius error, max abs error / max |ref|)."""
    fro = float(np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(out - ref).max() / max(np.abs(ref).max(), 1e-300))
    return fro, mx


def assert_gemm_close(out: np.ndarray, ref: np.ndarray, label=""):
    fro, mx = gemm_error(out, ref)
    assert fro <= GEMM_RTOL and mx <= GEMM_RTOL, f"{label}: rel err fro={fro:.3e} max={mx:.3e}"
    return fro, mx


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_oracle_case(case, transpose, want_ratio=True):
    return oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv,
                                           case.eps, transpose, want_ratio=want_ratio)


# e8m0 scales: relative distance of amax / 448 to a power of two within which
# the exponent byte may differ by one from the oracle's
BOUNDARY = 2.0 ** -20


def compare_e8m0(codes, sbytes, ref, M, G, transpose, label):
    """e8m0 norm-quant bar: exponent bytes equal to the oracle's except, by
    one, where the group's amax / 448 lies within BOUNDARY of a power of two
    (those groups' codes are not compared); other codes within 1 e4m3 ULP,
    any difference next to a rounding midpoint, >= CODE_EXACT_FRACTION
    identical, no NaN code.  Returns (exact fraction, groups whose exponent
    differs)."""
    rs = ref["scale"].astype(np.int64)
    gs = sbytes.astype(np.int64)
    to_mg = (lambda a: a.reshape(G, M).T) if transpose else (lambda a: a.reshape(M, G))
    rs, gs = to_mg(rs), to_mg(gs)
    diff = rs != gs
    ratio = ref["ratio"].reshape(M, G, 128)
    rmax = np.abs(ratio).max(axis=2)                 # amax / s_oracle, in (224, 448] for live groups
    if diff.any():
        assert np.all(np.abs(gs[diff] - rs[diff]) == 1), f"{label}: exponent off by more than one"
        near = np.minimum(np.abs(rmax[diff] / 448 - 1), np.abs(rmax[diff] / 224 - 1))
        assert np.all(near <= BOUNDARY), f"{label}: exponent differs away from a power-of-two boundary"
    keep = np.repeat(~diff, 128, axis=1).reshape(M, G * 128)
    got, want = codes[keep], ref["q"][keep]
    assert not np.any((got & 0x7F) == 0x7F), f"{label}: NaN code"
    d = np.abs(e4m3_ord(got) - e4m3_ord(want))
    assert d.max(initial=0) <= 1, f"{label}: code off by {d.max()} ULP"
    if (d != 0).any():
        near = e4m3_midpoint_distance(ref["ratio"][keep][d != 0])
        assert np.all(near <= MIDPOINT_WINDOW), f"{label}: code mismatch away from a midpoint"
    exact = float((d == 0).mean()) if d.size else 1.0
    if d.size >= 10_000:
        assert exact >= CODE_EXACT_FRACTION, f"{label}: only {exact:.5f} exact"
    return exact, int(diff.sum())
