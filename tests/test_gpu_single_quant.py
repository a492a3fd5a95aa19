"""GPU parity of the single-input quantisations (HIP, gfx950) against the CPU
oracle, through the C ABI: the RMSNorm + per-1x128 FP8 group quant of one
activation (PRHub digest of SGLang PR #27289, "实现拆解" item 2) and the
norm-less per-1x128 dynamic quant (the same digest's
aiter_w8a8_block_fp8_linear excerpt, branch B; GitHub page of vLLM PR
#53540, "Purpose": the second step of the unfused pipeline).

Cases: the q-latent width (1536) at decode and prefill batch sizes, a strided
column slice of a wider buffer, a wide 7168 row, the largest width (8192) on
the generic path, ragged / tiny / unaligned shapes, outliers with an all-zero
group per row, both scale layouts.  Bar: as for the dual operation (codes
within 1 e4m3 ULP, >= 99.9 % identical, mismatches only next to a midpoint
of the oracle's exact x/s; RMSNorm scales within 1e-6 relative).  The
norm-less quant is exact on both sides (scales one correctly rounded
division of exact values, codes the single rounding of the exact quotient),
so there codes and scales must be bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_fp8_block_amd as mi
from rmsnorm_fp8_block_amd import workloads as W

from helpers import compare_quant, dev_u16_as_bf16, gpu_or_skip, scale_buffer
from test_gpu_normquant import exhaustive_bf16_rows

pytestmark = pytest.mark.gpu


def upload(x: np.ndarray, dev) -> torch.Tensor:
    """A 2-D uint16 view with unit inner stride -> a device view with the
    same row stride (the padding columns are zero)."""
    M, N = x.shape
    stride = x.strides[0] // x.itemsize if M > 1 else N
    if stride == N:
        return dev_u16_as_bf16(x, dev)
    padded = np.zeros((M, stride), np.uint16)
    padded[:, :N] = x
    return dev_u16_as_bf16(padded, dev)[:, :N]


def run(x, gamma, transpose, dev, normalize=True, eps=W.EPS, xd=None):
    xd = upload(x, dev) if xd is None else xd
    if normalize:
        codes, scale = mi.mi_rmsnorm_group_quant(xd, dev_u16_as_bf16(gamma, dev), eps, transpose)
    else:
        codes, scale = mi.mi_group_quant_1x128(xd, transpose)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scale_buffer(scale)


def ref(x, gamma, transpose, normalize=True, eps=W.EPS):
    if normalize:
        return oracle.rmsnorm_group_quant(x, gamma, eps, transpose, want_ratio=True)
    return oracle.group_quant(x, transpose, want_ratio=True)


def assert_parity(got, r, normalize, label):
    if not normalize:
        mis = np.flatnonzero(got[0] != r["q"])
        assert mis.size == 0, f"{label}: {mis.size} codes differ, first at {mis[:4]}"
    stats = compare_quant(*got, r, label=label, scale_rtol=1e-6 if normalize else 0.0)
    print(f"{label}: {stats}")


def check(x, gamma, transpose, dev, normalize, label, eps=W.EPS):
    got = run(x, gamma, transpose, dev, normalize, eps)
    assert_parity(got, ref(x, gamma, transpose, normalize, eps), normalize, label)
    return got


WORKLOADS = {
    "decode_M1_N1536": dict(M=1, N=1536),
    "batch_M64_N1536_strided": dict(M=64, N=1536, pad=512),
    "batch_M256_N7168": dict(M=256, N=7168),
    "prefill_M8192_N1536": dict(M=8192, N=1536),
}


@pytest.mark.parametrize("normalize", [True, False], ids=["rmsnorm_quant", "quant"])
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name, normalize):
    dev = gpu_or_skip()
    x, gamma = W.single_input(**WORKLOADS[name])
    for t in (0, 1):
        check(x, gamma, t, dev, normalize, f"{name} normalize={normalize} t={t}")


@pytest.mark.parametrize("normalize", [True, False], ids=["rmsnorm_quant", "quant"])
@pytest.mark.parametrize("M,N,pad,seed", [(1, 128, 0, 21), (3, 256, 0, 22), (7, 640, 0, 23),
                                          (5, 8192, 0, 24), (33, 1024, 8, 25), (4099, 1536, 0, 26),
                                          (9, 7168, 128, 27), (2, 4096, 0, 28), (3, 2048, 0, 30),
                                          (1500, 7168, 0, 31), (2047, 2560, 8, 32), (2048, 3584, 0, 33)])
def test_generic_shapes(M, N, pad, seed, normalize):
    """Tiny, ragged (partial 512-element chunks, rows not a multiple of the
    rows per block), strided and largest widths, both layouts; below 2048
    rows, rows of 4 or more chunks are split over 2 or 4 waves (2048 x 3584
    is just above that, on one wave per row)."""
    dev = gpu_or_skip()
    x, gamma = W.single_input(M, N, seed=seed, pad=pad)
    for t in (0, 1):
        check(x, gamma, t, dev, normalize, f"M{M} N{N} pad{pad} normalize={normalize} t={t}")


@pytest.mark.parametrize("normalize", [True, False], ids=["rmsnorm_quant", "quant"])
def test_unaligned_rows_equal_aligned(normalize):
    """Row stride 1537 and a view starting one element in: no 16-byte
    alignment; oracle parity and bit-identity with the aligned run."""
    dev = gpu_or_skip()
    M, N = 10, 1536
    r = np.random.default_rng(29)
    wide = W.f32_to_bf16_bits(r.standard_normal((M, N + 1)).astype(np.float32))
    x_np = wide[:, 1:]
    _, gamma = W.single_input(1, N, seed=29)
    xd = dev_u16_as_bf16(wide, dev)[:, 1:]
    for t in (0, 1):
        got = run(x_np, gamma, t, dev, normalize, xd=xd)
        assert_parity(got, ref(x_np, gamma, t, normalize), normalize, f"unaligned t{t}")
        aligned = run(np.ascontiguousarray(x_np), gamma, t, dev, normalize)
        for a, b in zip(got, aligned):
            assert np.array_equal(a, b)


def test_rmsnorm_quant_equals_the_dual_ops_q_outputs():
    """Same q rows through the single-input and the dual entry point: the q
    path is the same computation, so codes and scales agree bit for bit."""
    dev = gpu_or_skip()
    for case in (W.strided_batch(64), W.prefill(1024)):
        buf = dev_u16_as_bf16(case.buffer, dev)
        q, kv = buf[:, :W.NQ], buf[:, W.NQ:]
        gq, gk = dev_u16_as_bf16(case.gamma_q, dev), dev_u16_as_bf16(case.gamma_kv, dev)
        for t in (0, 1):
            dq, ds, _ = mi.mi_fused_dual_rmsnorm_group_quant(q, kv, gq, gk, case.eps, t)
            sq, ss = mi.mi_rmsnorm_group_quant(q, gq, case.eps, t)
            assert torch.equal(dq, sq)
            assert np.array_equal(scale_buffer(ds), scale_buffer(ss))


def test_quant_is_rne_of_every_bf16_value():
    """Every bf16 magnitude in [2^-20, 448] with both signs, with 448 first
    in each group: s = 448 / 448 = 1 exactly, so every code is the single
    RNE rounding of a bf16 value (midpoints and subnormals included) and
    equals torch's cast."""
    dev = gpu_or_skip()
    x = exhaustive_bf16_rows()
    for t in (0, 1):
        got = run(x, None, t, dev, normalize=False)
        r = oracle.group_quant(x, t)
        assert np.all(r["scale"] == 1.0)
        assert np.array_equal(got[0], r["q"])
        assert np.array_equal(got[1], r["scale"])
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    assert np.array_equal(got[0], xt.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_pipeline_two_step_matches_oracle_sequential():
    """Unfused pipeline on the device: the oracle's RMSNorm rounded to bf16,
    then the device per-1x128 quant, equals the oracle's sequential mode of
    the dual operation bit for bit."""
    dev = gpu_or_skip()
    case = W.producer_activations(64)
    seq = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, case.eps, False,
                                          sequential=True, want_ratio=True)
    fused = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, case.eps, False,
                                            want_ratio=True)
    y_bf16 = np.vectorize(oracle.bf16_encode, otypes=[np.uint16])(fused["y"])
    got = run(y_bf16, None, 0, dev, normalize=False)
    assert_parity(got, seq, False, "two-step")


@pytest.mark.parametrize("normalize", [True, False], ids=["rmsnorm_quant", "quant"])
def test_zero_rows_is_a_noop(normalize):
    dev = gpu_or_skip()
    x = torch.zeros((0, 1536), dtype=torch.bfloat16, device=dev)
    g = torch.ones(1536, dtype=torch.bfloat16, device=dev)
    if normalize:
        codes, scale = mi.mi_rmsnorm_group_quant(x, g, W.EPS, True)
    else:
        codes, scale = mi.mi_group_quant_1x128(x, True)
    assert codes.shape == (0, 1536) and scale.shape == (0, 12)
