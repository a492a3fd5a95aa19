"""GPU parity of the one-call decode step (mi_fused_normquant_gemm_pair):
the fused dual RMSNorm + per-1x128 FP8 group quant of the q/kv latents
(GitHub page of vLLM PR #53540, "Purpose") and both block-scaled FP8
consumers of its (q_fp8, scale) pair (PRHub digest of the same PR, the
apply_pre_quantized_block_scaled_mm excerpt), in one launch for decode
batches of the MLA shape.

Bar: all five outputs bit-identical to the two calls it replaces
(mi_fused_dual_rmsnorm_group_quant, then mi_block_scaled_fp8_gemm_pair), at
every batch size of the one-launch path, both scale layouts, both weight
layouts, and on the shapes that fall back to two launches; against the
oracle chain, the norm-quant bar of the dual operation and the GEMM's
relative error bar on sampled column blocks; also when the inputs change
between calls that reuse the output buffers, and under graph replay.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_fp8_block_amd as mi
from rmsnorm_fp8_block_amd import workloads as W

from helpers import (assert_gemm_close, bf16_to_f64, compare_e8m0, compare_normquant, dev_f32, dev_u16_as_bf16,
                     dev_u8, gpu_or_skip, host_bf16_bits, scale_buffer)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def weights():
    """W_a [24576, 1536] and W_b [8192, 1536] (host codes and scales, device
    copies row-major and tiled)."""
    dev = gpu_or_skip()
    out = {}
    for name, (shape, seed) in (("W_a", (W.W_A_SHAPE, W.W_A_SEED)), ("W_b", (W.W_B_SHAPE, W.W_B_SEED))):
        wt = W.block_fp8_weight(*shape, seed)
        d = dev_u8(wt.codes, dev)
        out[name] = dict(host=wt, row=d, tiled=mi.relayout_weight(d), scale=dev_f32(wt.scale, dev))
    return out


def device_case(case, dev):
    if case.buffer is not None:
        buf = dev_u16_as_bf16(case.buffer, dev)
        q, kv = buf[:, :case.q.shape[1]], buf[:, case.q.shape[1]:]
    else:
        q, kv = dev_u16_as_bf16(case.q, dev), dev_u16_as_bf16(case.kv, dev)
    return q, kv, dev_u16_as_bf16(case.gamma_q, dev), dev_u16_as_bf16(case.gamma_kv, dev)


def two_calls(q, kv, gq, gk, t, w1, s1, w2, s2):
    codes, scale, kvo = mi.mi_fused_dual_rmsnorm_group_quant(q, kv, gq, gk, W.EPS, t)
    o1, o2 = mi.mi_block_scaled_fp8_gemm_pair(codes, scale, w1, s1, w2, s2)
    return codes, scale, kvo, o1, o2


def host(outs):
    codes, scale, kvo, o1, o2 = outs
    return (codes.cpu().numpy(), scale_buffer(scale), host_bf16_bits(kvo), host_bf16_bits(o1), host_bf16_bits(o2))


def assert_same(got, want, label):
    for name, g, w in zip(("q_fp8", "scale", "kv", "out1", "out2"), host(got), host(want)):
        assert np.array_equal(g, w), f"{label}: {name} differs"


@pytest.mark.parametrize("layout", ["tiled", "row"])
@pytest.mark.parametrize("M", [1, 2, 5, 8, 15, 16, 17, 20, 32, 33, 48, 64])
def test_step_equals_the_two_calls(M, layout, weights):
    """One launch up to 16 rows, two launches above (the query says which),
    ragged sizes, both scale layouts, both weight layouts: bit-identical to
    the two calls."""
    dev = gpu_or_skip()
    q, kv, gq, gk = device_case(W.producer_activations(M), dev)
    wa, wb = weights["W_a"], weights["W_b"]
    assert mi.mi_fused_normquant_gemm_pair_launches(M, 1536, 512, 24576, 8192) == (1 if M <= 16 else 2)
    for t in (0, 1):
        args = (wa[layout], wa["scale"], wb[layout], wb["scale"])
        got = mi.mi_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, t, *args)
        want = two_calls(q, kv, gq, gk, t, *args)
        torch.cuda.synchronize()
        assert_same(got, want, f"M{M} {layout} t{t}")


@pytest.mark.parametrize("M", [16, 64])
def test_step_vs_oracle(M, weights):
    """M = 16 (one launch) and 64 (two), column-major scales, tiled
    weights: the norm-quant outputs to the dual operation's bar, both GEMM
    outputs on sampled 128-column blocks against the oracle chain on the
    same inputs."""
    dev = gpu_or_skip()
    case = W.strided_batch(M)
    q, kv, gq, gk = device_case(case, dev)
    wa, wb = weights["W_a"], weights["W_b"]
    codes, scale, kvo, o1, o2 = mi.mi_fused_normquant_gemm_pair(
        q, kv, gq, gk, case.eps, True, wa["tiled"], wa["scale"], wb["tiled"], wb["scale"])
    torch.cuda.synchronize()
    ref = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, case.eps, True,
                                          want_ratio=True)
    compare_normquant(codes.cpu().numpy(), scale_buffer(scale), host_bf16_bits(kvo), ref, label=f"step M{M}")
    for name, out in (("W_a", o1), ("W_b", o2)):
        wt = weights[name]["host"]
        nb = wt.codes.shape[0] // 128
        blocks = np.unique([0, 1, nb // 2, nb - 1])
        cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
        gref = oracle.block_scaled_fp8_gemm(ref["q"], ref["scale"], True, wt.codes[cols], wt.scale[blocks])
        assert_gemm_close(bf16_to_f64(out)[:, cols], gref, f"step {name}")


@pytest.mark.parametrize("M", [16, 64])
def test_step_every_column_vs_oracle(M, weights):
    """The decode-step configurations at their full widths (W_a [24576, 1536]
    and W_b [8192, 1536], all 32 768 output columns; M = 16 in one launch,
    64 in two): every GEMM output element against the oracle GEMM on the
    step's own quantised pair, to the element-wise bar: bf16 rounding of the
    result plus an accumulation error of at most 2^-12 of the sum of the
    scaled |a| |w| products."""
    dev = gpu_or_skip()
    case = W.strided_batch(M)
    q, kv, gq, gk = device_case(case, dev)
    wa, wb = weights["W_a"], weights["W_b"]
    codes, scale, _, o1, o2 = mi.mi_fused_normquant_gemm_pair(
        q, kv, gq, gk, case.eps, True, wa["tiled"], wa["scale"], wb["tiled"], wb["scale"])
    torch.cuda.synchronize()
    q_np, s_np = codes.cpu().numpy(), scale_buffer(scale)
    a_abs = np.abs(oracle.e4m3_decode_array(q_np)) * np.repeat(s_np.reshape(12, M).T.astype(np.float64), 128, axis=1)
    for name, out in (("W_a", o1), ("W_b", o2)):
        wt = weights[name]["host"]
        ref = oracle.block_scaled_fp8_gemm(q_np, s_np, True, wt.codes, wt.scale)
        w_abs = np.abs(oracle.e4m3_decode_array(wt.codes)) * np.repeat(
            np.repeat(wt.scale.astype(np.float64), 128, axis=0), 128, axis=1)
        mag = a_abs @ w_abs.T
        got = bf16_to_f64(out)
        err = np.abs(got - ref)
        fro, mx = assert_gemm_close(got, ref, f"step M{M} {name} all columns")
        print(f"step M{M} {name} [{wt.codes.shape[0]} columns]: fro {fro:.2e} max {mx:.2e} "
              f"max(err/mag) {np.max(err / mag):.3e}")
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * mag), f"step M{M} {name}"


def test_step_back_to_back_with_changing_inputs(weights):
    """Calls on one stream sharing the output buffers, with new activations
    every call and batch sizes 16, 1, 64, 7, 33, 64, 17, 16 (one and two
    launches in turn): each call equals the two calls on its own inputs."""
    dev = gpu_or_skip()
    wa, wb = weights["W_a"], weights["W_b"]
    bufs = {k: None for k in ("q", "s", "kv", "o1", "o2")}
    Ms = (16, 1, 64, 7, 33, 64, 17, 16)
    for i, M in enumerate(Ms):
        q, kv, gq, gk = device_case(W.producer_activations(M, seed=40 + i), dev)
        if bufs["q"] is None or bufs["q"].shape[0] != M:
            bufs = dict(q=torch.empty((M, 1536), dtype=torch.uint8, device=dev),
                        s=torch.empty(M * 12, dtype=torch.float32, device=dev),
                        kv=torch.empty((M, 512), dtype=torch.bfloat16, device=dev),
                        o1=torch.empty((M, 24576), dtype=torch.bfloat16, device=dev),
                        o2=torch.empty((M, 8192), dtype=torch.bfloat16, device=dev))
        got = mi.mi_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, True, wa["tiled"], wa["scale"], wb["tiled"],
                                              wb["scale"], out_q=bufs["q"], out_scale=bufs["s"], out_kv=bufs["kv"],
                                              out1=bufs["o1"], out2=bufs["o2"])
        want = two_calls(q, kv, gq, gk, True, wa["tiled"], wa["scale"], wb["tiled"], wb["scale"])
        torch.cuda.synchronize()
        assert_same(got, want, f"call {i} M{M}")


@pytest.mark.parametrize("M,Nq,Nkv,N1,N2", [(65, 1536, 512, 24576, 8192), (100, 1536, 512, 24576, 8192),
                                            (64, 1536, 512, 3072, 1024), (16, 1024, 512, 24576, 8192),
                                            (8, 1536, 448, 24576, 8192), (200, 1536, 512, 3072, 1024)])
def test_step_shapes_that_take_two_launches(M, Nq, Nkv, N1, N2):
    """Beyond 64 rows (three launches over the full weights, two over a
    TP-8 shard pair), narrow weights, other latent widths: the same results
    as the two calls."""
    dev = gpu_or_skip()
    r = np.random.default_rng(M + Nq + N1)
    buf = W.f32_to_bf16_bits(r.standard_normal((M, Nq + Nkv), dtype=np.float32))
    gq, gk = W.gammas(Nq, Nkv)
    d = dev_u16_as_bf16(buf, dev)
    q, kv = d[:, :Nq], d[:, Nq:]
    gq, gk = dev_u16_as_bf16(gq, dev), dev_u16_as_bf16(gk, dev)
    w1 = W.block_fp8_weight(N1, Nq, 60)
    w2 = W.block_fp8_weight(N2, Nq, 61)
    args = (dev_u8(w1.codes, dev), dev_f32(w1.scale, dev), dev_u8(w2.codes, dev), dev_f32(w2.scale, dev))
    got = mi.mi_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, True, *args)
    want = two_calls(q, kv, gq, gk, True, *args)
    torch.cuda.synchronize()
    assert_same(got, want, f"M{M} Nq{Nq} Nkv{Nkv} N{N1}+{N2}")
    narrow_above_64 = M > 64 and Nq == 1536 and (N1 + N2) // 16 <= 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    assert mi.mi_fused_normquant_gemm_pair_launches(M, Nq, Nkv, N1, N2) == (2 if narrow_above_64 or M <= 64 else 3)


@pytest.mark.parametrize("M", [16, 64])
def test_step_graph_replays(M, weights):
    """The step captured in a HIP graph (one launch at 16 rows, two at 64):
    four replays, the input rewritten by eager work between them, each
    replay equal to the eager two calls on that input."""
    dev = gpu_or_skip()
    wa, wb = weights["W_a"], weights["W_b"]
    case = W.strided_batch(M)
    q, kv, gq, gk = device_case(case, dev)
    buf = q._base if q._base is not None else None
    assert buf is not None and buf.shape == (M, 2048)
    outs = (torch.empty((M, 1536), dtype=torch.uint8, device=dev), torch.empty(M * 12, dtype=torch.float32, device=dev),
            torch.empty((M, 512), dtype=torch.bfloat16, device=dev),
            torch.empty((M, 24576), dtype=torch.bfloat16, device=dev),
            torch.empty((M, 8192), dtype=torch.bfloat16, device=dev))
    call = mi.prepare_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, True, wa["tiled"], wa["scale"], wb["tiled"],
                                                wb["scale"], *outs)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture (sets the kernel's LDS attribute)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        r = np.random.default_rng(70 + i)
        buf.copy_(dev_u16_as_bf16(W.f32_to_bf16_bits(r.standard_normal((M, 2048), dtype=np.float32)), dev))
        g.replay()
        torch.cuda.synchronize()
        want = two_calls(q, kv, gq, gk, True, wa["tiled"], wa["scale"], wb["tiled"], wb["scale"])
        got = (outs[0], outs[1].view(12, M).T, outs[2], outs[3], outs[4])
        torch.cuda.synchronize()
        assert_same(got, want, f"replay {i}")


def test_step_unaligned_views_take_two_launches(weights):
    """q and kv as views of a [16, 2049] buffer one element in (rows and
    slices not 16-byte aligned): the call takes the two launches (whose
    kernels handle any alignment) and equals the two calls."""
    dev = gpu_or_skip()
    M = 16
    r = np.random.default_rng(81)
    buf = dev_u16_as_bf16(W.f32_to_bf16_bits(r.standard_normal((M, 2049), dtype=np.float32)), dev)
    q, kv = buf[:, 1:1537], buf[:, 1537:]
    gq, gk = (dev_u16_as_bf16(g, dev) for g in W.gammas())
    wa, wb = weights["W_a"], weights["W_b"]
    for t in (0, 1):
        args = (wa["tiled"], wa["scale"], wb["tiled"], wb["scale"])
        got = mi.mi_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, t, *args)
        want = two_calls(q, kv, gq, gk, t, *args)
        torch.cuda.synchronize()
        assert_same(got, want, f"unaligned t{t}")


def test_step_zero_rows(weights):
    dev = gpu_or_skip()
    q = torch.zeros((0, 1536), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((0, 512), dtype=torch.bfloat16, device=dev)
    gq, gk = (dev_u16_as_bf16(g, dev) for g in W.gammas())
    wa, wb = weights["W_a"], weights["W_b"]
    codes, scale, kvo, o1, o2 = mi.mi_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, True, wa["tiled"], wa["scale"],
                                                                wb["tiled"], wb["scale"])
    assert codes.shape == (0, 1536) and scale.shape == (0, 12) and kvo.shape == (0, 512)
    assert o1.shape == (0, 24576) and o2.shape == (0, 8192)


# ---------------------------------------------------------------------------
# the step with e8m0 (power-of-two) scales on both sides: the e8m0 norm-quant
# (exponent bytes) feeding the e8m0 pair, whose matrix cores apply the
# activation and weight exponents (PRHub digest of vLLM PR #56560)


@pytest.fixture(scope="module")
def weights_e8m0():
    dev = gpu_or_skip()
    out = {}
    for name, (shape, seed) in (("W_a", (W.W_A_SHAPE, W.W_A_SEED)), ("W_b", (W.W_B_SHAPE, W.W_B_SEED))):
        wt = W.block_fp8_weight_e8m0(*shape, seed)
        d = dev_u8(wt.codes, dev)
        out[name] = dict(host=wt, row=d, tiled=mi.relayout_weight(d), scale=dev_u8(wt.scale, dev))
    return out


def two_calls_e8m0(q, kv, gq, gk, t, w1, s1, w2, s2):
    codes, scale, kvo = mi.mi_fused_dual_rmsnorm_group_quant_e8m0(q, kv, gq, gk, W.EPS, t)
    o1, o2 = mi.mi_block_scaled_fp8_gemm_pair(codes, scale, w1, s1, w2, s2)
    return codes, scale, kvo, o1, o2


@pytest.mark.parametrize("layout", ["tiled", "row"])
@pytest.mark.parametrize("M", [1, 7, 16, 33, 64])
def test_step_e8m0_equals_the_two_calls(M, layout, weights_e8m0):
    """e8m0 scales: one launch up to 16 rows, two above; both scale layouts:
    bit-identical to the e8m0 norm-quant followed by the e8m0 pair."""
    dev = gpu_or_skip()
    q, kv, gq, gk = device_case(W.producer_activations(M), dev)
    wa, wb = weights_e8m0["W_a"], weights_e8m0["W_b"]
    for t in (0, 1):
        args = (wa[layout], wa["scale"], wb[layout], wb["scale"])
        got = mi.mi_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, t, *args)
        assert got[1].dtype == torch.uint8
        want = two_calls_e8m0(q, kv, gq, gk, t, *args)
        torch.cuda.synchronize()
        assert_same(got, want, f"e8m0 M{M} {layout} t{t}")


def test_step_e8m0_vs_oracle(weights_e8m0):
    """M = 16 (one launch), column-major exponent bytes: the norm-quant
    outputs to the e8m0 bar against the e8m0 oracle, both GEMM outputs on
    sampled column blocks against the fp64 oracle GEMM on the decoded
    scales of the oracle's own quantised pair."""
    dev = gpu_or_skip()
    case = W.strided_batch(16)
    q, kv, gq, gk = device_case(case, dev)
    wa, wb = weights_e8m0["W_a"], weights_e8m0["W_b"]
    codes, scale, kvo, o1, o2 = mi.mi_fused_normquant_gemm_pair(
        q, kv, gq, gk, case.eps, True, wa["tiled"], wa["scale"], wb["tiled"], wb["scale"])
    _, _, kv32 = mi.mi_fused_dual_rmsnorm_group_quant(q, kv, gq, gk, case.eps, True)
    torch.cuda.synchronize()
    assert torch.equal(kvo, kv32), "kv must equal the fp32-scale call's"
    ref = oracle.dual_rmsnorm_group_quant_e8m0(case.q, case.kv, case.gamma_q, case.gamma_kv, case.eps, True,
                                               want_ratio=True)
    compare_e8m0(codes.cpu().numpy(), scale_buffer(scale), ref, 16, 12, True, "e8m0 step M16")
    asf = oracle.e8m0_decode_array(ref["scale"]).astype(np.float32)
    for name, out in (("W_a", o1), ("W_b", o2)):
        wt = weights_e8m0[name]["host"]
        nb = wt.codes.shape[0] // 128
        blocks = np.unique([0, 1, nb // 2, nb - 1])
        cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
        bsf = oracle.e8m0_decode_array(wt.scale[blocks]).astype(np.float32)
        gref = oracle.block_scaled_fp8_gemm(ref["q"], asf, True, wt.codes[cols], bsf)
        assert_gemm_close(bf16_to_f64(out)[:, cols], gref, f"e8m0 step {name}")


def test_step_refuses_mixed_scale_types(weights, weights_e8m0):
    """Both weights' scales, and a given out_scale, must be of one type."""
    dev = gpu_or_skip()
    q, kv, gq, gk = device_case(W.producer_activations(4), dev)
    wa, wb = weights["W_a"], weights_e8m0["W_b"]
    with pytest.raises(ValueError):
        mi.mi_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, True, wa["tiled"], wa["scale"], wb["tiled"],
                                        wb["scale"])
    with pytest.raises(ValueError):
        mi.mi_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, True, wa["tiled"], wa["scale"], wa["tiled"],
                                        wa["scale"], out_scale=torch.empty(48, dtype=torch.uint8, device=dev))


def test_step_e8m0_graph_replays(weights_e8m0):
    """The e8m0 one-launch step captured in a HIP graph: three replays with
    the input rewritten by eager work between them, each equal to the eager
    e8m0 two calls on that input."""
    dev = gpu_or_skip()
    wa, wb = weights_e8m0["W_a"], weights_e8m0["W_b"]
    M = 16
    case = W.strided_batch(M)
    q, kv, gq, gk = device_case(case, dev)
    buf = q._base
    assert buf is not None and buf.shape == (M, 2048)
    outs = (torch.empty((M, 1536), dtype=torch.uint8, device=dev), torch.empty(M * 12, dtype=torch.uint8, device=dev),
            torch.empty((M, 512), dtype=torch.bfloat16, device=dev),
            torch.empty((M, 24576), dtype=torch.bfloat16, device=dev),
            torch.empty((M, 8192), dtype=torch.bfloat16, device=dev))
    call = mi.prepare_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, True, wa["tiled"], wa["scale"], wb["tiled"],
                                                wb["scale"], *outs)
    assert call.name == "mi_fused_normquant_gemm_pair_e8m0"
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture (sets the kernel's LDS attribute)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        r = np.random.default_rng(90 + i)
        buf.copy_(dev_u16_as_bf16(W.f32_to_bf16_bits(r.standard_normal((M, 2048), dtype=np.float32)), dev))
        g.replay()
        torch.cuda.synchronize()
        want = two_calls_e8m0(q, kv, gq, gk, True, wa["tiled"], wa["scale"], wb["tiled"], wb["scale"])
        got = (outs[0], outs[1].view(12, M).T, outs[2], outs[3], outs[4])
        torch.cuda.synchronize()
        assert_same(got, want, f"e8m0 replay {i}")
