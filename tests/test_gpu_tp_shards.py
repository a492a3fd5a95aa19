"""GPU parity of the block-scaled FP8 GEMM at tensor-parallel shard shapes.

Under column parallelism each rank holds N/TP rows of both consumer weights
(W_a [24576, 1536] and W_b [8192, 1536]) with their 128x128 block scales,
and multiplies the replicated (q_fp8, scale) pair.  The PRHub report of vLLM
PR #56433 ("功能与动机") records that the silent As layout mismatch only
showed at TP >= 4 shapes (TP4/TP8 for DeepSeek V3/R1, TP > 2 for Kimi-K2),
so every shard shape is checked here: TP in {1, 2, 4, 8} (the last rank's
rows, so shard offsets matter), M in {1, 16, 64, 256}, both As layouts, the
two-consumer launch against two single launches bit for bit and against the
oracle on sampled column blocks; and, for M > 1, the wrong layout flag must
give a large error at every shard shape (the bytes differ).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import rmsnorm_fp8_block_amd as mi
from rmsnorm_fp8_block_amd import _binding as B
from rmsnorm_fp8_block_amd import workloads as W

from helpers import (assert_gemm_close, bf16_to_f64, dev_f32, dev_u8, dev_u16_as_bf16, gemm_error,
                     gpu_or_skip, host_bf16_bits)

pytestmark = pytest.mark.gpu

_W = {}


def full_weights():
    if not _W:
        _W["a"] = W.block_fp8_weight(*W.W_A_SHAPE, W.W_A_SEED)
        _W["b"] = W.block_fp8_weight(*W.W_B_SHAPE, W.W_B_SEED)
    return _W["a"], _W["b"]


def shard(wt, tp, rank):
    n = wt.codes.shape[0] // tp
    return wt.codes[rank * n:(rank + 1) * n], wt.scale[rank * n // 128:(rank + 1) * n // 128]


def sampled_ref(codes, scale_q, layout, wc, ws, seed):
    nb = wc.shape[0] // 128
    r = np.random.default_rng(seed)
    blocks = np.unique(np.concatenate([[0, nb - 1], r.choice(nb, size=min(2, nb), replace=False)]))
    cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    return cols, oracle.block_scaled_fp8_gemm(codes, scale_q, layout, wc[cols], ws[blocks])


@pytest.mark.parametrize("M", [1, 16, 64, 256])
@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_shard_pair_vs_oracle_and_singles(tp, M):
    dev = gpu_or_skip()
    wa, wb = full_weights()
    (ca, sa), (cb, sb) = shard(wa, tp, tp - 1), shard(wb, tp, tp - 1)
    case = W.producer_activations(M)
    buf = dev_u16_as_bf16(case.buffer, dev)
    dca, dsa, dcb, dsb = dev_u8(ca, dev), dev_f32(sa, dev), dev_u8(cb, dev), dev_f32(sb, dev)
    for layout in (False, True):
        codes, scale, _ = mi.mi_fused_dual_rmsnorm_group_quant(
            buf[:, :W.NQ], buf[:, W.NQ:], dev_u16_as_bf16(case.gamma_q, dev),
            dev_u16_as_bf16(case.gamma_kv, dev), W.EPS, layout)
        o1, o2 = mi.mi_block_scaled_fp8_gemm_pair(codes, scale, dca, dsa, dcb, dsb)
        s1 = mi.mi_block_scaled_fp8_gemm(codes, scale, dca, dsa)
        s2 = mi.mi_block_scaled_fp8_gemm(codes, scale, dcb, dsb)
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16_bits(o1), host_bf16_bits(s1)), f"TP{tp} M{M} W_a shard"
        assert np.array_equal(host_bf16_bits(o2), host_bf16_bits(s2)), f"TP{tp} M{M} W_b shard"
        # the oracle takes the device's quantised pair (the norm-quant's own
        # parity is covered elsewhere): this isolates the GEMM at this shape
        q_np = codes.cpu().numpy()
        s_np = scale.T.contiguous().reshape(-1).cpu().numpy() if layout else \
            scale.contiguous().reshape(-1).cpu().numpy()
        for o, wc, ws, name in ((o1, ca, sa, "W_a"), (o2, cb, sb, "W_b")):
            cols, ref = sampled_ref(q_np, s_np, layout, wc, ws, seed=tp * 100 + M)
            fro, mx = assert_gemm_close(bf16_to_f64(o)[:, cols], ref, f"TP{tp} {name} M{M} t{layout}")
            print(f"TP{tp} {name}/{tp} [{wc.shape[0]}, 1536] M={M} t={int(layout)}: fro {fro:.2e} max {mx:.2e}")


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_shard_wrong_layout_flag_is_caught_by_a_large_error(tp):
    """Row-major As bytes declared column-major: same logical shape, wrong
    numbers for M > 1 at every shard shape (and harmless at M = 1)."""
    dev = gpu_or_skip()
    wa, _ = full_weights()
    ca, sa = shard(wa, tp, tp - 1)
    for M, expect_ok in ((1, True), (16, False)):
        r = np.random.default_rng(tp + M)
        a = r.integers(0, 0x78, size=(M, 1536), dtype=np.uint8)
        As = np.exp2(r.uniform(-8, 0, (M, 12))).astype(np.float32)
        cols, ref = sampled_ref(a, As.reshape(-1), False, ca, sa, seed=tp)
        da, das, dw, dbs = dev_u8(a, dev), dev_f32(As, dev), dev_u8(ca, dev), dev_f32(sa, dev)
        out = torch.empty((M, ca.shape[0]), dtype=torch.bfloat16, device=dev)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        st = mi.lib().mi_block_scaled_fp8_gemm(p(da), p(das), 1, p(dw), p(dbs), p(out), M, ca.shape[0], 1536,
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == B.MI_OK
        torch.cuda.synchronize()
        fro, _ = gemm_error(bf16_to_f64(out)[:, cols], ref)
        assert (fro <= 2e-2) if expect_ok else (fro > 0.1), f"TP{tp} M{M}: fro {fro:.3e}"


@pytest.mark.parametrize("M", [1, 7, 16])
def test_split_k_equals_the_k_loop_kernels(M):
    """A TP-8 shard gives each CU at most one 16-row subtile, where the GEMM
    of up to 16 rows splits K over the waves of a block and folds the
    partial sums in K-block order afterwards.  Its output must equal, bit
    for bit, the same shard's
    output from a K-loop kernel: the shard paired with a full consumer
    weight (a grid too wide for the split), both As layouts, row-major and
    tiled weights."""
    dev = gpu_or_skip()
    wa, wb = full_weights()
    r = np.random.default_rng(500 + M)
    a = dev_u8(r.integers(0, 0x100, size=(M, 1536), dtype=np.uint8) & 0xF7, dev)   # no NaN codes
    As = np.exp2(r.uniform(-8, 0, (M, 12))).astype(np.float32)
    for shard_w, other in ((shard(wa, 8, 7), wb), (shard(wb, 8, 7), wa)):
        (cs, ss) = shard_w
        for tiled in (False, True):
            dw = dev_u8(cs, dev)
            dw = mi.relayout_weight(dw) if tiled else dw
            do = dev_u8(other.codes, dev)
            do = mi.relayout_weight(do) if tiled else do
            dss, dos = dev_f32(ss, dev), dev_f32(other.scale, dev)
            for layout in (False, True):
                das = dev_f32(As.T.copy(), dev).T if layout else dev_f32(As, dev)
                single = mi.mi_block_scaled_fp8_gemm(a, das, dw, dss)
                paired, _ = mi.mi_block_scaled_fp8_gemm_pair(a, das, dw, dss, do, dos)
                torch.cuda.synchronize()
                assert np.array_equal(host_bf16_bits(single), host_bf16_bits(paired)), \
                    f"M{M} [{cs.shape[0]}] tiled={tiled} t={layout}"


@pytest.mark.parametrize("M", [1, 16, 40])
@pytest.mark.parametrize("N", [12288, 16384, 20480])
def test_one_subtile_per_wave_equals_the_two_subtile_kernel(N, M):
    """Weights of three to five 16-row subtiles per CU (N = 12288, 16384,
    20480 on 256 CUs) at up to 16 rows run the stream kernel with one subtile
    per wave and a wave per subtile, and at 40 rows the wide kernel (three
    subtiles per block at N = 12288); paired with W_a the same weight runs
    the stream kernel with two subtiles per wave.  The outputs must be equal
    bit for bit, tiled weights, both As layouts."""
    dev = gpu_or_skip()
    wa, _ = full_weights()
    wt = W.block_fp8_weight(N, 1536, 700 + N // 4096)
    r = np.random.default_rng(800 + M + N)
    a = dev_u8(r.integers(0, 0x100, size=(M, 1536), dtype=np.uint8) & 0xF7, dev)   # no NaN codes
    As = np.exp2(r.uniform(-8, 0, (M, 12))).astype(np.float32)
    dw, ds = mi.relayout_weight(dev_u8(wt.codes, dev)), dev_f32(wt.scale, dev)
    da, dsa = mi.relayout_weight(dev_u8(wa.codes, dev)), dev_f32(wa.scale, dev)
    for layout in (False, True):
        das = dev_f32(As.T.copy(), dev).T if layout else dev_f32(As, dev)
        single = mi.mi_block_scaled_fp8_gemm(a, das, dw, ds)
        paired, _ = mi.mi_block_scaled_fp8_gemm_pair(a, das, dw, ds, da, dsa)
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16_bits(single), host_bf16_bits(paired)), f"N{N} M{M} t={layout}"


@pytest.mark.parametrize("which", ["W_b", "TP2 W_a"])
def test_a_row_does_not_depend_on_its_batch(which):
    """Every output row depends only on its own activation row and scales, and
    every kernel folds the K blocks in the same order, so a row must come out
    bit for bit the same whatever batch it is computed in: 256 rows (the stream
    kernel in 64-row chunks) against slices of 16 (one subtile per wave), 64,
    100 and 200 rows, for W_b and the last TP-2 shard of W_a, both As layouts."""
    dev = gpu_or_skip()
    wa, wb = full_weights()
    codes, scale = (wb.codes, wb.scale) if which == "W_b" else shard(wa, 2, 1)
    r = np.random.default_rng(900 + (which == "W_b"))
    a = r.integers(0, 0x100, size=(256, 1536), dtype=np.uint8) & 0xF7   # no NaN codes
    As = np.exp2(r.uniform(-8, 0, (256, 12))).astype(np.float32)
    dw, ds = mi.relayout_weight(dev_u8(codes, dev)), dev_f32(scale, dev)
    for layout in (False, True):
        def run(lo, hi):
            das = dev_f32(As[lo:hi].T.copy(), dev).T if layout else dev_f32(As[lo:hi].copy(), dev)
            out = mi.mi_block_scaled_fp8_gemm(dev_u8(a[lo:hi].copy(), dev), das, dw, ds)
            torch.cuda.synchronize()
            return host_bf16_bits(out)
        full = run(0, 256)
        for lo, hi in ((0, 16), (240, 256), (64, 128), (3, 103), (0, 200), (56, 256)):
            assert np.array_equal(run(lo, hi), full[lo:hi]), f"{which} rows {lo}:{hi} t={layout}"


@pytest.mark.parametrize("M", [20, 40, 64, 128, 200, 256])
def test_one_subtile_blocks_equal_the_slab_kernels(M):
    """Between 17 and 64 rows a weight of at most one 16-row subtile per CU
    (a TP-8 shard, alone or paired with the other shard) runs the wide
    kernel with one subtile per block; above 64 rows the TP-8 W_a shard runs
    64-row chunks of three-subtile slabs and the W_b shard of two-subtile
    slabs, and the TP-4 W_a shard three-subtile slabs of half the rows.
    Paired with a full consumer weight the same shard runs in slabs of four
    to six subtiles.  Outputs must be equal bit for bit, row-major
    and tiled weights, both As layouts, and match the oracle on sampled
    column blocks."""
    dev = gpu_or_skip()
    wa, wb = full_weights()
    r = np.random.default_rng(600 + M)
    a_np = r.integers(0, 0x100, size=(M, 1536), dtype=np.uint8) & 0xF7   # no NaN codes
    a = dev_u8(a_np, dev)
    As = np.exp2(r.uniform(-8, 0, (M, 12))).astype(np.float32)
    for shard_w, other in ((shard(wa, 8, 7), wb), (shard(wb, 8, 7), wa), (shard(wa, 4, 3), wb)):
        cs, ss = shard_w
        for tiled in (False, True):
            dw = dev_u8(cs, dev)
            dw = mi.relayout_weight(dw) if tiled else dw
            do = dev_u8(other.codes, dev)
            do = mi.relayout_weight(do) if tiled else do
            dss, dos = dev_f32(ss, dev), dev_f32(other.scale, dev)
            for layout in (False, True):
                das = dev_f32(As.T.copy(), dev).T if layout else dev_f32(As, dev)
                single = mi.mi_block_scaled_fp8_gemm(a, das, dw, dss)
                paired, _ = mi.mi_block_scaled_fp8_gemm_pair(a, das, dw, dss, do, dos)
                torch.cuda.synchronize()
                assert np.array_equal(host_bf16_bits(single), host_bf16_bits(paired)), \
                    f"M{M} [{cs.shape[0]}] tiled={tiled} t={layout}"
            cols, ref = sampled_ref(a_np, As.reshape(-1), False, cs, ss, seed=M)
            assert_gemm_close(bf16_to_f64(single)[:, cols], ref, f"M{M} [{cs.shape[0]}] tiled={tiled}")
