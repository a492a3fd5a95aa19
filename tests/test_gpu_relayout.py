"""GPU checks of the load-time weight relayout (PRHub report of vLLM PR
#56433, "实现拆解" items 1-3: a GEMM that wants its weight relaid out says so
with a capability flag; the relayout is applied once, at load time; it is
a permutation, not an involution).

- the device relayout equals the oracle's tiled order bit for bit (full W_a
  and W_b included), and the inverse restores the weight exactly;
- every GEMM path (decode, wide, row-split, v0, the two-consumer launch,
  tensor-parallel shards) gives bit-identical results on the tiled and on
  the row-major weight;
- tiled bytes declared row-major (the silent failure of a layout mix-up)
  give a large error.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import rmsnorm_fp8_block_amd as mi
from rmsnorm_fp8_block_amd import _binding as B
from rmsnorm_fp8_block_amd import workloads as W

from helpers import assert_gemm_close, bf16_to_f64, dev_f32, dev_u8, gemm_error, gpu_or_skip, host_bf16_bits

pytestmark = pytest.mark.gpu


def operands(M, N, K, seed):
    r = np.random.default_rng(seed)
    a = r.integers(0, 256, size=(M, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38
    As = np.exp2(r.uniform(-10, 0, (M, K // 128))).astype(np.float32)
    Bs = np.exp2(r.uniform(-10, 0, (N // 128, K // 128))).astype(np.float32)
    return a, As, w, Bs


@pytest.mark.parametrize("N,K", [(16, 128), (128, 256), (384, 640), (W.W_B_SHAPE[0], W.W_B_SHAPE[1]),
                                 (W.W_A_SHAPE[0], W.W_A_SHAPE[1])])
def test_device_relayout_equals_oracle_and_round_trips(N, K):
    dev = gpu_or_skip()
    w = np.random.default_rng(N + K).integers(0, 256, size=(N, K), dtype=np.uint8)
    dw = dev_u8(w, dev)
    tw = mi.relayout_weight(dw)
    back = mi.untile_weight(tw)
    torch.cuda.synchronize()
    assert np.array_equal(tw.data.cpu().numpy(), oracle.tile_weight(w))
    assert np.array_equal(back.cpu().numpy(), w)


def test_same_layout_is_a_copy():
    dev = gpu_or_skip()
    w = dev_u8(np.random.default_rng(1).integers(0, 256, size=(128, 256), dtype=np.uint8), dev)
    dst = torch.empty_like(w)
    st = mi.lib().mi_relayout_weight(ctypes.c_void_p(w.data_ptr()), 1, ctypes.c_void_p(dst.data_ptr()), 1,
                                     128, 256, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == B.MI_OK
    torch.cuda.synchronize()
    assert torch.equal(dst, w)


# (M, N, K): stream kernel (M <= 64 over at least 6 subtiles per CU, K/128 in
# {4, 8, 12}); decode kernel (M <= 32 over more than 4 subtiles per CU where
# the stream kernel does not apply: K/128 = 16, or 5 subtiles per CU); wide
# kernel (M <= 256, K/128 in {4, 8, 12, 16}); row-split wide kernel (few
# slabs, M > 64); v0 (M > 256, or K/128 = 5)
@pytest.mark.parametrize("M,N,K,seed", [(1, 24576, 1536, 1), (16, 24576, 1536, 2), (32, 16384, 1024, 3),
                                        (64, 8192, 1536, 4), (100, 1536, 1536, 5), (256, 3072, 1536, 6),
                                        (256, 24576, 1536, 7), (300, 1280, 1536, 8), (40, 1280, 640, 9),
                                        (5, 256, 2048, 10), (16, 24576, 2048, 11), (8, 20480, 1536, 12),
                                        (32, 20480, 1024, 13)])
def test_tiled_gemm_equals_row_major(M, N, K, seed):
    dev = gpu_or_skip()
    a, As, w, Bs = operands(M, N, K, seed)
    da, dbs, dw = dev_u8(a, dev), dev_f32(Bs, dev), dev_u8(w, dev)
    tw = mi.relayout_weight(dw)
    for t in (False, True):
        das = dev_f32(As.T.copy(), dev).T if t else dev_f32(As, dev)
        plain = mi.mi_block_scaled_fp8_gemm(da, das, dw, dbs)
        tiled = mi.mi_block_scaled_fp8_gemm(da, das, tw, dbs)
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16_bits(plain), host_bf16_bits(tiled)), f"M{M} N{N} K{K} t{t}"
    nb = N // 128
    blocks = np.unique([0, nb // 2, nb - 1])
    cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    ref = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w[cols], Bs[blocks])
    assert_gemm_close(bf16_to_f64(tiled)[:, cols], ref, f"tiled M{M} N{N} K{K}")


@pytest.mark.parametrize("M", [1, 16, 64, 100])
@pytest.mark.parametrize("tp", [1, 4, 8])
def test_tiled_pair_equals_row_major_on_shards(tp, M):
    dev = gpu_or_skip()
    wa = W.block_fp8_weight(*W.W_A_SHAPE, W.W_A_SEED)
    wb = W.block_fp8_weight(*W.W_B_SHAPE, W.W_B_SEED)
    na, nb = wa.codes.shape[0] // tp, wb.codes.shape[0] // tp
    r = np.random.default_rng(tp * 10 + M)
    a = dev_u8(r.integers(0, 0x78, size=(M, 1536), dtype=np.uint8), dev)
    asc = dev_f32(np.exp2(r.uniform(-8, 0, (12, M))).astype(np.float32), dev).T
    dwa, dwb = dev_u8(wa.codes[:na], dev), dev_u8(wb.codes[:nb], dev)
    sa, sb = dev_f32(wa.scale[:na // 128], dev), dev_f32(wb.scale[:nb // 128], dev)
    p1, p2 = mi.mi_block_scaled_fp8_gemm_pair(a, asc, dwa, sa, dwb, sb)
    t1, t2 = mi.mi_block_scaled_fp8_gemm_pair(a, asc, mi.relayout_weight(dwa), sa, mi.relayout_weight(dwb), sb)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(p1), host_bf16_bits(t1))
    assert np.array_equal(host_bf16_bits(p2), host_bf16_bits(t2))
    with pytest.raises(ValueError):   # one layout for both weights of a pair
        mi.mi_block_scaled_fp8_gemm_pair(a, asc, dwa, sa, mi.relayout_weight(dwb), sb)


def test_tiled_bytes_declared_row_major_are_wrong():
    dev = gpu_or_skip()
    M, N, K = 16, 1024, 1536
    a, As, w, Bs = operands(M, N, K, 30)
    ref = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w, Bs)
    tw = mi.relayout_weight(dev_u8(w, dev))
    da, das, dbs = dev_u8(a, dev), dev_f32(As, dev), dev_f32(Bs, dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = mi.lib().mi_block_scaled_fp8_gemm_ex(p(da), p(das), 0, p(tw.data), B.MI_WEIGHT_ROW_MAJOR, p(dbs), p(out),
                                              M, N, K, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == B.MI_OK
    torch.cuda.synchronize()
    fro, _ = gemm_error(bf16_to_f64(out), ref)
    assert fro > 0.1, "a weight layout mix-up must show up as a large error"
