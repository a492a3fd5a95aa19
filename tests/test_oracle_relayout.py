"""Pins for the oracle's load-time weight relayout (the tiled byte order of
the library's GEMMs).  The PRHub report of vLLM PR #56433 ("功能与动机",
"实现拆解" items 1-3) fixes what matters about such a relayout: it is a
permutation, applied once at load time, not an involution, and a GEMM on
the relaid weight must equal the GEMM on the plain one.  The byte order
itself is this library's contract (the order in which the 16x16x128 matrix
instruction takes a 16-row x 128-byte tile: lane L = 16 q + r holds row r,
bytes 32 q .. 32 q + 31); it is pinned here by what it is for rather than by
retyping its index formula:
  - a bijection, undone exactly by the inverse;
  - each 2 KB tile holds exactly the bytes of one 16 x 128 block of the
    weight, tiles in (subtile, K-block) order, each subtile's tiles
    contiguous;
  - each 16-byte chunk stays whole and each lane slot of a tile carries
    chunks of a single row, lanes 0-15 rows 0-15 in order, and the four
    lanes of one row hold its 8 chunks in K order;
  - applying it twice is neither the identity nor the single relayout (not
    an involution);
  - the oracle GEMM on the weight recovered from the tiled bytes equals the
    GEMM on the original.
The device GEMMs reading this order give the same bits as on row-major
weights (GPU tests), which pins the lane assignment itself.
"""
import numpy as np
import pytest

import oracle


def tagged_weight(N, K):
    """Every 16-byte chunk tagged: byte 0 = row % 256, byte 1 = chunk index
    within the row % 256, the rest random."""
    r = np.random.default_rng(N * 1000 + K)
    w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    w[:, 0::16] = (np.arange(N)[:, None] % 256).astype(np.uint8)
    w[:, 1::16] = (np.arange(K // 16)[None, :] % 256).astype(np.uint8)
    return w


@pytest.mark.parametrize("N,K", [(16, 128), (32, 256), (48, 640), (128, 1536)])
def test_bijection_and_round_trip(N, K):
    r = np.random.default_rng(N + K)
    w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    t = oracle.tile_weight(w)
    assert t.shape == (N * K,)
    assert np.array_equal(np.sort(t), np.sort(w.reshape(-1)))
    assert np.array_equal(oracle.untile_weight(t, N, K), w)
    if N * K <= 65536:
        pos = np.arange(N * K, dtype=np.uint32).reshape(N, K)
        lo = oracle.tile_weight((pos & 0xFF).astype(np.uint8)).astype(np.uint32)
        hi = oracle.tile_weight((pos >> 8).astype(np.uint8)).astype(np.uint32)
        assert np.array_equal(np.sort(lo | (hi << 8)), np.arange(N * K))


@pytest.mark.parametrize("N,K", [(32, 256), (64, 1536)])
def test_tiles_chunks_and_lanes(N, K):
    w = tagged_weight(N, K)
    t = oracle.tile_weight(w).reshape(N // 16, K // 128, 2, 64, 16)     # s, kb, h, lane, b
    for s in range(N // 16):
        for kb in range(K // 128):
            block = w[16 * s:16 * s + 16, 128 * kb:128 * kb + 128]
            tile = t[s, kb]
            assert np.array_equal(np.sort(tile.reshape(-1)), np.sort(block.reshape(-1)))
            # every 16-byte chunk of the tile is a whole chunk of the block
            chunks = {bytes(c) for c in block.reshape(16, 8, 16).reshape(-1, 16)}
            assert {bytes(c) for c in tile.reshape(-1, 16)} == chunks
            rows = tile[:, :, 0].astype(int)            # [h, lane]: the row tag of each lane slot
            cidx = (tile[:, :, 1].astype(int) - 8 * kb) % 256   # chunk index within the K-block
            # a lane slot carries a single row; lanes 0..15 are rows 0..15 of the subtile
            assert np.all(rows[0] == rows[1])
            assert np.array_equal(rows[0][:16], (16 * s + np.arange(16)) % 256)
            assert np.array_equal(rows[0].reshape(4, 16), np.tile(rows[0][:16], (4, 1)))
            # the 4 lanes of one row hold its 8 chunks in K order
            for rr in range(16):
                lanes = [rr + 16 * q for q in range(4)]
                order = [cidx[h, L] for L in lanes for h in range(2)]
                assert order == list(range(8))


def test_not_an_involution():
    r = np.random.default_rng(7)
    for N, K in ((16, 128), (16, 256), (64, 1536)):
        w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
        once = oracle.tile_weight(w)
        twice = oracle.tile_weight(once.reshape(N, K))
        assert not np.array_equal(twice, w.reshape(-1))
        assert not np.array_equal(twice, once)


def test_gemm_on_recovered_weight_is_unchanged():
    r = np.random.default_rng(8)
    M, N, K = 5, 256, 512
    a = r.integers(0, 0x78, size=(M, K), dtype=np.uint8)
    w = r.integers(0, 0x78, size=(N, K), dtype=np.uint8)
    As = np.exp2(r.uniform(-6, 0, (M, K // 128))).astype(np.float32)
    Bs = np.exp2(r.uniform(-6, 0, (N // 128, K // 128))).astype(np.float32)
    ref = oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, w, Bs)
    back = oracle.untile_weight(oracle.tile_weight(w), N, K)
    assert np.array_equal(oracle.block_scaled_fp8_gemm(a, As.reshape(-1), False, back, Bs), ref)
