"""Pins for the oracle's load-time weight relayout (the tiled byte order of
the library's GEMMs).  The PRHub report of vLLM PR #56433 ("功能与动机",
"实现拆解" items 1-3) fixes what matters about such a relayout: it is a
permutation, applied once at load time, not an involution, and a GEMM on
the relaid weight must equal the GEMM on the plain one.  The byte order
itself is this library's contract; it is pinned here by what it is for,
not by retyping its index formula:
  - a bijection, undone exactly by the inverse;
  - each 2 KB tile holds exactly the bytes of one 16 x 128 block of the
    weight, tiles in (subtile, K-block) order, each subtile's tiles
    contiguous;
  - each 128-byte piece of a tile holds exactly one 128-byte row segment, the
    rows in order, and the 16-byte chunks of a row only move inside it;
  - the bank-conflict property the order exists for: within one 1 KB half,
    a given chunk of the 8 rows lands at 8 distinct positions;
  - applying it twice differs from applying it once and from the identity
    (not an involution) from two K-blocks on;
  - the oracle GEMM on the weight recovered from the tiled bytes equals the
    GEMM on the original.
The exact choice among conflict-free swizzles (r ^ g) is pinned only by
the device GEMM reading it (tiled results equal row-major ones bit for bit).
"""
import numpy as np
import pytest

import oracle


def distinct_weight(N, K):
    """Every 16-byte chunk tagged by (row, chunk) in its first two bytes, so
    positions can be traced; the rest random."""
    r = np.random.default_rng(N * 1000 + K)
    w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    rows = np.arange(N)[:, None]
    chunks = np.arange(K // 16)[None, :]
    w[:, 0::16] = (rows % 256).astype(np.uint8)
    w[:, 1::16] = (chunks % 256).astype(np.uint8)   # chunk index in the row
    return w


@pytest.mark.parametrize("N,K", [(16, 128), (32, 256), (48, 640), (128, 1536)])
def test_bijection_and_round_trip(N, K):
    r = np.random.default_rng(N + K)
    w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    t = oracle.tile_weight(w)
    assert t.shape == (N * K,)
    assert np.array_equal(np.sort(t), np.sort(w.reshape(-1)))
    assert np.array_equal(oracle.untile_weight(t, N, K), w)
    # index-level bijection: tile the positions themselves (N*K < 2^16 here
    # for the small cases, so two bytes of a position fit in two weights)
    if N * K <= 65536:
        pos = np.arange(N * K, dtype=np.uint32).reshape(N, K)
        lo = oracle.tile_weight((pos & 0xFF).astype(np.uint8)).astype(np.uint32)
        hi = oracle.tile_weight((pos >> 8).astype(np.uint8)).astype(np.uint32)
        src = lo | (hi << 8)
        assert np.array_equal(np.sort(src), np.arange(N * K))


@pytest.mark.parametrize("N,K", [(32, 256), (64, 1536)])
def test_tiles_rows_and_chunks_stay_local(N, K):
    w = distinct_weight(N, K)
    t = oracle.tile_weight(w).reshape(N // 16, K // 128, 2, 8, 8, 16)   # s, kb, g, r, p, b
    for s in range(N // 16):
        for kb in range(K // 128):
            block = w[16 * s:16 * s + 16, 128 * kb:128 * kb + 128]
            tile = t[s, kb]
            assert np.array_equal(np.sort(tile.reshape(-1)), np.sort(block.reshape(-1)))
            for g in range(2):
                for rr in range(8):
                    piece = tile[g, rr]                     # 8 chunks of 16 bytes
                    row = block[8 * g + rr].reshape(8, 16)  # the row segment's chunks
                    # same chunks, only reordered
                    got = sorted(map(bytes, piece))
                    assert got == sorted(map(bytes, row))
                    # every chunk of the piece is tagged with this row
                    assert np.all(piece[:, 0] == (16 * s + 8 * g + rr) % 256)


@pytest.mark.parametrize("K", [128, 1536])
def test_same_chunk_of_eight_rows_in_eight_positions(K):
    """For each 1 KB half and each source chunk c, the 8 rows put c at 8
    distinct 16-byte positions (distinct LDS banks for the 8 lanes that
    read chunk c of rows 0..7 together)."""
    N = 32
    w = distinct_weight(N, K)
    t = oracle.tile_weight(w).reshape(N // 16, K // 128, 2, 8, 8, 16)
    for s in range(N // 16):
        for kb in range(K // 128):
            for g in range(2):
                # chunk index within the K-block, from the tag byte
                c = (t[s, kb, g, :, :, 1].astype(np.int64) - 8 * kb) % 256   # [r, p]
                for chunk in range(8):
                    r_idx, p_idx = np.nonzero(c == chunk)
                    assert sorted(r_idx) == list(range(8))
                    assert len(set(p_idx)) == 8


def test_not_an_involution():
    """From two K-blocks on, relaying out twice is neither the identity nor
    the single relayout.  With a single K-block (K = 128) the order is only a
    per-row XOR swizzle of the chunks, which is its own inverse."""
    r = np.random.default_rng(7)
    for N, K in ((16, 256), (32, 384), (64, 1536)):
        w = r.integers(0, 256, size=(N, K), dtype=np.uint8)
        once = oracle.tile_weight(w)
        twice = oracle.tile_weight(once.reshape(N, K))
        assert not np.array_equal(twice, w.reshape(-1))
        assert not np.array_equal(twice, once)
    w = r.integers(0, 256, size=(32, 128), dtype=np.uint8)
    assert np.array_equal(oracle.tile_weight(oracle.tile_weight(w).reshape(32, 128)), w.reshape(-1))


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
