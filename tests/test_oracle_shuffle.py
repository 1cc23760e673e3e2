"""Pins of the pre-shuffled weight layout (oracle/shuffle.py, readings P1-P2).

The layout is this library's own definition (the pages name shuffled weights
and swizzled scales without giving one), so it is pinned by hand-worked byte
positions, exhaustive bijection checks and round trips, not by a page value.
"""

import numpy as np
import pytest

import oracle
from oracle.shuffle import chunk_swizzle


def test_swizzle_is_a_permutation_of_chunks_for_every_row():
    for x in range(256):
        perm = [p ^ int(chunk_swizzle(x)) for p in range(8)]
        assert sorted(perm) == list(range(8))
    # Over 16 consecutive rows the swizzle takes both parities of every pair.
    assert sorted({int(chunk_swizzle(x)) for x in range(16)}) == list(range(8))


def test_sizes():
    assert oracle.shuffled_sizes(256, 256) == (32768, 8192)
    assert oracle.shuffled_sizes(257, 1280) == (2 * 5 * 32768, 2 * 2 * 8192)


def test_hand_worked_code_position():
    """N = K = 512: codes[258, 130] -> tile 1, row x = 2, step 1, logical chunk 0,
    byte 2; swz(2) = 2 so physical chunk 2: (1*2 + 1)*32768 + 2*128 + 2*16 + 2."""
    codes = np.zeros((512, 256), dtype=np.uint8)
    scales = np.zeros((512, 16), dtype=np.uint8)
    codes[258, 130] = 0xA5
    sh, _ = oracle.shuffle_b(codes, scales)
    assert np.flatnonzero(sh).tolist() == [98594]
    assert sh[98594] == 0xA5


def test_hand_worked_scale_position():
    """N = 512, K = 2048: scales[300, 37] -> tile 1, x = 44 = 32*1 + 12 (h 0, t 1,
    r 12); column 37 = 32*1 + 4*1 + 1 -> chunk 1, half-step 1, byte 1;
    stored half-step 1 ^ ((12 >> 1) & 7) = 7:
    (1*2 + 1)*8192 + 128*12 + 16*7 + 4*1 + 1 = 26229."""
    codes = np.zeros((512, 1024), dtype=np.uint8)
    scales = np.zeros((512, 64), dtype=np.uint8)
    scales[300, 37] = 0x7B
    _, sh = oracle.shuffle_b(codes, scales)
    assert np.flatnonzero(sh).tolist() == [26229]


@pytest.mark.parametrize("N,K", [(256, 256), (32, 1024), (300, 1280), (512, 2048), (96, 768)])
def test_round_trip_and_bijection(N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(N, K // 32), dtype=np.uint8)
    cs, ss = oracle.shuffle_b(codes, scales)
    assert (cs.size, ss.size) == oracle.shuffled_sizes(N, K)
    c2, s2 = oracle.unshuffle_b(cs, ss, N, K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # Every plain byte appears exactly once; everything else is zero padding.
    ids = np.arange(1, N * (K // 2) + 1, dtype=np.int64).reshape(N, K // 2)
    hit = np.zeros(cs.size, dtype=np.int64)
    from oracle.shuffle import _code_index
    row, col = _code_index(N, K)
    ok = row >= 0
    hit[ok] = ids[row[ok], col[ok]]
    assert np.array_equal(np.sort(hit[hit > 0]), ids.ravel())
    assert ok.sum() == N * (K // 2)
    pad_rows = -(-N // 256) * 256 - N
    assert (~ok).sum() == pad_rows * (K // 2)
