"""Plain CPU oracle for stochastic-rounding MXFP4 quantize.

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import this module. The HIP library never
does, and this module imports nothing from it: the two sides share no code.

Sources:
  * NVIDIA/TransformerEngine #3809, description: stochastic rounding takes one
    Philox4x32 draw per output block, keyed by the block's coordinates and by
    the direction (rowwise or columnwise), and each draw is plain Philox4x32
    of a known counter.
  * Philox4x32 itself: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
    "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, the Philox
    construction (two 32x32 -> 64-bit products per round, a Weyl-sequence key
    schedule) with the multipliers and key increments the paper gives for
    four 32-bit words, and 10 rounds (the paper's default variant).

Readings taken here (the pages leave them open):
  S1  The scale byte is the one of round-to-nearest quantize (readings R2 of
      mxfp4_ref): stochastic rounding changes only the element codes.
  S2  Randomness per element: 8 bits. An MXFP4 block has 32 elements and one
      draw gives 128 bits, so each half block (16 elements) takes its own draw:
      counter (block column j, row r, direction d, half h), key (seed mod 2**32,
      seed >> 32). d = 0 for the rowwise output and 1 for the columnwise one
      (where r is the column of X and j the block index along M). Element
      16 h + i uses byte i % 4 (least significant first) of word i // 4.
  S3  Rounding: v = x * 2**-e lies between the E2M1 magnitudes lo <= |v| < hi
      (|v| >= 6 saturates to 6 and draws nothing). With frac = (|v| - lo) /
      (hi - lo) and u the element's random byte, the magnitude is hi when
      floor(256 * frac) + u >= 256, else lo: the byte is added to the eight
      bits just below the grid spacing and the sum truncated. A value then
      rounds up with probability floor(256 frac) / 256, which is exactly frac
      whenever |v| >= 1/4 (frac then has at most 8 bits); below that the
      result is biased toward zero by less than 1/256 of the grid spacing.
  S4  The sign bit of x is kept, also on magnitude 0 (as in R3 of mxfp4_ref).
  S5  "The block's coordinates" are its coordinates in the whole input: a
      part of X holding rows row0 .. row0 + M - 1 draws with the global rows
      (rowwise) and the global row blocks row0 / 32 + j (columnwise), so that
      its outputs are the matching part of the whole input's.
Everything below is computed exactly (integers and float64).
"""

import numpy as np

from .mxfp4_ref import BLOCK, bf16_bits_to_f64, scale_exponent

# Philox4x32 constants from the SC'11 paper: the two round multipliers and the
# two Weyl-sequence key increments.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
PHILOX_ROUNDS = 10

DIR_ROWWISE = 0
DIR_COLUMNWISE = 1

_MASK32 = np.uint64(0xFFFFFFFF)
_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def philox4x32(counters, key, rounds=PHILOX_ROUNDS):
    """Philox4x32-`rounds` of each 128-bit counter under one 64-bit key.

    counters: uint32 [..., 4] (words c0..c3); key: (k0, k1) 32-bit ints.
    One round maps (c0, c1, c2, c3) to
        (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
    where hi/lo are the upper and lower 32 bits of the 64-bit product; the
    key gains (W0, W1) modulo 2**32 after every round.
    """
    c = np.asarray(counters, dtype=np.uint32).astype(np.uint64)
    if c.shape[-1] != 4:
        raise ValueError("counters must have 4 words in the last axis")
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = int(key[0]) & 0xFFFFFFFF
    k1 = int(key[1]) & 0xFFFFFFFF
    for _ in range(rounds):
        p0 = np.uint64(PHILOX_M0) * c0          # < 2**64: exact in uint64
        p1 = np.uint64(PHILOX_M1) * c2
        n0 = (p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0)
        n2 = (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1)
        c0, c1, c2, c3 = n0, p1 & _MASK32, n2, p0 & _MASK32
        k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
        k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def seed_key(seed):
    """S2: the Philox key of a 64-bit seed, (low word, high word)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def sr_random_bytes(row_ids, nblocks, seed, direction, block0=0):
    """S2: the random byte of every element of the given rows.

    row_ids: row indices r (of the output being written); nblocks: blocks
    per row, whose block columns are block0 .. block0 + nblocks - 1 (S5).
    Returns uint8 [len(row_ids), nblocks * 32].
    """
    rows = np.asarray(row_ids, dtype=np.int64).reshape(-1)
    R = rows.size
    ctr = np.zeros((R, nblocks, 2, 4), dtype=np.uint32)
    ctr[..., 0] = (block0 + np.arange(nblocks, dtype=np.int64)).astype(np.uint32)[None, :, None]
    ctr[..., 1] = rows.astype(np.uint32)[:, None, None]
    ctr[..., 2] = np.uint32(direction)
    ctr[..., 3] = np.arange(2, dtype=np.uint32)[None, None, :]
    words = philox4x32(ctr, seed_key(seed))             # [R, nblocks, 2, 4]
    shifts = np.array([0, 8, 16, 24], dtype=np.uint32)
    b = (words[..., None] >> shifts) & np.uint32(0xFF)  # [R, nblocks, 2, 4, 4]
    return b.astype(np.uint8).reshape(R, nblocks * BLOCK)


def sr_magnitude_index(mag, rand_bytes):
    """S3: E2M1 magnitude index (0..7) of |v| = `mag` under random bytes."""
    mag = np.asarray(mag, dtype=np.float64)
    u = np.asarray(rand_bytes, dtype=np.int64)
    sat = mag >= 6.0
    lo_idx = np.searchsorted(_MAGNITUDES, mag, side="right") - 1   # lo <= mag
    lo_idx = np.clip(lo_idx, 0, 6)
    lo = _MAGNITUDES[lo_idx]
    hi = _MAGNITUDES[lo_idx + 1]
    frac = (mag - lo) / (hi - lo)           # exact: a power-of-two spacing
    f8 = np.floor(frac * 256.0).astype(np.int64)
    up = (f8 + u) >= 256
    idx = np.where(sat, 7, lo_idx + up.astype(np.int64))
    return idx.astype(np.uint8)


def quantize_sr_with_bytes(x_bits, rand_bytes):
    """S1, S3, S4 with the random bytes given: uint8 [M, K] (one per element).

    Returns (codes uint8 [M, K/2], scales uint8 [M, K/32]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    rand_bytes = np.asarray(rand_bytes, dtype=np.uint8)
    if rand_bytes.shape != (M, K):
        raise ValueError("one random byte per element is required")
    x = bf16_bits_to_f64(x_bits).reshape(M, K // BLOCK, BLOCK)
    e = scale_exponent(np.abs(x).max(axis=2))
    scales = (e + 127).astype(np.uint8)
    v = np.ldexp(x, -e[..., None])          # exact
    idx = sr_magnitude_index(np.abs(v), rand_bytes.reshape(M, K // BLOCK, BLOCK))
    code = (idx | (np.signbit(x).astype(np.uint8) << 3)).reshape(M, K)
    codes = code[:, 0::2] | (code[:, 1::2] << 4)
    return codes.astype(np.uint8), scales


def quantize_sr(x_bits, seed, direction=DIR_ROWWISE, row_ids=None, block0=0):
    """Row-wise MXFP4 with stochastic rounding (S1-S5).

    x_bits: uint16 [M, K] BF16 bits. row_ids: the output row index of each
    given row (default 0..M-1), so that sampled rows, or a row shard, of a
    large input take the random bytes of their real coordinates; block0: the
    global block column of the first block of a row.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if row_ids is None:
        row_ids = np.arange(M)
    rb = sr_random_bytes(row_ids, K // BLOCK, seed, direction, block0)
    return quantize_sr_with_bytes(x_bits, rb)


def quantize_2d_sr(x_bits, seed, row0=0):
    """Rowwise (direction 0) and columnwise (direction 1: the rowwise form of
    X^T) stochastic-rounding MXFP4 of X [M, K], M and K multiples of 32;
    X may be rows row0 .. row0 + M - 1 of a larger input (row0 % 32 == 0, S5).

    Returns (codes [M, K/2], scales [M, K/32], codes_t [K, M/2], scales_t
    [K, M/32]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if row0 % BLOCK:
        raise ValueError("row0 must be a multiple of 32")
    M = x_bits.shape[0]
    codes, scales = quantize_sr(x_bits, seed, DIR_ROWWISE, row_ids=row0 + np.arange(M))
    codes_t, scales_t = quantize_sr(np.ascontiguousarray(x_bits.T), seed, DIR_COLUMNWISE,
                                    block0=row0 // BLOCK)
    return codes, scales, codes_t, scales_t
