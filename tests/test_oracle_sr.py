"""Pins of the stochastic-rounding oracle (oracle/stochastic.py).

Philox4x32-10 is pinned against an independent implementation run at test
time (Triton's, executed by its CPU interpreter) and against the mixing
property that its round count buys; the rounding rule is pinned by
exhaustive enumeration of every random byte for every BF16 value, checked
exactly (float64 on dyadic values, rationals on samples): each result is one
of the two grid neighbours found by search, the bytes that round up are the
largest ones, and the mean over all bytes is the input itself wherever frac
has at most 8 bits; a row shard keyed by its global rows (reading S5) gives the
matching part of the whole input's outputs. Readings S1-S5 are those stated in
oracle/stochastic.py.
"""

import os
import subprocess
import sys
import textwrap
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import bf16_matrix

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
        Fraction(2), Fraction(3), Fraction(4), Fraction(6)]

def _triton_philox(counters, seeds, tmp_path):
    """Philox4x32-10 outputs from Triton's implementation (tl.philox), run by
    its CPU interpreter in a child process. Returns None if Triton is absent."""
    try:
        import triton  # noqa: F401
    except ImportError:
        return None
    np.save(tmp_path / "ctr.npy", counters)
    script = textwrap.dedent("""
        import os, sys
        os.environ["TRITON_INTERPRET"] = "1"
        import numpy as np, torch, triton, triton.language as tl

        @triton.jit
        def philox_kernel(c_ptr, out_ptr, seed, BLOCK: tl.constexpr):
            i = tl.arange(0, BLOCK)
            c0 = tl.load(c_ptr + 4 * i + 0)
            c1 = tl.load(c_ptr + 4 * i + 1)
            c2 = tl.load(c_ptr + 4 * i + 2)
            c3 = tl.load(c_ptr + 4 * i + 3)
            r0, r1, r2, r3 = tl.philox(seed, c0, c1, c2, c3)
            tl.store(out_ptr + 4 * i + 0, r0.to(tl.int32, bitcast=True))
            tl.store(out_ptr + 4 * i + 1, r1.to(tl.int32, bitcast=True))
            tl.store(out_ptr + 4 * i + 2, r2.to(tl.int32, bitcast=True))
            tl.store(out_ptr + 4 * i + 3, r3.to(tl.int32, bitcast=True))

        d = sys.argv[1]
        ctr = np.load(os.path.join(d, "ctr.npy"))
        outs = []
        for seed in [int(s) for s in sys.argv[2:]]:
            c = torch.from_numpy(ctr.view(np.int32).copy())
            out = torch.zeros_like(c)
            philox_kernel[(1,)](c, out, seed, BLOCK=c.shape[0])
            outs.append(out.numpy().view(np.uint32).copy())
        np.save(os.path.join(d, "out.npy"), np.stack(outs))
    """)
    env = dict(os.environ, TRITON_INTERPRET="1")
    subprocess.run([sys.executable, "-c", script, str(tmp_path)] + [str(s) for s in seeds],
                   check=True, env=env, timeout=600)
    return np.load(tmp_path / "out.npy")


def test_philox_matches_independent_implementation(tmp_path):
    """Philox4x32-10 against Triton's tl.philox (same published algorithm,
    independent code, key = (seed low word, seed high word))."""
    rng = np.random.default_rng(11)
    ctr = rng.integers(0, 2**32, size=(256, 4), dtype=np.uint64).astype(np.uint32)
    ctr[:16] = 0
    ctr[:16, 0] = np.arange(16)                 # small structured counters too
    ctr[16:20] = 0xFFFFFFFF
    seeds = [0, 1, 0x12345678, 0x0123456789ABCDEF, 2**63 - 1]
    ref = _triton_philox(ctr, seeds, tmp_path)
    if ref is None:
        pytest.skip("Triton is not installed: no independent Philox to compare with")
    for s, want in zip(seeds, ref):
        got = oracle.philox4x32(ctr, oracle.seed_key(s))
        assert np.array_equal(got, want), hex(s)


def _avalanche_means(rounds, flip_key):
    rng = np.random.default_rng(12)
    n = 512
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = (0x9A3B1C2D, 0x55AA1234)
    base = oracle.philox4x32(ctr, key, rounds)
    means = []
    for bit in range(64 if flip_key else 128):
        if flip_key:
            k = [key[0], key[1]]
            k[bit // 32] ^= 1 << (bit % 32)
            out = oracle.philox4x32(ctr, k, rounds)
        else:
            c = ctr.copy()
            c[:, bit // 32] ^= np.uint32(1 << (bit % 32))
            out = oracle.philox4x32(c, key, rounds)
        diff = np.unpackbits((base ^ out).view(np.uint8), axis=1).sum(axis=1)
        means.append(diff.mean())
    return np.array(means)


def test_philox_avalanche():
    """Ten rounds mix fully: flipping any one counter or key bit flips 64 of
    the 128 output bits on average (standard error about 0.25 here). One
    round does not, which shows the check can tell the difference."""
    for flip_key in (False, True):
        m = _avalanche_means(10, flip_key)
        assert np.all(np.abs(m - 64.0) < 2.0), (flip_key, m.min(), m.max())
    weak = _avalanche_means(1, False)
    assert np.any(np.abs(weak - 64.0) > 10.0)


def test_draws_are_distinct_across_coordinates():
    """S2: every (row, block, direction, half) gets its own 128-bit draw."""
    seen = set()
    for d in (oracle.DIR_ROWWISE, oracle.DIR_COLUMNWISE):
        b = oracle.sr_random_bytes(np.arange(8), 8, seed=77, direction=d)
        halves = b.reshape(8, 8, 2, 16)
        for r in range(8):
            for j in range(8):
                for h in range(2):
                    seen.add(halves[r, j, h].tobytes())
    assert len(seen) == 2 * 8 * 8 * 2


def _neighbours(mag):
    """Grid neighbours of a Fraction magnitude, by search (6 saturates)."""
    if mag >= 6:
        return Fraction(6), Fraction(6)
    lo = max(g for g in GRID if g <= mag)
    hi = min(g for g in GRID if g > mag)
    return lo, hi


_GRID_F64 = np.array([float(g) for g in GRID])


@pytest.mark.parametrize("partner_hex", ["40c0", "3f80", "4000", "0100", "0008", "7f7f"])
def test_sr_every_bf16_every_byte(partner_hex):
    """S3 by exhaustion. For every BF16 x with |x| <= amax (a partner element
    fixes amax, hence the scale) and every byte u in 0..255:
      * the magnitude is one of the two grid neighbours of |v| = |x| 2^-e,
        found by a search over the grid;
      * the bytes that round up are the largest ones;
      * the mean over all bytes equals x exactly when 1/4 <= |v| < 6, and
        lies below |x| by less than 1/256 of the spacing (1/2) under 1/4;
      * the sign bit is that of x.
    All values here are dyadic with few bits, so float64 sums and
    differences are exact; a sample is re-checked in rationals."""
    partner = int(partner_hex, 16)
    pos = np.arange(0, partner + 1, dtype=np.uint16)
    xs = np.concatenate([pos, pos | np.uint16(0x8000)])
    n = xs.size
    nb = -(-n // 31)
    slots = np.zeros(nb * 31, dtype=np.uint16)
    slots[:n] = xs
    blk = np.empty((nb, 32), dtype=np.uint16)
    blk[:, 0] = partner
    blk[:, 1:] = slots.reshape(nb, 31)
    blocks = np.tile(blk, (256, 1))                     # byte u: rows u*nb ..
    rb = np.repeat(np.arange(256, dtype=np.uint8), nb)[:, None].repeat(32, axis=1)
    codes, scales = oracle.quantize_sr_with_bytes(blocks, rb)
    assert np.all(scales == scales[0, 0])
    e = int(scales[0, 0]) - 127
    c = oracle.unpack_codes(codes).reshape(256, nb, 32)[:, :, 1:].reshape(256, nb * 31)[:, :n]
    mag = oracle.E2M1_VALUES[c & 7]                    # [256, n]
    x = oracle.bf16_bits_to_f64(xs)
    v = np.abs(np.ldexp(x, -e))
    below = np.where(_GRID_F64[None, :] <= v[:, None], _GRID_F64[None, :], -1.0)
    above = np.where(_GRID_F64[None, :] > v[:, None], _GRID_F64[None, :], np.inf)
    lo = below.max(axis=1)
    hi = np.minimum(above.min(axis=1), 6.0)
    lo = np.where(v >= 6, 6.0, lo)
    assert np.all((mag == lo[None, :]) | (mag == hi[None, :]))
    up = (mag == hi[None, :]) & (hi != lo)[None, :]
    nup = up.sum(axis=0)
    u = np.arange(256)[:, None]
    assert np.array_equal(up, u >= (256 - nup)[None, :])
    signed = np.where(np.signbit(x)[None, :], -mag, mag)
    mean = np.ldexp(signed.sum(axis=0) / 256.0, e)     # exact: dyadic
    mid = (v >= 0.25) & (v < 6)
    assert np.array_equal(mean[mid], x[mid])
    small = v < 0.25
    gap = np.ldexp(np.abs(x[small]) - np.abs(mean[small]), -e)
    assert np.all((gap >= 0) & (gap < 0.5 / 256))
    assert np.all(((c >> 3) & 1) == (xs >> 15)[None, :])
    # Rational re-check of the count of round-ups on a sample.
    rng = np.random.default_rng(int(partner_hex, 16))
    for i in rng.choice(n, size=min(n, 200), replace=False):
        vv = abs(Fraction(float(x[i]))) * Fraction(2) ** (-e)
        lo_f, hi_f = _neighbours(vv)
        want = 0 if hi_f == lo_f else int((vv - lo_f) / (hi_f - lo_f) * 256)
        assert nup[i] == want, hex(xs[i])


def test_sr_mean_over_all_bytes_is_the_input():
    """E[SR(x)] = x on random rows, in exact rationals: the mean of the
    dequantized value over all 256 bytes equals x when |x| 2^-e >= 1/4 (and
    below 6)."""
    x = bf16_matrix((8, 32), ("normal", 1.0, 0.0, 1.0), 13)
    for r in range(8):
        row = np.repeat(x[r:r + 1], 256, axis=0)
        rb = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 32, axis=1)
        codes, scales = oracle.quantize_sr_with_bytes(row, rb)
        dq = oracle.dequantize(codes, scales)
        e = int(scales[0, 0]) - 127
        vals = oracle.bf16_bits_to_f64(x[r])
        for k in range(32):
            xv = Fraction(float(vals[k]))
            v = abs(xv) * Fraction(2) ** (-e)
            if Fraction(1, 4) <= v < 6:
                mean = sum(Fraction(float(d)) for d in dq[:, k]) / 256
                assert mean == xv


def test_sr_scales_match_rne_and_grid_values_are_fixed():
    """S1: the scales are those of round-to-nearest quantize; values already
    on the grid come out unchanged whatever the random bytes."""
    rng = np.random.default_rng(14)
    x = bf16_matrix((16, 256), ("normal", 1.0, 0.0, 1.0), 14)
    _, s_rne = oracle.quantize(x)
    for seed in (0, 5, 2**40 + 3):
        _, s_sr = oracle.quantize_sr(x, seed)
        assert np.array_equal(s_sr, s_rne)
    grid_codes = rng.integers(0, 16, size=(16, 256), dtype=np.uint8)
    grid_codes[:, ::32] = 7                            # amax 6 in every block
    vals = oracle.E2M1_VALUES[grid_codes] * 2.0 ** rng.integers(-8, 8, size=(16, 1))
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    c_rne, _ = oracle.quantize(bits)
    for seed in (1, 99):
        c_sr, _ = oracle.quantize_sr(bits, seed)
        assert np.array_equal(c_sr, c_rne)


def test_sr_byte_layout():
    """S2 wiring: with every element at |v| = 1/4 (halfway from 0 to 1/2) an
    element rounds up exactly when bit 7 of its byte is set, so the codes
    expose the bytes. They must be byte i % 4 of word i // 4 of the draw for
    counter (block, row, direction, half)."""
    M, K, seed = 3, 96, 0xDEADBEEF12345678
    x = np.full((M, K), 0x3E80, dtype=np.uint16)      # 0.25
    x[:, ::32] = 0x40C0                                # 6.0: e = 0
    for d in (oracle.DIR_ROWWISE, oracle.DIR_COLUMNWISE):
        codes, _ = oracle.quantize_sr(x, seed, direction=d, row_ids=np.array([5, 0, 9]))
        c = oracle.unpack_codes(codes)
        for i, r in enumerate([5, 0, 9]):
            for j in range(K // 32):
                for h in range(2):
                    w = oracle.philox4x32(np.array([j, r, d, h], dtype=np.uint32),
                                          oracle.seed_key(seed))
                    for t in range(16):
                        k = 32 * j + 16 * h + t
                        if k % 32 == 0:
                            continue
                        byte = (int(w[t // 4]) >> (8 * (t % 4))) & 0xFF
                        assert c[i, k] == (1 if byte >= 128 else 0), (d, r, j, h, t)


def test_sr_2d_is_rowwise_of_transpose_with_direction_1():
    x = bf16_matrix((64, 96), ("laplace", 1.0), 15)
    c, s, ct, st = oracle.quantize_2d_sr(x, 1234)
    c1, s1 = oracle.quantize_sr(x, 1234, oracle.DIR_ROWWISE)
    c2, s2 = oracle.quantize_sr(np.ascontiguousarray(x.T), 1234, oracle.DIR_COLUMNWISE)
    assert np.array_equal(c, c1) and np.array_equal(s, s1)
    assert np.array_equal(ct, c2) and np.array_equal(st, s2)
    c3, _ = oracle.quantize_sr(np.ascontiguousarray(x.T), 1234, oracle.DIR_ROWWISE)
    assert not np.array_equal(ct, c3)                  # the direction is keyed


def test_sr_seed_changes_codes_and_is_deterministic():
    x = bf16_matrix((8, 128), ("normal", 1.0, 0.0, 1.0), 16)
    a, _ = oracle.quantize_sr(x, 1)
    b, _ = oracle.quantize_sr(x, 1)
    c, _ = oracle.quantize_sr(x, 2)
    d, _ = oracle.quantize_sr(x, 1 + (1 << 32))        # high key word
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert not np.array_equal(a, d)


def test_sr_row_shards_are_parts_of_the_whole():
    """Reading S5: a row shard keyed by its global rows and row blocks gives
    exactly the matching rows (row-wise) and columns (column-wise) of the
    whole input's outputs, and keying it from row 0 instead does not."""
    x = bf16_matrix((160, 96), ("laplace", 1.0), 17)
    c, s, ct, st = oracle.quantize_2d_sr(x, 99)
    for row0, m in [(0, 64), (32, 96), (128, 32)]:
        part = x[row0:row0 + m]
        pc, ps, pct, pst = oracle.quantize_2d_sr(part, 99, row0=row0)
        assert np.array_equal(pc, c[row0:row0 + m]) and np.array_equal(ps, s[row0:row0 + m])
        assert np.array_equal(pct, ct[:, row0 // 2:(row0 + m) // 2])
        assert np.array_equal(pst, st[:, row0 // 32:(row0 + m) // 32])
        rc, rs = oracle.quantize_sr(part, 99, row_ids=row0 + np.arange(m))
        assert np.array_equal(rc, pc) and np.array_equal(rs, ps)
        if row0:
            qc, _, qct, _ = oracle.quantize_2d_sr(part, 99)
            assert not np.array_equal(qc, pc) and not np.array_equal(qct, pct)
    with pytest.raises(ValueError):
        oracle.quantize_2d_sr(x[16:48], 99, row0=16)
