"""Pins of the CPU oracle against things other than itself.

Each test ties one part of the oracle to a hand-worked example, a closed form,
an exhaustive brute force in a different formulation, exact rational
arithmetic, or a library routine. Format source for all of them: "Integrate
MXFP4 hipblaslt GEMM support" (ROCm/TransformerEngine #697), Changes list
(E2M1 elements, UE8M0 block-32 scales, TN GEMM); the numeric readings R1-R6
are those stated in oracle/mxfp4_ref.py.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden, read_golden_table
from synth import large_block_first, random_codes, random_scales, random_bf16_bits

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
        Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _f2bits(vals):
    """BF16 bits of values that are exactly BF16 (checked)."""
    f32 = np.asarray(vals, dtype=np.float32)
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f32)
    return bits


# --------------------------------------------------------------------- R1
def test_e2m1_table_matches_bitfield_definition():
    """E2M1 = 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is
    subnormal. Decoding each code from its bit fields must give the table."""
    for c in range(16):
        s, E, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if E == 0 else (1 + m / 2) * 2.0 ** (E - 1)
        val = -mag if s else mag
        assert oracle.E2M1_VALUES[c] == val
        assert np.signbit(oracle.E2M1_VALUES[c]) == bool(s)
    mags = sorted(set(abs(v) for v in oracle.E2M1_VALUES))
    assert mags == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


# --------------------------------------------------------------------- R2
def test_scale_byte_bruteforce_all_bf16_amax():
    """Every finite non-negative BF16 amax: the frexp exponent of the oracle
    against the closed form on bits, byte = max(E_field - 2, 0)."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)          # +0 .. BF16 max
    amax = oracle.bf16_bits_to_f64(bits)
    got = oracle.scale_exponent(amax) + 127
    want = np.maximum((bits.astype(np.int64) >> 7) - 2, 0)
    assert np.array_equal(got, want)


def test_scale_spot_values():
    for hexbits, _name, byte, code in read_golden_table("scale_spots.txt"):
        b = np.zeros((1, 32), dtype=np.uint16)
        b[0, 0] = int(hexbits, 16)
        codes, scales = oracle.quantize(b)
        assert scales[0, 0] == int(byte), hexbits
        assert (codes[0, 0] & 0xF) == int(code), hexbits
        assert np.all(codes[0, 1:] == 0) and (codes[0, 0] >> 4) == 0


# --------------------------------------------------------------------- R3
def _threshold_code(v):
    """Independent encoder: count the grid midpoints below |v|; a value on a
    midpoint goes to the even neighbour. Midpoints 0.25 .. 5 alternate
    odd/even lower neighbours, hence the alternating strict/non-strict tests."""
    a = np.abs(v)
    return ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0))


@pytest.mark.parametrize("partner_hex", ["40c0", "3f80", "0100", "0008", "7f7f", "3ca4"])
def test_rne_bruteforce_every_bf16(partner_hex):
    """Every finite BF16 x in a block whose other 31 entries are one fixed
    partner value: oracle codes vs the midpoint-count encoder, with the
    scale from the bit-field closed form."""
    xs = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    xs = xs[(xs & 0x7F80) != 0x7F80]
    blocks = np.full((xs.size, 32), int(partner_hex, 16), dtype=np.uint16)
    blocks[:, 7] = xs
    codes, scales = oracle.quantize(blocks)
    amax_bits = np.maximum(xs & 0x7FFF, int(partner_hex, 16) & 0x7FFF)
    byte = np.maximum((amax_bits.astype(np.int64) >> 7) - 2, 0)
    assert np.array_equal(scales[:, 0], byte)
    v = np.ldexp(oracle.bf16_bits_to_f64(xs), 127 - byte)
    want = _threshold_code(v) | (((xs >> 15) & 1).astype(np.uint8) << 3)
    got = codes[:, 3] >> 4                                  # element 7 = high nibble of byte 3
    assert np.array_equal(got, want)


def test_rne_fraction_nearest_search_random():
    """Random finite BF16 blocks: each code against an exact nearest-grid
    search in rational arithmetic (ties to the even index)."""
    bits = random_bf16_bits((64, 32), seed=7)
    codes, scales = oracle.quantize(bits)
    c = oracle.unpack_codes(codes)
    for r in range(bits.shape[0]):
        e = int(scales[r, 0]) - 127
        for i in range(32):
            x = Fraction(float(oracle.bf16_bits_to_f64(bits[r, i])))
            v = abs(x) / Fraction(2) ** e
            d = [abs(v - g) for g in GRID]
            best = min(range(8), key=lambda j: (d[j], j % 2))
            sign = int(bits[r, i]) >> 15
            assert c[r, i] == best | (sign << 3), (r, i)


# --------------------------------------------------------- R2-R4 worked examples
def test_q1_hand_worked():
    g = read_golden("q1_block.txt")
    x = _f2bits([float(v) for v in g["input"]])[None, :]
    codes, scales = oracle.quantize(x)
    assert scales.tolist() == [[int(g["scale"][0])]]
    assert oracle.unpack_codes(codes)[0].tolist() == [int(v, 16) for v in g["codes"]]
    assert codes[0].tolist() == [int(v, 16) for v in g["packed"]]
    dq = oracle.dequantize(codes, scales)[0]
    assert dq.tolist() == [float(v) for v in g["dequant"]]


def test_q2_hand_worked():
    g = read_golden("q2_block.txt")
    x = _f2bits([float(v) for v in g["input"]])[None, :]
    codes, scales = oracle.quantize(x)
    assert scales.tolist() == [[int(g["scale"][0])]]
    assert oracle.unpack_codes(codes)[0].tolist() == [int(v, 16) for v in g["codes"]]


def test_quantize_2d_columns_hand_worked():
    """Columnwise form (NVIDIA/TransformerEngine #3809, bidimensional quantize):
    a 32 x 64 X whose column 5 is the hand-worked Q1 block (others zero) must
    give Q1's packed codes and scale in row 5 of the transposed output, and
    Q1-free rows elsewhere; the rowwise form is the plain quantize."""
    g = read_golden("q1_block.txt")
    x = np.zeros((32, 64), dtype=np.uint16)
    x[:, 5] = _f2bits([float(v) for v in g["input"]])
    codes, scales, codes_t, scales_t = oracle.quantize_2d(x)
    assert codes_t.shape == (64, 16) and scales_t.shape == (64, 1)
    assert codes_t[5].tolist() == [int(v, 16) for v in g["packed"]]
    assert scales_t[5].tolist() == [int(g["scale"][0])]
    others = np.delete(np.arange(64), 5)
    assert np.all(codes_t[others] == 0) and np.all(scales_t[others] == 0)
    rc, rs = oracle.quantize(x)
    assert np.array_equal(codes, rc) and np.array_equal(scales, rs)


def test_quantize_2d_transpose_symmetry():
    """The columnwise outputs of X are the rowwise outputs of X^T and back."""
    x = random_bf16_bits((64, 96), 12345)
    c, s, ct, st = oracle.quantize_2d(x)
    c2, s2, ct2, st2 = oracle.quantize_2d(np.ascontiguousarray(x.T))
    assert np.array_equal(ct, c2) and np.array_equal(st, s2)
    assert np.array_equal(c, ct2) and np.array_equal(s, st2)


# --------------------------------------------------------------- invariants
def test_sign_flip_invariant():
    bits = random_bf16_bits((16, 256), seed=11)
    c1, s1 = oracle.quantize(bits)
    c2, s2 = oracle.quantize(bits ^ np.uint16(0x8000))
    assert np.array_equal(s1, s2)
    assert np.array_equal(c2, c1 ^ np.uint8(0x88))


def test_power_of_two_scaling_invariant():
    """q(2**j x) keeps the codes and adds j to every scale byte when no
    clamping occurs (normal N(0,1) data far from both ends)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c0, s0 = oracle.quantize(bits)
    for j in (-20, -1, 1, 7, 30):
        bj = (bits.astype(np.int32) + (j << 7)).astype(np.uint16)   # exponent field + j
        cj, sj = oracle.quantize(bj)
        assert np.array_equal(cj, c0)
        assert np.array_equal(sj.astype(int), s0.astype(int) + j)


def test_roundtrip_on_grid():
    """dq(q(x)) == x when every x / 2**e is an E2M1 value."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(32, 256))
    codes[:, ::32] = 7                         # amax 6 * 2**e in every block
    e = rng.integers(-100, 100, size=(32, 8))
    x = np.ldexp(oracle.E2M1_VALUES[codes].reshape(32, 8, 32), e[..., None]).reshape(32, 256)
    c, s = oracle.quantize(_f2bits(x))
    assert np.array_equal(s.astype(int), e + 127)
    assert np.array_equal(oracle.dequantize(c, s), x)


def test_zero_blocks():
    z = np.zeros((2, 64), dtype=np.uint16)
    z[1, :] = 0x8000                           # -0.0 keeps its sign bit
    c, s = oracle.quantize(z)
    assert np.all(s == 0)
    assert np.all(c[0] == 0) and np.all(c[1] == 0x88)


# ---------------------------------------------------------------------- R6
def test_dequant_bruteforce_all_codes_and_scales():
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256).repeat(255, axis=0)
    scales = np.arange(255, dtype=np.uint8)[:, None].repeat(16, axis=1)
    dq = oracle.dequantize(codes, scales)
    for s in (0, 1, 100, 127, 200, 254):
        for k in range(0, 512, 37):
            c = (k // 2) >> 4 if k % 2 else (k // 2) & 0xF
            want = GRID[c & 7] * (Fraction(2) ** (s - 127))
            want = -want if c >> 3 else want
            assert Fraction(dq[s, k]) == want


# -------------------------------------------------------------------- GEMM
SCALE_SET = [0, 1, 60, 119, 126, 127, 128, 200, 254]


def test_gemm_bruteforce_code_scale_pairs():
    """1 x 1 x 32 products of every code pair under every scale pair,
    against exact rationals: val(ca) * val(cb) * 2**(sa + sb - 254)."""
    rows = [(c, s) for c in range(16) for s in SCALE_SET]
    codes = np.zeros((len(rows), 16), dtype=np.uint8)
    scales = np.zeros((len(rows), 1), dtype=np.uint8)
    for i, (c, s) in enumerate(rows):
        codes[i, 5] = c << 4                  # element k = 11
        scales[i, 0] = s
    C, S = oracle.gemm(codes, scales, codes, scales)
    for i, (ca, sa) in enumerate(rows):
        va = (-1 if ca >> 3 else 1) * GRID[ca & 7]
        for j, (cb, sb) in enumerate(rows):
            vb = (-1 if cb >> 3 else 1) * GRID[cb & 7]
            want = va * vb * Fraction(2) ** (sa + sb - 254)
            assert Fraction(C[i, j]) == want
            assert Fraction(S[i, j]) == abs(want)


def test_g1_hand_worked_1x32x32():
    """A = the Q1 block; B row n holds code 2 (1.0) at k = n, scale 127, so
    C[0, n] is the n-th dequantized value of Q1."""
    g = read_golden("q1_block.txt")
    A = np.array([[int(v, 16) for v in g["packed"]]], dtype=np.uint8)
    As = np.array([[127]], dtype=np.uint8)
    Bc = np.zeros((32, 16), dtype=np.uint8)
    for n in range(32):
        Bc[n, n // 2] = 2 << (4 * (n % 2))
    Bs = np.full((32, 1), 127, dtype=np.uint8)
    C, _ = oracle.gemm(A, As, Bc, Bs)
    assert C[0].tolist() == [float(v) for v in g["dequant"]]


def test_g2_scale_rows():
    """All codes 2 (1.0); A scale[m, j] = 123 + j; B scale[n, :] = 126 + n % 3.
    Closed form: C = 32 * 2**(n%3 - 1) * sum_j 2**(j - 4) = 255 * 2**(n % 3)."""
    A = np.full((32, 128), 0x22, dtype=np.uint8)
    As = np.tile(np.arange(123, 131, dtype=np.uint8), (32, 1))
    Bs = (126 + np.arange(32) % 3).astype(np.uint8)[:, None].repeat(8, axis=1)
    C, S = oracle.gemm(A, As, A, Bs)
    want = 255.0 * 2.0 ** (np.arange(32) % 3)
    assert np.array_equal(C, np.tile(want, (32, 1)))
    assert np.array_equal(S, C)


def test_g3_nibble_pairing():
    """A bytes 0x13 (1.5 low, 0.5 high), B bytes 0x24 (2.0 low, 1.0 high):
    each byte pair gives 1.5*2 + 0.5*1 = 3.5, C = 128 * 3.5 = 448. Swapping
    one operand's nibbles would give 128 * 2.5 = 320."""
    A = np.full((32, 128), 0x13, dtype=np.uint8)
    B = np.full((32, 128), 0x24, dtype=np.uint8)
    s = np.full((32, 8), 127, dtype=np.uint8)
    C, _ = oracle.gemm(A, s, B, s)
    assert np.all(C == 448.0)
    Cswap, _ = oracle.gemm((A >> 4) | (A << 4), s, B, s)
    assert np.all(Cswap == 320.0)


def test_g4_scale_blocks():
    """A code j in K-block j, A scale[m, j] = 123 + j + m % 2; B code 2 with
    scale 125 + n % 4. Closed form: 32 * sum_j val(j) 2**j = 37408, so
    C[m, n] = 37408 * 2**(m%2 + n%4 - 6) = 2338 * 2**(m%2 + n%4 - 2)."""
    A = np.zeros((32, 128), dtype=np.uint8)
    for j in range(8):
        A[:, 16 * j:16 * (j + 1)] = j | (j << 4)
    As = (123 + np.arange(8)[None, :] + (np.arange(32) % 2)[:, None]).astype(np.uint8)
    B = np.full((32, 128), 0x22, dtype=np.uint8)
    Bs = (125 + np.arange(32) % 4).astype(np.uint8)[:, None].repeat(8, axis=1)
    C, _ = oracle.gemm(A, As, B, Bs)
    m = np.arange(32)[:, None]
    n = np.arange(32)[None, :]
    assert np.array_equal(C, 2338.0 * 2.0 ** ((m % 2) + (n % 4) - 2))


def test_gemm_fp64_equals_exact_rational():
    """Random 32x32x256 operands, scales in 127 +- 8: the float64 C and S
    equal the exact rational sums."""
    Ac, Bc = random_codes(32, 256, 21), random_codes(32, 256, 22)
    As, Bs = random_scales(32, 256, 23, 119, 135), random_scales(32, 256, 24, 119, 135)
    C, S = oracle.gemm(Ac, As, Bc, Bs)
    a = oracle.unpack_codes(Ac)
    b = oracle.unpack_codes(Bc)

    def val(c, s):
        v = GRID[c & 7] * Fraction(2) ** (int(s) - 127)
        return -v if c >> 3 else v

    av = [[val(a[i, k], As[i, k // 32]) for k in range(256)] for i in range(32)]
    bv = [[val(b[i, k], Bs[i, k // 32]) for k in range(256)] for i in range(32)]
    for i in range(32):
        for j in range(32):
            terms = [x * y for x, y in zip(av[i], bv[j])]
            assert Fraction(C[i, j]) == sum(terms)
            assert Fraction(S[i, j]) == sum(abs(t) for t in terms)


def test_gemm_entries_and_block_agree_with_full():
    Ac, Bc = random_codes(64, 512, 31), random_codes(96, 512, 32)
    As, Bs = random_scales(64, 512, 33), random_scales(96, 512, 34)
    C, S = oracle.gemm(Ac, As, Bc, Bs)
    mi = np.array([0, 5, 63, 17])
    ni = np.array([95, 0, 3, 40])
    ce, se = oracle.gemm_entries(Ac, As, Bc, Bs, mi, ni)
    assert np.allclose(ce, C[mi, ni], rtol=0, atol=1e-12 * S[mi, ni].max())
    assert np.allclose(se, S[mi, ni], rtol=1e-14)
    cb, _ = oracle.gemm_block(Ac, As, Bc, Bs, mi, ni)
    assert np.array_equal(cb, C[np.ix_(mi, ni)])


# ------------------------------------------------------- acceptance criteria
def test_round_to_bf16_matches_torch_on_float32_values():
    """For float32-representable values, direct float64->BF16 rounding must
    equal torch's float32->BF16 conversion (nearest even)."""
    rng = np.random.default_rng(9)
    raw = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f32 = raw.view(np.float32)
    f32 = f32[np.isfinite(f32) & (np.abs(f32) < 3.3e38)]
    want = torch.from_numpy(f32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(f32.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_to_bf16_ties_and_double_rounding():
    one = 1.0
    assert oracle.round_to_bf16(one + 2.0 ** -8) == one                 # tie -> even
    assert oracle.round_to_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6  # tie -> even
    # Above the tie by less than float32 can hold: must round up (a detour
    # through float32 would land on the tie and round down).
    assert oracle.round_to_bf16(one + 2.0 ** -8 + 2.0 ** -40) == one + 2.0 ** -7
    assert oracle.round_to_bf16(-(one + 2.0 ** -8 + 2.0 ** -40)) == -(one + 2.0 ** -7)


def test_bf16_ordinal_counts_steps():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    o = oracle.bf16_ordinal(bits)
    assert np.all(np.diff(o) == 1)
    neg = oracle.bf16_ordinal(bits | np.uint16(0x8000))
    assert np.array_equal(neg, -o)


def test_check_functions_reject_planted_errors():
    c_ref = np.array([100.0, -3.0, 1e-3, 0.0])
    s_ref = np.array([1000.0, 10.0, 5.0, 1.0])
    assert oracle.check_fp32(c_ref + 0.9e-5 * s_ref, c_ref, s_ref).all()
    assert not oracle.check_fp32(c_ref + 1.1e-5 * s_ref, c_ref, s_ref).any()
    r = oracle.round_to_bf16(c_ref)
    bits = oracle.bf16_bits_of(r)
    lit, rd = oracle.check_bf16(bits, c_ref, s_ref)
    assert lit.all() and rd.all()
    two_up = bits.copy()
    two_up[:3] += 2                            # two BF16 steps away
    lit, rd = oracle.check_bf16(two_up, c_ref, s_ref)
    assert not lit[:3].any()
    assert not rd[0]                           # 100 + 2 steps (0.5 each) >> 1e-5 * 1000 + ulp/2


def test_large_block_first_closed_form():
    """The FP32 worst-case operands of the GPU tests: the oracle's C and S
    equal the closed form 8192 + (K - 256) 2^-17 (all products positive)."""
    for K in (256, 512, 2048):
        ac, as_ = large_block_first(3, K, 127)
        bc, bs = large_block_first(5, K, 128)
        c, s = oracle.gemm(ac, as_, bc, bs)
        assert np.all(c == 8192.0 + (K - 256) * 2.0 ** -17) and np.array_equal(c, s)
