"""Pins of the fused-SwiGLU oracle (oracle/swiglu.py, readings W1-W4).

silu is pinned against torch's float64 SiLU and closed forms; the gate/up
split of the stacked weight against a GEMM whose outputs are known element
by element; the tolerance W4 against a brute-force search of its error box
plus torch's measured fp32 evaluation error (it must cover both and be at
most four times their sum), and against planted errors.
"""

import math

import numpy as np
import torch

import oracle
from conftest import read_golden


def test_silu_matches_torch_float64():
    z = np.concatenate([np.linspace(-60, 60, 20001), [-1e3, -745.2, 0.0, 1e-300, 700.0]])
    want = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    got = oracle.silu(z)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-300)


def test_silu_closed_forms():
    ln3 = math.log(3.0)
    assert oracle.silu(0.0) == 0.0
    assert math.isclose(oracle.silu(ln3), 0.75 * ln3, rel_tol=1e-15)      # sigmoid(ln 3) = 3/4
    assert math.isclose(oracle.silu(-ln3), -0.25 * ln3, rel_tol=1e-15)
    z = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)  # s(z)+s(-z)=1
    assert oracle.silu(-1e4) == 0.0 and oracle.silu(1e4) == 1e4


def test_silu_minimum():
    """The one critical point of silu, found by a fine grid search."""
    z = np.linspace(-3, 1, 4000001)
    v = oracle.silu(z)
    assert abs(z[np.argmin(v)] - oracle.SILU_ARGMIN) < 2e-6
    assert math.isclose(oracle.SILU_ARGMIN, -1.2784645427610738, rel_tol=1e-13)
    assert oracle.silu(z).min() >= oracle.silu(oracle.SILU_ARGMIN)


def _box_worst_case(g, u, sg, su, n=257):
    """Largest |silu(g') u' - silu(g) u| over a grid of the box |g' - g| <=
    1e-5 S_g, |u' - u| <= 1e-5 S_u (both ends included), in float64."""
    dg, du = 1e-5 * sg, 1e-5 * su
    gg = np.linspace(g - dg, g + dg, n)
    uu = np.linspace(u - du, u + du, n)
    ref = float(oracle.silu(g)) * u
    return float(np.abs(oracle.silu(gg)[:, None] * uu[None, :] - ref).max())


def _torch_fp32_error(g, u):
    """|fp32 silu(g) * u - exact| measured with torch on the fp32 inputs."""
    g32, u32 = torch.tensor(g, dtype=torch.float32), torch.tensor(u, dtype=torch.float32)
    got = float(torch.nn.functional.silu(g32) * u32)
    exact = float(oracle.silu(float(g32))) * float(u32)
    return abs(got - exact)


# (g, u, S_g, S_u): both tails of silu, its minimum, zeros, sums whose S is
# just |C| (one product) and sums whose S is far above |C| (cancellation),
# boxes wide enough that the cross term dominates.
_W4_SAMPLES = [
    (g, u, sg, su)
    for g in (-120.0, -95.0, -88.0, -30.0, -10.0, -3.0, oracle.SILU_ARGMIN, -1.0, -0.3,
              0.0, 1e-3, 0.5, 2.4, 5.0, 20.0, 90.0)
    for u in (-50.0, -1.0, -1e-3, 0.0, 0.7, 13.0)
    for sg, su in ((abs(g), abs(u)), (10 * abs(g) + 1, 10 * abs(u) + 1), (1e4, 1e4))
]


def test_w4_tolerance_is_a_tight_bound():
    """W4 covers the worst case of the GEMM bound through silu(g) u plus the
    fp32 evaluation error, and is at most 4x that sum. Where the fp32 exp of
    the kernel may overflow (g < -87) only validity is asserted: there W4
    allows the whole |act|."""
    loose = []
    for g, u, sg, su in _W4_SAMPLES:
        need = _box_worst_case(g, u, sg, su) + _torch_fp32_error(g, u)
        tol = float(oracle.swiglu_tolerance(g, u, sg, su))
        assert tol >= need, (g, u, sg, su, tol, need)
        if g >= -87.0 and need > 0:
            loose.append(tol / need)
            assert tol <= 4 * need, (g, u, sg, su, tol, need)
        if need == 0:
            assert tol == 0.0
    assert max(loose) < 4 and len(loose) > 200


def test_w4_slips_are_caught():
    """Plausible mistakes in W4 break one of the two bounds: the cross term
    dropped (g = u = 0 with a wide box), |silu'| <= 1.1 in place of the range
    of silu (g far below 0), and the box taken ten times too wide."""
    # Cross term only: g = u = 0, d = 0.1 -> max |s u'| = silu(0.1) * 0.1.
    need = _box_worst_case(0.0, 0.0, 1e4, 1e4)
    assert math.isclose(need, float(oracle.silu(0.1)) * 0.1, rel_tol=1e-12)
    assert float(oracle.swiglu_tolerance(0.0, 0.0, 1e4, 1e4)) >= need > 0
    # A first-order bound with |silu'| <= 1.1 is hundreds of times too loose at g = -10.
    g, u, sg, su = -10.0, 13.0, 101.0, 131.0
    need = _box_worst_case(g, u, sg, su) + _torch_fp32_error(g, u)
    first_order = 1e-5 * (1.1 * sg * abs(u) + abs(float(oracle.silu(g))) * su)
    assert first_order > 4 * need >= float(oracle.swiglu_tolerance(g, u, sg, su))
    # Ten times the box is outside the 4x bound.
    assert float(oracle.swiglu_tolerance(2.4, 13.0, 10 * 25.0, 10 * 131.0)) > 4 * (
        _box_worst_case(2.4, 13.0, 25.0, 131.0) + _torch_fp32_error(2.4, 13.0))


def _one_hot_b(Nh, K, pick):
    """B [2 Nh, K]: row n holds one code 2 (value 1.0) at k = pick[n], scale 127."""
    codes = np.zeros((2 * Nh, K), dtype=np.uint8)
    codes[np.arange(2 * Nh), pick] = 2
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return packed.astype(np.uint8), np.full((2 * Nh, K // 32), 127, dtype=np.uint8)


def test_gate_up_split_with_known_gemm_outputs():
    """W1: with A's row holding the Q1 values and B one-hot, g[j] = x[j] and
    u[j] = x[Nh + j] exactly, so act[j] = silu(x[j]) * x[Nh + j]."""
    g = read_golden("q1_block.txt")
    vals = np.array([float(v) for v in g["input"]])             # 32 BF16-exact values
    a_codes, a_scales = oracle.quantize(
        (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)[None, :])
    x = oracle.dequantize(a_codes, a_scales)[0]                  # what the GEMM sees
    Nh, K = 16, 32
    b_codes, b_scales = _one_hot_b(Nh, K, np.arange(2 * Nh))
    act, tol = oracle.swiglu_reference(a_codes, a_scales, b_codes, b_scales)
    want = np.array([x[j] / (1.0 + math.exp(-x[j])) * x[Nh + j] for j in range(Nh)])
    assert np.array_equal(act[0], want)
    # Swapping the halves of B changes the answer (the split is not symmetric).
    swapped = np.concatenate([np.arange(Nh, 2 * Nh), np.arange(Nh)])
    b2, s2 = _one_hot_b(Nh, K, swapped)
    act2, _ = oracle.swiglu_reference(a_codes, a_scales, b2, s2)
    assert not np.array_equal(act, act2)
    # One product per output: S_g = |g|, S_u = |u|; W4 covers the box.
    for j in range(Nh):
        need = _box_worst_case(x[j], x[Nh + j], abs(x[j]), abs(x[Nh + j]))
        assert tol[0, j] >= need


def test_act_check_accepts_rounded_and_rejects_planted_errors():
    rng = np.random.default_rng(3)
    a_codes = rng.integers(0, 256, size=(8, 128), dtype=np.uint8)
    a_scales = rng.integers(120, 128, size=(8, 8), dtype=np.uint8)
    b_codes = rng.integers(0, 256, size=(64, 128), dtype=np.uint8)
    b_scales = rng.integers(118, 126, size=(64, 8), dtype=np.uint8)
    act, tol = oracle.swiglu_reference(a_codes, a_scales, b_codes, b_scales)
    assert act.shape == (8, 32) and np.all(tol >= 0)
    ok_bits = oracle.bf16_bits_of(oracle.round_to_bf16(act))
    assert oracle.check_act_bf16(ok_bits, act, tol).all()
    # Move every element 3 tolerances plus 2 BF16 steps away: all must fail.
    bad = act + np.sign(act + 1e-30) * (3 * tol + 2 * oracle.bf16_ulp(act))
    bad_bits = oracle.bf16_bits_of(oracle.round_to_bf16(bad))
    assert not oracle.check_act_bf16(bad_bits, act, tol).any()


def test_row_subset_matches_full():
    rng = np.random.default_rng(4)
    a_codes = rng.integers(0, 256, size=(16, 64), dtype=np.uint8)
    a_scales = rng.integers(120, 128, size=(16, 4), dtype=np.uint8)
    b_codes = rng.integers(0, 256, size=(96, 64), dtype=np.uint8)
    b_scales = rng.integers(118, 126, size=(96, 4), dtype=np.uint8)
    act, tol = oracle.swiglu_reference(a_codes, a_scales, b_codes, b_scales)
    rows = np.array([0, 5, 15])
    act_r, tol_r = oracle.swiglu_reference(a_codes, a_scales, b_codes, b_scales, m_rows=rows)
    assert np.array_equal(act_r, act[rows]) and np.array_equal(tol_r, tol[rows])
