"""Pins of the fused-SwiGLU oracle (oracle/swiglu.py, readings W1-W3).

silu is pinned against torch's float64 SiLU and closed forms; the gate/up
split of the stacked weight against a GEMM whose outputs are known element
by element; the tolerance formula against its own stated bound on |silu'|
and against planted errors.
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


def test_silu_derivative_bound():
    """The tolerance uses |silu'| <= 1.1; the true maximum is about 1.0998."""
    z = np.linspace(-20, 20, 400001)
    d = np.gradient(oracle.silu(z), z)
    assert 1.09 < np.abs(d).max() <= 1.1


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
    # One product per output: S_g = |g|, S_u = |u|.
    s_g, s_u = np.abs(x[:Nh]), np.abs(x[Nh:])
    exp_tol = (1e-5 * (1.1 * s_g * s_u + np.abs(oracle.silu(x[:Nh])) * s_u
                       + 1.1e-5 * s_g * s_u) + 2.0 ** -16 * np.abs(want))
    assert np.allclose(tol[0], exp_tol, rtol=1e-12, atol=0)


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
