"""Plain CPU oracle for the gate+up GEMM with a fused SwiGLU and MXFP4
requantize of its output.

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import this module. The HIP library never
does, and this module imports nothing from it: the two sides share no code.

What is computed. In a Llama-style MLP the gate and up projections are one
GEMM against the stacked weight [W_gate; W_up] (N = 2 Nh rows), followed by
SwiGLU, act = Swish(g) * u with Swish(z) = z * sigmoid(z) (Shazeer, "GLU
Variants Improve Transformer", 2020, the SwiGLU variant with beta = 1), and
the down projection consumes act as its MXFP4 A operand. The MXFP4 GEMM
contract of "Integrate MXFP4 hipblaslt GEMM support" (ROCm/TransformerEngine
#697, Changes list) has no activation epilogue; fusing one is a widening of
that GEMM, defined here as:
  W1  g[m, j] = C[m, j], u[m, j] = C[m, Nh + j] for j < Nh, with C the MXFP4
      GEMM of mxfp4_ref (float64 sum of dequantized products).
  W2  act[m, j] = silu(g) * u, silu(z) = z / (1 + exp(-z)), float64.
  W3  The kernel rounds its act to BF16 (nearest even) and quantizes those
      BF16 values exactly as mxfp4_ref.quantize does (blocks of 32 along j).
Readings (the pages are silent): the kernel evaluates W2 in fp32 from fp32
GEMM sums, and W4 bounds how far its act may lie from the float64 act:
  W4  tol = E_gemm + E_eval.
      E_gemm is the largest |silu(g') u' - silu(g) u| over the box
      |g' - g| <= 1e-5 S_g, |u' - u| <= 1e-5 S_u, i.e. the GEMM's FP32 bound
      (1e-5 * S, with S_g, S_u the sums of |products| from
      mxfp4_ref.gemm_block) carried through W2 exactly. silu has one
      minimum, at z* = -(1 + exp(z*)) = -1.27846..., and is monotone on each
      side of it, so over an interval of g' its values fill [lo, hi] with
      hi taken at an end of the interval and lo at an end or at z*; the
      product s u' is bilinear, so its extremes over [lo, hi] x [u - du,
      u + du] lie at the four corners.
      E_eval covers the fp32 evaluation z * rcp(1 + exp2(-z * log2 e)) * u:
      the product -z log2 e is rounded (relative 2^-24, and the constant
      itself 2^-25), which moves exp by about 1.5 |z| units of 2^-24; exp2,
      the add, the reciprocal and the two products add at most 7 more.
      E_eval = (2 |g| + 16) 2^-24 |act| leaves margin over that. For
      g < -87 the fp32 exp overflows (or its reciprocal falls below the
      normal range) and the kernel's silu is 0, so there E_eval also holds
      |act| itself.
A BF16 act output then lies within tol + half a BF16 step of act
(compare.check_act_bf16).
"""

import numpy as np

from .mxfp4_ref import gemm_block

GEMM_REL_TOL = 1e-5
EVAL_ULP = 2.0 ** -24
# g below which the fp32 evaluation of silu returns 0 (exp2 of more than 125.5
# overflows or its reciprocal leaves the normal range).
FP32_SILU_FLUSH = -87.0


def _silu_argmin():
    """z* with silu'(z*) = 0, the only critical point of silu: sigma(z)(1 + z
    sigma(-z)) = 0 means z = -(1 + exp(z)); Newton's method from -1."""
    z = -1.0
    for _ in range(50):
        z -= (z + 1.0 + np.exp(z)) / (1.0 + np.exp(z))
    return float(z)


SILU_ARGMIN = _silu_argmin()


def silu(z):
    """W2: z * sigmoid(z) = z / (1 + exp(-z)) in float64 (exp overflow -> 0)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_range(lo, hi):
    """(min, max) of silu over [lo, hi] (elementwise arrays, lo <= hi)."""
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    s_lo, s_hi = silu(lo), silu(hi)
    smin = np.minimum(s_lo, s_hi)
    smin = np.where((lo <= SILU_ARGMIN) & (SILU_ARGMIN <= hi), silu(SILU_ARGMIN), smin)
    return smin, np.maximum(s_lo, s_hi)


def swiglu_tolerance(g, u, sg, su):
    """W4: tol = E_gemm + E_eval for float64 g, u and their S_g, S_u."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    dg = GEMM_REL_TOL * np.asarray(sg, dtype=np.float64)
    du = GEMM_REL_TOL * np.asarray(su, dtype=np.float64)
    act = silu(g) * u
    smin, smax = silu_range(g - dg, g + dg)
    e_gemm = np.zeros_like(act)
    for s in (smin, smax):
        for uu in (u - du, u + du):
            e_gemm = np.maximum(e_gemm, np.abs(s * uu - act))
    e_eval = (2.0 * np.abs(g) + 16.0) * EVAL_ULP * np.abs(act)
    e_eval = np.where(g < FP32_SILU_FLUSH, e_eval + np.abs(act), e_eval)
    return e_gemm + e_eval


def swiglu_reference(A_codes, A_scales, B_codes, B_scales, m_rows=None):
    """W1, W2 for the rows m_rows of A (all if None), and W4's tolerance.

    B_codes [N, K/2] / B_scales [N, K/32] hold W_gate in rows 0..Nh-1 and
    W_up in rows Nh..N-1. Returns (act, tol), float64 [rows, Nh].
    """
    B_codes = np.asarray(B_codes)
    N = B_codes.shape[0]
    if N % 2:
        raise ValueError("the stacked gate+up weight needs an even row count")
    C, S = gemm_block(A_codes, A_scales, B_codes, B_scales, m_rows=m_rows)
    Nh = N // 2
    g, u = C[:, :Nh], C[:, Nh:]
    act = silu(g) * u
    return act, swiglu_tolerance(g, u, S[:, :Nh], S[:, Nh:])
