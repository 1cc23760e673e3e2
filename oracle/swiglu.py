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
GEMM sums. Its act may differ from the float64 act by the GEMM tolerance
propagated through W2 plus the fp32 evaluation error:
  tol = 1e-5 * (1.1 * S_g * |u| + |silu(g)| * S_u + 1.1e-5 * S_g * S_u)
        + 2**-16 * |act|
where S_g, S_u are the sums of |products| of g and u (mxfp4_ref.gemm_block),
1e-5 * S is the GEMM's FP32 bound, 1.1 bounds |silu'| (its maximum is
1.0998), the S_g S_u term is the product of the two errors, and 2**-16 covers
the exp, reciprocal and products in fp32 (a few units in the last place,
plus |g| ulps of exp's argument for |g| up to about 100). A BF16 act output
then lies within tol + half a BF16 step of act (compare.check_act_bf16).
"""

import numpy as np

from .mxfp4_ref import gemm_block

SILU_DERIV_MAX = 1.1
GEMM_REL_TOL = 1e-5
EVAL_REL_TOL = 2.0 ** -16


def silu(z):
    """W2: z * sigmoid(z) = z / (1 + exp(-z)) in float64 (exp overflow -> 0)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_reference(A_codes, A_scales, B_codes, B_scales, m_rows=None):
    """W1, W2 for the rows m_rows of A (all if None).

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
    sg, su = S[:, :Nh], S[:, Nh:]
    sg_silu = silu(g)
    act = sg_silu * u
    tol = (GEMM_REL_TOL * (SILU_DERIV_MAX * sg * np.abs(u) + np.abs(sg_silu) * su
                           + SILU_DERIV_MAX * GEMM_REL_TOL * sg * su)
           + EVAL_REL_TOL * np.abs(act))
    return act, tol
