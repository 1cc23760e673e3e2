"""Acceptance criteria for GEMM outputs, measured against the oracle.

TEST INFRASTRUCTURE (see oracle/mxfp4_ref.py for who may use it).

  FP32 output: |C_out - C_ref| <= 1e-5 * S, S = sum_k |a_k * b_k|.
  BF16 output: C_out within one BF16 step of C_ref rounded to BF16
               (round to nearest even, straight from float64).

The pages fix neither; both are the stated acceptance bar of this library.
Past K = 8192 the FP32 bar widens with K (fp32_rel_tol): a kernel that adds
one rounded 64-wide MFMA sum per K slice into an fp32 accumulator takes
K/64 roundings in a row, each at most 2^-24 of the running |sum| <= S, so
its worst case is about (K/64 + 2) 2^-24 S, which passes 1e-5 S near
K = 10700.
A reading is added for BF16 (documented with the others): fp32 accumulation
along K is itself rounded, and near cancellation (|C| far below S) that error
can exceed one BF16 step of a tiny |C|. Such an element still passes the
"reading" criterion when it is the BF16 rounding of a value that meets the
FP32 bound: |C_out - C_ref| <= 1e-5 * S + ulp_bf16(C_out) / 2. Tests report
both counts.
"""

import numpy as np

FP32_REL_TOL = 1e-5


def fp32_rel_tol(K):
    """The FP32 bar for a sum over K: max(1e-5, (K/64 + 2) * 2^-24)."""
    return max(FP32_REL_TOL, (K / 64 + 2) * 2.0 ** -24)


def round_to_bf16(c):
    """float64 -> nearest BF16 value (ties to even), returned as float64.

    A BF16 value has 8 significant bits; with c = m * 2**E (0.5 <= |m| < 1)
    its spacing is 2**(E - 8) in the normal range and 2**-133 below 2**-126.
    Scaling by a power of two is exact, and np.rint rounds half to even.
    Results past the BF16 range become +-inf.
    """
    c = np.asarray(c, dtype=np.float64)
    _, E = np.frexp(c)
    q = np.ldexp(1.0, np.maximum(E.astype(np.int64), -125) - 8)
    r = np.rint(c / q) * q
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, c), r)
    return r


def bf16_bits_of(values):
    """BF16 bit patterns of float64 values that are exactly BF16 values."""
    f32 = np.asarray(values, dtype=np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_ordinal(bits):
    """Map BF16 bit patterns to integers whose difference counts BF16 steps.

    +0 and -0 both map to 0; adjacent finite BF16 values differ by 1.
    """
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = bits & 0x7FFF
    return np.where(bits & 0x8000, -mag, mag)


def bf16_ulp(values):
    """Spacing of BF16 values at `values` (the step above |v| in its binade)."""
    v = np.asarray(values, dtype=np.float64)
    _, E = np.frexp(v)
    E = np.where(v == 0, -125, E.astype(np.int64))
    return np.ldexp(1.0, np.maximum(E, -125) - 8)


def check_fp32(c_out, c_ref, s_ref, rel_tol=FP32_REL_TOL):
    """Boolean mask: FP32 output element within rel_tol * S of the oracle."""
    c_out = np.asarray(c_out, dtype=np.float64)
    return np.abs(c_out - c_ref) <= rel_tol * np.asarray(s_ref)


def check_bf16(out_bits, c_ref, s_ref, rel_tol=FP32_REL_TOL):
    """Masks (literal, reading) for BF16 output bits against the oracle.

    literal: at most one BF16 step from round_to_bf16(c_ref).
    reading: literal, or |c_out - c_ref| <= rel_tol * S + ulp_bf16(c_out) / 2.
    """
    out_bits = np.asarray(out_bits, dtype=np.uint16)
    ref_bits = bf16_bits_of(round_to_bf16(c_ref))
    steps = np.abs(bf16_ordinal(out_bits) - bf16_ordinal(ref_bits))
    literal = steps <= 1
    c_out = (out_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    near = np.abs(c_out - c_ref) <= rel_tol * np.asarray(s_ref) + 0.5 * bf16_ulp(c_out)
    return literal, literal | near


def check_act_bf16(act_bits, act_ref, tol):
    """Mask: a BF16 activation output within tol + half a BF16 step of the
    float64 reference (the fused SwiGLU's act, oracle.swiglu)."""
    act_bits = np.asarray(act_bits, dtype=np.uint16)
    got = (act_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.abs(got - act_ref) <= np.asarray(tol) + 0.5 * bf16_ulp(got)
