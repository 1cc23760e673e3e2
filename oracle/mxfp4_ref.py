"""Plain CPU oracle for MXFP4 quantize, dequantize and the block-scaled GEMM.

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import this module. The HIP library never
does, and this module imports nothing from it: the two sides share no code.

Sources, by page title and section:
  * "Integrate MXFP4 hipblaslt GEMM support" (ROCm/TransformerEngine #697),
    'Changes' list: an MXFP4 operand is FP4 E2M1 elements (HIP_R_4F_E2M1) with
    one UE8M0 power-of-two scale per 32 consecutive K elements (VEC32_UE8M0);
    the operands are plain (not shuffled) FP4 data and plain UE8M0 scales; the
    GEMM is TN, output BF16 or FP32, K % 256 == 0, M and N % 32 == 0, no bias,
    beta == 0.
  * "Initial integration of a4w4 GEMM" (ROCm/TransformerEngine #663), review
    comment on the CK call site: the a4w4 GEMM takes the FP4 operands with
    uint8 scale tensors.
  * "feat(ck-tile): aquant GEMM TE to dispatcher bridge" (ROCm/rocm-libraries
    #9980), pk_int4 heap-overflow fix: packed 4-bit data holds two values per
    byte.
  * NVIDIA/TransformerEngine #3809, description: a bidimensional quantize
    writes both the rowwise and the columnwise (transposed) quantized forms
    of one input (quantize_2d below).

The pages never state the numbers of the format. Readings taken here, the
plainest ones consistent with the pages:
  R1  E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; bit 3 of a code is the sign.
  R2  Shared exponent of a 32-element block: e = floor(log2(amax)) - 2, where
      amax is the largest |x| of the block's BF16 values (2 is the exponent of
      the largest E2M1 magnitude, 6 = 1.5 * 2**2). An all-zero block takes
      e = -127. e is clamped to [-127, 127]; the scale byte is e + 127.
  R3  Element code: x * 2**-e rounded to the nearest E2M1 magnitude, ties to
      the even code, magnitudes beyond 6 saturate to 6; the sign bit of x is
      kept, also when the magnitude rounds to 0.
  R4  Two codes per byte: element 2i in bits 3:0, element 2i+1 in bits 7:4.
  R5  Scales row-major [rows, K/32] uint8; B is stored N x K ("TN").
  R6  Dequantized value of code c under scale byte s: E2M1(c) * 2**(s - 127).
Everything is computed in float64, where every step above is exact.
"""

import numpy as np

BLOCK = 32

# R1: the sixteen E2M1 codes; index = code, bit 3 = sign.
E2M1_VALUES = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)
_MAGNITUDES = E2M1_VALUES[:8]

# Rows per chunk so that temporaries stay near a few hundred MB.
_CHUNK_ELEMS = 1 << 21


def bf16_bits_to_f64(bits):
    """Exact value of BF16 bit patterns (uint16 array) as float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def scale_exponent(amax):
    """R2: shared exponent e for block maxima `amax` (float64 array, >= 0).

    floor(log2(amax)) is taken exactly from frexp (amax = m * 2**E with
    0.5 <= m < 1, so floor(log2(amax)) = E - 1), never from a rounded log2.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(amax)
    e = np.where(amax > 0, E.astype(np.int64) - 1 - 2, -127)
    return np.clip(e, -127, 127)


def e2m1_nearest_even(mag):
    """R3: index (0..7) of the E2M1 magnitude nearest to `mag` (float64 >= 0).

    The nearest grid point wins; on an exact tie between two neighbours the
    even index wins. Values past 6 land on index 7 (6.0), which is the
    saturating behaviour, since 6 is the nearest grid point to all of them.
    """
    mag = np.asarray(mag, dtype=np.float64)
    dist = np.abs(mag[..., None] - _MAGNITUDES)
    best = np.argmin(dist, axis=-1)          # first (lower) index on a tie
    dmin = np.take_along_axis(dist, best[..., None], axis=-1)[..., 0]
    upper = np.minimum(best + 1, 7)
    dup = np.take_along_axis(dist, upper[..., None], axis=-1)[..., 0]
    tie = (upper != best) & (dup == dmin)
    # Neighbouring indices differ in parity: on a tie move to the even one.
    return np.where(tie & (best % 2 == 1), upper, best).astype(np.uint8)


def quantize(x_bits):
    """Row-wise BF16 -> MXFP4 (R2-R5).

    x_bits: uint16 [M, K] BF16 bit patterns, K % 32 == 0, finite values.
    Returns (codes uint8 [M, K/2], scales uint8 [M, K/32]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    codes = np.empty((M, K // 2), dtype=np.uint8)
    scales = np.empty((M, K // BLOCK), dtype=np.uint8)
    step = max(1, _CHUNK_ELEMS // max(K, 1))
    for r0 in range(0, M, step):
        r1 = min(M, r0 + step)
        x = bf16_bits_to_f64(x_bits[r0:r1]).reshape(r1 - r0, K // BLOCK, BLOCK)
        amax = np.abs(x).max(axis=2)
        e = scale_exponent(amax)
        scales[r0:r1] = (e + 127).astype(np.uint8)
        v = np.ldexp(x, -e[..., None])                     # exact
        mag = e2m1_nearest_even(np.abs(v))
        code = mag | (np.signbit(x).astype(np.uint8) << 3)
        code = code.reshape(r1 - r0, K)
        codes[r0:r1] = code[:, 0::2] | (code[:, 1::2] << 4)  # R4
    return codes, scales


def quantize_2d(x_bits):
    """Rowwise and columnwise MXFP4 of X [M, K] (BF16 bits): the rowwise form
    of X and the rowwise form of X^T, i.e. blocks of 32 consecutive rows of
    each column (R2-R5 applied to X^T). M and K must be multiples of 32.

    Returns (codes [M, K/2], scales [M, K/32], codes_t [K, M/2], scales_t
    [K, M/32]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    codes, scales = quantize(x_bits)
    codes_t, scales_t = quantize(np.ascontiguousarray(x_bits.T))
    return codes, scales, codes_t, scales_t


def unpack_codes(codes):
    """R4: uint8 [rows, K/2] packed codes -> uint8 [rows, K] codes."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def dequantize(codes, scales):
    """R6: packed codes [rows, K/2] + scales [rows, K/32] -> float64 [rows, K]."""
    c = unpack_codes(codes)
    rows, K = c.shape
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape != (rows, K // BLOCK):
        raise ValueError("scale tensor shape does not match the codes")
    vals = E2M1_VALUES[c].reshape(rows, K // BLOCK, BLOCK)
    exps = scales.astype(np.int64)[..., None] - 127
    return np.ldexp(vals, exps).reshape(rows, K)


def gemm_block(A_codes, A_scales, B_codes, B_scales, m_rows=None, n_rows=None):
    """C and S on the rows m_rows of A and rows n_rows of B (all if None).

    C[i, j] = sum_k dq(A)[m_i, k] * dq(B)[n_j, k]      (TN: B is N x K)
    S[i, j] = sum_k |dq(A)[m_i, k] * dq(B)[n_j, k]|    (the tolerance scale)
    Both float64, through a BLAS matmul of the dequantized operands.
    """
    A_codes = np.asarray(A_codes)
    B_codes = np.asarray(B_codes)
    A_scales = np.asarray(A_scales)
    B_scales = np.asarray(B_scales)
    if m_rows is not None:
        A_codes, A_scales = A_codes[m_rows], A_scales[m_rows]
    if n_rows is not None:
        B_codes, B_scales = B_codes[n_rows], B_scales[n_rows]
    a = dequantize(A_codes, A_scales)
    b = dequantize(B_codes, B_scales)
    if a.shape[1] != b.shape[1]:
        raise ValueError("A and B disagree on K")
    C = a @ b.T
    S = np.abs(a) @ np.abs(b).T
    return C, S


def gemm(A_codes, A_scales, B_codes, B_scales):
    """Full C, S (float64 [M, N]) for small problems."""
    return gemm_block(A_codes, A_scales, B_codes, B_scales)


def gemm_entries(A_codes, A_scales, B_codes, B_scales, m_idx, n_idx):
    """C and S at the index pairs (m_idx[t], n_idx[t]) only, as float64 [T]."""
    m_idx = np.asarray(m_idx)
    n_idx = np.asarray(n_idx)
    a = dequantize(np.asarray(A_codes)[m_idx], np.asarray(A_scales)[m_idx])
    b = dequantize(np.asarray(B_codes)[n_idx], np.asarray(B_scales)[n_idx])
    prod = a * b
    return prod.sum(axis=1), np.abs(prod).sum(axis=1)
