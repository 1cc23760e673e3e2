"""Plain CPU oracle for the fragment-order MXFP4 layout of the skinny GEMM.

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import this module. The HIP library never
does, and this module imports nothing from it: the two sides share no code.

Source: the a4w4 path of "Integrate MXFP4 hipblaslt GEMM support"
(ROCm/TransformerEngine #697, Changes list) and the call site reviewed on
"Initial integration of a4w4 GEMM" (#663) feed the GEMM operands re-arranged
ahead of time (B_shuffled, swizzled scales) so that it loads them without
address arithmetic. The pages give no layout. This one is this library's own
(reading F1): the order in which a GEMM that keeps its operands in registers
consumes them, so that each block-scaled MFMA operand is one contiguous run.

Reading F1. X is an MXFP4 operand of R rows and K columns (codes [R, K/2],
scales [R, K/32], R % 32 == 0, K % 256 == 0). Cut it into tiles of 32 rows
(t) and steps of 256 K (s, KS = K / 256 steps; 8 blocks of 32 elements per
row per step). Write h in {0, 1}, q in {0..3} and l = r + 32 h for a "lane"
l in 0..63 holding row r of the tile.
  Codes: tile t, step s is one 4096-byte block at byte (t KS + s) 4096. Its
    byte 1024 q + 16 l + c (c < 16) is code byte 16 (4 h + q) + c of row
    32 t + r in step s, i.e. codes[32 t + r, 128 s + 16 (4 h + q) + c]:
    block 4 h + q of the step, whole.
  Scales: tile t, step s is one 256-byte block at byte (t KS + s) 256. Its
    byte 4 l + q is the scale of block 4 h + q of row 32 t + r in step s,
    i.e. scales[32 t + r, 8 s + 4 h + q].
Both are permutations of the plain bytes (no padding, same sizes); from_frag
inverts them.
"""

import numpy as np

TILE = 32
STEP_K = 256


def _check(R, K):
    if R % TILE or K % STEP_K or R <= 0 or K <= 0:
        raise ValueError("fragment order needs R % 32 == 0 and K % 256 == 0")


def _code_source(R, K):
    """F1 codes: for every fragment-order byte, the (row, byte column) it holds."""
    ks = K // STEP_K
    off = np.arange(R * K // 2, dtype=np.int64)
    blk, inb = off // 4096, off % 4096
    t, s = blk // ks, blk % ks
    q, l, c = inb // 1024, (inb % 1024) // 16, inb % 16
    r, h = l % 32, l // 32
    return TILE * t + r, 128 * s + 16 * (4 * h + q) + c


def _scale_source(R, K):
    """F1 scales: for every fragment-order byte, the (row, scale column) it holds."""
    ks = K // STEP_K
    off = np.arange(R * K // 32, dtype=np.int64)
    blk, inb = off // 256, off % 256
    t, s = blk // ks, blk % ks
    l, q = inb // 4, inb % 4
    r, h = l % 32, l // 32
    return TILE * t + r, 8 * s + 4 * h + q


def to_frag(codes, scales):
    """Plain codes [R, K/2] and scales [R, K/32] (uint8) -> F1 codes and scales
    as flat uint8 arrays of the same sizes."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, Kh = codes.shape
    K = 2 * Kh
    _check(R, K)
    if scales.shape != (R, K // 32):
        raise ValueError("scales must be [R, K/32]")
    row, col = _code_source(R, K)
    out_c = codes[row, col]
    row, col = _scale_source(R, K)
    out_s = scales[row, col]
    return out_c, out_s


def from_frag(codes_f, scales_f, R, K):
    """Inverse of to_frag: F1 flat bytes -> plain codes [R, K/2], scales [R, K/32]."""
    _check(R, K)
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    row, col = _code_source(R, K)
    codes[row, col] = np.asarray(codes_f, dtype=np.uint8)
    scales = np.zeros((R, K // 32), dtype=np.uint8)
    row, col = _scale_source(R, K)
    scales[row, col] = np.asarray(scales_f, dtype=np.uint8)
    return codes, scales
