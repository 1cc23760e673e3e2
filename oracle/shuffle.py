"""Plain CPU oracle for the pre-shuffled MXFP4 weight layout.

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import this module. The HIP library never
does, and this module imports nothing from it: the two sides share no code.

Source: the AITER a4w4 path of "Integrate MXFP4 hipblaslt GEMM support"
(ROCm/TransformerEngine #697, Changes list) and the a4w4 call site reviewed on
"Initial integration of a4w4 GEMM" (#663) take the weight as B_shuffled with
swizzled UE8M0 scales: a one-time re-arrangement of the weight so that the
GEMM loads it without address arithmetic. The pages name the idea but not a
layout; the layout below is this library's own (reading P1), chosen to be
the byte order in which its tile GEMM consumes B.

Readings:
  P1  Codes. B is cut into tiles of 256 rows (n) and steps of 256 K (128 code
      bytes per row). Tile nt, step ks is one 32 KiB block at byte offset
      (nt * KS + ks) * 32768, KS = K / 256, tiles in order of nt. Inside a
      block, row x (0..255) takes bytes x * 128 .. x * 128 + 127 as eight
      16-byte chunks; physical chunk p holds the row's logical chunk
      p ^ swz(x), swz(x) = (x & 6) | ((x ^ (x >> 3)) & 1) (an XOR on the low
      four bits of x). Logical chunk c of row x is codes[256 nt + x,
      128 ks + 16 c .. + 15]. Rows at or past N are zero.
  P2  Scales. Steps of 1024 K (eight "half-steps" of 128 K; a half-step of a
      row is one 4-byte word: the row's four scale bytes of those 128 K, in
      order). Tile nt, chunk ch is one 8 KiB block at byte offset
      (nt * NC + ch) * 8192, NC = ceil(K / 1024). Inside a block the word of
      row x = 128 h + 32 t + r (h < 2, t < 4, r < 32) and half-step s lies at
      byte 128 (32 h + r) + 16 (s ^ ((r >> 1) & 7)) + 4 t. Rows at or past N
      and half-steps past K / 128 are zero.
Both are permutations of the plain bytes plus zero padding; unshuffle_b
inverts them.
"""

import numpy as np

TILE_N = 256
STEP_K = 256
CHUNK_K = 1024
CODE_BLOCK = TILE_N * STEP_K // 2       # 32768 bytes
SCALE_BLOCK = TILE_N * (CHUNK_K // 32)  # 8192 bytes


def chunk_swizzle(x):
    """P1: swz(x) for row index x (int or array)."""
    x = np.asarray(x)
    return (x & 6) | ((x ^ (x >> 3)) & 1)


def shuffled_sizes(N, K):
    """Bytes of the shuffled codes and scales of a [N, K] MXFP4 operand."""
    nt = -(-N // TILE_N)
    return nt * (K // STEP_K) * CODE_BLOCK, nt * (-(-K // CHUNK_K)) * SCALE_BLOCK


def _code_index(N, K):
    """For every shuffled code byte: (row, byte column) of its source, or row
    -1 for padding. Arrays of length shuffled_sizes(N, K)[0]."""
    nt_n, ks_n = -(-N // TILE_N), K // STEP_K
    off = np.arange(nt_n * ks_n * CODE_BLOCK, dtype=np.int64)
    blk, inb = off // CODE_BLOCK, off % CODE_BLOCK
    nt, ks = blk // ks_n, blk % ks_n
    x, p, c = inb // 128, (inb % 128) // 16, inb % 16
    row = TILE_N * nt + x
    col = 128 * ks + 16 * (p ^ chunk_swizzle(x)) + c
    return np.where(row < N, row, -1), col


def _scale_index(N, K):
    """For every shuffled scale byte: (row, scale column) of its source, or
    row -1 for padding (past N or past K)."""
    nt_n, nc = -(-N // TILE_N), -(-K // CHUNK_K)
    off = np.arange(nt_n * nc * SCALE_BLOCK, dtype=np.int64)
    blk, inb = off // SCALE_BLOCK, off % SCALE_BLOCK
    nt, ch = blk // nc, blk % nc
    hr, rest = inb // 128, inb % 128            # hr = 32 h + r
    h, r = hr // 32, hr % 32
    sp, t, byte = rest // 16, (rest % 16) // 4, rest % 4
    s = sp ^ ((r >> 1) & 7)
    row = TILE_N * nt + 128 * h + 32 * t + r
    col = 4 * (8 * ch + s) + byte                # scale column: 4 per half-step
    ok = (row < N) & (col < K // 32)
    return np.where(ok, row, -1), col


def shuffle_b(codes, scales):
    """Plain codes [N, K/2] and scales [N, K/32] (uint8) -> shuffled (P1, P2)
    codes and scales as flat uint8 arrays."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N, Kh = codes.shape
    K = 2 * Kh
    if K % STEP_K or scales.shape != (N, K // 32):
        raise ValueError("need K % 256 == 0 and scales [N, K/32]")
    row, col = _code_index(N, K)
    out_c = np.zeros(row.shape, dtype=np.uint8)
    ok = row >= 0
    out_c[ok] = codes[row[ok], col[ok]]
    row, col = _scale_index(N, K)
    out_s = np.zeros(row.shape, dtype=np.uint8)
    ok = row >= 0
    out_s[ok] = scales[row[ok], col[ok]]
    return out_c, out_s


def unshuffle_b(codes_sh, scales_sh, N, K):
    """Inverse of shuffle_b: back to plain codes [N, K/2] and scales [N, K/32]."""
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    row, col = _code_index(N, K)
    ok = row >= 0
    codes[row[ok], col[ok]] = np.asarray(codes_sh, dtype=np.uint8)[ok]
    scales = np.zeros((N, K // 32), dtype=np.uint8)
    row, col = _scale_index(N, K)
    ok = row >= 0
    scales[row[ok], col[ok]] = np.asarray(scales_sh, dtype=np.uint8)[ok]
    return codes, scales
