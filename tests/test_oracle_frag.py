"""Pins of the fragment-order layout (oracle/frag.py, reading F1).

The layout is this library's own definition (the pages name pre-arranged
weights and swizzled scales without giving a layout), so it is pinned by
hand-worked byte positions, bijection and round-trip checks, and a GEMM
computed by walking the fragments the way the block-scaled MFMA pairs them,
compared with the plain-definition GEMM.
"""

import numpy as np
import pytest

import oracle


def test_hand_worked_code_position():
    """R = 64, K = 512: codes[45, 200] -> tile 1, r = 13; byte column 200 is
    step 1, byte 72 of the step = block 4 (h = 1, q = 0), byte 8 of it; lane
    13 + 32 = 45: (1*2 + 1)*4096 + 1024*0 + 16*45 + 8 = 13016."""
    codes = np.zeros((64, 256), dtype=np.uint8)
    scales = np.zeros((64, 16), dtype=np.uint8)
    codes[45, 200] = 0x5A
    cf, sf = oracle.to_frag(codes, scales)
    assert np.flatnonzero(cf).tolist() == [13016]
    assert cf[13016] == 0x5A and not sf.any()


def test_hand_worked_scale_position():
    """R = 64, K = 512: scales[33, 13] -> tile 1, r = 1; column 13 is step 1,
    block 5 (h = 1, q = 1); lane 33: (1*2 + 1)*256 + 4*33 + 1 = 901."""
    codes = np.zeros((64, 256), dtype=np.uint8)
    scales = np.zeros((64, 16), dtype=np.uint8)
    scales[33, 13] = 0x81
    _, sf = oracle.to_frag(codes, scales)
    assert np.flatnonzero(sf).tolist() == [901]


def test_lane_word_is_four_consecutive_scales():
    """The 4-byte word of lane l in a step holds the row's scale bytes
    4h..4h+3 of that step, in order (one dword per lane, byte q picked by the
    MFMA's scale byte select)."""
    R, K = 32, 256
    scales = np.arange(R * K // 32, dtype=np.uint8).reshape(R, K // 32)
    _, sf = oracle.to_frag(np.zeros((R, K // 2), np.uint8), scales)
    words = sf.reshape(64, 4)
    for l in range(64):
        r, h = l % 32, l // 32
        assert words[l].tolist() == scales[r, 4 * h:4 * h + 4].tolist()


@pytest.mark.parametrize("R,K", [(32, 256), (64, 512), (96, 768), (128, 8192), (32, 2560)])
def test_round_trip_and_bijection(R, K):
    rng = np.random.default_rng(R * 7 + K)
    codes = rng.integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(R, K // 32), dtype=np.uint8)
    cf, sf = oracle.to_frag(codes, scales)
    assert cf.shape == (R * K // 2,) and sf.shape == (R * K // 32,)
    c2, s2 = oracle.from_frag(cf, sf, R, K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # A permutation: distinct plain positions map to distinct fragment bytes.
    ident = np.arange(R * K // 2, dtype=np.int64).reshape(R, K // 2)
    row, col = oracle.frag._code_source(R, K)
    assert np.array_equal(np.sort(ident[row, col]), np.arange(R * K // 2))
    ident = np.arange(R * K // 32, dtype=np.int64).reshape(R, K // 32)
    row, col = oracle.frag._scale_source(R, K)
    assert np.array_equal(np.sort(ident[row, col]), np.arange(R * K // 32))


def test_rejects_unsupported_shapes():
    with pytest.raises(ValueError):
        oracle.to_frag(np.zeros((33, 128), np.uint8), np.zeros((33, 8), np.uint8))
    with pytest.raises(ValueError):
        oracle.to_frag(np.zeros((32, 64), np.uint8), np.zeros((32, 4), np.uint8))


def _frag_values(cf, sf, R, K):
    """Dequantized fragment-order operand as [tile, step, q, lane, 32] fp64."""
    ks = K // 256
    lo = cf & 0x0F
    hi = cf >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(R // 32, ks, 4, 64, 32)
    val = oracle.E2M1_VALUES[nib]
    sc = np.ldexp(1.0, sf.astype(np.int64) - 127).reshape(R // 32, ks, 64, 4)
    return val * np.moveaxis(sc, 3, 2)[..., None]


def test_gemm_by_mfma_pairing_equals_plain_gemm():
    """C computed the way the GEMM consumes fragments: per step s and slice q,
    lane (r, h) of A and lane (r', h) of B hold the same K block 4h + q, so
    C[32 ta + r, 32 tb + r'] = sum over s, q, h of the dot product of those two
    32-element blocks. Small integer codes and scales near 127 keep every sum
    exact, so it must equal oracle.gemm bit for bit."""
    rng = np.random.default_rng(5)
    M, N, K = 64, 96, 768
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    as_ = rng.integers(124, 131, size=(M, K // 32), dtype=np.uint8)
    bs = rng.integers(124, 131, size=(N, K // 32), dtype=np.uint8)
    c_ref, _ = oracle.gemm(ac, as_, bc, bs)
    fa = _frag_values(*oracle.to_frag(ac, as_), M, K)
    fb = _frag_values(*oracle.to_frag(bc, bs), N, K)
    c = np.zeros((M, N))
    for ta in range(M // 32):
        for tb in range(N // 32):
            for h in range(2):
                xa = fa[ta, :, :, 32 * h:32 * h + 32, :]   # [ks, q, r, 32]
                xb = fb[tb, :, :, 32 * h:32 * h + 32, :]
                c[32 * ta:32 * ta + 32, 32 * tb:32 * tb + 32] += np.einsum(
                    "sqre,sqte->rt", xa, xb)
    assert np.array_equal(c, c_ref)
