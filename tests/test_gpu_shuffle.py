"""GPU parity of the weight pre-shuffle and of the GEMM on pre-shuffled B.

The shuffle is a byte permutation with zero padding (readings P1-P2 of
oracle/shuffle.py): bit-exact with the oracle. The GEMM on shuffled B runs
the same tile kernel and MFMA sequence as the GEMM on plain B, so for
M > 128 its output must equal mxfp4_gemm's bit for bit; against the oracle
it meets the GEMM tolerance (R9/R10).
"""

import numpy as np
import pytest
import torch

import block_scaled_microscaling_amd as mx
import oracle
from gpu_helpers import DEV, announce, bf16_to_dev, check_gemm_output, u8_to_dev


pytestmark = pytest.mark.gpu


def _random_operand(rows, K, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(118, 128, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("N,K", [(256, 256), (300, 1280), (32, 768), (544, 2048), (8192, 1024)])
def test_shuffle_bit_exact(N, K):
    announce(f"shuffle_b {N}x{K}")
    codes, scales = _random_operand(N, K, N + K)
    cs, ss = mx.shuffle_b(u8_to_dev(codes), u8_to_dev(scales))
    torch.cuda.synchronize()
    rc, rs = oracle.shuffle_b(codes, scales)
    assert np.array_equal(cs.cpu().numpy(), rc)
    assert np.array_equal(ss.cpu().numpy(), rs)


def test_shuffle_writes_exactly_its_buffers():
    announce("shuffle_b canary")
    N, K = 300, 1280
    codes, scales = _random_operand(N, K, 3)
    rc_, cb, sb = mx.mxfp4_shuffle_b_sizes(N, K)
    pad = 4096
    cbuf = torch.full((cb + 2 * pad,), 0xAB, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((sb + 2 * pad,), 0xCD, dtype=torch.uint8, device=DEV)
    c_d, s_d = u8_to_dev(codes), u8_to_dev(scales)
    assert mx.mxfp4_shuffle_b(c_d.data_ptr(), s_d.data_ptr(), N, K, cbuf.data_ptr() + pad,
                              sbuf.data_ptr() + pad, None) == 0
    torch.cuda.synchronize()
    c, s = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(c[:pad] == 0xAB) and np.all(c[-pad:] == 0xAB)
    assert np.all(s[:pad] == 0xCD) and np.all(s[-pad:] == 0xCD)
    rc, rs = oracle.shuffle_b(codes, scales)
    assert np.array_equal(c[pad:-pad], rc) and np.array_equal(s[pad:-pad], rs)


@pytest.mark.parametrize("M,N,K,out", [
    (256, 256, 256, torch.float32),
    (288, 544, 1280, torch.bfloat16),   # ragged tiles, K % 1024 != 0
    (512, 288, 2048, torch.float32),    # N = 288: a partial B tile
    (64, 256, 1024, torch.bfloat16),    # M <= 128 on the tile kernel
])
def test_shuffled_gemm_matches_oracle(M, N, K, out):
    announce(f"gemm_bshuffled {M}x{N}x{K} {out}")
    a_c, a_s = _random_operand(M, K, M * 3 + K)
    b_c, b_s = _random_operand(N, K, N * 5 + K)
    bc, bs = mx.shuffle_b(u8_to_dev(b_c), u8_to_dev(b_s))
    got = mx.gemm_bshuffled(u8_to_dev(a_c), u8_to_dev(a_s), bc, bs, N, out_dtype=out)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.gemm(a_c, a_s, b_c, b_s)
    check_gemm_output(got, c_ref, s_ref)


@pytest.mark.parametrize("M,N,K", [(512, 768, 2048), (288, 544, 1280)])
def test_shuffled_gemm_equals_plain_gemm(M, N, K):
    """Same tile kernel (mxfp4_gemm_tile), same MFMA order: identical bits."""
    announce(f"gemm_bshuffled == gemm_tile {M}x{N}x{K}")
    a_c, a_s = _random_operand(M, K, 11)
    b_c, b_s = _random_operand(N, K, 12)
    A, As_, B, Bs = (u8_to_dev(t) for t in (a_c, a_s, b_c, b_s))
    bc, bs = mx.shuffle_b(B, Bs)
    for dt in (torch.float32, torch.bfloat16):
        plain = mx.gemm_tile(A, As_, B, Bs, out_dtype=dt)
        shuf = mx.gemm_bshuffled(A, As_, bc, bs, N, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(plain, shuf)
