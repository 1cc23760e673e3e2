"""GPU parity of the fragment-order path: quantize into fragment order, the
re-layout of plain MXFP4 bytes, and the register-ring GEMM reading both
operands in that order (reading F1 of oracle/frag.py).

Quantize and re-layout are byte work: bit-exact with the oracle. The GEMM
runs the same K order, MFMA sequence and reduction as mxfp4_gemm's M <= 128
kernel, so for M <= 128 it must return identical bits; against the oracle it
meets the GEMM tolerance (FP32 within 1e-5 * sum|a*b|, BF16 within one BF16
step of the rounded oracle).
"""

import numpy as np
import pytest
import torch

import block_scaled_microscaling_amd as mx
import oracle
from gpu_helpers import DEV, announce, bf16_to_dev, check_gemm_output, sample_pairs, u8_to_dev
from synth import WORKLOADS, bf16_matrix

pytestmark = pytest.mark.gpu


def _random_operand(rows, K, seed, lo=118, hi=128):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("M,K", [(32, 256), (64, 768), (96, 8192), (128, 2560), (160, 1024)])
def test_quantize_frag_bit_exact(M, K):
    announce(f"quantize_frag {M}x{K}")
    bits = bf16_matrix((M, K), ("normal", 1.0, 0.01, 100.0), M * 3 + K)
    cf, sf = mx.quantize_frag(bf16_to_dev(bits))
    torch.cuda.synchronize()
    rc, rs = oracle.to_frag(*oracle.quantize(bits))
    assert np.array_equal(cf.cpu().numpy(), rc)
    assert np.array_equal(sf.cpu().numpy(), rs)


def test_quantize_frag_special_blocks():
    """Zero blocks, -0.0, subnormal and largest-BF16 blocks, saturating and
    tie values: every decision of the quantize, in fragment order."""
    M, K = 32, 512
    announce(f"quantize_frag special blocks {M}x{K}")
    rng = np.random.default_rng(77)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 32:64] = -0.0
    x[2, 64:96] = np.float32(1.5 * 2.0 ** -126) * rng.standard_normal(32).astype(np.float32)
    x[3, 96:128] = np.float32(3.0e38) * np.sign(rng.standard_normal(32)).astype(np.float32)
    x[4, :32] = np.array([6, -6, 3, -3, 1.5, .5, 0, -0, 4, 2, 1, -1, .25, .75, 1.25, 1.75,
                          2.5, 3.5, 5, -5, .125, -.125, 5.5, -2.5, -.25, -.75, 4.5, 2.75,
                          .375, -1.625, 3.875, -4.125], dtype=np.float32)
    x[5, 256:288] = 7.9375
    from synth import f32_to_bf16_bits
    bits = f32_to_bf16_bits(x)
    cf, sf = mx.quantize_frag(bf16_to_dev(bits))
    torch.cuda.synchronize()
    rc, rs = oracle.to_frag(*oracle.quantize(bits))
    assert np.array_equal(cf.cpu().numpy(), rc)
    assert np.array_equal(sf.cpu().numpy(), rs)


def test_quantize_frag_ragged_workload_activation():
    """The ragged workload's activation X [4128, 7936] (Laplace(0, 1)): 129
    row tiles, 31 K steps."""
    w = WORKLOADS["ragged"]
    announce(f"quantize_frag {w.M}x{w.K}")
    bits = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    cf, sf = mx.quantize_frag(bf16_to_dev(bits))
    torch.cuda.synchronize()
    rc, rs = oracle.to_frag(*oracle.quantize(bits))
    assert np.array_equal(cf.cpu().numpy(), rc)
    assert np.array_equal(sf.cpu().numpy(), rs)


def test_frag_entries_write_exactly_their_buffers():
    announce("quantize_frag / to_frag canary")
    M, K, pad = 64, 512, 4096
    bits = bf16_matrix((M, K), ("normal", 1.0, 0.0, 1.0), 9)
    x = bf16_to_dev(bits)
    cbuf = torch.full((M * K // 2 + 2 * pad,), 0xAB, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((M * K // 32 + 2 * pad,), 0xCD, dtype=torch.uint8, device=DEV)
    assert mx.mxfp4_quantize_frag(x.data_ptr(), M, K, cbuf.data_ptr() + pad,
                                  sbuf.data_ptr() + pad, None) == 0
    torch.cuda.synchronize()
    c, s = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (c[:pad] == 0xAB).all() and (c[-pad:] == 0xAB).all()
    assert (s[:pad] == 0xCD).all() and (s[-pad:] == 0xCD).all()
    rc, rs = oracle.to_frag(*oracle.quantize(bits))
    assert np.array_equal(c[pad:-pad], rc) and np.array_equal(s[pad:-pad], rs)
    codes, scales = _random_operand(M, K, 4)
    cbuf.fill_(0xAB)
    sbuf.fill_(0xCD)
    c_d, s_d = u8_to_dev(codes), u8_to_dev(scales)
    assert mx.mxfp4_to_frag(c_d.data_ptr(), s_d.data_ptr(), M, K, cbuf.data_ptr() + pad,
                            sbuf.data_ptr() + pad, None) == 0
    torch.cuda.synchronize()
    c, s = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (c[:pad] == 0xAB).all() and (c[-pad:] == 0xAB).all()
    assert (s[:pad] == 0xCD).all() and (s[-pad:] == 0xCD).all()
    rc, rs = oracle.to_frag(codes, scales)
    assert np.array_equal(c[pad:-pad], rc) and np.array_equal(s[pad:-pad], rs)


@pytest.mark.parametrize("R,K", [(32, 256), (96, 2304), (8192, 1024), (320, 7936)])
def test_to_frag_bit_exact(R, K):
    announce(f"to_frag {R}x{K}")
    codes, scales = _random_operand(R, K, R + K, 0, 256)
    cf, sf = mx.to_frag(u8_to_dev(codes), u8_to_dev(scales))
    torch.cuda.synchronize()
    rc, rs = oracle.to_frag(codes, scales)
    assert np.array_equal(cf.cpu().numpy(), rc)
    assert np.array_equal(sf.cpu().numpy(), rs)


# K = 256 leaves 7 of the 8 waves without a step, 2304 gives waves 0 and 1 a
# second step, 8192 four steps each (the register ring's depth), 14336 seven
# (a full round of four plus a remainder).
@pytest.mark.parametrize("M,N,K", [(32, 64, 256), (32, 256, 2304), (64, 96, 8192),
                                   (128, 160, 768), (32, 128, 14336), (96, 8192, 1024)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_frag_equals_gemm_and_oracle(M, N, K, out_dtype):
    announce(f"gemm_frag {M}x{N}x{K} {out_dtype}")
    ac, as_ = _random_operand(M, K, 11 + M)
    bc, bs = _random_operand(N, K, 13 + N)
    ac_d, as_d, bc_d, bs_d = (u8_to_dev(t) for t in (ac, as_, bc, bs))
    plain = mx.gemm(ac_d, as_d, bc_d, bs_d, out_dtype=out_dtype)
    af, asf = mx.to_frag(ac_d, as_d)
    bf, bsf = mx.to_frag(bc_d, bs_d)
    got = mx.gemm_frag(af, asf, bf, bsf, M, N, K, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32 if out_dtype == torch.float32 else torch.int16),
                       plain.view(torch.int32 if out_dtype == torch.float32 else torch.int16))
    if M * N * K <= 64 * 96 * 8192:
        c_ref, s_ref = oracle.gemm(ac, as_, bc, bs)
        check_gemm_output(got, c_ref, s_ref)
    else:
        m_idx, n_idx = sample_pairs(M, N, 1500, seed=K)
        c_ref, s_ref = oracle.gemm_entries(ac, as_, bc, bs, m_idx, n_idx)
        check_gemm_output(got[torch.from_numpy(m_idx).to(DEV), torch.from_numpy(n_idx).to(DEV)],
                          c_ref, s_ref)


@pytest.mark.parametrize("M", [160, 224, 320])
def test_gemm_frag_many_row_tiles(M):
    """Past the 128 rows mxfp4_gemm sends to this arithmetic, against the
    oracle only: 5 row tiles run as groups of 3 + 2 (two launches), 7 as
    3 + 2 + 2, 10 as 3 + 3 + 2 + 2."""
    N, K = 96, 512
    announce(f"gemm_frag {M}x{N}x{K}")
    ac, as_ = _random_operand(M, K, 21)
    bc, bs = _random_operand(N, K, 22)
    af, asf = oracle.to_frag(ac, as_)
    bf, bsf = oracle.to_frag(bc, bs)
    got = mx.gemm_frag(u8_to_dev(af), u8_to_dev(asf), u8_to_dev(bf), u8_to_dev(bsf), M, N, K,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.gemm(ac, as_, bc, bs)
    check_gemm_output(got, c_ref, s_ref)


def test_gemm_frag_output_written_exactly_in_bounds():
    announce("gemm_frag output canary")
    M, N, K, pad = 32, 64, 512, 1024
    ac, as_ = _random_operand(M, K, 31)
    bc, bs = _random_operand(N, K, 32)
    af, asf = (u8_to_dev(t) for t in oracle.to_frag(ac, as_))
    bf, bsf = (u8_to_dev(t) for t in oracle.to_frag(bc, bs))
    buf = torch.full((M * N + 2 * pad,), -7.0, dtype=torch.float32, device=DEV)
    assert mx.mxfp4_gemm_frag(af.data_ptr(), asf.data_ptr(), bf.data_ptr(), bsf.data_ptr(), M, N,
                              K, mx.OUT_FP32, buf.data_ptr() + 4 * pad, None) == 0
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[:pad] == -7.0).all() and (host[-pad:] == -7.0).all()
    c_ref, s_ref = oracle.gemm(ac, as_, bc, bs)
    check_gemm_output(buf[pad:-pad].view(M, N), c_ref, s_ref)


@pytest.mark.parametrize("name", ["skinny", "decode128"])
def test_skinny_workload_full_size_pipeline(name):
    """The decode-shaped workloads (32 or 128 x 8192 x 8192, BF16 out)
    through the fragment path: activation quantized into fragment order per
    call, the weight quantized row-major then re-laid out. Equal bit for bit
    to quantize + mxfp4_gemm on the same inputs, and within tolerance of the
    oracle at every output."""
    w = WORKLOADS[name]
    announce(f"fragment pipeline {w.M}x{w.N}x{w.K}, full C")
    a_bits = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    b_bits = bf16_matrix((w.N, w.K), w.b_dist, w.b_seed)
    x, wt = bf16_to_dev(a_bits), bf16_to_dev(b_bits)
    bc, bs = mx.quantize(wt)
    bf, bsf = mx.to_frag(bc, bs)
    af, asf = mx.quantize_frag(x)
    got = mx.gemm_frag(af, asf, bf, bsf, w.M, w.N, w.K)
    ac, as_ = mx.quantize(x)
    plain = mx.gemm(ac, as_, bc, bs)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), plain.view(torch.int16))
    ra_c, ra_s = oracle.quantize(a_bits)
    rb_c, rb_s = oracle.quantize(b_bits)
    assert np.array_equal(af.cpu().numpy(), oracle.to_frag(ra_c, ra_s)[0])
    c_ref, s_ref = oracle.gemm(ra_c, ra_s, rb_c, rb_s)
    check_gemm_output(got, c_ref, s_ref)
