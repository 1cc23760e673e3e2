"""GPU parity at sizes whose byte offsets pass 2^31 and 2^32.

Operations: the row-wise and bidimensional quantize, round to nearest and
stochastic, and the FP4 x FP4 GEMM ("Initial integration of a4w4 GEMM",
ROCm/TransformerEngine #663; gates of "Integrate MXFP4 hipblaslt GEMM
support", #697, Changes list) with its fused SwiGLU epilogue, whose contract
admits every buffer under 2^40 bytes. Each kernel forms 64-bit row bases and
32-bit offsets within a tile; these cases put checked rows on both sides of
the 2^31- and 2^32-byte marks of the quantize input, of A's and B's codes, of
C and of the BF16 activation, on the tile, split-K, pre-shuffled,
fragment-order and fused SwiGLU paths.

Operands of gigabytes are drawn on the GPU by torch's seeded generator
(synth.device_random_bytes, synth.device_normal_bf16); the rows and columns
the oracle checks are copied back. Quantize outputs are compared bit for
bit, GEMM outputs within the tolerances of oracle/compare.py.
"""

import numpy as np
import pytest
import torch

import block_scaled_microscaling_amd as mx
import oracle
from gpu_helpers import DEV, announce, bf16_bits_of_tensor, check_gemm_output
from synth import device_normal_bf16, device_random_bytes

pytestmark = pytest.mark.gpu

K = 1024          # 512 code bytes and 32 scale bytes per row
BIG = 5 << 20     # rows of a 2.5 GiB code array at K = 1024 (row 2^22 starts at 2^31 B)


def _sample(n, seed, count=48):
    """Row indexes: both ends, both sides of rows 2^20 .. 2^23 (the 2^31 and
    2^32 byte marks of the arrays here), and `count` random rows."""
    rng = np.random.default_rng(seed)
    pts = [0, 1, n - 2, n - 1]
    for b in (1 << 20, 1 << 21, 1 << 22, 1 << 23):
        if b < n:
            pts += [b - 1, b]
    pts += rng.integers(0, n, size=count).tolist()
    return np.unique(np.array(pts, dtype=np.int64))


def _rows(t, idx):
    return t[torch.from_numpy(idx).to(DEV)].cpu().numpy()


def _operand(rows, seed):
    return (device_random_bytes((rows, K // 2), seed),
            device_random_bytes((rows, K // 32), seed + 1, lo=118, hi=134))


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_quantize_input_past_4gib():
    """X [2^21 + 96, 1024] BF16 (4 GiB + 192 KiB): row-wise quantize and both
    outputs of the bidimensional quantize against the oracle on sampled rows
    (past 2^31 and 2^32 bytes of X) and on whole sampled columns."""
    M = (1 << 21) + 96
    announce(f"quantize past 4 GiB: X [{M}, {K}]")
    x = device_normal_bf16((M, K), 5001)
    codes, scales = mx.quantize(x)
    cr, sr, cc, sc = mx.quantize_2d(x)
    torch.cuda.synchronize()
    rows = _sample(M, 5002)
    want_c, want_s = oracle.quantize(bf16_bits_of_tensor(x[torch.from_numpy(rows).to(DEV)]))
    for got_c, got_s in ((codes, scales), (cr, sr)):
        assert np.array_equal(_rows(got_c, rows), want_c)
        assert np.array_equal(_rows(got_s, rows), want_s)
    cols = np.array([0, 1, 517, K - 1], dtype=np.int64)
    xt = x[:, torch.from_numpy(cols).to(DEV)].t().contiguous()
    want_c, want_s = oracle.quantize(bf16_bits_of_tensor(xt))
    assert np.array_equal(_rows(cc, cols), want_c)
    assert np.array_equal(_rows(sc, cols), want_s)
    print(f"[gpu] quantize past 4 GiB: {rows.size} rows, {cols.size} columns bit-exact",
          flush=True)
    del x, codes, scales, cr, sr, cc, sc, xt
    _free()


def test_gemm_a_and_c_past_2gib():
    """A [5 Mi, 1024] (2.5 GiB of codes) x B [256, 1024], BF16 C (2.5 GiB), on
    the tile kernel: sampled rows of C, past row 2^22, against the oracle."""
    N = 256
    announce(f"gemm A past 2 GiB: {BIG}x{N}x{K} bf16 (tile kernel)")
    ac, as_ = _operand(BIG, 5011)
    bc, bs = _operand(N, 5013)
    out = mx.gemm(ac, as_, bc, bs, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _sample(BIG, 5015)
    c_ref, s_ref = oracle.gemm(_rows(ac, rows), _rows(as_, rows), bc.cpu().numpy(),
                               bs.cpu().numpy())
    misses = check_gemm_output(out[torch.from_numpy(rows).to(DEV)], c_ref, s_ref)
    print(f"[gpu] A past 2 GiB: {rows.size} rows x {N}, literal BF16 misses {misses}",
          flush=True)
    del ac, as_, bc, bs, out
    _free()


@pytest.mark.parametrize("M,out_dtype", [(32, torch.bfloat16), (288, torch.float32)])
def test_gemm_b_past_2gib(M, out_dtype):
    """B [5 Mi, 1024] (2.5 GiB of codes): M = 32 on the split-K kernel (and
    the fragment-order GEMM, which must give the same bits), M = 288 on the
    tile kernel with FP32 C of 5.6 GiB (rows past 2^31 and 2^32 bytes) and
    on pre-shuffled B (the same bits); sampled columns of C, past column
    2^22, against the oracle."""
    announce(f"gemm B past 2 GiB: {M}x{BIG}x{K} {out_dtype}")
    ac, as_ = _operand(M, 5021)
    bc, bs = _operand(BIG, 5023)
    out = mx.gemm(ac, as_, bc, bs, out_dtype=out_dtype)
    torch.cuda.synchronize()
    cols = _sample(BIG, 5025)
    cols_t = torch.from_numpy(cols).to(DEV)
    c_ref, s_ref = oracle.gemm(ac.cpu().numpy(), as_.cpu().numpy(), _rows(bc, cols),
                               _rows(bs, cols))
    misses = check_gemm_output(out[:, cols_t].contiguous(), c_ref, s_ref)
    print(f"[gpu] B past 2 GiB, M={M}: {M} x {cols.size} outputs, literal BF16 misses "
          f"{misses}", flush=True)
    if M <= 128:
        announce(f"gemm_frag B past 2 GiB: {M}x{BIG}x{K}")
        af, asf = mx.to_frag(ac, as_)
        bf, bsf = mx.to_frag(bc, bs)
        got = mx.gemm_frag(af, asf, bf, bsf, M, BIG, K, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(got, out), "fragment-order GEMM differs from mxfp4_gemm"
        del af, asf, bf, bsf, got
    else:
        announce(f"gemm_bshuffled B past 2 GiB: {M}x{BIG}x{K}")
        bsh, bssh = mx.shuffle_b(bc, bs)
        got = mx.gemm_bshuffled(ac, as_, bsh, bssh, BIG, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(got, out), "pre-shuffled GEMM differs from mxfp4_gemm"
        del bsh, bssh, got
    del ac, as_, bc, bs, out
    _free()


def test_quantize_sr_input_past_4gib():
    """Stochastic rounding on the same 4 GiB shape: row-wise and both outputs
    of the bidimensional form against the oracle's draws at the sampled
    rows' own coordinates (rows past 2^31 and 2^32 bytes of X) and on whole
    sampled columns."""
    M, seed = (1 << 21) + 96, 0x0123456789ABCDEF
    announce(f"stochastic quantize past 4 GiB: X [{M}, {K}]")
    x = device_normal_bf16((M, K), 5031)
    codes, scales = mx.quantize_sr(x, seed)
    cr, sr, cc, sc = mx.quantize_2d_sr(x, seed)
    torch.cuda.synchronize()
    rows = _sample(M, 5032)
    xb = bf16_bits_of_tensor(x[torch.from_numpy(rows).to(DEV)])
    want_c, want_s = oracle.quantize_sr(xb, seed, oracle.DIR_ROWWISE, row_ids=rows)
    for got_c, got_s in ((codes, scales), (cr, sr)):
        assert np.array_equal(_rows(got_c, rows), want_c)
        assert np.array_equal(_rows(got_s, rows), want_s)
    cols = np.array([0, 1, 517, K - 1], dtype=np.int64)
    xt = bf16_bits_of_tensor(x[:, torch.from_numpy(cols).to(DEV)].t().contiguous())
    want_c, want_s = oracle.quantize_sr(xt, seed, oracle.DIR_COLUMNWISE, row_ids=cols)
    assert np.array_equal(_rows(cc, cols), want_c)
    assert np.array_equal(_rows(sc, cols), want_s)
    print(f"[gpu] stochastic quantize past 4 GiB: {rows.size} rows, {cols.size} columns "
          f"bit-exact", flush=True)
    del x, codes, scales, cr, sr, cc, sc
    _free()


def test_gemm_swiglu_a_and_act_past_2gib():
    """Fused SwiGLU gate+up GEMM with A [5 Mi, 1024] (2.5 GiB of codes) and
    B = [W_gate; W_up] of 2 x 256 rows: the BF16 activation (2.5 GiB) within
    the oracle's tolerance and its codes and scales bit-exact with the
    oracle's quantize of it, at sampled rows past row 2^22."""
    N = 512
    announce(f"gemm_swiglu A past 2 GiB: {BIG}x{N}x{K}")
    ac = device_random_bytes((BIG, K // 2), 5041)
    as_ = device_random_bytes((BIG, K // 32), 5042, lo=122, hi=130)
    bc = device_random_bytes((N, K // 2), 5043)
    bs = device_random_bytes((N, K // 32), 5044, lo=112, hi=120)
    codes, scales, act = mx.gemm_swiglu(ac, as_, bc, bs, want_act=True)
    torch.cuda.synchronize()
    rows = _sample(BIG, 5045)
    rows_t = torch.from_numpy(rows).to(DEV)
    ref, tol = oracle.swiglu_reference(_rows(ac, rows), _rows(as_, rows), bc.cpu().numpy(),
                                       bs.cpu().numpy())
    act_bits = bf16_bits_of_tensor(act[rows_t])
    ok = oracle.check_act_bf16(act_bits, ref, tol)
    assert ok.all(), f"{int((~ok).sum())} activations outside tolerance"
    q_codes, q_scales = oracle.quantize(act_bits)
    assert np.array_equal(_rows(codes, rows), q_codes)
    assert np.array_equal(_rows(scales, rows), q_scales)
    print(f"[gpu] gemm_swiglu A past 2 GiB: {rows.size} rows x {N // 2} activations", flush=True)
    del ac, as_, bc, bs, codes, scales, act
    _free()
