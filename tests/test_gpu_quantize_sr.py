"""GPU parity of the stochastic-rounding quantize kernels against the oracle.

Codes and scales must match bit for bit: the random bytes are Philox4x32-10
draws keyed by block coordinates and direction (the stochastic-rounding
design described on NVIDIA/TransformerEngine #3809), computed independently
on each side, and the rounding rule is reading S3 of oracle/stochastic.py.
"""

import numpy as np
import pytest
import torch

import block_scaled_microscaling_amd as mx
import oracle
from gpu_helpers import DEV, announce, bf16_to_dev
from synth import WORKLOADS, bf16_matrix, random_bf16_bits

pytestmark = pytest.mark.gpu

SEEDS = [0, 1, 0xFFFFFFFF, 1 << 32, 0x0123456789ABCDEF, (1 << 64) - 1]


def _diff(name, g, r):
    bad = np.argwhere(g != r)
    assert bad.size == 0, f"{name}: {bad.shape[0]} bytes differ, first {bad[:4].tolist()}"


def _assert_same_sr(bits, seed):
    x = bf16_to_dev(bits)
    gc, gs = mx.quantize_sr(x, seed)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_sr(bits, seed)
    _diff("scales", gs.cpu().numpy(), rs)
    _diff("codes", gc.cpu().numpy(), rc)


def _assert_same_2d_sr(bits, seed):
    x = bf16_to_dev(bits)
    out = [t.cpu().numpy() for t in mx.quantize_2d_sr(x, seed)]
    torch.cuda.synchronize()
    ref = oracle.quantize_2d_sr(bits, seed)
    for name, g, r in zip(("codes", "scales", "codes_t", "scales_t"), out, ref):
        _diff(name, g, r)


@pytest.mark.parametrize("partner_hex", ["40c0", "3f80", "0100", "0008", "7f7f", "0000"])
def test_sr_every_bf16_value(partner_hex):
    """All finite BF16 values, each at 16 positions of blocks of a fixed
    partner (so at 16 different random bytes, in both signs): every rounding
    case, saturation, signed zero, subnormal inputs and many scale bytes."""
    announce(f"quantize_sr exhaustive, partner {partner_hex}")
    xs = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    xs = xs[(xs & 0x7F80) != 0x7F80]
    blocks = np.full((xs.size, 32), int(partner_hex, 16), dtype=np.uint16)
    for k in range(1, 32, 2):
        blocks[:, k] = xs if k % 4 == 1 else xs ^ np.uint16(0x8000)
    _assert_same_sr(blocks.reshape(-1, 256), seed=int(partner_hex, 16) * 31 + 7)


@pytest.mark.parametrize("seed", SEEDS)
def test_sr_seeds(seed):
    """Seeds with zero, all-ones and mixed key words."""
    announce(f"quantize_sr seed {seed:#x}")
    _assert_same_sr(bf16_matrix((64, 1024), ("normal", 1.0, 0.01, 100.0), 3), seed)


@pytest.mark.parametrize("M,K", [(1, 32), (1, 64), (3, 96), (5, 7936), (17, 1056), (129, 4128),
                                 (1000, 2016), (2, 1 << 16)])
def test_sr_ragged_sizes(M, K):
    """Block counts that leave partial wavefronts and workgroups, one block per
    row, and long rows (block coordinates from the flat index)."""
    announce(f"quantize_sr ragged M={M} K={K}")
    _assert_same_sr(bf16_matrix((M, K), ("laplace", 1.0), M * 7 + K), seed=M + K)


def test_sr_random_bit_patterns():
    announce("quantize_sr random finite bit patterns 512 x 1024")
    _assert_same_sr(random_bf16_bits((512, 1024), seed=4321), seed=99)


def test_sr_special_blocks():
    announce("quantize_sr zero, -0, subnormal and extreme blocks")
    rows = [np.zeros(64, np.uint16), np.full(64, 0x8000, np.uint16),
            np.arange(1, 65, dtype=np.uint16), np.full(64, 0x7F7F, np.uint16),
            np.tile(np.array([0x7F7F, 0x0001], np.uint16), 32),
            np.tile(np.array([0x40C0, 0x3E80, 0xBE80, 0x3F40], np.uint16), 16)]
    _assert_same_sr(np.stack(rows), seed=5)


def test_sr_deterministic_and_seed_dependent():
    announce("quantize_sr determinism")
    bits = bf16_matrix((128, 512), ("normal", 1.0, 0.0, 1.0), 8)
    x = bf16_to_dev(bits)
    a, _ = mx.quantize_sr(x, 17)
    b, _ = mx.quantize_sr(x, 17)
    c, _ = mx.quantize_sr(x, 18)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


def test_sr_mean_tracks_input():
    """Averaged over many seeds the dequantized values approach x (the point
    of stochastic rounding); RNE keeps a systematic error on the same data."""
    announce("quantize_sr mean over 64 seeds")
    bits = bf16_matrix((32, 256), ("normal", 1.0, 0.0, 1.0), 21)
    x = bf16_to_dev(bits)
    acc = np.zeros((32, 256))
    for s in range(64):
        c, sc = mx.quantize_sr(x, 1000 + s)
        acc += oracle.dequantize(c.cpu().numpy(), sc.cpu().numpy())
    mean = acc / 64
    xv = oracle.bf16_bits_to_f64(bits)
    rc, rs = oracle.quantize(bits)
    err_sr = np.abs(mean - xv).mean()
    err_rne = np.abs(oracle.dequantize(rc, rs) - xv).mean()
    assert err_sr < 0.35 * err_rne, (err_sr, err_rne)


def test_sr_outputs_written_exactly_in_bounds():
    announce("quantize_sr canary")
    M, K = 37, 96
    bits = bf16_matrix((M, K), ("normal", 1.0, 0.0, 1.0), 5)
    pad = 256
    cbuf = torch.full((M * K // 2 + 2 * pad,), 0xAB, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((M * K // 32 + 2 * pad,), 0xCD, dtype=torch.uint8, device=DEV)
    codes = cbuf[pad:pad + M * K // 2].view(M, K // 2)
    scales = sbuf[pad:pad + M * K // 32].view(M, K // 32)
    mx.quantize_sr(bf16_to_dev(bits), 3, codes, scales)
    torch.cuda.synchronize()
    c = cbuf.cpu().numpy()
    s = sbuf.cpu().numpy()
    assert np.all(c[:pad] == 0xAB) and np.all(c[-pad:] == 0xAB)
    assert np.all(s[:pad] == 0xCD) and np.all(s[-pad:] == 0xCD)
    rc, rs = oracle.quantize_sr(bits, 3)
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("name", ["square", "ragged"])
def test_sr_workload_sampled_rows(name):
    """Full-size stochastic quantize of the workload's activation; the oracle
    recomputes sampled rows with their real row coordinates."""
    w = WORKLOADS[name]
    announce(f"quantize_sr workload {name}: {w.M}x{w.K}")
    bits = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    seed = 0x5EED0000 + w.M
    gc, gs = mx.quantize_sr(bf16_to_dev(bits), seed)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([rng.integers(0, w.M, 120), [0, 1, w.M - 2, w.M - 1]]))
    rc, rs = oracle.quantize_sr(bits[rows], seed, row_ids=rows)
    _diff("scales", gs.cpu().numpy()[rows], rs)
    _diff("codes", gc.cpu().numpy()[rows], rc)


# ------------------------------------------- bidimensional, stochastic
@pytest.mark.parametrize("M,K", [(32, 32), (128, 128), (256, 384), (160, 96), (96, 4128),
                                 (1056, 352)])
def test_sr_2d_random(M, K):
    announce(f"quantize_2d_sr random {M}x{K}")
    _assert_same_2d_sr(random_bf16_bits((M, K), seed=M * 5 + K), seed=M * K)


def test_sr_2d_every_bf16_value():
    """Every finite BF16 value as a column element (row 5, negated at row 30,
    in a column of a fixed partner), and along rows of the row-wise output."""
    announce("quantize_2d_sr exhaustive")
    xs = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    xs = xs[(xs & 0x7F80) != 0x7F80][:65280]
    cols = np.full((32, xs.size), 0x40C0, dtype=np.uint16)
    cols[5] = xs
    cols[30] = xs ^ np.uint16(0x8000)
    _assert_same_2d_sr(cols, seed=(1 << 64) - 3)


def test_sr_2d_rowwise_equals_rowwise_kernel():
    """The 2-D kernel's row-wise output is the row-wise kernel's, byte for byte."""
    announce("quantize_2d_sr vs quantize_sr")
    bits = bf16_matrix((512, 640), ("laplace", 1.0), 6)
    x = bf16_to_dev(bits)
    c, s, _, _ = mx.quantize_2d_sr(x, 77)
    c1, s1 = mx.quantize_sr(x, 77)
    torch.cuda.synchronize()
    assert torch.equal(c, c1) and torch.equal(s, s1)


@pytest.mark.parametrize("name", ["ragged", "square"])
def test_sr_2d_workload(name):
    w = WORKLOADS[name]
    announce(f"quantize_2d_sr workload {name}: {w.M}x{w.K}")
    bits = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    seed = 0xC0FFEE + w.K
    if name == "ragged":
        _assert_same_2d_sr(bits, seed)
        return
    gc, gs, gct, gst = mx.quantize_2d_sr(bf16_to_dev(bits), seed)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = np.sort(rng.choice(w.M, 48, replace=False))
    cols = np.sort(rng.choice(w.K, 48, replace=False))
    rc, rs = oracle.quantize_sr(bits[rows], seed, oracle.DIR_ROWWISE, row_ids=rows)
    _diff("codes", gc.cpu().numpy()[rows], rc)
    _diff("scales", gs.cpu().numpy()[rows], rs)
    rct, rst = oracle.quantize_sr(np.ascontiguousarray(bits[:, cols].T), seed,
                                  oracle.DIR_COLUMNWISE, row_ids=cols)
    _diff("codes_t", gct.cpu().numpy()[cols], rct)
    _diff("scales_t", gst.cpu().numpy()[cols], rst)


@pytest.mark.parametrize("row0,m", [(0, 160), (160, 96), (256, 256), (480, 32)])
def test_sr_row_shard_is_part_of_the_whole(row0, m):
    """mxfp4_quantize_sr_rows and mxfp4_quantize_2d_sr_rows on rows row0 ..
    row0 + m - 1 of X [512, 384]: byte for byte the matching part of the
    whole input's outputs, and equal to the oracle keyed by global rows."""
    announce(f"quantize_sr row shard {row0}+{m}")
    bits = bf16_matrix((512, 384), ("laplace", 1.0), 23)
    seed = 0x5EED
    x = bf16_to_dev(bits)
    wc, ws = [t.cpu().numpy() for t in mx.quantize_sr(x, seed)]
    wc2, ws2, wct, wst = [t.cpu().numpy() for t in mx.quantize_2d_sr(x, seed)]
    part = bf16_to_dev(np.ascontiguousarray(bits[row0:row0 + m]))
    pc, ps = [t.cpu().numpy() for t in mx.quantize_sr(part, seed, row0=row0)]
    qc, qs, qct, qst = [t.cpu().numpy() for t in mx.quantize_2d_sr(part, seed, row0=row0)]
    torch.cuda.synchronize()
    _diff("codes", pc, wc[row0:row0 + m])
    _diff("scales", ps, ws[row0:row0 + m])
    _diff("2d codes", qc, wc2[row0:row0 + m])
    _diff("2d scales", qs, ws2[row0:row0 + m])
    _diff("codes_t", qct, wct[:, row0 // 2:(row0 + m) // 2])
    _diff("scales_t", qst, wst[:, row0 // 32:(row0 + m) // 32])
    ref = oracle.quantize_2d_sr(np.ascontiguousarray(bits[row0:row0 + m]), seed, row0=row0)
    for name, g, r in zip(("codes", "scales", "codes_t", "scales_t"), (qc, qs, qct, qst), ref):
        _diff("oracle " + name, g, r)
