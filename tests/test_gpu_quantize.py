"""GPU parity of the BF16 -> MXFP4 quantize kernel against the CPU oracle.

Codes and scales must match bit for bit. The format is the MXFP4 of
"Integrate MXFP4 hipblaslt GEMM support" (ROCm/TransformerEngine #697,
Changes list); the readings (exponent floor(log2 amax) - 2, nearest-even
E2M1, signed zero, low nibble first) are those of oracle/mxfp4_ref.py.
"""

import numpy as np
import pytest
import torch

import block_scaled_microscaling_amd as mx
import oracle
from gpu_helpers import DEV, announce, bf16_to_dev
from synth import WORKLOADS, bf16_matrix, random_bf16_bits

pytestmark = pytest.mark.gpu


def _gpu_quantize(bits):
    x = bf16_to_dev(bits)
    codes, scales = mx.quantize(x)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _assert_same(bits):
    gc, gs = _gpu_quantize(bits)
    rc, rs = oracle.quantize(bits)
    bad_s = np.argwhere(gs != rs)
    assert bad_s.size == 0, f"{bad_s.shape[0]} scale bytes differ, first {bad_s[:4].tolist()}"
    bad_c = np.argwhere(gc != rc)
    assert bad_c.size == 0, f"{bad_c.shape[0]} code bytes differ, first {bad_c[:4].tolist()}"


def test_library_available():
    announce("mxfp4_available")
    assert mx.mxfp4_available() == 1


@pytest.mark.parametrize("partner_hex", ["40c0", "3f80", "0100", "0080", "0008", "7f7f", "3ca4",
                                         "0000"])
def test_every_bf16_value_in_fixed_context(partner_hex):
    """All 65280 finite BF16 values, each in a block whose other 31 entries are
    one partner value: covers every rounding case, ties, saturation, signed
    zeros, subnormal inputs and scale bytes 0..252."""
    announce(f"quantize exhaustive, partner {partner_hex}")
    xs = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    xs = xs[(xs & 0x7F80) != 0x7F80]
    blocks = np.full((xs.size, 32), int(partner_hex, 16), dtype=np.uint16)
    blocks[:, 5] = xs
    blocks[:, 30] = xs ^ np.uint16(0x8000)
    _assert_same(blocks)


def test_random_bit_patterns():
    announce("quantize random finite bit patterns 1000 x 1024")
    _assert_same(random_bf16_bits((1000, 1024), seed=1234))


@pytest.mark.parametrize("M,K", [(1, 32), (1, 64), (3, 96), (5, 7936), (17, 1056), (129, 4128),
                                 (1000, 2016)])
def test_ragged_sizes(M, K):
    """Block counts that leave partial wavefronts and workgroups."""
    announce(f"quantize ragged M={M} K={K}")
    _assert_same(bf16_matrix((M, K), ("laplace", 1.0), M * 7 + K))


def test_special_blocks():
    announce("quantize zero, -0, subnormal and extreme blocks")
    rows = []
    rows.append(np.zeros(64, np.uint16))                        # all +0
    rows.append(np.full(64, 0x8000, np.uint16))                 # all -0
    rows.append(np.arange(1, 65, dtype=np.uint16))              # subnormals only
    rows.append(np.full(64, 0x7F7F, np.uint16))                 # BF16 max
    rows.append(np.tile(np.array([0x7F7F, 0x0001], np.uint16), 32))
    r = np.zeros(64, np.uint16)
    r[::2] = 0x00C0                                             # 1.5 * 2^-126
    rows.append(r)
    _assert_same(np.stack(rows))


@pytest.mark.parametrize("name", ["tiny", "skinny", "ragged"])
def test_workload_inputs_full(name):
    w = WORKLOADS[name]
    announce(f"quantize full inputs of workload {name}")
    a = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    _assert_same(a)
    b = bf16_matrix((w.N, w.K), w.b_dist, w.b_seed)
    _assert_same(b)


@pytest.mark.parametrize("name", ["square", "mlp_gate_up", "mlp_down"])
def test_workload_inputs_sampled_rows(name):
    """Full-size GPU quantize; the oracle recomputes 384 sampled rows (rows
    are independent)."""
    w = WORKLOADS[name]
    rng = np.random.default_rng(77)
    for label, rows, dist, seed in (("A", w.M, w.a_dist, w.a_seed), ("B", w.N, w.b_dist, w.b_seed)):
        announce(f"quantize {name} operand {label} [{rows}, {w.K}]")
        bits = bf16_matrix((rows, w.K), dist, seed)
        gc, gs = _gpu_quantize(bits)
        pick = np.unique(np.concatenate([rng.integers(0, rows, 380), [0, 1, rows - 2, rows - 1]]))
        rc, rs = oracle.quantize(bits[pick])
        assert np.array_equal(gs[pick], rs)
        assert np.array_equal(gc[pick], rc)
        assert gs.max() <= 252


def test_misaligned_input_rejected():
    announce("quantize misaligned pointer")
    base = torch.zeros(4 * 64 + 4, dtype=torch.bfloat16, device=DEV)
    x = base[4:].view(4, 64)                                    # 8-byte offset
    codes = torch.empty((4, 32), dtype=torch.uint8, device=DEV)
    scales = torch.empty((4, 2), dtype=torch.uint8, device=DEV)
    rc = mx.mxfp4_quantize(x.data_ptr(), 4, 64, codes.data_ptr(), scales.data_ptr())
    assert rc == -4


def test_outputs_written_exactly_in_bounds():
    """Guard bytes around codes and scales stay untouched."""
    announce("quantize canary")
    M, K = 37, 96
    bits = bf16_matrix((M, K), ("normal", 1.0, 0.0, 1.0), 5)
    pad = 256
    cbuf = torch.full((M * K // 2 + 2 * pad,), 0xAB, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((M * K // 32 + 2 * pad,), 0xCD, dtype=torch.uint8, device=DEV)
    codes = cbuf[pad:pad + M * K // 2].view(M, K // 2)
    scales = sbuf[pad:pad + M * K // 32].view(M, K // 32)
    mx.quantize(bf16_to_dev(bits), codes, scales)
    torch.cuda.synchronize()
    c = cbuf.cpu().numpy()
    s = sbuf.cpu().numpy()
    assert np.all(c[:pad] == 0xAB) and np.all(c[-pad:] == 0xAB)
    assert np.all(s[:pad] == 0xCD) and np.all(s[-pad:] == 0xCD)
    rc, rs = oracle.quantize(bits)
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)


def test_side_stream_and_null_stream_entry():
    announce("quantize on a side stream and through the 5-argument entry")
    bits = bf16_matrix((64, 512), ("normal", 1.0, 0.01, 100.0), 9)
    rc, rs = oracle.quantize(bits)
    x = bf16_to_dev(bits)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        codes, scales = mx.quantize(x)
    s.synchronize()
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)
    c2 = torch.empty_like(codes)
    s2 = torch.empty_like(scales)
    torch.cuda.synchronize()
    assert mx.mxfp4_quantize(x.data_ptr(), 64, 512, c2.data_ptr(), s2.data_ptr()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), rc) and np.array_equal(s2.cpu().numpy(), rs)


# ------------------------------------------------- bidimensional quantize
# Rowwise + columnwise MXFP4 in one pass (the bidimensional quantize of
# NVIDIA/TransformerEngine #3809, description): both outputs bit-exact with
# the oracle's quantize of X and of X^T.
def _assert_same_2d(bits):
    x = bf16_to_dev(bits)
    gc, gs, gct, gst = (t.cpu().numpy() for t in mx.quantize_2d(x))
    torch.cuda.synchronize()
    rc, rs, rct, rst = oracle.quantize_2d(bits)
    for name, g, r in (("codes", gc, rc), ("scales", gs, rs), ("codes_t", gct, rct),
                       ("scales_t", gst, rst)):
        bad = np.argwhere(g != r)
        assert bad.size == 0, f"{name}: {bad.shape[0]} bytes differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("M,K", [(32, 32), (128, 128), (256, 384), (160, 96), (4128, 7936),
                                 (96, 4128), (1056, 352), (288, 800), (512, 1024)])
def test_quantize_2d_random(M, K):
    """Random finite bit patterns; shapes with whole and ragged 256 x 256
    tiles (the kernel's), down to a single 32-element block past the last
    whole tile (K = 800), and more tiles than one pass of the persistent grid
    (4128 x 7936)."""
    announce(f"quantize_2d random {M}x{K}")
    _assert_same_2d(random_bf16_bits((M, K), seed=M * 7 + K))


def test_quantize_2d_every_bf16_value():
    """All finite BF16 values as columns' elements: 65280 columns of 32 rows,
    each holding the value at row 5 and its negation at row 30 in a column of
    a fixed partner value (the exhaustive rowwise test, transposed), plus the
    same values along rows."""
    announce("quantize_2d exhaustive")
    xs = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    xs = xs[(xs & 0x7F80) != 0x7F80][:65280]
    cols = np.full((32, xs.size), 0x40c0, dtype=np.uint16)
    cols[5] = xs
    cols[30] = xs ^ np.uint16(0x8000)
    _assert_same_2d(cols)


@pytest.mark.parametrize("name", ["ragged", "square"])
def test_quantize_2d_workload(name):
    """The workload's activation at full size; the square one is compared on
    sampled rows of both outputs (the oracle quantizes those rows itself)."""
    w = WORKLOADS[name]
    announce(f"quantize_2d workload {name}: {w.M}x{w.K}")
    bits = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    if name == "ragged":
        _assert_same_2d(bits)
        return
    gc, gs, gct, gst = mx.quantize_2d(bf16_to_dev(bits))
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(w.M, 64, replace=False))
    cols = np.sort(rng.choice(w.K, 64, replace=False))
    rc, rs = oracle.quantize(bits[rows])
    assert np.array_equal(gc.cpu().numpy()[rows], rc)
    assert np.array_equal(gs.cpu().numpy()[rows], rs)
    rct, rst = oracle.quantize(np.ascontiguousarray(bits[:, cols].T))
    assert np.array_equal(gct.cpu().numpy()[cols], rct)
    assert np.array_equal(gst.cpu().numpy()[cols], rst)
