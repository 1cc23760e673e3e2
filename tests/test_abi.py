"""Host-side checks of the C ABI in libmxfp4.so (no GPU work is launched).

Return codes follow the stub/probe convention reviewed on "Initial
integration of a4w4 GEMM" (ROCm/TransformerEngine #663); the argument gates
are those of the hipBLASLt MXFP4 path on "Integrate MXFP4 hipblaslt GEMM
support" (#697, Changes list). Every call here fails validation, or finds no
gfx950 device, before anything is enqueued.
"""

import os
import re

import pytest

import block_scaled_microscaling_amd as mx

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "mxfp4.h")

OK, EINVAL, EUNSUPPORTED, ELAUNCH, EALIGN = 0, -1, -2, -3, -4
P16 = 1 << 20           # stand-in pointer values: never dereferenced here
P_ODD = (1 << 20) + 2


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp4_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = mx.load_library()
    names = _declared_functions()
    assert names == ["mxfp4_available", "mxfp4_gemm", "mxfp4_gemm_bshuffled",
                     "mxfp4_gemm_frag", "mxfp4_gemm_swiglu", "mxfp4_gemm_tile", "mxfp4_quantize",
                     "mxfp4_quantize_2d", "mxfp4_quantize_2d_sr", "mxfp4_quantize_2d_sr_rows",
                     "mxfp4_quantize_async", "mxfp4_quantize_frag", "mxfp4_quantize_sr",
                     "mxfp4_quantize_sr_rows", "mxfp4_shuffle_b",
                     "mxfp4_shuffle_b_sizes", "mxfp4_strerror", "mxfp4_to_frag"]
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_texts():
    for rc in (OK, EINVAL, EUNSUPPORTED, ELAUNCH, EALIGN):
        assert mx.mxfp4_strerror(rc) and "unknown" not in mx.mxfp4_strerror(rc)
    assert "unknown" in mx.mxfp4_strerror(12345)


@pytest.mark.parametrize("M,N,K", [
    (0, 32, 256), (32, 0, 256), (32, 32, 0), (-32, 32, 256),
    (33, 32, 256), (32, 48, 256), (32, 32, 128), (32, 32, 384),
    (1 << 31, 32, 256), (32, 32, (1 << 31) + 256), (32, 32, (1 << 24) + 256),
])
def test_gemm_rejects_bad_sizes(M, N, K):
    for fn in (mx.mxfp4_gemm, mx.mxfp4_gemm_tile):
        assert fn(P16, P16, P16, P16, M, N, K, mx.OUT_BF16, P16, None) == EINVAL


def test_gemm_rejects_bad_dtype_and_nulls():
    for fn in (mx.mxfp4_gemm, mx.mxfp4_gemm_tile):
        assert fn(P16, P16, P16, P16, 32, 32, 256, 2, P16, None) == EINVAL
        assert fn(P16, P16, P16, P16, 32, 32, 256, -1, P16, None) == EINVAL
        for i in range(5):
            ptrs = [P16] * 5
            ptrs[i] = None
            a, as_, b, bs, c = ptrs
            assert fn(a, as_, b, bs, 32, 32, 256, mx.OUT_FP32, c, None) == EINVAL


@pytest.mark.parametrize("M,N,K", [
    (0, 256, 256), (32, 0, 256), (32, 256, 0), (33, 256, 256), (32, 96, 256), (32, 64, 256),
    (32, 384, 256), (32, 256, 128), (32, 256, (1 << 24) + 256), (32, 1 << 14, 1 << 18),
])
def test_gemm_swiglu_rejects_bad_sizes(M, N, K):
    assert mx.mxfp4_gemm_swiglu(P16, P16, P16, P16, M, N, K, P16, P16, None, None) == EINVAL


def test_gemm_swiglu_rejects_nulls_and_misalignment():
    args = [P16, P16, P16, P16, 64, 256, 256, P16, P16, P16, None]
    for i in (0, 1, 2, 3, 7, 8):
        bad = list(args)
        bad[i] = None
        assert mx.mxfp4_gemm_swiglu(*bad) == EINVAL
    for i, off in ((0, 8), (2, 8), (1, 2), (3, 1), (7, 8), (9, 8)):
        bad = list(args)
        bad[i] = P16 + off
        assert mx.mxfp4_gemm_swiglu(*bad) == EALIGN, i


def test_shuffle_sizes_match_the_oracle_layout():
    import oracle
    for N, K in [(1, 256), (256, 256), (257, 1280), (8192, 8192), (6176, 7936)]:
        rc, cb, sb = mx.mxfp4_shuffle_b_sizes(N, K)
        assert rc == OK and (cb, sb) == oracle.shuffled_sizes(N, K)
    for N, K in [(0, 256), (32, 128), (32, 300), (32, 0), (1 << 31, 256), (32, (1 << 24) + 256)]:
        assert mx.mxfp4_shuffle_b_sizes(N, K)[0] == EINVAL


def test_shuffle_and_shuffled_gemm_reject_bad_arguments():
    assert mx.mxfp4_shuffle_b(None, P16, 32, 256, P16, P16, None) == EINVAL
    assert mx.mxfp4_shuffle_b(P16, P16, 32, 300, P16, P16, None) == EINVAL
    assert mx.mxfp4_shuffle_b(P16 + 8, P16, 32, 256, P16, P16, None) == EALIGN
    assert mx.mxfp4_shuffle_b(P16, P16 + 2, 32, 256, P16, P16, None) == EALIGN
    assert mx.mxfp4_shuffle_b(P16, P16, 32, 256, P16 + 8, P16, None) == EALIGN
    for M, N, K in [(0, 32, 256), (33, 32, 256), (32, 48, 256), (32, 32, 128)]:
        assert mx.mxfp4_gemm_bshuffled(P16, P16, P16, P16, M, N, K, mx.OUT_BF16, P16,
                                       None) == EINVAL
    assert mx.mxfp4_gemm_bshuffled(P16, P16, P16, P16, 32, 32, 256, 7, P16, None) == EINVAL
    assert mx.mxfp4_gemm_bshuffled(P16, P16, P16 + 8, P16, 32, 32, 256, mx.OUT_BF16, P16,
                                   None) == EALIGN


def test_gemm_rejects_oversized_buffers():
    # M * N * 4 bytes >= 2^40
    assert mx.mxfp4_gemm(P16, P16, P16, P16, 1 << 20, 1 << 18, 256, mx.OUT_FP32, P16,
                         None) == EINVAL
    # M * N * 4 past int64 (M = N = 2^31 - 32): rejected, not wrapped negative.
    big = (1 << 31) - 32
    for dt in (mx.OUT_BF16, mx.OUT_FP32):
        assert mx.mxfp4_gemm(P16, P16, P16, P16, big, big, 256, dt, P16, None) == EINVAL
        assert mx.mxfp4_gemm_tile(P16, P16, P16, P16, big, big, 256, dt, P16, None) == EINVAL
        assert mx.mxfp4_gemm_bshuffled(P16, P16, P16, P16, big, big, 256, dt, P16,
                                       None) == EINVAL
        assert mx.mxfp4_gemm_frag(P16, P16, P16, P16, big, big, 256, dt, P16, None) == EINVAL


@pytest.mark.parametrize("out", [mx.OUT_BF16, mx.OUT_FP32])
def test_gemm_rejects_past_2_28_columns(out):
    # The tile epilogue's store resource covers rows of C within 2^31 bytes
    # (N <= 2^28); the buffer sizes alone (256 x (2^28 + 32) x 4 bytes <
    # 2^40) would pass.
    N = (1 << 28) + 32
    assert mx.mxfp4_gemm(P16, P16, P16, P16, 256, N, 256, out, P16, None) == EINVAL
    assert mx.mxfp4_gemm(P16, P16, P16, P16, 32, N, 256, out, P16, None) == EINVAL
    assert mx.mxfp4_gemm_tile(P16, P16, P16, P16, 256, N, 256, out, P16, None) == EINVAL
    assert mx.mxfp4_gemm_bshuffled(P16, P16, P16, P16, 256, N, 256, out, P16, None) == EINVAL
    assert mx.mxfp4_gemm_frag(P16, P16, P16, P16, 32, N, 256, out, P16, None) == EINVAL


def test_gemm_rejects_misaligned():
    args = dict(A=P16, As=P16, B=P16, Bs=P16, C=P16)
    for key, bad in [("A", P_ODD), ("B", P_ODD), ("C", P16 + 8), ("As", P16 + 2),
                     ("Bs", P16 + 1)]:
        a = dict(args)
        a[key] = bad
        for fn in (mx.mxfp4_gemm, mx.mxfp4_gemm_tile):
            rc = fn(a["A"], a["As"], a["B"], a["Bs"], 32, 32, 256, mx.OUT_BF16, a["C"], None)
            assert rc == EALIGN, key


@pytest.mark.parametrize("M,K", [(0, 32), (-1, 32), (4, 0), (4, 16), (4, 48), (4, 33),
                                 (1 << 31, 32), (1 << 20, 1 << 20)])
def test_quantize_rejects_bad_sizes(M, K):
    assert mx.mxfp4_quantize(P16, M, K, P16, P16) == EINVAL
    assert mx.mxfp4_quantize_async(P16, M, K, P16, P16, None) == EINVAL
    assert mx.mxfp4_quantize_sr(P16, M, K, 7, P16, P16, None) == EINVAL


@pytest.mark.parametrize("M,row0", [(4, -1), (4, (1 << 31) - 4), (1, (1 << 31) - 1),
                                    ((1 << 31) - 1, 1)])
def test_quantize_sr_rows_rejects_bad_offsets(M, row0):
    """A row shard must lie within rows 0 .. 2^31 - 2 of the whole input."""
    assert mx.mxfp4_quantize_sr_rows(P16, M, 32, row0, 7, P16, P16, None) == EINVAL


@pytest.mark.parametrize("row0", [-32, 16, 1, (1 << 31) - 64])
def test_quantize_2d_sr_rows_rejects_bad_offsets(row0):
    """Bidimensional shards start on a 32-row block and stay below 2^31 - 1 rows."""
    assert mx.mxfp4_quantize_2d_sr_rows(P16, 64, 64, row0, 3, P16, P16, P16, P16,
                                        None) == EINVAL


def test_quantize_rejects_nulls_and_misalignment():
    assert mx.mxfp4_quantize(None, 4, 32, P16, P16) == EINVAL
    assert mx.mxfp4_quantize(P16, 4, 32, None, P16) == EINVAL
    assert mx.mxfp4_quantize(P16, 4, 32, P16, None) == EINVAL
    assert mx.mxfp4_quantize(P16 + 8, 4, 32, P16, P16) == EALIGN
    assert mx.mxfp4_quantize(P16, 4, 32, P16 + 2, P16) == EALIGN
    assert mx.mxfp4_quantize_sr(None, 4, 32, 1, P16, P16, None) == EINVAL
    assert mx.mxfp4_quantize_sr(P16, 4, 32, 1, None, P16, None) == EINVAL
    assert mx.mxfp4_quantize_sr(P16, 4, 32, 1, P16, None, None) == EINVAL
    assert mx.mxfp4_quantize_sr(P16 + 8, 4, 32, 1, P16, P16, None) == EALIGN
    assert mx.mxfp4_quantize_sr(P16, 4, 32, 1, P16 + 2, P16, None) == EALIGN


@pytest.mark.parametrize("M,K", [(0, 32), (32, 0), (16, 32), (32, 16), (48, 64), (64, 48),
                                 (1 << 31, 32), (1 << 20, 1 << 20)])
def test_quantize_2d_rejects_bad_sizes(M, K):
    assert mx.mxfp4_quantize_2d(P16, M, K, P16, P16, P16, P16, None) == EINVAL
    assert mx.mxfp4_quantize_2d_sr(P16, M, K, 3, P16, P16, P16, P16, None) == EINVAL


def test_quantize_2d_rejects_nulls_and_misalignment():
    args = [P16, 64, 64, P16, P16, P16, P16, None]
    for i in (0, 3, 4, 5, 6):
        bad = list(args)
        bad[i] = None
        assert mx.mxfp4_quantize_2d(*bad) == EINVAL
    for i in (0, 3, 5):
        bad = list(args)
        bad[i] = P16 + 8
        assert mx.mxfp4_quantize_2d(*bad) == EALIGN
    sr_args = [P16, 64, 64, 2**64 - 1, P16, P16, P16, P16, None]
    for i in (0, 4, 5, 6, 7):
        bad = list(sr_args)
        bad[i] = None
        assert mx.mxfp4_quantize_2d_sr(*bad) == EINVAL
    for i in (0, 4, 6):
        bad = list(sr_args)
        bad[i] = P16 + 8
        assert mx.mxfp4_quantize_2d_sr(*bad) == EALIGN


def test_no_device_reports_unsupported():
    """Valid arguments with no gfx950 device current: rc -2, nothing launched."""
    if mx.mxfp4_available() != 0:
        pytest.skip("a gfx950 device is present; stand-in pointers must not reach it")
    assert mx.mxfp4_gemm(P16, P16, P16, P16, 32, 32, 256, mx.OUT_BF16, P16, None) == EUNSUPPORTED
    assert mx.mxfp4_gemm_tile(P16, P16, P16, P16, 32, 32, 256, mx.OUT_BF16, P16,
                              None) == EUNSUPPORTED
    assert mx.mxfp4_quantize(P16, 4, 32, P16, P16) == EUNSUPPORTED
    assert mx.mxfp4_quantize_2d(P16, 32, 32, P16, P16, P16, P16, None) == EUNSUPPORTED
    assert mx.mxfp4_quantize_sr(P16, 4, 32, 5, P16, P16, None) == EUNSUPPORTED
    assert mx.mxfp4_gemm_swiglu(P16, P16, P16, P16, 32, 256, 256, P16, P16, None,
                                None) == EUNSUPPORTED
    assert mx.mxfp4_shuffle_b(P16, P16, 32, 256, P16, P16, None) == EUNSUPPORTED
    assert mx.mxfp4_gemm_bshuffled(P16, P16, P16, P16, 32, 32, 256, mx.OUT_BF16, P16,
                                   None) == EUNSUPPORTED
    assert mx.mxfp4_quantize_2d_sr(P16, 32, 32, 5, P16, P16, P16, P16, None) == EUNSUPPORTED
    assert mx.mxfp4_quantize_sr_rows(P16, 4, 32, 64, 5, P16, P16, None) == EUNSUPPORTED
    assert mx.mxfp4_quantize_2d_sr_rows(P16, 32, 32, 64, 5, P16, P16, P16, P16,
                                        None) == EUNSUPPORTED
    assert mx.mxfp4_quantize_frag(P16, 32, 256, P16, P16, None) == EUNSUPPORTED
    assert mx.mxfp4_to_frag(P16, P16, 32, 256, P16, P16, None) == EUNSUPPORTED
    assert mx.mxfp4_gemm_frag(P16, P16, P16, P16, 32, 32, 256, mx.OUT_BF16, P16,
                              None) == EUNSUPPORTED


def test_tensor_layer_validates_before_calling():
    import torch
    x = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(TypeError):
        mx.quantize(x)
    with pytest.raises(ValueError):
        mx.quantize(torch.zeros(4, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        mx.quantize_sr(x, 1)
    with pytest.raises(ValueError):
        mx.quantize_sr(torch.zeros((4, 64), dtype=torch.bfloat16), -1)


@pytest.mark.parametrize("M,K", [(0, 256), (16, 256), (48, 256), (32, 128), (32, 288),
                                 (32, 1 << 25), (1 << 31, 256)])
def test_frag_quantize_and_relayout_reject_bad_sizes(M, K):
    assert mx.mxfp4_quantize_frag(P16, M, K, P16, P16, None) == EINVAL
    assert mx.mxfp4_to_frag(P16, P16, M, K, P16, P16, None) == EINVAL


def test_frag_entries_reject_nulls_and_misalignment():
    assert mx.mxfp4_quantize_frag(None, 32, 256, P16, P16, None) == EINVAL
    assert mx.mxfp4_quantize_frag(P16, 32, 256, None, P16, None) == EINVAL
    assert mx.mxfp4_quantize_frag(P16 + 8, 32, 256, P16, P16, None) == EALIGN
    assert mx.mxfp4_quantize_frag(P16, 32, 256, P16 + 4, P16, None) == EALIGN
    assert mx.mxfp4_to_frag(P16, None, 32, 256, P16, P16, None) == EINVAL
    for i, off in ((0, 8), (1, 2), (4, 8), (5, 2)):
        args = [P16, P16, 32, 256, P16, P16, None]
        args[i] = P16 + off
        assert mx.mxfp4_to_frag(*args) == EALIGN


@pytest.mark.parametrize("M,N,K", [(0, 32, 256), (32, 0, 256), (16, 32, 256), (32, 48, 256),
                                   (32, 32, 128), (32, 32, 1 << 25), (1 << 31, 32, 256),
                                   (32 * 65535, 32, 1 << 24), (1 << 26, 1 << 14, 256),
                                   (32 * 3 * 65536, 32, 256)])
def test_gemm_frag_rejects_bad_sizes(M, N, K):
    assert mx.mxfp4_gemm_frag(P16, P16, P16, P16, M, N, K, mx.OUT_BF16, P16, None) == EINVAL


def test_gemm_frag_rejects_bad_dtype_nulls_and_misalignment():
    assert mx.mxfp4_gemm_frag(P16, P16, P16, P16, 32, 32, 256, 3, P16, None) == EINVAL
    assert mx.mxfp4_gemm_frag(P16, P16, None, P16, 32, 32, 256, mx.OUT_BF16, P16, None) == EINVAL
    for i, off in ((0, 8), (1, 2), (2, 8), (3, 2), (8, 8)):
        args = [P16, P16, P16, P16, 32, 32, 256, mx.OUT_BF16, P16, None]
        args[i] = P16 + off
        assert mx.mxfp4_gemm_frag(*args) == EALIGN
