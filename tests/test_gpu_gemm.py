"""GPU parity of the MXFP4 GEMM against the CPU oracle.

Operation: the FP4 x FP4 ("a4w4") GEMM of "Initial integration of a4w4 GEMM"
(ROCm/TransformerEngine #663) under the gates of the hipBLASLt MXFP4 path on
"Integrate MXFP4 hipblaslt GEMM support" (#697, Changes list). FP32 output
must be within 1e-5 * sum|a*b| of the float64 oracle; BF16 output within one
BF16 step of the oracle rounded to BF16 (with the near-cancellation reading
documented in oracle/compare.py). The non-zero count check guards against the
silent all-zeros failure reported on "feat(ck-tile): aquant GEMM TE to
dispatcher bridge" (rocm-libraries #9980, GPU validation).

mxfp4_gemm runs M <= 128, and problems of at most CUs / 8 tiles of 256 x 256,
on the split-K kernel and larger problems on the 256 x 256 tile kernel;
mxfp4_gemm_tile runs the tile kernel whatever the shape. Each layout case runs
at M = 32 (or the case's own small M), and again with its rows repeated past
128 through mxfp4_gemm (split-K kernel, several row tiles) and through
mxfp4_gemm_tile.
"""

import numpy as np
import pytest
import torch

import block_scaled_microscaling_amd as mx
import oracle
from conftest import read_golden
from gpu_helpers import (DEV, announce, bf16_bits_of_tensor, bf16_to_dev, check_gemm_output,
                         sample_pairs, u8_to_dev)
from synth import WORKLOADS, bf16_matrix, large_block_first, random_codes, random_scales

pytestmark = pytest.mark.gpu


def _assert_not_silent_zeros(got, c_ref, s_ref):
    """Every output the oracle puts clearly away from zero is non-zero."""
    significant = np.abs(c_ref) > 2 * oracle.FP32_REL_TOL * s_ref
    assert significant.sum() > 0
    assert np.count_nonzero(got[significant]) == int(significant.sum())


# (rows, entry point): the split-K kernel at one and at five row tiles
# (mxfp4_gemm), the tile kernel (mxfp4_gemm_tile).
KERNEL_CASES = [(32, "auto"), (160, "auto"), (160, "tile")]
ENTRY = {"auto": mx.gemm, "tile": mx.gemm_tile}


def _rep(x, rows):
    """Repeat a 32-row operand (or expected C) down to `rows` rows."""
    return np.tile(x, (rows // x.shape[0],) + (1,) * (x.ndim - 1))


def _gemm(Ac, As, Bc, Bs, out_dtype, kernel="auto"):
    out = ENTRY[kernel](u8_to_dev(Ac), u8_to_dev(As), u8_to_dev(Bc), u8_to_dev(Bs),
                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("rows,kernel", KERNEL_CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_single_tile_random(out_dtype, rows, kernel):
    """One 32 x 32 x 256 problem: pins the MFMA operand/scale lane layout."""
    announce(f"gemm {rows}x32x256 random {out_dtype} ({kernel})")
    Ac, Bc = random_codes(rows, 256, 1), random_codes(32, 256, 2)
    As, Bs = random_scales(rows, 256, 3), random_scales(32, 256, 4)
    out = _gemm(Ac, As, Bc, Bs, out_dtype, kernel)
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    check_gemm_output(out, c_ref, s_ref)


@pytest.mark.parametrize("rows,kernel", KERNEL_CASES)
def test_hand_worked_g1_padded(rows, kernel):
    """Q1 block x unit B rows (1 x 32 x 32 by hand), padded to rows x 32 x 256
    with zero codes: row 0 of C is the dequantized Q1 block."""
    announce(f"gemm G1 padded to {rows} rows ({kernel})")
    g = read_golden("q1_block.txt")
    Ac = np.zeros((rows, 128), np.uint8)
    Ac[0, :16] = [int(v, 16) for v in g["packed"]]
    As = np.full((rows, 8), 127, np.uint8)
    Bc = np.zeros((32, 128), np.uint8)
    for n in range(32):
        Bc[n, n // 2] = 2 << (4 * (n % 2))
    out = _gemm(Ac, As, Bc, As[:32], torch.float32, kernel).cpu().numpy()
    assert out[0].tolist() == [float(v) for v in g["dequant"]]
    assert np.all(out[1:] == 0)


@pytest.mark.parametrize("rows,kernel", KERNEL_CASES)
def test_hand_worked_g2_g3_g4(rows, kernel):
    announce(f"gemm G2 G3 G4 at {rows} rows ({kernel})")
    n = np.arange(32)
    m = np.arange(32)[:, None]
    # G2: C = 255 * 2^(n % 3)
    A = np.full((32, 128), 0x22, np.uint8)
    As = np.tile(np.arange(123, 131, dtype=np.uint8), (32, 1))
    Bs = (126 + n % 3).astype(np.uint8)[:, None].repeat(8, axis=1)
    for dt in (torch.float32, torch.bfloat16):
        out = _gemm(_rep(A, rows), _rep(As, rows), A, Bs, dt, kernel).float().cpu().numpy()
        assert np.array_equal(out, np.tile(255.0 * 2.0 ** (n % 3), (rows, 1)))
    # G3: nibble pairing, C = 448 everywhere
    s = np.full((32, 8), 127, np.uint8)
    out = _gemm(_rep(np.full((32, 128), 0x13, np.uint8), rows), _rep(s, rows),
                np.full((32, 128), 0x24, np.uint8), s, torch.float32, kernel).cpu().numpy()
    assert out.shape == (rows, 32) and np.all(out == 448.0)
    # G4: scale-to-block mapping, C = 2338 * 2^(m%2 + n%4 - 2)
    A = np.zeros((32, 128), np.uint8)
    for j in range(8):
        A[:, 16 * j:16 * (j + 1)] = j | (j << 4)
    As = (123 + np.arange(8)[None, :] + (np.arange(32) % 2)[:, None]).astype(np.uint8)
    B = np.full((32, 128), 0x22, np.uint8)
    Bs = (125 + n % 4).astype(np.uint8)[:, None].repeat(8, axis=1)
    out = _gemm(_rep(A, rows), _rep(As, rows), B, Bs, torch.float32, kernel).cpu().numpy()
    assert np.array_equal(out, _rep(2338.0 * 2.0 ** ((m % 2) + (n[None, :] % 4) - 2), rows))


@pytest.mark.parametrize("M,N,K", [(32, 32, 256), (256, 256, 256), (288, 544, 512),
                                   (544, 288, 1024), (64, 800, 768), (512, 96, 2304),
                                   (800, 1056, 256), (160, 64, 512),
                                   # split-K kernel: K steps not a multiple of its 8
                                   # waves, a single step (7 idle waves), long K
                                   (96, 320, 2304), (128, 64, 256), (128, 288, 768),
                                   (32, 96, 14336), (64, 2080, 7936)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("kernel", ["auto", "tile"])
def test_random_operands_many_tiles(M, N, K, out_dtype, kernel):
    """Uniform random code bytes (every code, both signs) and scales 117..137,
    shapes spanning several 256-tiles with ragged M and N edges, through
    mxfp4_gemm (the split-K kernel at these sizes) and the tile kernel."""
    announce(f"gemm random {M}x{N}x{K} {out_dtype} ({kernel})")
    Ac, Bc = random_codes(M, K, M + 1), random_codes(N, K, N + 2)
    As, Bs = random_scales(M, K, K + 3), random_scales(N, K, K + 4)
    out = _gemm(Ac, As, Bc, Bs, out_dtype, kernel)
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    check_gemm_output(out, c_ref, s_ref)
    _assert_not_silent_zeros(out.float().cpu().numpy(), c_ref, s_ref)


def _sweep_shapes(n=20, seed=20261203):
    """Seeded shapes: M, N multiples of 32 up to 768, K a multiple of 256 up
    to 2048 (ragged tile edges, one or several K steps and scale chunks)."""
    rng = np.random.default_rng(seed)
    return [(32 * int(rng.integers(1, 25)), 32 * int(rng.integers(1, 25)),
             256 * int(rng.integers(1, 9))) for _ in range(n)]


@pytest.mark.parametrize("idx", range(20))
def test_random_shape_sweep(idx):
    """Seeded random shapes through both kernels (mxfp4_gemm: split-K for
    these sizes; mxfp4_gemm_tile: the tile kernel with edge tiles), BF16 and
    FP32 out alternating, against the oracle."""
    M, N, K = _sweep_shapes()[idx]
    out_dtype = torch.bfloat16 if idx % 2 == 0 else torch.float32
    announce(f"gemm sweep {idx}: {M}x{N}x{K} {out_dtype}")
    Ac, Bc = random_codes(M, K, 900 + idx), random_codes(N, K, 950 + idx)
    As, Bs = random_scales(M, K, 1000 + idx), random_scales(N, K, 1050 + idx)
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    for kernel in ("auto", "tile"):
        out = _gemm(Ac, As, Bc, Bs, out_dtype, kernel)
        check_gemm_output(out, c_ref, s_ref)
        _assert_not_silent_zeros(out.float().cpu().numpy(), c_ref, s_ref)


@pytest.mark.parametrize("N", [2048, 2080])
def test_kernel_choice_boundary(N):
    """1024 x N: 4 x 8 = 32 tiles of 256 x 256 (CUs / 8 on a 256-CU part:
    mxfp4_gemm runs the split-K kernel) and 4 x 9 = 36 tiles (the tile kernel,
    so its bits equal mxfp4_gemm_tile's). Both against the oracle."""
    M, K = 1024, 512
    workers = torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8
    tiles = (M // 256) * (-(-N // 256))
    announce(f"gemm kernel choice {M}x{N}x{K}: {tiles} tiles, {workers} workgroups")
    Ac, Bc = random_codes(M, K, 71), random_codes(N, K, 72)
    As, Bs = random_scales(M, K, 73), random_scales(N, K, 74)
    args = [u8_to_dev(t) for t in (Ac, As, Bc, Bs)]
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    for dt in (torch.bfloat16, torch.float32):
        auto = mx.gemm(*args, out_dtype=dt)
        tile = mx.gemm_tile(*args, out_dtype=dt)
        torch.cuda.synchronize()
        if tiles * 8 > workers:
            assert torch.equal(auto, tile)
        check_gemm_output(auto, c_ref, s_ref)
        check_gemm_output(tile, c_ref, s_ref)


def _tile_of(pid, tiles_m, tiles_n, n_xcd=8, group_m=4):
    """The tile kernel's XCD-aware tile order (tile id -> tile row, column)."""
    total = tiles_m * tiles_n
    q, rem = divmod(total, n_xcd)
    xcd, idx = pid % n_xcd, pid // n_xcd
    p = xcd * q + min(xcd, rem) + idx
    width = group_m * tiles_n
    first_m = (p // width) * group_m
    in_group = p - (p // width) * width
    gsize = min(tiles_m - first_m, group_m)
    return first_m + in_group % gsize, in_group // gsize


def _edge_transitions(M, N, workers):
    """(whole -> edge, edge -> whole) tile successions over the persistent
    workgroups: a BF16 tile's C stores overlap the next tile's first loads
    only after a tile that lies wholly inside C."""
    tiles_m, tiles_n = -(-M // 256), -(-N // 256)
    total = tiles_m * tiles_n
    wp = pw = 0
    for b in range(min(workers, total)):
        prev = None
        for p in range(b, total, workers):
            tm, tn = _tile_of(p, tiles_m, tiles_n)
            whole = 256 * tm + 256 <= M and 256 * tn + 256 <= N
            if prev is not None:
                wp += prev and not whole
                pw += whole and not prev
            prev = whole
    return wp, pw


@pytest.mark.parametrize("M,N,K", [(4384, 4128, 256), (4128, 4384, 1280)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_persistent_edge_tiles(M, N, K, out_dtype):
    """More tiles than workgroups with ragged M and N: workgroups run whole
    tiles followed by edge tiles (and the reverse), whose epilogues mask
    rows and columns in their stores, on plain and on pre-shuffled B."""
    workers = torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8
    wp, pw = _edge_transitions(M, N, workers)
    announce(f"gemm {out_dtype} {M}x{N}x{K}: {workers} workgroups, whole->edge {wp}, "
             f"edge->whole {pw}")
    assert wp > 0
    Ac, Bc = random_codes(M, K, M + 7), random_codes(N, K, N + 8)
    As, Bs = random_scales(M, K, K + 9), random_scales(N, K, K + 10)
    A, As_d, B, Bs_d = (u8_to_dev(t) for t in (Ac, As, Bc, Bs))
    plain = mx.gemm(A, As_d, B, Bs_d, out_dtype=out_dtype)
    tile = mx.gemm_tile(A, As_d, B, Bs_d, out_dtype=out_dtype)
    bc, bs = mx.shuffle_b(B, Bs_d)
    shuf = mx.gemm_bshuffled(A, As_d, bc, bs, N, out_dtype=out_dtype)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    check_gemm_output(plain, c_ref, s_ref)
    assert torch.equal(plain, tile), "mxfp4_gemm did not run the tile kernel at this size"
    assert torch.equal(plain, shuf)


@pytest.mark.parametrize("M,kernel", [(96, "auto"), (288, "auto"), (288, "tile")])
def test_wide_scale_range(M, kernel):
    """Scales 100..150 on both sides: products span 2^-54 .. 2^46."""
    announce(f"gemm wide scale range M={M} ({kernel})")
    N, K = 160, 1280
    Ac, Bc = random_codes(M, K, 31), random_codes(N, K, 32)
    As, Bs = random_scales(M, K, 33, 100, 150), random_scales(N, K, 34, 100, 150)
    out = _gemm(Ac, As, Bc, Bs, torch.float32, kernel)
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    check_gemm_output(out, c_ref, s_ref)


@pytest.mark.parametrize("M,kernel", [(64, "auto"), (288, "auto"), (288, "tile")])
def test_scale_doubling_is_exact(M, kernel):
    """Adding 1 to every A scale of one row doubles that C row bit for bit
    (power-of-two scaling commutes with fp32 rounding) and leaves the others."""
    announce(f"gemm scale doubling invariant M={M} ({kernel})")
    N, K = 288, 1024
    Ac, Bc = random_codes(M, K, 41), random_codes(N, K, 42)
    As, Bs = random_scales(M, K, 43), random_scales(N, K, 44)
    c0 = _gemm(Ac, As, Bc, Bs, torch.float32, kernel).cpu().numpy()
    As2 = As.copy()
    As2[17] += 1
    c1 = _gemm(Ac, As2, Bc, Bs, torch.float32, kernel).cpu().numpy()
    assert np.array_equal(c1[17], 2 * c0[17])
    assert np.array_equal(np.delete(c1, 17, axis=0), np.delete(c0, 17, axis=0))


@pytest.mark.parametrize("M,kernel", [(96, "auto"), (288, "auto"), (288, "tile"),
                                      (544, "tile")])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_output_written_exactly_in_bounds(M, kernel, out_dtype):
    """C inside a larger buffer: nothing before or after it is written (the
    tile epilogue's masked lanes are dropped by the store resource)."""
    announce(f"gemm canary M={M} {out_dtype} ({kernel})")
    N, K = 320, 512
    Ac, Bc = random_codes(M, K, 51), random_codes(N, K, 52)
    As, Bs = random_scales(M, K, 53), random_scales(N, K, 54)
    pad = 4 * 256 * N  # past the last row, four tiles' worth of rows
    buf = torch.full((M * N + 2 * pad,), 12288.0, dtype=out_dtype, device=DEV)
    out = buf[pad:pad + M * N].view(M, N)
    ENTRY[kernel](u8_to_dev(Ac), u8_to_dev(As), u8_to_dev(Bc), u8_to_dev(Bs), out=out)
    torch.cuda.synchronize()
    b = buf.float().cpu().numpy()
    assert np.all(b[:pad] == 12288.0) and np.all(b[-pad:] == 12288.0)
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    check_gemm_output(out, c_ref, s_ref)


@pytest.mark.parametrize("M", [64, 256])
def test_side_stream(M):
    announce(f"gemm on a side stream M={M}")
    N, K = 512, 768
    Ac, Bc = random_codes(M, K, 61), random_codes(N, K, 62)
    As, Bs = random_scales(M, K, 63), random_scales(N, K, 64)
    args = [u8_to_dev(t) for t in (Ac, As, Bc, Bs)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = mx.gemm(*args, out_dtype=torch.bfloat16)
    s.synchronize()
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    check_gemm_output(out, c_ref, s_ref)


def _workload_operands(w):
    a_bits = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    b_bits = bf16_matrix((w.N, w.K), w.b_dist, w.b_seed)
    ac, as_ = mx.quantize(bf16_to_dev(a_bits))
    bc, bs = mx.quantize(bf16_to_dev(b_bits))
    out_dtype = torch.float32 if w.out_dtype == mx.OUT_FP32 else torch.bfloat16
    return a_bits, b_bits, ac, as_, bc, bs, out_dtype


@pytest.mark.parametrize("name", ["tiny", "skinny", "square", "ragged"])
def test_workload_full_size(name):
    """The workload end to end at full size, every output compared: GPU
    quantize of A and B (bit-exact with the oracle's quantize of all rows),
    GPU GEMM against the oracle's float64 C and S computed from the oracle's
    own codes. The square workload also runs the GEMM on pre-shuffled B (the
    bench step's GEMM), which must give the same bits."""
    w = WORKLOADS[name]
    announce(f"workload {name}: {w.M}x{w.N}x{w.K} out={'fp32' if w.out_dtype else 'bf16'}, full C")
    a_bits, b_bits, ac, as_, bc, bs, out_dtype = _workload_operands(w)
    out = mx.gemm(ac, as_, bc, bs, out_dtype=out_dtype)
    shuf = None
    if name == "square":
        bsh, bssh = mx.shuffle_b(bc, bs)
        shuf = mx.gemm_bshuffled(ac, as_, bsh, bssh, w.N, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ra_c, ra_s = oracle.quantize(a_bits)
    del a_bits
    assert np.array_equal(ac.cpu().numpy(), ra_c) and np.array_equal(as_.cpu().numpy(), ra_s)
    rb_c, rb_s = oracle.quantize(b_bits)
    del b_bits
    assert np.array_equal(bc.cpu().numpy(), rb_c) and np.array_equal(bs.cpu().numpy(), rb_s)
    c_ref, s_ref = oracle.gemm(ra_c, ra_s, rb_c, rb_s)
    misses = check_gemm_output(out, c_ref, s_ref)
    print(f"[gpu] {name}: all {w.M * w.N} outputs compared, literal BF16 misses {misses}",
          flush=True)
    _assert_not_silent_zeros(out.float().cpu().numpy(), c_ref, s_ref)
    if shuf is not None:
        assert torch.equal(out, shuf), "pre-shuffled GEMM differs from mxfp4_gemm"


def _tile_class_rows(M, count, seed):
    """Whole-row sample: rows at every offset class of a 256-row tile (MFMA
    tile row, lane row), spread over tile rows, plus the first and last."""
    rng = np.random.default_rng(seed)
    tiles = rng.integers(0, M // 256, size=count)
    offs = (32 * (np.arange(count) % 8) + rng.integers(0, 32, size=count))
    return np.unique(np.concatenate([256 * tiles + offs, [0, M - 1]]))


@pytest.mark.parametrize("name", ["mlp_gate_up", "mlp_down"])
def test_workload_mlp_whole_rows(name):
    """Llama-MLP shapes at full size: whole rows of C (every column, so every
    tile column, wave and MFMA column of the kernel) at rows of every offset
    class within a tile, and the codes of all of B and of those rows of A
    bit-exact with the oracle's."""
    w = WORKLOADS[name]
    announce(f"workload {name}: {w.M}x{w.N}x{w.K} bf16, whole rows")
    a_bits, b_bits, ac, as_, bc, bs, out_dtype = _workload_operands(w)
    out = mx.gemm(ac, as_, bc, bs, out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = _tile_class_rows(w.M, 40, seed=len(name))
    ra_c, ra_s = oracle.quantize(a_bits[rows])
    del a_bits
    ridx = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(ac[ridx].cpu().numpy(), ra_c)
    assert np.array_equal(as_[ridx].cpu().numpy(), ra_s)
    rb_c, rb_s = oracle.quantize(b_bits)
    del b_bits
    assert np.array_equal(bc.cpu().numpy(), rb_c) and np.array_equal(bs.cpu().numpy(), rb_s)
    c_ref, s_ref = oracle.gemm(ra_c, ra_s, rb_c, rb_s)
    got = out[ridx]
    misses = check_gemm_output(got, c_ref, s_ref)
    print(f"[gpu] {name}: {rows.size} whole rows ({rows.size * w.N} outputs), literal BF16 "
          f"misses {misses}", flush=True)
    _assert_not_silent_zeros(got.float().cpu().numpy(), c_ref, s_ref)


@pytest.mark.parametrize("M", [32, 256])
def test_maximum_k_closed_form(M):
    """K = 2^24, the largest K the GEMM accepts, on both kernels (mxfp4_gemm
    runs the split-K kernel at both M, mxfp4_gemm_tile the tile kernel), on
    the pre-shuffled path and (M = 32) on the fragment-order path. A is all 1.0 (scale 127); row n of B holds 1.0 at
    every k with k % 8192 == 2 n (2048 of them) under scale 127 + n % 3, so
    C[m, n] = 2048 * 2^(n % 3) exactly: every K block of the range counts,
    and any offset overflow along K would change the sums."""
    K, N = 1 << 24, 64
    announce(f"maximum K: M={M} N={N} K={K}")
    a_codes = torch.full((M, K // 2), 0x22, dtype=torch.uint8, device=DEV)
    a_scales = torch.full((M, K // 32), 127, dtype=torch.uint8, device=DEV)
    b_codes = torch.zeros((N, K // 2), dtype=torch.uint8, device=DEV)
    n = torch.arange(N, device=DEV)
    cols = (4096 * torch.arange(K // 8192, device=DEV))[None, :] + n[:, None]   # byte of k = 2n + 8192 t
    b_codes.scatter_(1, cols, 0x02)
    b_scales = (127 + (n % 3)).to(torch.uint8)[:, None].expand(N, K // 32).contiguous()
    want = (2048.0 * 2.0 ** (n % 3).float())[None, :].expand(M, N)
    for dt in (torch.float32, torch.bfloat16):
        for entry in (mx.gemm, mx.gemm_tile):
            got = entry(a_codes, a_scales, b_codes, b_scales, out_dtype=dt)
            torch.cuda.synchronize()
            assert torch.equal(got.float(), want), (dt, entry.__name__)
            del got
    bc, bs = mx.shuffle_b(b_codes, b_scales)
    got = mx.gemm_bshuffled(a_codes, a_scales, bc, bs, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    del bc, bs
    if M <= 128:
        af, asf = mx.to_frag(a_codes, a_scales)
        bf, bsf = mx.to_frag(b_codes, b_scales)
        got = mx.gemm_frag(af, asf, bf, bsf, M, N, K, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, want)


@pytest.mark.parametrize("K", [8192, 14336, 65536])
@pytest.mark.parametrize("M", [32, 256])
def test_fp32_accumulation_worst_case(M, K):
    """A large partial sum first and half-ulp slices after it: every
    sequential fp32 rounding loses its slice. The closed form of C is
    8192 + (K - 256) 2^-17 (all products positive, so S = C); the error must
    stay within fp32_rel_tol(K) * S on the split-K (mxfp4_gemm at both M),
    tile (mxfp4_gemm_tile) and fragment-order kernels, and within 1e-5 * S up
    to K = 8192."""
    N = 64
    announce(f"fp32 accumulation worst case M={M} K={K}")
    ac, as_ = large_block_first(M, K, 127)
    bc, bs = large_block_first(N, K, 128)
    exact = 8192.0 + (K - 256) * 2.0 ** -17
    A, As_, B, Bs = (u8_to_dev(t) for t in (ac, as_, bc, bs))
    outs = {"gemm": mx.gemm(A, As_, B, Bs, out_dtype=torch.float32),
            "gemm_tile": mx.gemm_tile(A, As_, B, Bs, out_dtype=torch.float32)}
    if M <= 128:
        af, asf = mx.to_frag(A, As_)
        bf, bsf = mx.to_frag(B, Bs)
        outs["gemm_frag"] = mx.gemm_frag(af, asf, bf, bsf, M, N, K, out_dtype=torch.float32)
    torch.cuda.synchronize()
    tol = oracle.fp32_rel_tol(K)
    for name, out in outs.items():
        err = np.abs(out.cpu().numpy().astype(np.float64) - exact).max()
        print(f"[gpu] {name}: max error {err:.6g} = {err / exact:.3e} S (bar {tol:.3e} S)",
              flush=True)
        assert err <= tol * exact, name
        if K <= 8192:
            assert err <= oracle.FP32_REL_TOL * exact, name


@pytest.mark.parametrize("K", [65536, 262144])
@pytest.mark.parametrize("M,kernel", [(32, "auto"), (160, "tile")])
def test_fp32_random_operands_long_k(M, kernel, K):
    """Random codes and scales at K far past the workloads' 14336, on both
    kernels, against the oracle at fp32_rel_tol(K)."""
    N = 64
    announce(f"gemm random fp32 {M}x{N}x{K} ({kernel})")
    Ac, Bc = random_codes(M, K, K + M), random_codes(N, K, K + 1)
    As, Bs = random_scales(M, K, K + 2), random_scales(N, K, K + 3)
    out = _gemm(Ac, As, Bc, Bs, torch.float32, kernel)
    c_ref, s_ref = oracle.gemm(Ac, As, Bc, Bs)
    check_gemm_output(out, c_ref, s_ref, K=K)
    _assert_not_silent_zeros(out.cpu().numpy(), c_ref, s_ref)
