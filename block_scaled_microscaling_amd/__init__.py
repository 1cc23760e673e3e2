"""MXFP4 quantize and block-scaled GEMM on AMD gfx950 (MI355X).

A thin binding over the C ABI of libmxfp4.so (include/mxfp4.h). Every step
of the computation runs in the library's HIP kernels; this module only
marshals arguments. PyTorch supplies device memory and streams.

Two layers, same names as the C ABI:
  * mxfp4_available, mxfp4_strerror, mxfp4_quantize, mxfp4_quantize_async,
    mxfp4_quantize_2d, mxfp4_quantize_sr, mxfp4_quantize_2d_sr,
    mxfp4_quantize_sr_rows, mxfp4_quantize_2d_sr_rows, mxfp4_gemm,
    mxfp4_gemm_tile, mxfp4_gemm_swiglu, mxfp4_shuffle_b(_sizes), mxfp4_gemm_bshuffled,
    mxfp4_quantize_frag, mxfp4_to_frag, mxfp4_gemm_frag take raw device
    pointers (ints) and return the C status code.
  * quantize(x), quantize_2d(x), quantize_sr(x, seed, row0=0),
    quantize_2d_sr(x, seed, row0=0), gemm(...), gemm_tile(...) and
    gemm_swiglu(...) take torch tensors,
    check their dtype, device, shape and contiguity, allocate outputs when none
    are given, enqueue on torch's current stream and raise Mxfp4Error on a
    non-zero status.

If the library is missing the functions raise: there is no fallback path.
"""

import ctypes
import os

__all__ = [
    "Mxfp4Error", "OUT_BF16", "OUT_FP32", "library_path", "load_library",
    "mxfp4_available", "mxfp4_strerror", "mxfp4_quantize", "mxfp4_quantize_async",
    "mxfp4_quantize_2d", "mxfp4_quantize_sr", "mxfp4_quantize_2d_sr", "mxfp4_quantize_sr_rows",
    "mxfp4_quantize_2d_sr_rows", "mxfp4_gemm",
    "mxfp4_gemm_tile", "mxfp4_gemm_swiglu", "quantize", "quantize_2d", "quantize_sr",
    "quantize_2d_sr", "gemm", "gemm_tile",
    "gemm_swiglu", "mxfp4_shuffle_b_sizes", "mxfp4_shuffle_b", "mxfp4_gemm_bshuffled",
    "shuffle_b", "gemm_bshuffled", "mxfp4_quantize_frag", "mxfp4_to_frag", "mxfp4_gemm_frag",
    "quantize_frag", "to_frag", "gemm_frag",
]

OUT_BF16 = 0
OUT_FP32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmxfp4.so")
_lib = None


class Mxfp4Error(RuntimeError):
    def __init__(self, rc, what):
        super().__init__(f"{what} failed: rc={rc} ({mxfp4_strerror(rc)})")
        self.rc = rc


def load_library():
    """Load libmxfp4.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it with "
                "`python -m block_scaled_microscaling_amd.build`")
        lib = ctypes.CDLL(library_path)
        vp, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
        lib.mxfp4_available.argtypes = []
        lib.mxfp4_available.restype = i32
        lib.mxfp4_strerror.argtypes = [i32]
        lib.mxfp4_strerror.restype = ctypes.c_char_p
        lib.mxfp4_quantize.argtypes = [vp, i64, i64, vp, vp]
        lib.mxfp4_quantize.restype = i32
        lib.mxfp4_quantize_async.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.mxfp4_quantize_async.restype = i32
        lib.mxfp4_quantize_2d.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        lib.mxfp4_quantize_2d.restype = i32
        lib.mxfp4_quantize_sr.argtypes = [vp, i64, i64, u64, vp, vp, vp]
        lib.mxfp4_quantize_sr.restype = i32
        lib.mxfp4_quantize_2d_sr.argtypes = [vp, i64, i64, u64, vp, vp, vp, vp, vp]
        lib.mxfp4_quantize_2d_sr.restype = i32
        lib.mxfp4_quantize_sr_rows.argtypes = [vp, i64, i64, i64, u64, vp, vp, vp]
        lib.mxfp4_quantize_sr_rows.restype = i32
        lib.mxfp4_quantize_2d_sr_rows.argtypes = [vp, i64, i64, i64, u64, vp, vp, vp, vp, vp]
        lib.mxfp4_quantize_2d_sr_rows.restype = i32
        lib.mxfp4_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
        lib.mxfp4_gemm.restype = i32
        lib.mxfp4_gemm_tile.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
        lib.mxfp4_gemm_tile.restype = i32
        lib.mxfp4_gemm_swiglu.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp]
        lib.mxfp4_gemm_swiglu.restype = i32
        lib.mxfp4_shuffle_b_sizes.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.mxfp4_shuffle_b_sizes.restype = i32
        lib.mxfp4_shuffle_b.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        lib.mxfp4_shuffle_b.restype = i32
        lib.mxfp4_gemm_bshuffled.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
        lib.mxfp4_gemm_bshuffled.restype = i32
        lib.mxfp4_quantize_frag.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.mxfp4_quantize_frag.restype = i32
        lib.mxfp4_to_frag.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        lib.mxfp4_to_frag.restype = i32
        lib.mxfp4_gemm_frag.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
        lib.mxfp4_gemm_frag.restype = i32
        _lib = lib
    return _lib


# ----------------------------------------------------------- raw C ABI names
def mxfp4_available():
    return int(load_library().mxfp4_available())


def mxfp4_strerror(rc):
    return load_library().mxfp4_strerror(int(rc)).decode()


def mxfp4_quantize(x_bf16, M, K, codes_out, scales_out):
    return int(load_library().mxfp4_quantize(x_bf16, M, K, codes_out, scales_out))


def mxfp4_quantize_async(x_bf16, M, K, codes_out, scales_out, stream):
    return int(load_library().mxfp4_quantize_async(x_bf16, M, K, codes_out, scales_out, stream))


def mxfp4_quantize_2d(x_bf16, M, K, codes_row, scales_row, codes_col, scales_col, stream):
    return int(load_library().mxfp4_quantize_2d(x_bf16, M, K, codes_row, scales_row, codes_col,
                                                scales_col, stream))


def mxfp4_quantize_sr(x_bf16, M, K, seed, codes_out, scales_out, stream):
    return int(load_library().mxfp4_quantize_sr(x_bf16, M, K, seed, codes_out, scales_out,
                                                stream))


def mxfp4_quantize_2d_sr(x_bf16, M, K, seed, codes_row, scales_row, codes_col, scales_col,
                         stream):
    return int(load_library().mxfp4_quantize_2d_sr(x_bf16, M, K, seed, codes_row, scales_row,
                                                   codes_col, scales_col, stream))


def mxfp4_quantize_sr_rows(x_bf16, M, K, row0, seed, codes_out, scales_out, stream):
    return int(load_library().mxfp4_quantize_sr_rows(x_bf16, M, K, row0, seed, codes_out,
                                                     scales_out, stream))


def mxfp4_quantize_2d_sr_rows(x_bf16, M, K, row0, seed, codes_row, scales_row, codes_col,
                              scales_col, stream):
    return int(load_library().mxfp4_quantize_2d_sr_rows(x_bf16, M, K, row0, seed, codes_row,
                                                        scales_row, codes_col, scales_col,
                                                        stream))


def mxfp4_gemm(A_codes, A_scales, B_codes, B_scales, M, N, K, out_dtype, C, stream):
    return int(load_library().mxfp4_gemm(A_codes, A_scales, B_codes, B_scales, M, N, K,
                                         out_dtype, C, stream))


def mxfp4_gemm_tile(A_codes, A_scales, B_codes, B_scales, M, N, K, out_dtype, C, stream):
    return int(load_library().mxfp4_gemm_tile(A_codes, A_scales, B_codes, B_scales, M, N, K,
                                              out_dtype, C, stream))


def mxfp4_gemm_swiglu(A_codes, A_scales, B_codes, B_scales, M, N, K, act_codes, act_scales,
                      act_bf16, stream):
    return int(load_library().mxfp4_gemm_swiglu(A_codes, A_scales, B_codes, B_scales, M, N, K,
                                                act_codes, act_scales, act_bf16, stream))


def mxfp4_shuffle_b_sizes(N, K):
    """(rc, code_bytes, scale_bytes) of the pre-shuffled layout of B [N, K]."""
    cb, sb = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = int(load_library().mxfp4_shuffle_b_sizes(N, K, ctypes.byref(cb), ctypes.byref(sb)))
    return rc, cb.value, sb.value


def mxfp4_shuffle_b(codes, scales, N, K, codes_sh, scales_sh, stream):
    return int(load_library().mxfp4_shuffle_b(codes, scales, N, K, codes_sh, scales_sh, stream))


def mxfp4_gemm_bshuffled(A_codes, A_scales, Bsh_codes, Bsh_scales, M, N, K, out_dtype, C, stream):
    return int(load_library().mxfp4_gemm_bshuffled(A_codes, A_scales, Bsh_codes, Bsh_scales, M, N,
                                                   K, out_dtype, C, stream))


def mxfp4_quantize_frag(x_bf16, M, K, codes_frag, scales_frag, stream):
    return int(load_library().mxfp4_quantize_frag(x_bf16, M, K, codes_frag, scales_frag, stream))


def mxfp4_to_frag(codes, scales, R, K, codes_frag, scales_frag, stream):
    return int(load_library().mxfp4_to_frag(codes, scales, R, K, codes_frag, scales_frag, stream))


def mxfp4_gemm_frag(A_frag, A_scales_frag, B_frag, B_scales_frag, M, N, K, out_dtype, C, stream):
    return int(load_library().mxfp4_gemm_frag(A_frag, A_scales_frag, B_frag, B_scales_frag, M, N,
                                              K, out_dtype, C, stream))


# ------------------------------------------------------- torch tensor layer
def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(t, name, dtype, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def quantize(x, codes=None, scales=None, stream=None):
    """Row-wise BF16 -> MXFP4. x: bfloat16 [M, K] on the GPU.

    Returns (codes uint8 [M, K/2], scales uint8 [M, K/32]).
    """
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    _check(x, "x", torch.bfloat16, (M, K))
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check(codes, "codes", torch.uint8, (M, K // 2))
    _check(scales, "scales", torch.uint8, (M, K // 32))
    rc = mxfp4_quantize_async(x.data_ptr(), M, K, codes.data_ptr(), scales.data_ptr(),
                              _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_quantize")
    return codes, scales


def quantize_2d(x, stream=None):
    """Row-wise and column-wise BF16 -> MXFP4 in one pass. x: bfloat16 [M, K].

    Returns (codes [M, K/2], scales [M, K/32], codes_t [K, M/2], scales_t
    [K, M/32]), uint8: the MXFP4 forms of x and of x^T.
    """
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    _check(x, "x", torch.bfloat16, (M, K))
    dev = x.device
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    codes_t = torch.empty((K, M // 2), dtype=torch.uint8, device=dev)
    scales_t = torch.empty((K, M // 32), dtype=torch.uint8, device=dev)
    rc = mxfp4_quantize_2d(x.data_ptr(), M, K, codes.data_ptr(), scales.data_ptr(),
                           codes_t.data_ptr(), scales_t.data_ptr(), _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_quantize_2d")
    return codes, scales, codes_t, scales_t


def _seed(seed):
    seed = int(seed)
    if not 0 <= seed < (1 << 64):
        raise ValueError("seed must be in [0, 2**64)")
    return seed


def quantize_sr(x, seed, codes=None, scales=None, stream=None, row0=0):
    """Row-wise BF16 -> MXFP4 with stochastic rounding (Philox4x32-10 keyed by
    block coordinates and the 64-bit `seed`). x: bfloat16 [M, K] on the GPU,
    rows row0 .. row0 + M - 1 of a larger input (the draws key by those
    global rows; row0 = 0 is the plain call).

    Returns (codes uint8 [M, K/2], scales uint8 [M, K/32]).
    """
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    _check(x, "x", torch.bfloat16, (M, K))
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check(codes, "codes", torch.uint8, (M, K // 2))
    _check(scales, "scales", torch.uint8, (M, K // 32))
    rc = mxfp4_quantize_sr_rows(x.data_ptr(), M, K, int(row0), _seed(seed), codes.data_ptr(),
                                scales.data_ptr(), _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_quantize_sr_rows")
    return codes, scales


def quantize_2d_sr(x, seed, stream=None, row0=0):
    """Row-wise and column-wise BF16 -> MXFP4 with stochastic rounding; x
    may be rows row0 .. of a larger input (row0 % 32 == 0), whose global
    rows and row blocks key the draws.

    Returns (codes [M, K/2], scales [M, K/32], codes_t [K, M/2], scales_t
    [K, M/32]), uint8.
    """
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    _check(x, "x", torch.bfloat16, (M, K))
    dev = x.device
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    codes_t = torch.empty((K, M // 2), dtype=torch.uint8, device=dev)
    scales_t = torch.empty((K, M // 32), dtype=torch.uint8, device=dev)
    rc = mxfp4_quantize_2d_sr_rows(x.data_ptr(), M, K, int(row0), _seed(seed), codes.data_ptr(),
                                   scales.data_ptr(), codes_t.data_ptr(), scales_t.data_ptr(),
                                   _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_quantize_2d_sr_rows")
    return codes, scales, codes_t, scales_t


def gemm(A_codes, A_scales, B_codes, B_scales, out_dtype=None, out=None, stream=None):
    """C[M, N] = dq(A) @ dq(B)^T from packed MXFP4 operands (B is N x K).

    out_dtype: torch.bfloat16 (default) or torch.float32.
    """
    return _gemm_call(mxfp4_gemm, "mxfp4_gemm", A_codes, A_scales, B_codes, B_scales, out_dtype,
                      out, stream)


def gemm_tile(A_codes, A_scales, B_codes, B_scales, out_dtype=None, out=None, stream=None):
    """gemm() on the 256 x 256 tile kernel whatever the shape."""
    return _gemm_call(mxfp4_gemm_tile, "mxfp4_gemm_tile", A_codes, A_scales, B_codes, B_scales,
                      out_dtype, out, stream)


def _gemm_call(fn, name, A_codes, A_scales, B_codes, B_scales, out_dtype, out, stream):
    import torch
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if A_codes.dim() != 2 or B_codes.dim() != 2:
        raise ValueError("code tensors must be 2-D")
    M, K = A_codes.shape[0], A_codes.shape[1] * 2
    N = B_codes.shape[0]
    _check(A_codes, "A_codes", torch.uint8, (M, K // 2))
    _check(B_codes, "B_codes", torch.uint8, (N, K // 2))
    _check(A_scales, "A_scales", torch.uint8, (M, K // 32))
    _check(B_scales, "B_scales", torch.uint8, (N, K // 32))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A_codes.device)
    _check(out, "out", out_dtype, (M, N))
    code = OUT_FP32 if out_dtype == torch.float32 else OUT_BF16
    rc = fn(A_codes.data_ptr(), A_scales.data_ptr(), B_codes.data_ptr(), B_scales.data_ptr(), M, N,
            K, code, out.data_ptr(), _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, name)
    return out


def gemm_swiglu(A_codes, A_scales, B_codes, B_scales, want_act=False, stream=None):
    """Gate+up GEMM with the SwiGLU + MXFP4 requantize epilogue.

    B_codes [N, K/2] / B_scales [N, K/32] hold the stacked [W_gate; W_up]
    (N/2 rows each). Returns (act_codes uint8 [M, N/4], act_scales uint8
    [M, N/64]) and, with want_act, also the BF16 act [M, N/2] the codes were
    quantized from.
    """
    import torch
    M, Kh = A_codes.shape
    K = 2 * Kh
    N = B_codes.shape[0]
    _check(A_codes, "A_codes", torch.uint8, (M, K // 2))
    _check(A_scales, "A_scales", torch.uint8, (M, K // 32))
    _check(B_codes, "B_codes", torch.uint8, (N, K // 2))
    _check(B_scales, "B_scales", torch.uint8, (N, K // 32))
    dev = A_codes.device
    Nh = N // 2
    codes = torch.empty((M, Nh // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, max(Nh // 32, 0)), dtype=torch.uint8, device=dev)
    act = torch.empty((M, Nh), dtype=torch.bfloat16, device=dev) if want_act else None
    rc = mxfp4_gemm_swiglu(A_codes.data_ptr(), A_scales.data_ptr(), B_codes.data_ptr(),
                           B_scales.data_ptr(), M, N, K, codes.data_ptr(), scales.data_ptr(),
                           None if act is None else act.data_ptr(), _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_gemm_swiglu")
    return (codes, scales, act) if want_act else (codes, scales)


def shuffle_b(B_codes, B_scales, stream=None):
    """Pre-shuffle an MXFP4 weight for gemm_bshuffled. Returns (codes_sh,
    scales_sh) as flat uint8 device tensors in the library's block layout."""
    import torch
    N, Kh = B_codes.shape
    K = 2 * Kh
    _check(B_codes, "B_codes", torch.uint8, (N, K // 2))
    _check(B_scales, "B_scales", torch.uint8, (N, K // 32))
    rc, cb, sb = mxfp4_shuffle_b_sizes(N, K)
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_shuffle_b_sizes")
    dev = B_codes.device
    codes_sh = torch.empty(cb, dtype=torch.uint8, device=dev)
    scales_sh = torch.empty(sb, dtype=torch.uint8, device=dev)
    rc = mxfp4_shuffle_b(B_codes.data_ptr(), B_scales.data_ptr(), N, K, codes_sh.data_ptr(),
                         scales_sh.data_ptr(), _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_shuffle_b")
    return codes_sh, scales_sh


def gemm_bshuffled(A_codes, A_scales, Bsh_codes, Bsh_scales, N, out_dtype=None, out=None,
                   stream=None):
    """gemm() with B pre-shuffled by shuffle_b (N: rows of B)."""
    import torch
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    M, K = A_codes.shape[0], A_codes.shape[1] * 2
    _check(A_codes, "A_codes", torch.uint8, (M, K // 2))
    _check(A_scales, "A_scales", torch.uint8, (M, K // 32))
    rc, cb, sb = mxfp4_shuffle_b_sizes(N, K)
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_shuffle_b_sizes")
    _check(Bsh_codes, "Bsh_codes", torch.uint8, (cb,))
    _check(Bsh_scales, "Bsh_scales", torch.uint8, (sb,))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A_codes.device)
    _check(out, "out", out_dtype, (M, N))
    code = OUT_FP32 if out_dtype == torch.float32 else OUT_BF16
    rc = mxfp4_gemm_bshuffled(A_codes.data_ptr(), A_scales.data_ptr(), Bsh_codes.data_ptr(),
                              Bsh_scales.data_ptr(), M, N, K, code, out.data_ptr(),
                              _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_gemm_bshuffled")
    return out


def quantize_frag(x, codes=None, scales=None, stream=None):
    """Row-wise BF16 -> MXFP4 written in fragment order. x: bfloat16 [M, K]
    (M % 32 == 0, K % 256 == 0). Returns flat uint8 (codes [M*K/2], scales
    [M*K/32])."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    _check(x, "x", torch.bfloat16, (M, K))
    if codes is None:
        codes = torch.empty(M * K // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(M * K // 32, dtype=torch.uint8, device=x.device)
    _check(codes, "codes", torch.uint8, (M * K // 2,))
    _check(scales, "scales", torch.uint8, (M * K // 32,))
    rc = mxfp4_quantize_frag(x.data_ptr(), M, K, codes.data_ptr(), scales.data_ptr(),
                             _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_quantize_frag")
    return codes, scales


def to_frag(codes, scales, stream=None):
    """Plain MXFP4 codes [R, K/2] and scales [R, K/32] -> fragment order (flat
    uint8 codes [R*K/2], scales [R*K/32])."""
    import torch
    R, Kh = codes.shape
    K = 2 * Kh
    _check(codes, "codes", torch.uint8, (R, K // 2))
    _check(scales, "scales", torch.uint8, (R, K // 32))
    cf = torch.empty(R * K // 2, dtype=torch.uint8, device=codes.device)
    sf = torch.empty(R * K // 32, dtype=torch.uint8, device=codes.device)
    rc = mxfp4_to_frag(codes.data_ptr(), scales.data_ptr(), R, K, cf.data_ptr(), sf.data_ptr(),
                       _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_to_frag")
    return cf, sf


def gemm_frag(A_frag, A_scales_frag, B_frag, B_scales_frag, M, N, K, out_dtype=None, out=None,
              stream=None):
    """gemm() with both operands in fragment order (flat uint8 tensors)."""
    import torch
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    _check(A_frag, "A_frag", torch.uint8, (M * K // 2,))
    _check(A_scales_frag, "A_scales_frag", torch.uint8, (M * K // 32,))
    _check(B_frag, "B_frag", torch.uint8, (N * K // 2,))
    _check(B_scales_frag, "B_scales_frag", torch.uint8, (N * K // 32,))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A_frag.device)
    _check(out, "out", out_dtype, (M, N))
    code = OUT_FP32 if out_dtype == torch.float32 else OUT_BF16
    rc = mxfp4_gemm_frag(A_frag.data_ptr(), A_scales_frag.data_ptr(), B_frag.data_ptr(),
                         B_scales_frag.data_ptr(), M, N, K, code, out.data_ptr(),
                         _stream_handle(stream))
    if rc != 0:
        raise Mxfp4Error(rc, "mxfp4_gemm_frag")
    return out
