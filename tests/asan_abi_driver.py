"""Child-process driver for the host-ASan check of the C ABI (run by
tests/test_abi_asan.py with the ASan runtime preloaded; not a pytest module).

Calls every entry point of the ASan-instrumented library through ctypes
with null, misaligned and out-of-range arguments, and, when no gfx950
device is present, with valid arguments (which must report "no device"),
asserting each return code. Stand-in pointer values are never dereferenced:
every call here is rejected before anything is launched.

Usage: python asan_abi_driver.py <libmxfp4_asan.so>
"""

import ctypes
import sys

OK, EINVAL, EUNSUPPORTED, ELAUNCH, EALIGN = 0, -1, -2, -3, -4
P = 1 << 20   # 16-byte-aligned stand-in pointer value


def main(path):
    lib = ctypes.CDLL(path)
    vp, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
    sigs = {
        "mxfp4_available": ([], i32),
        "mxfp4_strerror": ([i32], ctypes.c_char_p),
        "mxfp4_quantize": ([vp, i64, i64, vp, vp], i32),
        "mxfp4_quantize_async": ([vp, i64, i64, vp, vp, vp], i32),
        "mxfp4_quantize_2d": ([vp, i64, i64, vp, vp, vp, vp, vp], i32),
        "mxfp4_quantize_sr": ([vp, i64, i64, u64, vp, vp, vp], i32),
        "mxfp4_quantize_2d_sr": ([vp, i64, i64, u64, vp, vp, vp, vp, vp], i32),
        "mxfp4_quantize_sr_rows": ([vp, i64, i64, i64, u64, vp, vp, vp], i32),
        "mxfp4_quantize_2d_sr_rows": ([vp, i64, i64, i64, u64, vp, vp, vp, vp, vp], i32),
        "mxfp4_gemm": ([vp, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "mxfp4_gemm_tile": ([vp, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "mxfp4_gemm_swiglu": ([vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp], i32),
        "mxfp4_shuffle_b_sizes": ([i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)], i32),
        "mxfp4_shuffle_b": ([vp, vp, i64, i64, vp, vp, vp], i32),
        "mxfp4_gemm_bshuffled": ([vp, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
        "mxfp4_quantize_frag": ([vp, i64, i64, vp, vp, vp], i32),
        "mxfp4_to_frag": ([vp, vp, i64, i64, vp, vp, vp], i32),
        "mxfp4_gemm_frag": ([vp, vp, vp, vp, i64, i64, i64, i32, vp, vp], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, res
    L = lib
    checks = 0

    def expect(rc, want, what):
        nonlocal checks
        checks += 1
        if rc != want:
            raise SystemExit(f"{what}: rc {rc}, expected {want}")

    for rc in range(-8, 3):
        text = L.mxfp4_strerror(rc)
        assert text and len(text) > 3, rc
    present = L.mxfp4_available()
    assert present in (0, 1)

    # Rejected before any device check: invalid sizes, nulls, misalignment.
    for M, N, K in [(0, 32, 256), (32, 0, 256), (32, 32, 0), (31, 32, 256), (32, 33, 256),
                    (32, 32, 255), (32, 32, 1 << 25), (1 << 31, 32, 256)]:
        expect(L.mxfp4_gemm(P, P, P, P, M, N, K, 0, P, None), EINVAL, f"gemm {M}x{N}x{K}")
        expect(L.mxfp4_gemm_tile(P, P, P, P, M, N, K, 0, P, None), EINVAL, "gemm_tile")
        expect(L.mxfp4_gemm_bshuffled(P, P, P, P, M, N, K, 0, P, None), EINVAL, "bshuffled")
        expect(L.mxfp4_gemm_frag(P, P, P, P, M, N, K, 0, P, None), EINVAL, "frag")
    # M * N * 4 past int64 (M = N = 2^31 - 32, FP32): rejected, never wrapped.
    big = (1 << 31) - 32
    for dt in (0, 1):
        expect(L.mxfp4_gemm(P, P, P, P, big, big, 256, dt, P, None), EINVAL, "gemm M*N huge")
        expect(L.mxfp4_gemm_tile(P, P, P, P, big, big, 256, dt, P, None), EINVAL,
               "gemm_tile M*N huge")
        expect(L.mxfp4_gemm_bshuffled(P, P, P, P, big, big, 256, dt, P, None), EINVAL,
               "bshuffled M*N huge")
        expect(L.mxfp4_gemm_frag(P, P, P, P, big, big, 256, dt, P, None), EINVAL,
               "frag M*N huge")
    expect(L.mxfp4_gemm_swiglu(P, P, P, P, big, (1 << 31) - 256, 256, P, P, None, None), EINVAL,
           "swiglu M*N huge")
    expect(L.mxfp4_gemm(P, P, P, P, 32, 32, 256, 2, P, None), EINVAL, "gemm dtype")
    expect(L.mxfp4_gemm(None, P, P, P, 32, 32, 256, 0, P, None), EINVAL, "gemm null")
    expect(L.mxfp4_gemm(P + 8, P, P, P, 32, 32, 256, 0, P, None), EALIGN, "gemm align")
    expect(L.mxfp4_gemm(P, P + 2, P, P, 32, 32, 256, 0, P, None), EALIGN, "gemm scale align")
    expect(L.mxfp4_gemm(P, P, P, P, 32, 32, 256, 0, P + 8, None), EALIGN, "gemm C align")
    expect(L.mxfp4_gemm_tile(P + 8, P, P, P, 32, 32, 256, 0, P, None), EALIGN, "tile align")
    for M, K in [(0, 32), (4, 0), (4, 33), (1 << 31, 32), (1 << 21, 1 << 20)]:
        expect(L.mxfp4_quantize(P, M, K, P, P), EINVAL, f"quantize {M}x{K}")
        expect(L.mxfp4_quantize_async(P, M, K, P, P, None), EINVAL, "quantize_async")
        expect(L.mxfp4_quantize_sr(P, M, K, 7, P, P, None), EINVAL, "quantize_sr")
    expect(L.mxfp4_quantize(P + 8, 4, 32, P, P), EALIGN, "quantize align")
    expect(L.mxfp4_quantize(None, 4, 32, P, P), EINVAL, "quantize null")
    for M, K in [(16, 32), (32, 16), (48, 64), (1 << 31, 32)]:
        expect(L.mxfp4_quantize_2d(P, M, K, P, P, P, P, None), EINVAL, f"2d {M}x{K}")
        expect(L.mxfp4_quantize_2d_sr(P, M, K, 3, P, P, P, P, None), EINVAL, "2d_sr")
    expect(L.mxfp4_quantize_2d(P, 32, 32, P, P, P + 8, P, None), EALIGN, "2d align")
    for M, row0 in [(4, -1), (4, (1 << 31) - 4), ((1 << 31) - 1, 1)]:
        expect(L.mxfp4_quantize_sr_rows(P, M, 32, row0, 7, P, P, None), EINVAL, "sr_rows")
    for row0 in (-32, 16, (1 << 31) - 64):
        expect(L.mxfp4_quantize_2d_sr_rows(P, 64, 64, row0, 3, P, P, P, P, None), EINVAL,
               "2d_sr_rows")
    for M, N, K in [(32, 128, 256), (32, 256, 128), (0, 256, 256)]:
        expect(L.mxfp4_gemm_swiglu(P, P, P, P, M, N, K, P, P, None, None), EINVAL, "swiglu")
    expect(L.mxfp4_gemm_swiglu(P, P, P, P, 32, 256, 256, P, P, P + 8, None), EALIGN,
           "swiglu act align")
    cb, sb = ctypes.c_int64(-1), ctypes.c_int64(-1)
    expect(L.mxfp4_shuffle_b_sizes(300, 1280, ctypes.byref(cb), ctypes.byref(sb)), OK, "sizes")
    assert (cb.value, sb.value) == (2 * 5 * 32768, 2 * 2 * 8192), (cb.value, sb.value)
    expect(L.mxfp4_shuffle_b_sizes(300, 1280, None, ctypes.byref(sb)), EINVAL, "sizes null")
    expect(L.mxfp4_shuffle_b_sizes(0, 1280, ctypes.byref(cb), ctypes.byref(sb)), EINVAL,
           "sizes N")
    expect(L.mxfp4_shuffle_b(P, P, 32, 100, P, P, None), EINVAL, "shuffle K")
    expect(L.mxfp4_shuffle_b(P, P + 2, 32, 256, P, P, None), EALIGN, "shuffle align")
    for R, K in [(16, 256), (32, 128), (32, 1 << 25)]:
        expect(L.mxfp4_quantize_frag(P, R, K, P, P, None), EINVAL, "quantize_frag")
        expect(L.mxfp4_to_frag(P, P, R, K, P, P, None), EINVAL, "to_frag")
    expect(L.mxfp4_to_frag(P, P, 32, 256, P + 4, P, None), EALIGN, "to_frag align")

    # Valid arguments: with no gfx950 device they must report "no device"
    # and launch nothing. With a device present they would launch, so the
    # stand-in pointers stay out of them.
    if present == 0:
        U = EUNSUPPORTED
        expect(L.mxfp4_gemm(P, P, P, P, 32, 32, 256, 0, P, None), U, "gemm")
        expect(L.mxfp4_gemm(P, P, P, P, 256, 256, 1024, 1, P, None), U, "gemm 256^2")
        expect(L.mxfp4_gemm_tile(P, P, P, P, 256, 256, 1024, 1, P, None), U, "gemm_tile")
        expect(L.mxfp4_quantize(P, 4, 32, P, P), U, "quantize")
        expect(L.mxfp4_quantize_2d(P, 32, 32, P, P, P, P, None), U, "2d")
        expect(L.mxfp4_quantize_sr(P, 4, 32, 5, P, P, None), U, "sr")
        expect(L.mxfp4_quantize_2d_sr(P, 32, 32, 5, P, P, P, P, None), U, "2d_sr")
        expect(L.mxfp4_quantize_sr_rows(P, 4, 32, 64, 5, P, P, None), U, "sr_rows")
        expect(L.mxfp4_quantize_2d_sr_rows(P, 32, 32, 64, 5, P, P, P, P, None), U,
               "2d_sr_rows")
        expect(L.mxfp4_gemm_swiglu(P, P, P, P, 32, 256, 256, P, P, None, None), U, "swiglu")
        expect(L.mxfp4_shuffle_b(P, P, 32, 256, P, P, None), U, "shuffle")
        expect(L.mxfp4_gemm_bshuffled(P, P, P, P, 32, 32, 256, 0, P, None), U, "bshuffled")
        expect(L.mxfp4_quantize_frag(P, 32, 256, P, P, None), U, "quantize_frag")
        expect(L.mxfp4_to_frag(P, P, 32, 256, P, P, None), U, "to_frag")
        expect(L.mxfp4_gemm_frag(P, P, P, P, 32, 32, 256, 0, P, None), U, "gemm_frag")
    with open("/proc/self/maps") as f:
        asan = "libclang_rt.asan" in f.read()
    print(f"checks {checks} device {present} asan_runtime_mapped {int(asan)}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
