"""Build libmxfp4.so for gfx950 with hipcc, in-tree next to this file.

    python -m block_scaled_microscaling_amd.build

Compiles every HIP source under csrc/ into one shared library. Packed FP32
instructions are switched off for all device code (-packed-fp32-ops).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxfp4.so")
SOURCES = ["api.hip", "quantize.hip", "quantize_sr.hip", "quantize2d.hip", "gemm.hip",
           "gemm_skinny.hip", "shuffle.hip"]
ARCH = "gfx950"


def hipcc_command(out=LIB):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return [
        hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument", "-Wno-inline-asm",
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose=True):
    """Compile the library; raises CalledProcessError on a compiler error."""
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so: harmless.
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + err + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd)
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, LIB)
    return LIB


# A plain C program that drives the library through include/mxfp4.h alone
# (tests/c_abi/c_abi_check.c), built next to the library by gcc: the C ABI
# used with no Python in the process.
C_CHECK_SRC = os.path.join(os.path.dirname(HERE), "tests", "c_abi", "c_abi_check.c")
C_CHECK_BIN = os.path.join(HERE, "c_abi_check")


def c_check_command(out=C_CHECK_BIN, libdir=HERE):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
            "-I" + os.path.join(rocm, "include"),
            "-I" + os.path.join(os.path.dirname(HERE), "include"), C_CHECK_SRC,
            "-L" + libdir, "-L" + os.path.join(rocm, "lib"), "-lmxfp4", "-lamdhip64",
            "-Wl,-rpath," + libdir, "-Wl,-rpath,$ORIGIN", "-o", str(out)]


def build_c_check(out=C_CHECK_BIN, libdir=HERE, verbose=True):
    """Compile the C ABI check program against libmxfp4.so in `libdir`."""
    cmd = c_check_command(out, libdir)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd)
    return str(out)


# The MFMA / LDS microbenchmark (probe/mfma_lds_probe.hip): a standalone
# executable, built next to the library and run by `python bench.py --probe`.
PROBE_SRC = os.path.join(HERE, "probe", "mfma_lds_probe.hip")
PROBE_BIN = os.path.join(HERE, "mfma_lds_probe")


def build_probe(out=PROBE_BIN, verbose=True):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-o", str(out), PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd)
    return str(out)


# Section timing of the tile GEMM (probe/gemm_sections.hip): a standalone
# executable that includes csrc/gemm.hip with its section timers switched on,
# run by `python bench.py --sections`.
SECTIONS_SRC = os.path.join(HERE, "probe", "gemm_sections.hip")
SECTIONS_BIN = os.path.join(HERE, "gemm_sections")


def build_sections(out=SECTIONS_BIN, verbose=True):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-Wno-inline-asm", "-o", str(out), SECTIONS_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd)
    return str(out)


# Host-only AddressSanitizer: the device code is built as usual and the host
# code (the C ABI's argument checks, launchers, per-device state) is
# instrumented. Loading the result needs the matching runtime preloaded
# (asan_runtime()). Each sanitizer flag applies to the host pass only.
ASAN_HOST_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer"


def asan_runtime():
    """Path of clang's shared ASan runtime next to hipcc, or None."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    res = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def build_asan(out, verbose=False):
    """Compile the library with host-side ASan into `out`."""
    cmd = hipcc_command(str(out))
    cmd = cmd[:1] + ["-O1", "-g"] + [a for a in cmd[1:] if a != "-O3"]
    cmd += ASAN_HOST_FLAGS.split() + ["-shared-libasan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd)
    return str(out)


if __name__ == "__main__":
    build()
    build_c_check()
    build_probe()
