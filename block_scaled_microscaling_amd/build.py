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


if __name__ == "__main__":
    build()
