"""The C ABI used from plain C (tests/c_abi/c_abi_check.c): no Python in the
process, only include/mxfp4.h, libmxfp4.so and the HIP runtime for device
memory. The program quantizes power-of-two operands, runs the GEMM on the
row-major and fragment-order paths into FP32 and BF16, checks every byte and
output against its closed form, and checks rejected calls' status codes.
"""

import os
import subprocess

import pytest

from block_scaled_microscaling_amd import build

LIB_DIR = os.path.dirname(build.LIB)


def test_c_program_compiles_against_the_header_and_runs(tmp_path):
    """CPU: the header compiles as C11 with -Wall -Wextra and links; without
    a gfx950 device the program reports it and exits 2 (with one, it runs
    its checks and must pass them)."""
    if not os.path.exists(build.LIB):
        pytest.skip("libmxfp4.so is not built")
    exe = build.build_c_check(tmp_path / "c_abi_check", verbose=False)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode in (0, 2), res.stdout + res.stderr
    if res.returncode == 2:
        assert "no gfx950 device" in res.stderr
    else:
        assert "c_abi_check: OK" in res.stdout


@pytest.mark.gpu
def test_c_program_checks_pass_on_the_gpu():
    exe = build.C_CHECK_BIN
    assert os.path.exists(exe), ("the C ABI check program is not built: run "
                                 "python -m block_scaled_microscaling_amd.build")
    print("\n[gpu] c_abi_check", flush=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c_abi_check: OK (0 failures)" in res.stdout
