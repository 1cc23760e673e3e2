"""The C ABI's host code under AddressSanitizer (CPU only).

Builds libmxfp4.so with the host pass instrumented (device code unchanged)
into a temporary directory, then drives every entry point's argument checks
in a child process with clang's ASan runtime preloaded
(tests/asan_abi_driver.py). Any heap, stack or global overflow in the
argument validation, the per-device state or the error-text table fails the
run. Leak detection is off: the HIP runtime's process-lifetime allocations
are not the library's.
"""

import os
import subprocess
import sys

import pytest

from block_scaled_microscaling_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_argument_checks_under_host_asan(tmp_path):
    runtime = build.asan_runtime()
    if runtime is None:
        pytest.skip("clang's shared ASan runtime is not installed next to hipcc")
    lib = build.build_asan(tmp_path / "libmxfp4_asan.so")
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    res = subprocess.run([sys.executable, os.path.join(HERE, "asan_abi_driver.py"), lib],
                         env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "asan_runtime_mapped 1" in res.stdout, out[-2000:]
