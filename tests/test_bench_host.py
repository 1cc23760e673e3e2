"""Host logic of bench.py (CPU only): the one-GPU refusal and the rule that
HBM traffic from rocprofv3 counters is reported only for the kernel sources
it was measured on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_device_work():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def _entry(tmp_path, sources, sha, nbytes=1234):
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"workloads": {"square": {
        "sources": sources, "sha256": sha, "bytes_per_launch": nbytes}}}))
    return str(path)


def test_traffic_reported_only_for_the_measured_sources(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    rel = os.path.relpath(src, ROOT)
    good = bench.source_digest([rel])
    assert bench.read_traffic(_entry(tmp_path, [rel], good), "square") == 1234
    # Any change to the sources makes the stored counters stale: null.
    src.write_text("kernel v2\n")
    assert bench.read_traffic(_entry(tmp_path, [rel], good), "square") is None
    # Unknown workload, missing file, malformed file: null.
    assert bench.read_traffic(_entry(tmp_path, [rel], good), "skinny") is None
    assert bench.read_traffic(str(tmp_path / "absent.json"), "square") is None
    bad = tmp_path / "bad.json"
    bad.write_text("{not json")
    assert bench.read_traffic(str(bad), "square") is None


def test_source_digest_depends_on_every_source_and_their_order(tmp_path):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("a\n")
    b.write_text("b\n")
    ra, rb = os.path.relpath(a, ROOT), os.path.relpath(b, ROOT)
    d_ab = bench.source_digest([ra, rb])
    assert d_ab == bench.source_digest([ra, rb])
    assert d_ab != bench.source_digest([rb, ra])
    assert d_ab != bench.source_digest([ra])


def test_operand_rotation_covers_twice_the_cache_with_a_cap():
    llc = bench.LLC_BYTES
    assert bench.copies_for(3 * llc) == 1
    assert bench.copies_for(llc // 2) == 4
    assert bench.copies_for(llc) == 2 and bench.copies_for(llc + 1) == 2
    assert bench.copies_for((2 * llc) // 3) == 4     # floored: 3 copies fall short
    assert bench.copies_for(1000) == bench.MAX_COPIES
    for nbytes in (35_651_584, 71_303_168, 205_520_896):
        n = bench.copies_for(nbytes)
        assert n * nbytes >= 2 * llc and (n - 1) * nbytes < 2 * llc


def test_roofline_bound_and_short_kernels():
    r = bench.gemm_roofline(8192, 8192, 8192, 2, 0.2)
    assert r["bound"] == "mfma" and abs(r["achieved"] - 2 * 8192 ** 3 / 0.2e-3 / 1e12) < 1e-6
    assert abs(r["frac"] - r["achieved"] / bench.FP4_DENSE_PEAK_TFLOPS) < 1e-12
    r = bench.gemm_roofline(32, 8192, 8192, 2, 0.008)
    nbytes = (32 + 8192) * (4096 + 256) + 32 * 8192 * 2
    assert r["bound"] == "hbm" and abs(r["achieved"] - nbytes / 8e-6 / 1e9) < 1e-6
    assert bench.is_short(32, 8192, 8192) and bench.is_short(256, 256, 256)
    assert not bench.is_short(4128, 6176, 7936) and not bench.is_short(8192, 8192, 8192)


def test_profiled_mfma_quotes_the_counter_profile():
    got = bench.profiled_mfma()
    assert got is not None, "the headline GEMM's row is missing from the MFMA profile"
    assert 0.5 < got["clock_ghz"] < 2.5
    assert 0.0 < got["mfma_busy"] <= 1.0
    assert got["source"] == "profiles/gemm_mfma_utilisation_counters.md"
    assert bench.profiled_mfma(kernel="no_such_kernel") is None
