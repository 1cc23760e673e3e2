"""Benchmark of the MXFP4 hot path on one MI355X (gfx950).

Headline step = row-wise BF16 -> MXFP4 quantize of the activation A [M, K]
(mxfp4_quantize) plus the block-scaled GEMM C = dq(A) dq(B)^T against
pre-quantized weights B [N, K] in their plain row-major layout (mxfp4_gemm,
the contract entry point), on the square workload M = N = K = 8192 with BF16
output. Inputs are seeded synthetic BF16 (N(0,1) with 1% of entries x100)
resident in HBM before the timed region; weight quantization happens before
it. The step rotates through several copies of its activation and weights
(more than twice the 256 MB last-level cache in all), so each step reads its
operands from HBM.

Order of work: inputs and weights are prepared, then every per-kernel time
of the headline workload is taken, then W untimed and K timed steps run.

Per-kernel times: each kernel runs at least 50 untimed launches (and at
least 100 ms) on the launch stream, then 10 groups of 10 back-to-back
launches, each group between one HIP event pair on that stream; the figure
is the median of the 10 group means (events between single launches would
add a few microseconds to each). Launches rotate through operand copies as
the step does.

Prints one JSON line:
  value        2*M*N*K / (time per step), TFLOP/s, whole step (quantize + GEMM)
  roofline     the step's GEMM kernel against the FP4 MFMA dense peak
               (10.1 PFLOP/s): achieved = 2*M*N*K / median launch time
  profiled_mfma  the headline GEMM's engine clock and MFMA utilisation as
               rocprofv3's counters measured them (quoted from the committed
               profile), against the 2400 MHz the peak assumes
  configs      every workload: GEMM time, its roofline (FP4 MFMA peak, or
               HBM for GEMMs with at most 128 rows of A, whose bytes are
               mostly B), quantize time and rate of its activation, the
               faster layout variant, and the oracle's rate on a sample
  cpu_baseline the float64 NumPy oracle on a bounded sample of the headline
               workload (an 8192 x 8192 block of C over the full K = the
               whole square GEMM, including the oracle's quantize of the
               operand rows it needs)

For skinny workloads a bounded spin kernel keeps the GPU busy for a few
milliseconds before each timed region while the host queues the timed
launches, so that the events time the GPU and not Python's launch rate (a
skinny GEMM runs for less time than one launch takes the host).
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP4_DENSE_PEAK_TFLOPS = 10100.0   # MI355X dense MXFP4 MFMA peak
HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 << 20             # MI355X last-level (Infinity) cache
HBM_BOUND_MAX_M = 128             # GEMMs with at most this many rows of A stream B
WARM_LAUNCHES = 50
WARM_MS = 100.0
GROUPS = 10
PER_GROUP = 10
CONFIG_ORDER = ["tiny", "skinny", "square", "mlp_gate_up", "mlp_down", "ragged"]
CONFIG_INDEX = {"tiny": "0", "skinny": "1", "square": "2", "mlp_gate_up": "3a",
                "mlp_down": "3b", "ragged": "4"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="square")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-workload sweep (headline workload only)")
    p.add_argument("--no-swiglu", action="store_true",
                   help="skip timing the fused SwiGLU gate+up GEMM at the Llama MLP shape")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "gemm_traffic.json"),
                   help="HBM bytes per GEMM launch from rocprofv3 counters, if measured")
    p.add_argument("--probe", action="store_true",
                   help="only run the MFMA / LDS microbenchmark (built by build.build_probe) "
                        "and print its cases as one JSON line")
    p.add_argument("--sections", action="store_true",
                   help="only run the tile GEMM's section timing (built by "
                        "build.build_sections) and print its workloads as one JSON line")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB three times and exit "
                        "(the known-size kernel that scales the FETCH_SIZE/WRITE_SIZE counters)")
    p.add_argument("--copy-rate-mib", type=int, default=0,
                   help="only time a plain device copy of this many MiB (read + write rate, "
                        "the practical ceiling of streaming kernels) and exit")
    return p.parse_args()


def source_digest(sources):
    """SHA-256 over the named kernel sources: counters taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(path, workload):
    """HBM bytes per GEMM launch measured by rocprofv3 for this workload, or None
    when not measured or measured on other kernel sources."""
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            entry = json.load(f)["workloads"].get(workload)
    except (OSError, ValueError, KeyError, AttributeError):
        return None
    if not entry or entry.get("sha256") != source_digest(entry.get("sources", [])):
        return None
    return entry.get("bytes_per_launch")


def copy_calibration(mib):
    import torch
    dev = torch.device("cuda:0")
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def copy_rate(mib):
    """Read + write rate of a plain device-to-device copy of `mib` MiB: the
    practical ceiling of kernels that stream HBM in and out. Two buffer pairs
    (beyond the last-level cache) alternate; after 20 untimed copies, the
    median of 10 groups of 10 copies, each group between one event pair on
    the stream the copies run on."""
    import torch
    dev = torch.device("cuda:0")
    n = mib << 20
    pairs = [(torch.ones(n // 4, dtype=torch.float32, device=dev),
              torch.empty(n // 4, dtype=torch.float32, device=dev)) for _ in range(2)]
    for i in range(20):
        src, dst = pairs[i % 2]
        dst.copy_(src)
    times = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(10):
            src, dst = pairs[i % 2]
            dst.copy_(src)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / 10)
    us = sorted(times)[len(times) // 2] * 1e3
    print(json.dumps({"copy_mib": mib, "copy_us": round(us, 2),
                      "read_write_tb_per_s": round(2 * n / (us * 1e-6) / 1e12, 3),
                      "frac_of_8_tb_per_s": round(2 * n / (us * 1e-6) / 8e12, 3)}), flush=True)


def run_sections():
    """The tile GEMM's section timing in a child process: per section of the
    kernel (K loop, step waits and barriers, epilogue parts) the mean cycles
    per wave and tile, on the tile-GEMM workloads."""
    import subprocess
    exe = os.path.join(ROOT, "block_scaled_microscaling_amd", "gemm_sections")
    if not os.path.exists(exe):
        raise RuntimeError(f"{exe} is missing: build it with build.build_sections()")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"gemm_sections failed with status {res.returncode}")
    cases = [json.loads(line) for line in res.stdout.splitlines() if line.startswith("{")]
    print(json.dumps({"sections": cases}), flush=True)


def run_probe():
    """The MFMA / LDS microbenchmark in a child process: the FP4 MFMA issue
    rate and clock with and without the tile GEMM's LDS fragment reads, and
    the LDS read bandwidth."""
    import subprocess
    exe = os.path.join(ROOT, "block_scaled_microscaling_amd", "mfma_lds_probe")
    if not os.path.exists(exe):
        raise RuntimeError(f"{exe} is missing: build it with build.build_probe()")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"mfma_lds_probe failed with status {res.returncode}")
    cases = [json.loads(line) for line in res.stdout.splitlines() if line.startswith("{")]
    print(json.dumps({"probe": cases}), flush=True)


def oracle_rate(a_bits, b_bits, K, rows, cols):
    """Wall time of the float64 oracle on a rows x cols block of C over the
    full K (quantize of those operand rows, dequantize, C and S matmuls)."""
    import oracle
    rows = min(rows, a_bits.shape[0])
    cols = min(cols, b_bits.shape[0])
    t0 = time.perf_counter()
    ac, as_ = oracle.quantize(a_bits[:rows])
    bc, bs = oracle.quantize(b_bits[:cols])
    oracle.gemm_block(ac, as_, bc, bs)
    dt = time.perf_counter() - t0
    return rows, cols, dt, 2.0 * rows * cols * K / dt / 1e12


def cpu_baseline(a_bits, b_bits, K, rows=8192, cols=8192):
    rows, cols, dt, tflops = oracle_rate(a_bits, b_bits, K, rows, cols)
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"C block {rows}x{cols} over K={K}: oracle quantize of {rows}+{cols} rows, "
                   f"float64 dequantize, C and S matmuls; {dt:.2f} s wall"),
    }


def profiled_mfma(kernel="gemm_tile_kernel<0, true, false>", shape="8192^3, BF16"):
    """Engine clock and MFMA utilisation of the headline GEMM as rocprofv3's
    counters measured them (profiles/gemm_mfma_utilisation_counters.md, the
    row of this kernel and shape), or None. A clock read beside the running
    GEMM from a spin kernel's cycle counter disagreed with the counters
    (2.34-2.41 against 1.78 GHz), so the line quotes the counters instead."""
    path = os.path.join(ROOT, "profiles", "gemm_mfma_utilisation_counters.md")
    try:
        with open(path) as f:
            for line in f:
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                if len(cells) >= 7 and cells[0] == f"`mxfp4::{kernel}`" and cells[1] == shape:
                    return {"clock_ghz": float(cells[5].split()[0]),
                            "mfma_busy": float(cells[6].rstrip("%")) / 100.0,
                            "source": "profiles/gemm_mfma_utilisation_counters.md"}
    except (OSError, ValueError, IndexError):
        return None
    return None


def make_holder(torch, stream):
    """Return hold(ms): keep the GPU busy for about ms milliseconds with
    torch's bounded spin kernel, so that the host queues the launches that
    follow before the GPU reaches them. Events recorded between those
    launches then time the GPU rather than the host's launch rate, which
    decides the reading for kernels of a few microseconds."""
    cycles = 1 << 22
    torch.cuda._sleep(cycles)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(cycles)
    e1.record(stream)
    torch.cuda.synchronize()
    per_ms = cycles / max(e0.elapsed_time(e1), 1e-3)

    def hold(ms):
        torch.cuda._sleep(int(per_ms * ms))
    return hold


def make_timer(torch, mx, stream, hold):
    """time_kernel(launch, name, short) -> median ms per launch (see the
    module docstring). short: the kernel is shorter than a host launch, so
    the GPU is held while the host queues the timed groups."""

    def once(launch, name, i):
        rc = launch(i)  # a C status from the raw entries; the helpers raise
        if isinstance(rc, int) and rc != 0:
            raise mx.Mxfp4Error(rc, name)

    def time_kernel(launch, name, short=False):
        i = 0
        t0 = time.perf_counter()
        while i < WARM_LAUNCHES or (time.perf_counter() - t0) * 1e3 < WARM_MS:
            once(launch, name, i)
            i += 1
            if i % 20 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(GROUPS)]
        if short:
            hold(5.0 + 0.06 * GROUPS * PER_GROUP)
        for e0, e1 in evs:
            e0.record(stream)
            for _ in range(PER_GROUP):
                once(launch, name, i)
                i += 1
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) / PER_GROUP for e0, e1 in evs]))

    return time_kernel


MAX_COPIES = 64


def copies_for(nbytes):
    """Operand copies to rotate through so that they cover twice the LLC (at
    most 64: smaller operand sets stay cache-resident, and say so)."""
    return min(MAX_COPIES, max(1, -(-2 * LLC_BYTES // max(nbytes, 1))))


def is_short(M, N, K):
    """A GEMM shorter than a host launch (skinny M, or under 0.1 TFLOP):
    time it with the GPU held while the host queues the launches."""
    return M <= HBM_BOUND_MAX_M or 2.0 * M * N * K < 1e11


def gemm_roofline(M, N, K, out_bytes, ms, traffic=None):
    flops = 2.0 * M * N * K
    nbytes = (M + N) * (K // 2 + K // 32) + M * N * out_bytes
    if M <= HBM_BOUND_MAX_M:
        gbps = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic}
    tflops = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": tflops, "peak": FP4_DENSE_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": tflops / FP4_DENSE_PEAK_TFLOPS, "traffic": traffic}


def to_dev(torch, bits, dev):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)


def bench_config(torch, mx, dev, stream, time_kernel, w, oracle_sample=True, traffic=None):
    """GEMM and activation-quantize times of workload `w` (contract entries,
    and a layout variant: fragment order for GEMMs shorter than a host launch
    (M <= 128 or under 0.1 TFLOP), pre-shuffled B otherwise), with operand
    copies rotated past the LLC."""
    from synth import bf16_matrix
    M, N, K = w.M, w.N, w.K
    print(f"bench: config {CONFIG_INDEX[w.name]} ({w.name}) {M}x{N}x{K}", file=sys.stderr,
          flush=True)
    a_bits = bf16_matrix((M, K), w.a_dist, w.a_seed)
    b_bits = bf16_matrix((N, K), w.b_dist, w.b_seed)
    x = to_dev(torch, a_bits, dev)
    bc, bs = mx.quantize(to_dev(torch, b_bits, dev))
    out_dtype = torch.float32 if w.out_dtype == mx.OUT_FP32 else torch.bfloat16
    out_bytes = 4 if w.out_dtype == mx.OUT_FP32 else 2
    op_bytes = (M + N) * (K // 2 + K // 32)
    n = copies_for(op_bytes)
    ac, as_ = mx.quantize(x)
    sets = [(ac, as_, bc, bs)] + [tuple(t.clone() for t in (ac, as_, bc, bs))
                                  for _ in range(n - 1)]
    c = torch.empty((M, N), dtype=out_dtype, device=dev)
    short = is_short(M, N, K)

    def gemm(i):
        a, a_s, b, b_s = sets[i % n]
        return mx.mxfp4_gemm(a.data_ptr(), a_s.data_ptr(), b.data_ptr(), b_s.data_ptr(), M, N, K,
                             w.out_dtype, c.data_ptr(), stream.cuda_stream)

    g_ms = time_kernel(gemm, "mxfp4_gemm", short)
    xs = [x] + [x.clone() for _ in range(copies_for(M * K * 2) - 1)]
    qc = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    qs = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)

    def quant(i):
        return mx.mxfp4_quantize_async(xs[i % len(xs)].data_ptr(), M, K, qc.data_ptr(),
                                       qs.data_ptr(), stream.cuda_stream)

    q_ms = time_kernel(quant, "mxfp4_quantize", short)
    q_bytes = M * K * 2 + M * K // 2 + M * K // 32
    out = {
        "shape": f"{M}x{N}x{K}", "out": "fp32" if out_bytes == 4 else "bf16",
        "gemm_us": g_ms * 1e3,
        "gemm_roofline": gemm_roofline(M, N, K, out_bytes, g_ms, traffic),
        "quantize_us": q_ms * 1e3,
        "quantize_gbps": q_bytes / (q_ms * 1e-3) / 1e9,
        "quantize_hbm_frac": q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "operand_copies_rotated": n,
        "llc_resident": n * op_bytes < 2 * LLC_BYTES,
    }
    if short and M % 32 == 0:
        frag = [(mx.to_frag(a, a_s), mx.to_frag(b, b_s)) for a, a_s, b, b_s in sets]

        def gemm_f(i):
            (af, asf), (bf, bsf) = frag[i % n]
            return mx.mxfp4_gemm_frag(af.data_ptr(), asf.data_ptr(), bf.data_ptr(),
                                      bsf.data_ptr(), M, N, K, w.out_dtype, c.data_ptr(),
                                      stream.cuda_stream)
        v_ms = time_kernel(gemm_f, "mxfp4_gemm_frag", short)
        out["variant"] = "fragment order (mxfp4_gemm_frag)"
        del frag
    else:
        shuf = [mx.shuffle_b(b, b_s) for _, _, b, b_s in sets]

        def gemm_s(i):
            a, a_s, _, _ = sets[i % n]
            bsh, bssh = shuf[i % n]
            return mx.mxfp4_gemm_bshuffled(a.data_ptr(), a_s.data_ptr(), bsh.data_ptr(),
                                           bssh.data_ptr(), M, N, K, w.out_dtype, c.data_ptr(),
                                           stream.cuda_stream)
        v_ms = time_kernel(gemm_s, "mxfp4_gemm_bshuffled", short)
        out["variant"] = "pre-shuffled B (mxfp4_gemm_bshuffled)"
        del shuf
    out["variant_gemm_us"] = v_ms * 1e3
    out["variant_gemm_roofline_frac"] = gemm_roofline(M, N, K, out_bytes, v_ms)["frac"]
    del sets, xs, c
    if oracle_sample:
        rows, cols, dt, tflops = oracle_rate(a_bits, b_bits, K, 256, 1024)
        out["oracle"] = {"tflops": tflops, "sample": f"C block {rows}x{cols} over K={K}",
                         "sample_s": dt,
                         "full_gemm_s_at_that_rate": 2.0 * M * N * K / (tflops * 1e12)}
    return out


def time_swiglu(mx, torch, dev, stream, time_kernel):
    """The gate+up GEMM of the Llama-3-8B MLP shape (16384 x 28672 x 4096)
    with its fused SwiGLU + MXFP4 requantize epilogue, beside the plain GEMM
    of the same shape writing its 940 MB BF16 C, over the same operand
    copies (rotated past the LLC)."""
    from synth import WORKLOADS, bf16_matrix
    w = WORKLOADS["mlp_gate_up"]
    M, N, K = w.M, w.N, w.K
    print(f"bench: fused SwiGLU gate+up {M}x{N}x{K}", file=sys.stderr, flush=True)
    ac, as_ = mx.quantize(to_dev(torch, bf16_matrix((M, K), w.a_dist, w.a_seed), dev))
    bc, bs = mx.quantize(to_dev(torch, bf16_matrix((N, K), w.b_dist, w.b_seed), dev))
    n = copies_for((M + N) * (K // 2 + K // 32))
    sets = [(ac, as_, bc, bs)] + [tuple(t.clone() for t in (ac, as_, bc, bs))
                                  for _ in range(n - 1)]
    Nh = N // 2
    codes = torch.empty((M, Nh // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, Nh // 32), dtype=torch.uint8, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def fused(i):
        a, a_s, b, b_s = sets[i % n]
        return mx.mxfp4_gemm_swiglu(a.data_ptr(), a_s.data_ptr(), b.data_ptr(), b_s.data_ptr(),
                                    M, N, K, codes.data_ptr(), scales.data_ptr(), None,
                                    stream.cuda_stream)

    def plain(i):
        a, a_s, b, b_s = sets[i % n]
        return mx.mxfp4_gemm(a.data_ptr(), a_s.data_ptr(), b.data_ptr(), b_s.data_ptr(), M, N, K,
                             mx.OUT_BF16, c.data_ptr(), stream.cuda_stream)

    out = {"shape": f"{M}x{N}x{K}", "operand_copies_rotated": n}
    for name, fn in (("fused", fused), ("plain_bf16_gemm", plain)):
        ms = time_kernel(fn, name)
        out[name + "_ms"] = ms
        out[name + "_tflops"] = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path needs no collective; see the sharding notes)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.copy_rate_mib:
        copy_rate(args.copy_rate_mib)
        return
    if args.probe:
        run_probe()
        return
    if args.sections:
        run_sections()
        return

    import torch

    import block_scaled_microscaling_amd as mx
    from synth import WORKLOADS, bf16_matrix

    w = WORKLOADS[args.workload]
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if mx.mxfp4_available() != 1:
        raise RuntimeError("libmxfp4: no gfx950 device")
    stream = torch.cuda.current_stream()
    hbm_bound = M <= HBM_BOUND_MAX_M
    short = is_short(M, N, K)
    hold = make_holder(torch, stream)
    time_kernel = make_timer(torch, mx, stream, hold)

    print(f"bench: workload {w.name} M={M} N={N} K={K}; generating inputs", file=sys.stderr,
          flush=True)
    a_bits = bf16_matrix((M, K), w.a_dist, w.a_seed)
    b_bits = bf16_matrix((N, K), w.b_dist, w.b_seed)
    out_dtype = torch.float32 if w.out_dtype == mx.OUT_FP32 else torch.bfloat16
    out_bytes = 4 if w.out_dtype == mx.OUT_FP32 else 2

    # Copies of the step's inputs, rotated step by step: the activations X
    # and, separately, the GEMM operands (A's codes and scales, written by the
    # step's quantize, and the quantized weight B) each cover more than twice
    # the last-level cache, so every step reads them from HBM.
    x0 = to_dev(torch, a_bits, dev)
    bc0, bs0 = mx.quantize(to_dev(torch, b_bits, dev))
    op_bytes = (M + N) * (K // 2 + K // 32)
    x_copies = copies_for(M * K * 2)
    copies = copies_for(op_bytes)
    xs = [x0] + [x0.clone() for _ in range(x_copies - 1)]
    ws = [(bc0, bs0)] + [(bc0.clone(), bs0.clone()) for _ in range(copies - 1)]
    acs = [(torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
            torch.empty((M, K // 32), dtype=torch.uint8, device=dev)) for _ in range(copies)]
    c = torch.empty((M, N), dtype=out_dtype, device=dev)
    for i in range(copies):
        mx.quantize(xs[i % x_copies], *acs[i])

    def gemm_launch(i):
        (a, a_s), (b, b_s) = acs[i % copies], ws[i % copies]
        return mx.mxfp4_gemm(a.data_ptr(), a_s.data_ptr(), b.data_ptr(), b_s.data_ptr(), M, N, K,
                             w.out_dtype, c.data_ptr(), stream.cuda_stream)

    def quantize_launch(i):
        a, a_s = acs[i % copies]
        return mx.mxfp4_quantize_async(xs[i % x_copies].data_ptr(), M, K, a.data_ptr(),
                                       a_s.data_ptr(), stream.cuda_stream)

    def step(i):
        quantize_launch(i)
        gemm_launch(i)

    # Per-kernel times of the headline workload (the GEMM's is the roofline),
    # and the engine clock the GEMM runs at.
    g_ms = time_kernel(gemm_launch, "mxfp4_gemm", short)
    q_ms = time_kernel(quantize_launch, "mxfp4_quantize", short)
    flops = 2.0 * M * N * K
    q_bytes = M * K * 2 + M * K // 2 + M * K // 32
    traffic = read_traffic(args.traffic_json, w.name)
    roofline = gemm_roofline(M, N, K, out_bytes, g_ms, traffic)

    # The quantize widenings on the same activation copies.
    seed = 0x5EED
    a_sr, s_sr = acs[0]
    qsr_ms = time_kernel(lambda i: mx.mxfp4_quantize_sr(
        xs[i % x_copies].data_ptr(), M, K, seed, a_sr.data_ptr(), s_sr.data_ptr(),
        stream.cuda_stream), "mxfp4_quantize_sr", short)
    q2_ms = q2sr_ms = None
    if M % 32 == 0:
        q2_out = (torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                  torch.empty((M, K // 32), dtype=torch.uint8, device=dev),
                  torch.empty((K, M // 2), dtype=torch.uint8, device=dev),
                  torch.empty((K, M // 32), dtype=torch.uint8, device=dev))
        ptrs = [t.data_ptr() for t in q2_out]
        q2_ms = time_kernel(lambda i: mx.mxfp4_quantize_2d(
            xs[i % x_copies].data_ptr(), M, K, *ptrs, stream.cuda_stream), "mxfp4_quantize_2d",
            short)
        q2sr_ms = time_kernel(lambda i: mx.mxfp4_quantize_2d_sr(
            xs[i % x_copies].data_ptr(), M, K, seed, *ptrs, stream.cuda_stream),
            "mxfp4_quantize_2d_sr", short)
        del q2_out
    q2_bytes = 2 * M * K + 2 * (M * K // 2 + M * K // 32)

    # W untimed steps, then K timed steps with nothing between the two events.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    hold_ms = 2.0 + 0.3 * args.steps if short else 0.0
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    if short:
        hold(hold_ms)
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    del xs, ws, acs, c

    def gbps(nbytes, ms):
        return None if ms is None else nbytes / (ms * 1e-3) / 1e9

    result = {
        "metric": "MXFP4 GEMM TFLOP/s (2MNK) at 8192^3 + % of FP4 MFMA peak; quantize GB/s",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: quantize A[{M},{K}] BF16 -> MXFP4 (mxfp4_quantize), then "
                         f"mxfp4_gemm {M}x{N}x{K} against pre-quantized row-major B[{N},{K}], "
                         f"{'fp32' if out_bytes == 4 else 'bf16'} out; {x_copies} copies of X "
                         f"and {copies} of the GEMM operands rotated (each set past twice the "
                         f"256 MiB last-level cache)"),
            "M": M, "N": N, "K": K,
            "out_dtype": "fp32" if out_bytes == 4 else "bf16",
        },
        "roofline": roofline,
        "profiled_mfma": profiled_mfma() if w.name == "square" else None,
        "engine_clock_peak_mhz": 2400,
        "gemm_us": g_ms * 1e3,
        "gemm_tflops": flops / (g_ms * 1e-3) / 1e12,
        "quantize_us": q_ms * 1e3,
        "quantize_gbps": gbps(q_bytes, q_ms),
        "quantize_hbm_frac": gbps(q_bytes, q_ms) / HBM_PEAK_GBPS,
        "quantize_sr_gbps": gbps(q_bytes, qsr_ms),
        "quantize_2d_gbps": gbps(q2_bytes, q2_ms),
        "quantize_2d_sr_gbps": gbps(q2_bytes, q2sr_ms),
        "timing": (f"per-kernel: median of {GROUPS} groups of {PER_GROUP} back-to-back launches "
                   f"after >= {WARM_LAUNCHES} launches and >= {WARM_MS:.0f} ms untimed, taken "
                   f"before the step warm-up; step: {args.steps} steps between one event pair"),
        "wall_s_timed": t_wall,
    }
    if not args.no_configs:
        result["configs"] = {
            CONFIG_INDEX[name]: bench_config(torch, mx, dev, stream, time_kernel, WORKLOADS[name],
                                             oracle_sample=not args.no_cpu_baseline,
                                             traffic=read_traffic(args.traffic_json, name))
            for name in CONFIG_ORDER
        }
    if not args.no_swiglu:
        result["swiglu_gate_up"] = time_swiglu(mx, torch, dev, stream, time_kernel)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(a_bits, b_bits, K)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
