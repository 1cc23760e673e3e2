"""Benchmark of the MXFP4 hot path on one MI355X (gfx950).

One step = row-wise BF16 -> MXFP4 quantize of the activation A [M, K] plus the
block-scaled GEMM C = dq(A) dq(B)^T against pre-quantized weights B [N, K],
on the square workload M = N = K = 8192 with BF16 output (the headline MXFP4
GEMM shape). Inputs are seeded synthetic BF16 (N(0,1) with 1% of entries x100)
resident in HBM before the timed region. Weight preparation (quantize, and
for the tile kernel the one-time pre-shuffle of B) happens before it; the
GEMM on B in its plain layout is timed alone beside it.

Prints one JSON line:
  value        2*M*N*K / (time per step), TFLOP/s, whole step (quantize + GEMM)
  roofline     the GEMM kernel against the FP4 MFMA dense peak (10.1 PFLOP/s):
               achieved = 2*M*N*K / mean GEMM launch time; for GEMMs with at
               most 128 rows of A (skinny) against HBM (8 TB/s): achieved =
               algorithmic bytes (A, B codes + scales, C) / mean launch time,
               with B rotated through enough copies that it is read from HBM
               each launch. Launch times come from back-to-back launches on
               the launch stream with one HIP event pair around them (events
               between launches add a few microseconds to each); so does
               every other per-kernel time in the line. The timed steps have
               no events inside.
  cpu_baseline the float64 NumPy oracle on a bounded sample of the same
               workload (up to an 8192 x 8192 block of C over the full K, the
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # 200 untimed steps (about 60 ms of GPU work): measured, the square GEMM
    # reads 9% slower after 10 warm-up steps than after 300, while the
    # engine clock and caches settle.
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="square")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-swiglu", action="store_true",
                   help="skip timing the fused SwiGLU gate+up GEMM at the Llama MLP shape")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "gemm_traffic.json"),
                   help="HBM bytes per GEMM launch from rocprofv3 counters, if measured")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB three times and exit "
                        "(the known-size kernel that scales the FETCH_SIZE/WRITE_SIZE counters)")
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


def cpu_baseline(a_bits, b_bits, K, rows=8192, cols=8192):
    import oracle
    cores = len(os.sched_getaffinity(0))
    rows = min(rows, a_bits.shape[0])
    cols = min(cols, b_bits.shape[0])
    t0 = time.perf_counter()
    ac, as_ = oracle.quantize(a_bits[:rows])
    bc, bs = oracle.quantize(b_bits[:cols])
    c, _s = oracle.gemm_block(ac, as_, bc, bs)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * cols * K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"C block {rows}x{cols} over K={K}: oracle quantize of {rows}+{cols} rows, "
                   f"float64 dequantize, C and S matmuls; {dt:.2f} s wall"),
    }


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


def time_swiglu(mx, torch, dev, stream, reps=10):
    """The gate+up GEMM of the Llama-3-8B MLP shape (16384 x 28672 x 4096)
    with its fused SwiGLU + MXFP4 requantize epilogue, timed alone, beside
    the plain GEMM of the same shape writing its 940 MB BF16 C."""
    from synth import WORKLOADS, bf16_matrix
    w = WORKLOADS["mlp_gate_up"]
    M, N, K = w.M, w.N, w.K
    print(f"bench: fused SwiGLU gate+up {M}x{N}x{K}", file=sys.stderr, flush=True)
    a = torch.from_numpy(bf16_matrix((M, K), w.a_dist, w.a_seed).view(np.int16))
    ac, as_ = mx.quantize(a.view(torch.bfloat16).to(dev))
    b = torch.from_numpy(bf16_matrix((N, K), w.b_dist, w.b_seed).view(np.int16))
    bc, bs = mx.quantize(b.view(torch.bfloat16).to(dev))
    del a, b
    Nh = N // 2
    codes = torch.empty((M, Nh // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, Nh // 32), dtype=torch.uint8, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def fused():
        rc = mx.mxfp4_gemm_swiglu(ac.data_ptr(), as_.data_ptr(), bc.data_ptr(), bs.data_ptr(),
                                  M, N, K, codes.data_ptr(), scales.data_ptr(), None,
                                  stream.cuda_stream)
        if rc != 0:
            raise mx.Mxfp4Error(rc, "mxfp4_gemm_swiglu")

    def plain():
        mx.gemm(ac, as_, bc, bs, out=c)

    # Both kernels warm up together (the first kernel timed after a cold
    # start otherwise reads 10-15% slow), then each is timed twice,
    # alternating, and the two means are averaged.
    for _ in range(10):
        fused()
        plain()
    torch.cuda.synchronize()
    out = {"shape": f"{M}x{N}x{K}"}
    times = {"fused": [], "plain_bf16_gemm": []}
    for _ in range(2):
        for name, fn in (("fused", fused), ("plain_bf16_gemm", plain)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / reps)
    for name, ts in times.items():
        ms = float(np.mean(ts))
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

    import torch

    import block_scaled_microscaling_amd as mx
    from synth import WORKLOADS, bf16_matrix

    w = WORKLOADS[args.workload]
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if mx.mxfp4_available() != 1:
        raise RuntimeError("libmxfp4: no gfx950 device")

    print(f"bench: workload {w.name} M={M} N={N} K={K}; generating inputs", file=sys.stderr,
          flush=True)
    a_bits = bf16_matrix((M, K), w.a_dist, w.a_seed)
    b_bits = bf16_matrix((N, K), w.b_dist, w.b_seed)
    x = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    wts = torch.from_numpy(b_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    out_dtype = torch.float32 if w.out_dtype == mx.OUT_FP32 else torch.bfloat16

    # Pre-quantized weights and preallocated buffers: nothing is allocated
    # inside the timed region.
    bc, bs = mx.quantize(wts)
    del wts
    # A GEMM with few rows of A streams B from HBM; a single B would stay in
    # the 256 MB last-level cache between steps, so such workloads rotate
    # through enough copies of B to cover twice that cache.
    hbm_bound = M <= HBM_BOUND_MAX_M
    b_bytes = bc.numel() + bs.numel()
    copies = max(1, -(-2 * LLC_BYTES // b_bytes)) if hbm_bound else 1
    weights = [(bc, bs)] + [(bc.clone(), bs.clone()) for _ in range(copies - 1)]
    # Larger GEMMs run on the tile kernel with B pre-shuffled once (part of
    # the weight preparation, like its quantization). Skinny ones run the
    # register-ring kernel on fragment-order operands: the weight copies are
    # re-laid out once, and the activation is quantized straight into
    # fragment order each step.
    shuffled = not hbm_bound
    frag = hbm_bound and M % 32 == 0 and K % 256 == 0
    if shuffled:
        bsh = mx.shuffle_b(bc, bs)
    if frag:
        weights_f = [mx.to_frag(wb, ws) for wb, ws in weights]
        af = torch.empty(M * K // 2, dtype=torch.uint8, device=dev)
        asf = torch.empty(M * K // 32, dtype=torch.uint8, device=dev)
    ac = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    as_ = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    c = torch.empty((M, N), dtype=out_dtype, device=dev)
    stream = torch.cuda.current_stream()

    counter = [0]

    def gemm_step(i):
        if frag:
            wf, wsf = weights_f[i % copies]
            mx.gemm_frag(af, asf, wf, wsf, M, N, K, out=c)
        elif shuffled:
            mx.gemm_bshuffled(ac, as_, bsh[0], bsh[1], N, out=c)
        else:
            wb, ws = weights[i % copies]
            mx.gemm(ac, as_, wb, ws, out=c)

    def quantize_step():
        if frag:
            mx.quantize_frag(x, af, asf)
        else:
            mx.quantize(x, ac, as_)

    def step():
        quantize_step()
        gemm_step(counter[0])
        counter[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    # Skinny steps are shorter than the host's launch time: a spin before
    # `start` lets the host queue them ahead of the GPU. Not for the large
    # workloads: there the GPU is the slower side anyway, and an idle spin
    # before MFMA-heavy work was measured to slow the next 50 steps by 12%
    # while the clocks readjust.
    hold = make_holder(torch, stream) if hbm_bound else (lambda ms: None)
    hold_ms = 2.0 + 0.3 * args.steps if hbm_bound else 0.0
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    hold(hold_ms)
    # Nothing but the steps between the two events: events recorded between
    # launches add a few microseconds of their own to each.
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall

    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    flops = 2.0 * M * N * K
    q_bytes = M * K * 2 + M * K // 2 + M * K // 32

    # Launch times of the step's kernels and of the widenings, each over
    # back-to-back launches on the launch stream (3 untimed, then `reps`
    # between one event pair).
    def time_alone(launch, name, reps=20):
        def once(i):
            rc = launch(i)  # a C status from the raw entries; the helpers raise
            if isinstance(rc, int) and rc != 0:
                raise mx.Mxfp4Error(rc, name)
        for i in range(3):
            once(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # Long enough for the host to queue every launch first, also under a
        # profiler, which slows each launch to tens of microseconds.
        hold(5.0 + 0.06 * reps)
        e0.record(stream)
        for i in range(reps):
            once(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # The step's GEMM (skinny: B rotated through its copies, so each launch
    # reads B from HBM) and the step's quantize.
    reps_gemm = 10 * copies if hbm_bound else 20
    g_ms = time_alone(gemm_step, "gemm", reps=reps_gemm)
    q_ms = time_alone(lambda i: quantize_step(), "quantize")
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    quant_gbps = q_bytes / (q_ms * 1e-3) / 1e9

    # The GEMM on operands in their plain row-major layout, timed alone (for
    # skinny workloads over the same rotated weight copies), and the
    # row-major quantize beside the fragment-order one.
    def plain_gemm(i):
        wb, ws = weights[i % copies]
        return mx.mxfp4_gemm(ac.data_ptr(), as_.data_ptr(), wb.data_ptr(), ws.data_ptr(), M, N, K,
                             w.out_dtype, c.data_ptr(), stream.cuda_stream)
    mx.quantize(x, ac, as_)
    gplain_ms = time_alone(plain_gemm, "mxfp4_gemm", reps=reps_gemm)
    qplain_ms = time_alone(lambda i: mx.quantize(x, ac, as_), "quantize") if frag else q_ms

    seed = 0x5EED
    qsr_ms = time_alone(lambda i: mx.mxfp4_quantize_sr(x.data_ptr(), M, K, seed, ac.data_ptr(),
                                                     as_.data_ptr(), stream.cuda_stream),
                        "mxfp4_quantize_sr")
    q2_out = (torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
              torch.empty((M, K // 32), dtype=torch.uint8, device=dev),
              torch.empty((K, M // 2), dtype=torch.uint8, device=dev),
              torch.empty((K, M // 32), dtype=torch.uint8, device=dev))
    q2_ms = q2sr_ms = None
    if M % 32 == 0:
        ptrs = [t.data_ptr() for t in q2_out]
        q2_ms = time_alone(lambda i: mx.mxfp4_quantize_2d(x.data_ptr(), M, K, *ptrs,
                                                        stream.cuda_stream),
                           "mxfp4_quantize_2d")
        q2sr_ms = time_alone(lambda i: mx.mxfp4_quantize_2d_sr(x.data_ptr(), M, K, seed, *ptrs,
                                                             stream.cuda_stream),
                             "mxfp4_quantize_2d_sr")
    q2_bytes = 2 * M * K + 2 * (M * K // 2 + M * K // 32)

    def gbps(nbytes, ms):
        return None if ms is None else nbytes / (ms * 1e-3) / 1e9

    traffic = read_traffic(args.traffic_json, w.name)
    out_bytes = 4 if w.out_dtype == mx.OUT_FP32 else 2
    gemm_bytes = (M + N) * (K // 2 + K // 32) + M * N * out_bytes
    gemm_gbps = gemm_bytes / (g_ms * 1e-3) / 1e9
    if hbm_bound:
        roofline = {"bound": "hbm", "achieved": gemm_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": gemm_gbps / HBM_PEAK_GBPS, "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "achieved": gemm_tflops, "peak": FP4_DENSE_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": gemm_tflops / FP4_DENSE_PEAK_TFLOPS,
                    "traffic": traffic}

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
            "workload": (f"{w.name}: quantize A[{M},{K}] BF16 -> MXFP4"
                         f"{' (fragment order)' if frag else ''}, then GEMM "
                         f"{M}x{N}x{K} against pre-quantized"
                         f"{', pre-shuffled' if shuffled else ''}"
                         f"{', fragment-order' if frag else ''} B[{N},{K}], "
                         f"{'fp32' if w.out_dtype else 'bf16'} out"),
            "M": M, "N": N, "K": K,
            "out_dtype": "fp32" if w.out_dtype else "bf16",
        },
        "gemm_tflops": gemm_tflops,
        "gemm_ms": g_ms,
        "quantize_gbps": quant_gbps,
        "quantize_ms": q_ms,
        "quantize_hbm_frac": quant_gbps / HBM_PEAK_GBPS,
        "gemm_b_layout": ("pre-shuffled" if shuffled else
                          "fragment order (A and B)" if frag else "plain"),
        "gemm_plain_b_ms": gplain_ms,
        "gemm_plain_b_tflops": flops / (gplain_ms * 1e-3) / 1e12,
        "gemm_plain_b_gbps_algorithmic": gemm_bytes / (gplain_ms * 1e-3) / 1e9,
        "quantize_row_major_ms": qplain_ms,
        "quantize_sr_ms": qsr_ms,
        "quantize_sr_gbps": gbps(q_bytes, qsr_ms),
        "quantize_2d_ms": q2_ms,
        "quantize_2d_gbps": gbps(q2_bytes, q2_ms),
        "quantize_2d_sr_ms": q2sr_ms,
        "quantize_2d_sr_gbps": gbps(q2_bytes, q2sr_ms),
        "wall_s_timed": t_wall,
        "gpu_hold_ms_before_timed": hold_ms,
        "gemm_gbps_algorithmic": gemm_gbps,
        "b_copies_rotated": copies,
        "roofline": roofline,
    }
    if not args.no_swiglu:
        result["swiglu_gate_up"] = time_swiglu(mx, torch, dev, stream)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(a_bits, b_bits, K)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
