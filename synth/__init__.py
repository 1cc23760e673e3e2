"""Seeded synthetic inputs, shared by the tests, bench.py and the smoke check.

This module holds none of the MXFP4 arithmetic: it only draws random numbers
(NumPy PCG64 from a fixed seed) and rounds float32 draws to BF16 with torch's
CPU conversion (round to nearest even). The oracle and the HIP library both
take its arrays as inputs; neither is imported here.

Workloads (shapes and value distributions):
  tiny        M=N=K=256, A and B ~ N(0,1), FP32 output
  skinny      M=32, N=K=8192, activations N(0,1), weights N(0,0.02), BF16 output
  square      M=N=K=8192, N(0,1) with 1% of entries x100, BF16 output
  mlp_gate_up M=16384, N=28672, K=4096, activations N(0,1), weights N(0,0.02)
  mlp_down    M=16384, N=4096, K=14336, same distributions
  ragged      X[4128, 7936] ~ Laplace(0,1), W[6176, 7936] ~ N(0,0.02), FP32 out
  decode64, decode128
              the skinny workload's shape and distributions at M = 64 and 128
              (larger decode batches against the same 8192 x 8192 weight)
The MLP shapes are those of a Llama-3-8B MLP at 16384 tokens; no weights of
any trained model are used.
"""

from dataclasses import dataclass

import numpy as np
import torch

OUT_BF16 = 0
OUT_FP32 = 1


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    out_dtype: int
    a_dist: tuple   # ("normal", std, outlier_frac, outlier_scale) | ("laplace", b)
    b_dist: tuple
    a_seed: int
    b_seed: int


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 256, 256, 256, OUT_FP32,
                 ("normal", 1.0, 0.0, 1.0), ("normal", 1.0, 0.0, 1.0), 1000, 2000),
        Workload("skinny", 32, 8192, 8192, OUT_BF16,
                 ("normal", 1.0, 0.0, 1.0), ("normal", 0.02, 0.0, 1.0), 1001, 2001),
        Workload("square", 8192, 8192, 8192, OUT_BF16,
                 ("normal", 1.0, 0.01, 100.0), ("normal", 1.0, 0.01, 100.0), 1002, 2002),
        Workload("mlp_gate_up", 16384, 28672, 4096, OUT_BF16,
                 ("normal", 1.0, 0.0, 1.0), ("normal", 0.02, 0.0, 1.0), 1003, 2003),
        Workload("mlp_down", 16384, 4096, 14336, OUT_BF16,
                 ("normal", 1.0, 0.0, 1.0), ("normal", 0.02, 0.0, 1.0), 3003, 4003),
        Workload("ragged", 4128, 6176, 7936, OUT_FP32,
                 ("laplace", 1.0), ("normal", 0.02, 0.0, 1.0), 1004, 2004),
        Workload("decode64", 64, 8192, 8192, OUT_BF16,
                 ("normal", 1.0, 0.0, 1.0), ("normal", 0.02, 0.0, 1.0), 1005, 2001),
        Workload("decode128", 128, 8192, 8192, OUT_BF16,
                 ("normal", 1.0, 0.0, 1.0), ("normal", 0.02, 0.0, 1.0), 1006, 2001),
    ]
}


def f32_to_bf16_bits(x):
    """float32 array -> uint16 BF16 bit patterns (torch CPU, nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def draw_f32(shape, dist, seed):
    """float32 draws of distribution `dist` (see Workload) from `seed`."""
    rng = np.random.default_rng(seed)
    if dist[0] == "normal":
        _, std, frac, big = dist
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        if frac > 0:
            mask = rng.random(shape, dtype=np.float32) < frac
            x[mask] *= np.float32(big)
        return x
    if dist[0] == "laplace":
        return rng.laplace(0.0, dist[1], size=shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def bf16_matrix(shape, dist, seed):
    """BF16 bit patterns (uint16) of a seeded draw."""
    return f32_to_bf16_bits(draw_f32(shape, dist, seed))


def workload_inputs(w):
    """(A_bf16_bits [M,K], B_bf16_bits [N,K]) of workload `w`."""
    a = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    b = bf16_matrix((w.N, w.K), w.b_dist, w.b_seed)
    return a, b


def random_codes(rows, K, seed):
    """Uniform random packed FP4 bytes, uint8 [rows, K/2]."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)


def random_scales(rows, K, seed, lo=117, hi=137):
    """Uniform random UE8M0 scale bytes in [lo, hi], uint8 [rows, K/32]."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(rows, K // 32), dtype=np.uint8)


def random_bf16_bits(shape, seed):
    """Uniform random finite BF16 bit patterns (any sign, exponent, mantissa)."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    exp_all_ones = (bits & 0x7F80) == 0x7F80
    bits[exp_all_ones] &= 0xBFFF      # inf/NaN patterns -> finite ones
    return bits


def large_block_first(rows, K, big_scale):
    """Packed codes and scales [rows, K/2], [rows, K/32] whose first 256 K
    hold code 6 (4.0) under scale byte big_scale and every later K code 1
    (0.5) under big_scale - 8: an input for testing fp32 accumulation with a
    large partial sum first and many small ones after it."""
    codes = np.full((rows, K // 2), 0x11, np.uint8)
    codes[:, :128] = 0x66
    scales = np.full((rows, K // 32), big_scale - 8, np.uint8)
    scales[:, :8] = big_scale
    return codes, scales


def device_random_bytes(shape, seed, lo=0, hi=255, device="cuda:0"):
    """Uniform random bytes in [lo, hi], uint8 of `shape`, drawn on `device`
    by torch's generator seeded with `seed`: for operands of gigabytes, too
    large to draw on the host. The oracle reads the rows it checks back from
    the device."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.uint8)


def device_normal_bf16(shape, seed, device="cuda:0"):
    """N(0, 1) BF16 values of `shape` drawn on `device` by torch's generator
    seeded with `seed` (as device_random_bytes)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
