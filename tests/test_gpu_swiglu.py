"""GPU parity of the gate+up GEMM with the fused SwiGLU + MXFP4 requantize.

Two checks per case, following readings W1-W3 of oracle/swiglu.py:
  * the BF16 activation the kernel quantized lies within the derived
    tolerance of the float64 act = silu(g) * u (oracle.swiglu_reference);
  * its codes and scales are bit-exact with the oracle's quantize of that
    same BF16 activation, so the quantize decision is compared in the
    kernel's own precision.
A run without the activation output must give the same bytes.
"""

import numpy as np
import pytest
import torch

import block_scaled_microscaling_amd as mx
import oracle
from gpu_helpers import announce, bf16_bits_of_tensor, bf16_to_dev
from synth import WORKLOADS, bf16_matrix

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed, a_dist=("normal", 1.0, 0.0, 1.0), b_dist=("normal", 0.02, 0.0, 1.0)):
    a = bf16_matrix((M, K), a_dist, seed)
    b = bf16_matrix((N, K), b_dist, seed + 1)
    ac, as_ = mx.quantize(bf16_to_dev(a))
    bc, bs = mx.quantize(bf16_to_dev(b))
    torch.cuda.synchronize()
    return ac, as_, bc, bs


def _check(ac, as_, bc, bs, rows=None):
    codes, scales, act = mx.gemm_swiglu(ac, as_, bc, bs, want_act=True)
    codes2, scales2 = mx.gemm_swiglu(ac, as_, bc, bs)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    h = [t.cpu().numpy() for t in (ac, as_, bc, bs)]
    act_bits = bf16_bits_of_tensor(act)
    g_codes, g_scales = codes.cpu().numpy(), scales.cpu().numpy()
    if rows is not None:
        act_bits, g_codes, g_scales = act_bits[rows], g_codes[rows], g_scales[rows]
    ref, tol = oracle.swiglu_reference(*h, m_rows=rows)
    ok = oracle.check_act_bf16(act_bits, ref, tol)
    bad = np.argwhere(~ok)
    assert ok.all(), f"{bad.shape[0]} activations outside tolerance, first {bad[:4].tolist()}"
    q_codes, q_scales = oracle.quantize(act_bits)
    assert np.array_equal(g_scales, q_scales), "scales differ from quantize(act)"
    assert np.array_equal(g_codes, q_codes), "codes differ from quantize(act)"
    return ref, act_bits


@pytest.mark.parametrize("M,N,K", [
    (256, 512, 256),      # one tile row, 2 activation tiles, K % 1024 != 0
    (64, 256, 1024),      # M < 256 (a partial tile row), one tile; K % 1024 == 0
    (32, 512, 768),       # M = 32: one MFMA row block, the rest clamped
    (288, 768, 1280),     # ragged M, Nh = 384 (3 tiles), K % 1024 != 0
    (544, 1280, 2048),    # several tiles both ways, Nh = 640
])
def test_swiglu_small(M, N, K):
    announce(f"gemm_swiglu {M}x{N}x{K}")
    _check(*_operands(M, N, K, seed=M + N + K))


def test_swiglu_large_values_and_saturation():
    """Activations spanning many binades (A with 1% of entries x100) and gate
    sums far into both tails of silu."""
    announce("gemm_swiglu wide dynamic range")
    _check(*_operands(256, 512, 512, seed=5, a_dist=("normal", 1.0, 0.01, 100.0),
                      b_dist=("normal", 0.1, 0.0, 1.0)))


def test_swiglu_feeds_down_gemm():
    """The activation codes are a plain MXFP4 A operand: the down GEMM on
    them matches the oracle GEMM of the same bytes."""
    announce("gemm_swiglu -> down GEMM")
    M, N, K, Nd = 256, 1024, 512, 256
    ac, as_, bc, bs = _operands(M, N, K, seed=9)
    codes, scales = mx.gemm_swiglu(ac, as_, bc, bs)
    w = bf16_matrix((Nd, N // 2), ("normal", 0.02, 0.0, 1.0), 10)
    wc, ws = mx.quantize(bf16_to_dev(w))
    out = mx.gemm(codes, scales, wc, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.gemm(codes.cpu().numpy(), scales.cpu().numpy(), wc.cpu().numpy(),
                               ws.cpu().numpy())
    assert oracle.check_fp32(out.cpu().numpy(), c_ref, s_ref).all()


def test_swiglu_mlp_gate_up_workload_sampled_rows():
    """The Llama-3-8B gate+up shape (16384 x 28672 x 4096) at full size; the
    oracle recomputes 24 sampled rows (28672 x 4096 products each)."""
    w = WORKLOADS["mlp_gate_up"]
    announce(f"gemm_swiglu workload {w.M}x{w.N}x{w.K}")
    a = bf16_matrix((w.M, w.K), w.a_dist, w.a_seed)
    b = bf16_matrix((w.N, w.K), w.b_dist, w.b_seed)
    ac, as_ = mx.quantize(bf16_to_dev(a))
    bc, bs = mx.quantize(bf16_to_dev(b))
    del a, b
    rng = np.random.default_rng(41)
    rows = np.unique(np.concatenate([rng.integers(0, w.M, 20), [0, 255, 256, w.M - 1]]))
    _check(ac, as_, bc, bs, rows=rows)
