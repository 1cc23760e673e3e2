"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A serving loop captures the per-call work once and replays it: here the
decode step (activation quantized into fragment order, then the
fragment-order GEMM against a re-laid-out weight), the tile path
(row-wise quantize, then the GEMM on a pre-shuffled weight) and the contract
path (row-wise quantize, then mxfp4_gemm on row-major B). The kernels
allocate nothing and launch only on the caller's stream, so they capture
as they are. Each replay runs on a new input written into the captured
buffer, with eager work and a synchronisation between replays, and must
equal the eager result on that input bit for bit.
"""

import numpy as np
import pytest
import torch

import block_scaled_microscaling_amd as mx
from gpu_helpers import DEV, announce, bf16_to_dev
from synth import bf16_matrix

pytestmark = pytest.mark.gpu


def _weights(N, K, seed):
    w = bf16_to_dev(bf16_matrix((N, K), ("normal", 0.02, 0.0, 1.0), seed))
    return mx.quantize(w)


# fragment160: 5 row tiles of A, which the fragment-order GEMM enqueues as
# two kernels (3 + 2 tiles per workgroup); both are captured. contract: the
# row-wise quantize and mxfp4_gemm on plain row-major B, at a size it runs
# on the split-K kernel (2 tiles of 256 x 256) and at one it runs on the
# tile kernel (48 tiles).
@pytest.mark.parametrize("path", ["fragment", "fragment160", "tile", "contract_splitk",
                                  "contract_tile"])
def test_captured_step_replays_equal_eager(path):
    M, N, K = {"fragment": (32, 2048, 4096), "fragment160": (160, 1024, 2048),
               "tile": (512, 768, 2048), "contract_splitk": (256, 512, 1024),
               "contract_tile": (2048, 1536, 1024)}[path]
    path = "fragment" if path.startswith("fragment") else path
    announce(f"graph capture, {path} path {M}x{N}x{K}")
    bc, bs = _weights(N, K, 41)
    if path == "fragment":
        wf, wsf = mx.to_frag(bc, bs)
        af = torch.empty(M * K // 2, dtype=torch.uint8, device=DEV)
        asf = torch.empty(M * K // 32, dtype=torch.uint8, device=DEV)
    else:
        bsh = mx.shuffle_b(bc, bs) if path == "tile" else None
        ac = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
        as_ = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def step():
        if path == "fragment":
            mx.quantize_frag(x, af, asf)
            mx.gemm_frag(af, asf, wf, wsf, M, N, K, out=c)
        elif path == "tile":
            mx.quantize(x, ac, as_)
            mx.gemm_bshuffled(ac, as_, bsh[0], bsh[1], N, out=c)
        else:
            mx.quantize(x, ac, as_)
            mx.gemm(ac, as_, bc, bs, out=c)

    inputs = [bf16_to_dev(bf16_matrix((M, K), ("normal", 1.0, 0.01, 100.0), 50 + i))
              for i in range(4)]
    # Warm up on a side stream (first calls check the device), then capture.
    x.copy_(inputs[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for i, inp in enumerate(inputs):
        x.copy_(inp)
        step()                      # eager reference on this input
        torch.cuda.synchronize()
        want = c.clone()
        c.fill_(float("nan"))       # the replay must rewrite every element
        x.copy_(inp)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), want.view(torch.int16)), f"replay {i}"
        assert torch.isfinite(c).all()
        # Other eager work between replays.
        _ = (inp.float() * 2).sum().item()
