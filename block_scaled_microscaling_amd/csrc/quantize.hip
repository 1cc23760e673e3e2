// Row-wise BF16 -> MXFP4 quantize for gfx950.
//
// The operation is the MXFP4 quantizer of "Integrate MXFP4 hipblaslt GEMM
// support" (ROCm/TransformerEngine #697): plain E2M1 codes with one UE8M0
// scale per 32 consecutive elements of a row. With K % 32 == 0 a row-major
// [M, K] matrix is a flat sequence of M*K/32 blocks of 64 bytes, each mapping
// to 16 code bytes and one scale byte, so the kernel ignores rows entirely.
//
// Work mapping (HBM-streaming, no LDS): four consecutive lanes own one block,
// 16 bytes (8 BF16) each, so a wavefront covers 16 blocks = 1 KiB of input
// per load instruction. Each thread keeps kUnroll such loads in flight.
// The register-resident design follows the row-wise g2r kernel described on
// NVIDIA/TransformerEngine #3809 (one wide load per block, no staging, no
// per-element divide); the block arithmetic (gfx950.h) is gfx950's: integer
// amax of the |BF16| patterns, the scale byte from its exponent field, and
// v_cvt_scalef32_pk_fp4_bf16 for the division, rounding and packing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950.h"
#include "kernels.h"

namespace mxfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void quantize_kernel(const u32x4_t* __restrict__ x,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            int64_t nquarters) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t base = wave * (64 * kUnroll) + lane;

  u32x4_t v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t q = base + (int64_t)u * 64;
    v[u] = q < nquarters ? __builtin_nontemporal_load(&x[q]) : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t q = base + (int64_t)u * 64;
    // All 64 lanes take part in the DPP moves; a block's four lanes are
    // either all in range or all out (nquarters is a multiple of 4).
    const uint32_t amax = quad_max(block_quarter_absmax(v[u]));
    const uint32_t byte = scale_byte_of(amax);
    const uint32_t c = encode8(v[u], __uint_as_float(byte << 23));
    if (q < nquarters) {
      codes[q] = c;
      if ((lane & 3) == 0) scales[q >> 2] = (uint8_t)byte;
    }
  }
}

// Fragment order: one workgroup per (32-row tile t, 256-K step s), flat
// index wg = t KS + s, which is also the index of its 4 KiB code block and
// 256-byte scale block in the output. The loads are those of
// quantize_kernel over the tile's 32 row segments of 512 bytes (two
// segments per wave instruction); block j = 4 h + q of row r of the step
// lands at code word 256 q + 4 (r + 32 h) + quarter and at scale byte
// 4 (r + 32 h) + q of its blocks.
__global__ __launch_bounds__(kThreads) void quantize_frag_kernel(const uint8_t* __restrict__ x,
                                                                 int K,
                                                                 uint32_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales) {
  const unsigned ks_n = (unsigned)K / 256u;
  const unsigned wg = blockIdx.x;
  const unsigned t = wg / ks_n, s = wg - t * ks_n;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (int64_t)32 * t * K * 2 + 512 * s);
  const int row_quarters = K / 8;  // 16-byte quarters per row of x

  u32x4_t v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int qi = u * kThreads + threadIdx.x;  // 0..1023 = 32 r + 4 j + quarter
    v[u] = __builtin_nontemporal_load(&src[(qi >> 5) * row_quarters + (qi & 31)]);
  }
  uint32_t* cblk = codes + (int64_t)wg * 1024;
  uint8_t* sblk = scales + (int64_t)wg * 256;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int qi = u * kThreads + threadIdx.x;
    const int r = qi >> 5, j = (qi >> 2) & 7, quarter = qi & 3;
    const int lane = r + 32 * (j >> 2), q = j & 3;
    const uint32_t amax = quad_max(block_quarter_absmax(v[u]));
    const uint32_t byte = scale_byte_of(amax);
    cblk[256 * q + 4 * lane + quarter] = encode8(v[u], __uint_as_float(byte << 23));
    if (quarter == 0) sblk[4 * lane + q] = (uint8_t)byte;
  }
}

}  // namespace

hipError_t launch_quantize_frag(const void* x_bf16, int64_t M, int64_t K, void* codes,
                                void* scales, hipStream_t stream) {
  const int64_t grid = (M / 32) * (K / 256);
  hipLaunchKernelGGL(quantize_frag_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(x_bf16), (int)K, static_cast<uint32_t*>(codes),
                     static_cast<uint8_t*>(scales));
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x_bf16, int64_t nblocks, void* codes, void* scales,
                           hipStream_t stream) {
  const int64_t nquarters = nblocks * 4;
  const int64_t per_block = (int64_t)kThreads * kUnroll;  // quarters per workgroup
  const int64_t grid = (nquarters + per_block - 1) / per_block;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(x_bf16), static_cast<uint32_t*>(codes),
                     static_cast<uint8_t*>(scales), nquarters);
  return hipGetLastError();
}

}  // namespace mxfp4
