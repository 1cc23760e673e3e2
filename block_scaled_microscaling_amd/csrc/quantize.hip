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
// per-element divide); the arithmetic below is gfx950's:
//   * |x| is the BF16 pattern with bit 15 cleared; non-negative floats order
//     as integers, so the block max is an integer max (packed u16 pairs),
//     finished across the four lanes with two quad-permute DPP moves.
//   * The shared exponent floor(log2 amax) - 2 comes from the exponent field:
//     scale byte = max(E_field(amax) - 2, 0); a zero or subnormal amax gives 0.
//   * v_cvt_scalef32_pk_fp4_bf16 divides two BF16 values by the scale and
//     rounds them to E2M1 (nearest even, saturating); the scale operand
//     carries the UE8M0 byte in its float exponent field.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mxfp4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ u16x2_t abs_pair(uint32_t w) {
  return __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
}

__device__ __forceinline__ uint32_t block_quarter_absmax(u32x4_t q) {
  u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(abs_pair(q.x), abs_pair(q.y)),
                                        __builtin_elementwise_max(abs_pair(q.z), abs_pair(q.w)));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Max over the four lanes 4i..4i+3 that hold one block.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  v = max(v, o);  // quad_perm [1,0,3,2]
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  return max(v, o);  // quad_perm [2,3,0,1]
}

// The word is passed by value: a bit cast applied straight to a vector
// element (q.y) was seen to read element 0 instead.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2_t, w);
}

__device__ __forceinline__ uint32_t encode8(u32x4_t q, float scale) {
  const uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3];
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w0), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w1), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w2), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w3), scale, 3);
  return r;
}

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
    const uint32_t byte = (uint32_t)max((int)(amax >> 7) - 2, 0);
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
    const uint32_t byte = (uint32_t)max((int)(amax >> 7) - 2, 0);
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
