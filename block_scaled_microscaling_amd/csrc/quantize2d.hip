// Bidimensional BF16 -> MXFP4 quantize for gfx950: one pass over X [M, K]
// writes both the row-wise MXFP4 form (blocks of 32 along K, as
// quantize.hip) and the column-wise form, i.e. the row-wise MXFP4 form of
// X^T (blocks of 32 along M), as [K, M/2] codes and [K, M/32] scales.
//
// The column-wise operand is what a GEMM contracting over M needs (the
// weight-gradient product of a linear layer). The single-pass design, row
// blocks straight from registers and only the transposed direction staged
// through on-chip memory, is the bidimensional quantize kernel described on
// NVIDIA/TransformerEngine #3809 (description); the block arithmetic is the
// one of quantize.hip (integer amax of |bits|, scale byte = max(E_field(amax)
// - 2, 0), v_cvt_scalef32_pk_fp4_bf16 for RNE E2M1 codes).
//
// Work mapping: a workgroup of 256 threads owns a 128 x 128 tile.
//   Row phase: thread t takes row t / 2, columns 64 (t % 2) .. +63 (two MX
//   blocks, eight 16-byte loads), encodes them from registers and parks the
//   tile in LDS (rows padded to 272 bytes so the 16-byte writes of 8 rows
//   fall on distinct banks).
//   Column phase: thread t takes columns 2 (t % 64), +1 and rows
//   32 (t / 64) .. +31: 32 dword reads (both columns at once), an integer
//   amax per column, 16 byte-permutes per column to pair consecutive rows,
//   and 16 conversions per column.
// Edge tiles (M or K not a multiple of 128) mask whole 32-element blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mxfp4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 128;
constexpr int kLdsRow = 2 * kTile + 16;  // bytes per LDS row (padded)

__device__ __forceinline__ u16x2_t abs_pair(uint32_t w) {
  return __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
}
__device__ __forceinline__ u16x2_t max2(u16x2_t a, u16x2_t b) {
  return __builtin_elementwise_max(a, b);
}
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2_t, w);
}
__device__ __forceinline__ uint32_t scale_byte(uint32_t amax_bits) {
  return (uint32_t)max((int)(amax_bits >> 7) - 2, 0);
}
// Four BF16 pairs (8 elements, element 2i in the low half of word i) to 8
// E2M1 codes, element 2i in the low nibble of byte i.
__device__ __forceinline__ uint32_t encode8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                            float scale) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w0), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w1), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w2), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w3), scale, 3);
  return r;
}

__global__ __launch_bounds__(kThreads) void quantize_2d_kernel(
    const uint8_t* __restrict__ x, int M, int K, uint8_t* __restrict__ codes_row,
    uint8_t* __restrict__ scales_row, uint8_t* __restrict__ codes_col,
    uint8_t* __restrict__ scales_col) {
  __shared__ __align__(16) uint8_t tile[kTile * kLdsRow];
  const int t = threadIdx.x;
  const int m0 = blockIdx.y * kTile;
  const int c0 = blockIdx.x * kTile;
  const int64_t row_bytes = 2 * (int64_t)K;

  // Row phase.
  {
    const int r = t >> 1;
    const int half = t & 1;
    const int m = m0 + r;
    const int cb = c0 + 64 * half;  // first column of this thread's two blocks
    u32x4_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int col = cb + 8 * i;
      v[i] = (m < M && col < K)
                 ? __builtin_nontemporal_load(
                       reinterpret_cast<const u32x4_t*>(x + m * row_bytes + 2 * (int64_t)col))
                 : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4_t*>(tile + r * kLdsRow + 128 * half + 16 * i) = v[i];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = cb + 32 * b;
      u16x2_t mx = abs_pair(v[4 * b][0]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = max2(mx, abs_pair(v[4 * b + i][j]));
      const uint32_t byte = scale_byte(max((uint32_t)mx.x, (uint32_t)mx.y));
      const float scale = __uint_as_float(byte << 23);
      u32x4_t out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_t q = v[4 * b + i];
        out[i] = encode8(q[0], q[1], q[2], q[3], scale);
      }
      if (m < M && col < K) {
        *reinterpret_cast<u32x4_t*>(codes_row + (int64_t)m * (K / 2) + col / 2) = out;
        scales_row[(int64_t)m * (K / 32) + col / 32] = (uint8_t)byte;
      }
    }
  }
  __syncthreads();

  // Column phase: columns k0 = c0 + 2 cp and k0 + 1, rows mb .. mb + 31.
  {
    const int cp = t & 63;
    const int rb = t >> 6;
    const int k0 = c0 + 2 * cp;
    const int mb = m0 + 32 * rb;
    uint32_t w[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      w[i] = *reinterpret_cast<const uint32_t*>(tile + (32 * rb + i) * kLdsRow + 4 * cp);
    u16x2_t mx = abs_pair(w[0]);
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = max2(mx, abs_pair(w[i]));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t byte = scale_byte(e == 0 ? (uint32_t)mx.x : (uint32_t)mx.y);
      const float scale = __uint_as_float(byte << 23);
      // Pair rows 2i, 2i + 1 of column k0 + e: bytes (2e, 2e + 1) of each word.
      const uint32_t sel = e == 0 ? 0x05040100u : 0x07060302u;
      u32x4_t out;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 8 * g + 2 * j;
          p[j] = __builtin_amdgcn_perm(w[i + 1], w[i], sel);
        }
        out[g] = encode8(p[0], p[1], p[2], p[3], scale);
      }
      const int k = k0 + e;
      if (k < K && mb < M) {
        *reinterpret_cast<u32x4_t*>(codes_col + (int64_t)k * (M / 2) + mb / 2) = out;
        scales_col[(int64_t)k * (M / 32) + mb / 32] = (uint8_t)byte;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize_2d(const void* x_bf16, int M, int K, void* codes_row, void* scales_row,
                              void* codes_col, void* scales_col, hipStream_t stream) {
  const dim3 grid((K + kTile - 1) / kTile, (M + kTile - 1) / kTile);
  hipLaunchKernelGGL(quantize_2d_kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(x_bf16), M, K,
                     static_cast<uint8_t*>(codes_row), static_cast<uint8_t*>(scales_row),
                     static_cast<uint8_t*>(codes_col), static_cast<uint8_t*>(scales_col));
  return hipGetLastError();
}

}  // namespace mxfp4
