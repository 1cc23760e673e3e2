// Device helpers shared by the gfx950 GEMM kernels: the block-scaled FP4
// MFMA, global -> LDS copies, the LDS row swizzle and BF16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4 (cbsz = blgp = 4).
// Per lane l, an operand is the 32 codes (16 bytes) of row l % 32 in K block
// l / 32 of a 64-wide K slice, and sx / sy hold that block's UE8M0 scale in
// byte SEL_X / SEL_Y. Accumulator register v of lane l holds (row of x)
// 8 (v / 4) + 4 (l / 32) + v % 4, (row of y) l % 32.
template <int SEL_X, int SEL_Y>
__device__ __forceinline__ v16f_t mfma_fp4(const uint4& x, const uint4& y, v16f_t c, uint32_t sx,
                                           uint32_t sy) {
  const v8i_t xv = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  const v8i_t yv = {(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xv, yv, c, 4, 4, SEL_X, (int)sx, SEL_Y,
                                                         (int)sy);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> a BF16 pair (round to nearest even, lo in the low half), one
// v_cvt_pk_bf16_f32 (converting the halves one by one costs four VALU ops).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// XOR swizzle of the 16-byte chunk index within a 128-byte LDS row: the
// lanes reading one chunk column of 16 consecutive rows fall on distinct
// banks (in groups of 8 and of 16).
__device__ __forceinline__ int chunk_swizzle(int row) {
  return (row & 6) | ((row ^ (row >> 3)) & 1);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Global -> LDS copies. lds is the wave-uniform LDS byte address of the
// destination; lane i's bytes land at lds + size * i. Inline assembly, so
// that the compiler, which cannot tell the LDS buffers apart, adds no wait
// for these loads before LDS reads: every wait on them is an explicit one.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds) : "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds) : "m0");
}

}  // namespace mxfp4
