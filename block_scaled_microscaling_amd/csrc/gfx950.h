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

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// A pointer the caller knows to be the same in every lane, read from lane 0
// into scalar registers (an inline-asm "s" operand must not be left to a
// divergence analysis that cannot see the value is uniform).
__device__ __forceinline__ const uint8_t* sgpr_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>((uint64_t)hi << 32 | lo);
}

// Buffer resources for raw (untyped, stride 0) buffer stores: word 3 sets
// the data format to 32 bits, which raw accesses need to be valid; an access
// whose offset lies at or past the resource's byte count is dropped by the
// hardware. Cache-policy bits of a buffer instruction: nt (stream past L2).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNt = 2;

// Row-wise MXFP4 block arithmetic (used by the quantize kernels and the
// fused SwiGLU epilogue). Four consecutive lanes hold one 32-element block,
// 16 bytes (8 BF16) each.
//   * |x| is the BF16 pattern with bit 15 cleared; non-negative floats order
//     as integers, so the block max is an integer max (packed u16 pairs),
//     finished across the four lanes with two quad-permute DPP moves.
//   * The shared exponent floor(log2 amax) - 2 comes from the exponent field:
//     scale byte = max(E_field(amax) - 2, 0); a zero or subnormal amax gives 0.
//   * v_cvt_scalef32_pk_fp4_bf16 divides two BF16 values by the scale and
//     rounds them to E2M1 (nearest even, saturating); the scale operand
//     carries the UE8M0 byte in its float exponent field.
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

// Scale byte of a block from its largest |BF16| pattern.
__device__ __forceinline__ uint32_t scale_byte_of(uint32_t amax) {
  return (uint32_t)max((int)(amax >> 7) - 2, 0);
}

// The word is passed by value: a bit cast applied straight to a vector
// element (q.y) was seen to read element 0 instead.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2_t, w);
}

// Eight BF16 values (one lane's quarter of a block) -> eight E2M1 codes,
// element 2i in bits 4i..4i+3 (the low nibble of byte i first).
__device__ __forceinline__ uint32_t encode8(u32x4_t q, float scale) {
  const uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3];
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w0), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w1), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w2), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w3), scale, 3);
  return r;
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
