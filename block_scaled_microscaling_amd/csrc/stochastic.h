// Device helpers for stochastic-rounding MXFP4 quantize on gfx950.
//
// Random bits: one Philox4x32-10 draw per 16-element half block. The
// generator is the Philox construction of Salmon, Moraes, Dror and Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): per round two
// 32x32 -> 64-bit products of the even counter words with the paper's
// multipliers, the high halves folded into the odd words with the round
// key, the key advanced by the paper's Weyl increments; 10 rounds. Keying
// each draw by the block's coordinates and the direction follows the
// stochastic-rounding design described on NVIDIA/TransformerEngine #3809
// (description): counter (block column, row, direction, half), key (seed
// low word, seed high word); element 16 h + i takes byte i % 4 of word i / 4.
//
// Rounding of one element with its random byte u: the block's scale byte b
// gives v = x * 2^(127 - b). The element is carried as y = v * 2^-126 in
// fp32, so the E2M1 grid lines up with the fp32 bit fields: an E2M1 value
// keeps the exponent field and mantissa bit 22 of y (E2M1's subnormal step
// 0.5 lands on fp32's subnormal range, where bit 22 is worth 0.5 * 2^-126),
// and bits 21..14 of y are floor(256 * frac) of the position between the two
// grid neighbours. Adding u at bit 14 carries into bit 22 exactly when
// floor(256 frac) + u >= 256; clearing bits 21..0 then leaves the lower or
// the upper neighbour (a carry out of bit 22 moves into the next binade,
// which is the next grid value). v_cvt_scalef32_pk_fp4_f32 with scale
// 2^-126 turns the result, already on the grid, into its code and saturates
// 8 to 6. The sign bit rides along untouched. fp32 denormals are preserved
// (the kernels run in IEEE denormal mode), which this relies on for |v| < 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

constexpr uint32_t kDirRowwise = 0;
constexpr uint32_t kDirColumnwise = 1;

struct Draw {
  uint32_t w[4];
};

// a ^ b ^ k with the round key k wave-uniform: one v_bitop3_b32 with the
// XOR3 truth table 0x96 (the compiler otherwise emits two v_xor_b32 per
// output word).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

__device__ __forceinline__ Draw philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return Draw{{c0, c1, c2, c3}};
}

// 2^-126 as the conversion's scale operand.
__device__ __forceinline__ float sr_cvt_scale() { return __uint_as_float(0x00800000u); }

// One element: x_f32 = the BF16 value as fp32 bits, n = 1 - scale byte,
// u = random byte (0..255). Returns the grid value times 2^-126.
__device__ __forceinline__ float sr_round(uint32_t x_f32, int n, uint32_t u) {
  const float y = __builtin_amdgcn_ldexpf(__uint_as_float(x_f32), n);
  return __uint_as_float((__float_as_uint(y) + (u << 14)) & 0xFFC00000u);
}

// Byte k (0..3) of a random word.
__device__ __forceinline__ uint32_t rand_byte(uint32_t w, int k) {
  return __builtin_amdgcn_ubfe(w, 8 * k, 8);
}

// Eight elements given as fp32 bit patterns (in element order) with their
// eight random bytes, bytes 0..3 in r0 and 4..7 in r1. Returns the four code
// bytes (element 2i in the low nibble of byte i).
__device__ __forceinline__ uint32_t sr_encode8_f32(const uint32_t (&x)[8], int n, uint32_t r0,
                                                   uint32_t r1) {
  const float s = sr_cvt_scale();
  uint32_t c = 0;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, sr_round(x[0], n, rand_byte(r0, 0)),
                                               sr_round(x[1], n, rand_byte(r0, 1)), s, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, sr_round(x[2], n, rand_byte(r0, 2)),
                                               sr_round(x[3], n, rand_byte(r0, 3)), s, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, sr_round(x[4], n, rand_byte(r1, 0)),
                                               sr_round(x[5], n, rand_byte(r1, 1)), s, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, sr_round(x[6], n, rand_byte(r1, 2)),
                                               sr_round(x[7], n, rand_byte(r1, 3)), s, 3);
  return c;
}

// Eight consecutive elements held as four BF16 pair words (the even element
// in the low half).
__device__ __forceinline__ uint32_t sr_encode8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                               int n, uint32_t r0, uint32_t r1) {
  const uint32_t x[8] = {w0 << 16, w0 & 0xFFFF0000u, w1 << 16, w1 & 0xFFFF0000u,
                         w2 << 16, w2 & 0xFFFF0000u, w3 << 16, w3 & 0xFFFF0000u};
  return sr_encode8_f32(x, n, r0, r1);
}

}  // namespace mxfp4
