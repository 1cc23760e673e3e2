/* Drives libmxfp4.so from plain C through include/mxfp4.h alone (the HIP
 * runtime supplies device memory): quantize two BF16 operands, run the
 * GEMM into FP32 and BF16 on the row-major and fragment-order paths, and
 * check every output against its closed form.
 *
 * Operands: A[m][k] = 2^(m % 4), B[n][k] = -2^(n % 5) when k % 3 == 0 and
 * +2^(n % 5) otherwise. Every 32-element block then has amax 2^j, scale
 * exponent j - 2 and every element quantizes to +-4 exactly (code 6, or 14
 * with the sign), so C[m][n] = 2^(m % 4 + n % 5) * (K - 2 * ceil(K / 3)),
 * exact in FP32 and in BF16.
 *
 * Exit status: 0 all checks passed, 1 a check failed, 2 no gfx950 device.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mxfp4.h"

enum { M = 64, N = 96, K = 512 };

static int failures = 0;

static void check(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
  }
}

static uint16_t bf16_pow2(int e, int negative) {
  return (uint16_t)((negative ? 0x8000u : 0u) | (uint32_t)(127 + e) << 7);
}

static double expected(int m, int n) {
  const int neg = (K + 2) / 3; /* k % 3 == 0 for k < K */
  return (double)(K - 2 * neg) * (double)(1u << (m % 4 + n % 5));
}

static float bf16_to_float(uint16_t b) {
  const uint32_t w = (uint32_t)b << 16;
  float f;
  memcpy(&f, &w, 4);
  return f;
}

#define HIP_OK(call) check((call) == hipSuccess, #call)

int main(void) {
  if (mxfp4_available() != 1) {
    fprintf(stderr, "no gfx950 device: %s\n", mxfp4_strerror(MXFP4_EUNSUPPORTED));
    return 2;
  }
  uint16_t* ha = malloc(sizeof(uint16_t) * M * K);
  uint16_t* hb = malloc(sizeof(uint16_t) * N * K);
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k) ha[m * K + k] = bf16_pow2(m % 4, 0);
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) hb[n * K + k] = bf16_pow2(n % 5, k % 3 == 0);

  void *xa, *xb, *ac, *as, *bc, *bs, *af, *asf, *bf, *bsf, *c32, *c16;
  HIP_OK(hipMalloc(&xa, sizeof(uint16_t) * M * K));
  HIP_OK(hipMalloc(&xb, sizeof(uint16_t) * N * K));
  HIP_OK(hipMalloc(&ac, M * K / 2));
  HIP_OK(hipMalloc(&as, M * K / 32));
  HIP_OK(hipMalloc(&bc, N * K / 2));
  HIP_OK(hipMalloc(&bs, N * K / 32));
  HIP_OK(hipMalloc(&af, M * K / 2));
  HIP_OK(hipMalloc(&asf, M * K / 32));
  HIP_OK(hipMalloc(&bf, N * K / 2));
  HIP_OK(hipMalloc(&bsf, N * K / 32));
  HIP_OK(hipMalloc(&c32, sizeof(float) * M * N));
  HIP_OK(hipMalloc(&c16, sizeof(uint16_t) * M * N));
  HIP_OK(hipMemcpy(xa, ha, sizeof(uint16_t) * M * K, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(xb, hb, sizeof(uint16_t) * N * K, hipMemcpyHostToDevice));

  /* Row-major path: the 5-argument quantize (null stream), then the GEMM. */
  check(mxfp4_quantize(xa, M, K, ac, as) == MXFP4_OK, "mxfp4_quantize A");
  check(mxfp4_quantize_async(xb, N, K, bc, bs, NULL) == MXFP4_OK, "mxfp4_quantize_async B");
  check(mxfp4_gemm(ac, as, bc, bs, M, N, K, MXFP4_OUT_FP32, c32, NULL) == MXFP4_OK,
        "mxfp4_gemm fp32");
  check(mxfp4_gemm(ac, as, bc, bs, M, N, K, MXFP4_OUT_BF16, c16, NULL) == MXFP4_OK,
        "mxfp4_gemm bf16");
  HIP_OK(hipDeviceSynchronize());

  uint8_t* hac = malloc(M * K / 2);
  uint8_t* has = malloc(M * K / 32);
  uint8_t* hbc = malloc(N * K / 2);
  uint8_t* hbs = malloc(N * K / 32);
  HIP_OK(hipMemcpy(hac, ac, M * K / 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(has, as, M * K / 32, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hbc, bc, N * K / 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hbs, bs, N * K / 32, hipMemcpyDeviceToHost));
  int bad_bytes = 0;
  for (int m = 0; m < M; ++m) {
    for (int i = 0; i < K / 2; ++i) bad_bytes += hac[m * K / 2 + i] != 0x66;
    for (int j = 0; j < K / 32; ++j) bad_bytes += has[m * K / 32 + j] != 127 + m % 4 - 2;
  }
  for (int n = 0; n < N; ++n) {
    for (int i = 0; i < K / 2; ++i) {
      const int lo = (2 * i) % 3 == 0 ? 0xE : 0x6, hi = (2 * i + 1) % 3 == 0 ? 0xE : 0x6;
      bad_bytes += hbc[n * K / 2 + i] != (uint8_t)(lo | hi << 4);
    }
    for (int j = 0; j < K / 32; ++j) bad_bytes += hbs[n * K / 32 + j] != 127 + n % 5 - 2;
  }
  check(bad_bytes == 0, "quantized codes and scales equal their closed form");

  float* h32 = malloc(sizeof(float) * M * N);
  uint16_t* h16 = malloc(sizeof(uint16_t) * M * N);
  HIP_OK(hipMemcpy(h32, c32, sizeof(float) * M * N, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h16, c16, sizeof(uint16_t) * M * N, hipMemcpyDeviceToHost));
  int bad32 = 0, bad16 = 0;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      bad32 += (double)h32[m * N + n] != expected(m, n);
      bad16 += (double)bf16_to_float(h16[m * N + n]) != expected(m, n);
    }
  check(bad32 == 0, "FP32 GEMM equals its closed form");
  check(bad16 == 0, "BF16 GEMM equals its closed form");

  /* Fragment-order path: quantize A straight into it, re-lay B, same C. */
  check(mxfp4_quantize_frag(xa, M, K, af, asf, NULL) == MXFP4_OK, "mxfp4_quantize_frag");
  check(mxfp4_to_frag(bc, bs, N, K, bf, bsf, NULL) == MXFP4_OK, "mxfp4_to_frag");
  HIP_OK(hipMemset(c32, 0, sizeof(float) * M * N));
  check(mxfp4_gemm_frag(af, asf, bf, bsf, M, N, K, MXFP4_OUT_FP32, c32, NULL) == MXFP4_OK,
        "mxfp4_gemm_frag");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h32, c32, sizeof(float) * M * N, hipMemcpyDeviceToHost));
  bad32 = 0;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) bad32 += (double)h32[m * N + n] != expected(m, n);
  check(bad32 == 0, "fragment-order FP32 GEMM equals its closed form");

  /* The tile kernel named explicitly: same closed form. */
  HIP_OK(hipMemset(c32, 0, sizeof(float) * M * N));
  check(mxfp4_gemm_tile(ac, as, bc, bs, M, N, K, MXFP4_OUT_FP32, c32, NULL) == MXFP4_OK,
        "mxfp4_gemm_tile");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h32, c32, sizeof(float) * M * N, hipMemcpyDeviceToHost));
  bad32 = 0;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) bad32 += (double)h32[m * N + n] != expected(m, n);
  check(bad32 == 0, "tile-kernel FP32 GEMM equals its closed form");

  /* Rejected calls return their status and launch nothing. */
  check(mxfp4_gemm(ac, as, bc, bs, M, N, 100, MXFP4_OUT_FP32, c32, NULL) == MXFP4_EINVAL,
        "K % 256 != 0 is rejected");
  check(mxfp4_gemm(ac, as, bc, bs, M, N, K, 7, c32, NULL) == MXFP4_EINVAL,
        "unknown out_dtype is rejected");
  check(mxfp4_gemm((char*)ac + 8, as, bc, bs, M, N, K, MXFP4_OUT_FP32, c32, NULL) ==
            MXFP4_EALIGN,
        "misaligned A is rejected");
  check(strlen(mxfp4_strerror(MXFP4_EALIGN)) > 0, "mxfp4_strerror text");

  hipFree(xa); hipFree(xb); hipFree(ac); hipFree(as); hipFree(bc); hipFree(bs);
  hipFree(af); hipFree(asf); hipFree(bf); hipFree(bsf); hipFree(c32); hipFree(c16);
  free(ha); free(hb); free(hac); free(has); free(hbc); free(hbs); free(h32); free(h16);
  printf("c_abi_check: %s (%d failures)\n", failures ? "FAILED" : "OK", failures);
  return failures ? 1 : 0;
}
