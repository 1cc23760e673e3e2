// Microbenchmark of the gfx950 limits the tile GEMM's design rests on:
//   * the block-scaled FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) issued
//     back to back, with one or two waves per SIMD, and the engine clock it
//     runs at (s_memtime against the 100 MHz s_memrealtime);
//   * the same MFMA stream with the tile GEMM's LDS operand reads
//     interleaved (8 ds_read_b128 per 16 MFMAs for 128 x 128 wave tiles, 6
//     per 8 for 128 x 64 wave tiles at two waves per SIMD), in the
//     compiler's order or in a fixed order (ORDER, sched_group_barrier):
//     per four MFMAs, MFMA read MFMA read MFMA MFMA (the tile GEMM's K
//     loop), MFMA MFMA read twice, or MFMA read read MFMA MFMA MFMA;
//   * LDS read bandwidth (ds_read_b128 only).
// One workgroup per CU (96 KiB of dynamic LDS each); every LDS access stays
// in the first 64 KiB; loops have fixed trip counts. Prints one JSON object
// per case. Built next to libmxfp4.so by build.build_probe(); run by
// `python bench.py --probe`.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                               \
    }                                                                         \
  } while (0)

__device__ __forceinline__ v16f mfma(const uint4& x, const uint4& y, v16f c, uint32_t s) {
  const v8i xv = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  const v8i yv = {(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xv, yv, c, 4, 4, 0, (int)s, 0, (int)s);
}

// Instruction order of one half iteration (16 MFMAs, 8 reads) for ORDER
// 1..3; 0 leaves it to the compiler.
template <int ORDER>
__device__ __forceinline__ void order16() {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if constexpr (ORDER == 1) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    } else if constexpr (ORDER == 2) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    } else if constexpr (ORDER == 3) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
  }
}

// Per K slice: NA A and NB B fragments (1 KiB each, contiguous) read from
// LDS when READS, NA * NB MFMAs on the previous slice's fragments when MFMA.
template <int NA, int NB, bool READS, bool MFMA, int WAVES, int ORDER = 0>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void probe(uint64_t* out, float* sink, int iters) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4096; i += blockDim.x)
    lds[i] = make_uint4(i * 2654435761u, (i ^ 0x5bd1e995u) * 40503u, i * 0x9E3779B9u,
                        ~(i * 747796405u));
  __syncthreads();
  v16f acc[NA][NB];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = v16f{};
  uint4 f0[NA + NB], f1[NA + NB];
#pragma unroll
  for (int q = 0; q < NA + NB; ++q) f0[q] = lds[(q * 64 + lane + wave * 512) & 4095];
  const uint32_t sc = 0x7f7f7f7fu;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 2) {
    const int base = ((it & 7) * 512 + wave * 64) & 4095;
#pragma unroll
    for (int q = 0; q < NA + NB; ++q) f1[q] = READS ? lds[(base + q * 64 + lane) & 4095] : f0[q];
    if (MFMA) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = mfma(f0[NA + b], f0[a], acc[a][b], sc);
      if constexpr (ORDER != 0) order16<ORDER>();
    }
#pragma unroll
    for (int q = 0; q < NA + NB; ++q)
      f0[q] = READS ? lds[(base + 2048 + q * 64 + lane) & 4095] : f1[q];
    if (MFMA) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = mfma(f1[NA + b], f1[a], acc[a][b], sc);
      if constexpr (ORDER != 0) order16<ORDER>();
    } else {
#pragma unroll
      for (int q = 0; q < NA + NB; ++q) acc[0][0][q & 15] += (float)(f0[q].x ^ f1[q].y);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int k = 0; k < 16; ++k) s += acc[a][b][k];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) {
    const int w = blockIdx.x * WAVES + wave;
    out[2 * w] = t1 - t0;
    out[2 * w + 1] = r1 - r0;
  }
}

template <int NA, int NB, bool READS, bool MFMA, int WAVES, int ORDER = 0>
int run(const char* name, int iters, int grid) {
  auto k = probe<NA, NB, READS, MFMA, WAVES, ORDER>;
  CHECK(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                            96 * 1024));
  const int nw = grid * WAVES;
  uint64_t* d_out = nullptr;
  float* d_sink = nullptr;
  CHECK(hipMalloc(&d_out, sizeof(uint64_t) * 2 * nw));
  CHECK(hipMalloc(&d_sink, sizeof(float) * nw * 64));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<uint64_t> h(2 * nw);
  float best = 1e30f;
  double cyc = 0, real = 0;
  for (int rep = 0; rep < 6; ++rep) {
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(k, dim3(grid), dim3(64 * WAVES), 96 * 1024, 0, d_out, d_sink, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipMemcpy(h.data(), d_out, sizeof(uint64_t) * 2 * nw, hipMemcpyDeviceToHost));
    uint64_t mc = 0, mr = 0;
    for (int w = 0; w < nw; ++w) {
      mc = std::max(mc, h[2 * w]);
      mr = std::max(mr, h[2 * w + 1]);
    }
    if (rep >= 2 && ms < best) {  // the first launches settle the clock
      best = ms;
      cyc = (double)mc;
      real = (double)mr;
    }
  }
  const double mhz = cyc / (real / 100.0);
  const double mfma_per_simd = MFMA ? (double)iters * NA * NB * WAVES / 4.0 : 0.0;
  const double busy = mfma_per_simd * 32.0 / cyc;  // 32 cycles per FP4 32x32x64 MFMA
  const double lds_bpc = READS ? (double)iters * (NA + NB) * 1024.0 * WAVES / cyc : 0.0;
  const double tflops =
      MFMA ? (double)grid * WAVES * iters * NA * NB * 131072.0 / (best * 1e-3) / 1e12 : 0.0;
  printf("{\"case\": \"%s\", \"waves_per_cu\": %d, \"ms\": %.4f, \"clock_mhz\": %.1f, "
         "\"mfma_busy\": %.4f, \"fp4_tflops\": %.1f, \"lds_bytes_per_clk_per_cu\": %.1f}\n",
         name, WAVES, best, mhz, busy, tflops, lds_bpc);
  fflush(stdout);
  CHECK(hipFree(d_out));
  CHECK(hipFree(d_sink));
  return 0;
}

int main() {
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  int r = 0;
  r |= run<4, 4, false, true, 4>("mfma only, 128x128 wave tiles", 8000, cus);
  r |= run<4, 2, false, true, 8>("mfma only, 128x64 wave tiles", 8000, cus);
  r |= run<4, 4, true, true, 4>("mfma + 8 LDS reads per 16 mfma", 8000, cus);
  r |= run<4, 4, true, true, 4, 1>("mfma + 8 LDS reads per 16 mfma, M r M r M M", 8000, cus);
  r |= run<4, 4, true, true, 4, 2>("mfma + 8 LDS reads per 16 mfma, M M r M M r", 8000, cus);
  r |= run<4, 4, true, true, 4, 3>("mfma + 8 LDS reads per 16 mfma, M r r M M M", 8000, cus);
  r |= run<4, 2, true, true, 8>("mfma + 6 LDS reads per 8 mfma", 8000, cus);
  r |= run<4, 4, true, false, 4>("LDS reads only", 8000, cus);
  r |= run<4, 4, true, false, 16>("LDS reads only", 8000, cus);
  return r;
}
