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
//   * the tile GEMM's whole K-loop instruction mix (probe_step): per 64
//     MFMAs (one 256-wide K step of a 128 x 128 wave tile), 32 fragment
//     reads in the K loop's order, 20 global -> LDS DMAs (16 code loads in
//     pairs, 4 scale loads) from an L2-resident 1 MiB buffer into LDS that
//     is never read, and one wait for every load plus a barrier;
//   * LDS read bandwidth (ds_read_b128 only).
// One workgroup per CU (96 KiB of dynamic LDS each); fragment reads stay in
// the first 64 KiB and DMAs land in 64 KiB .. 92 KiB; loops have fixed trip
// counts. Prints one JSON object per case. Built next to libmxfp4.so by build.build_probe(); run by
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

// One wave instruction of global -> LDS DMA (lane i's 16 bytes land at
// m0 + 16 i), or two 1 KiB apart from one M0 write, as the tile GEMM issues
// its code loads.
__device__ __forceinline__ void dma_x1(const uint8_t* g, uint32_t off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:0"
               :: "v"(off), "s"(g), "s"(m0) : "m0");
}
__device__ __forceinline__ void dma_x2(const uint8_t* g, uint32_t off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %0, %1 offset:0\n\t"
               "global_load_lds_dwordx4 %0, %1 offset:1024"
               :: "v"(off), "s"(g), "s"(m0) : "m0");
}
#define PROBE_FENCE() __builtin_amdgcn_sched_barrier(0)

// One group of the K loop: the four MFMAs of A tile a, a fragment read after
// each of the first two, then D DMA instructions (0, 1 or 2) before the last.
template <int D>
__device__ __forceinline__ void step_group(v16f (&acc)[4][4], const uint4 (&f)[8], int a,
                                           uint4& r0, uint4& r1, const uint4* lds, int i0,
                                           int i1, const uint8_t* g, uint32_t off, uint32_t m0,
                                           uint32_t sc) {
  acc[a][0] = mfma(f[4], f[a], acc[a][0], sc);
  r0 = lds[i0];
  PROBE_FENCE();
  acc[a][1] = mfma(f[5], f[a], acc[a][1], sc);
  r1 = lds[i1];
  PROBE_FENCE();
  acc[a][2] = mfma(f[6], f[a], acc[a][2], sc);
  if constexpr (D == 2) dma_x2(g, off, m0);
  if constexpr (D == 1) dma_x1(g, off, m0);
  PROBE_FENCE();
  acc[a][3] = mfma(f[7], f[a], acc[a][3], sc);
  PROBE_FENCE();
}

// K steps of the tile GEMM's loop on one 128 x 128 wave tile: four phases
// of 16 MFMAs and 8 fragment reads each, 5 DMA instructions per phase (2,
// 2, 1, 0 per group), and after phase 2 a wait for every load and a barrier.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void probe_step(const uint8_t* __restrict__ gbuf, uint64_t* out, float* sink, int steps) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4096; i += blockDim.x)
    lds[i] = make_uint4(i * 2654435761u, (i ^ 0x5bd1e995u) * 40503u, i * 0x9E3779B9u,
                        ~(i * 747796405u));
  __syncthreads();
  uint4 f0[8], f1[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) f0[q] = lds[(q * 64 + lane + wave * 512) & 4095];
  const uint32_t sc = 0x7f7f7f7fu;
  v16f acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = v16f{};
  const uint32_t lds_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base + 65536 + wave * 8192);
  const uint8_t* g = gbuf + (size_t)(blockIdx.x & 255) * 4096;  // within 1 MiB
  const uint32_t off = 16 * lane;                                // + 1024: < 2 KiB
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0t = __builtin_amdgcn_s_memrealtime();
  for (int st = 0; st < steps; ++st) {
#pragma unroll
    for (int ph = 0; ph < 4; ++ph) {
      const int base = ((2 * ph + (st & 3)) * 512 + wave * 64) & 4095;
      uint4(&fc)[8] = (ph & 1) ? f1 : f0;
      uint4(&fn)[8] = (ph & 1) ? f0 : f1;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int i0 = (base + (2 * a) * 64 + lane) & 4095;
        const int i1 = (base + (2 * a + 1) * 64 + lane) & 4095;
        if (a < 2)
          step_group<2>(acc, fc, a, fn[2 * a], fn[2 * a + 1], lds, i0, i1, g, off, m0, sc);
        else if (a == 2)
          step_group<1>(acc, fc, a, fn[2 * a], fn[2 * a + 1], lds, i0, i1, g, off, m0, sc);
        else
          step_group<0>(acc, fc, a, fn[2 * a], fn[2 * a + 1], lds, i0, i1, g, off, m0, sc);
      }
      if (ph == 2) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int k = 0; k < 16; ++k) s += acc[a][b][k];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) {
    const int w = blockIdx.x * 4 + wave;
    out[2 * w] = t1 - t0;
    out[2 * w + 1] = r1 - r0t;
  }
}

int run_step(const char* name, int steps, int grid) {
  CHECK(hipFuncSetAttribute((const void*)probe_step, hipFuncAttributeMaxDynamicSharedMemorySize,
                            96 * 1024));
  const int nw = grid * 4;
  uint64_t* d_out = nullptr;
  float* d_sink = nullptr;
  uint8_t* d_g = nullptr;
  CHECK(hipMalloc(&d_out, sizeof(uint64_t) * 2 * nw));
  CHECK(hipMalloc(&d_sink, sizeof(float) * nw * 64));
  CHECK(hipMalloc(&d_g, 1 << 20));
  CHECK(hipMemset(d_g, 0x3c, 1 << 20));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<uint64_t> h(2 * nw);
  float best = 1e30f;
  double cyc = 0, real = 0;
  for (int rep = 0; rep < 6; ++rep) {
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(probe_step, dim3(grid), dim3(256), 96 * 1024, 0, d_g, d_out, d_sink, steps);
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
    if (rep >= 2 && ms < best) {
      best = ms;
      cyc = (double)mc;
      real = (double)mr;
    }
  }
  const double mhz = cyc / (real / 100.0);
  const double busy = (double)steps * 64 * 32.0 / cyc;
  const double lds_bpc = (double)steps * (32 + 20) * 1024.0 * 4 / cyc;
  const double tflops = (double)grid * 4 * steps * 64 * 131072.0 / (best * 1e-3) / 1e12;
  printf("{\"case\": \"%s\", \"waves_per_cu\": 4, \"ms\": %.4f, \"clock_mhz\": %.1f, "
         "\"mfma_busy\": %.4f, \"fp4_tflops\": %.1f, \"lds_bytes_per_clk_per_cu\": %.1f, "
         "\"cycles_per_k_step\": %.0f}\n",
         name, best, mhz, busy, tflops, lds_bpc, cyc / steps);
  fflush(stdout);
  CHECK(hipFree(d_out));
  CHECK(hipFree(d_sink));
  CHECK(hipFree(d_g));
  return 0;
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
  r |= run_step("K-loop mix: 64 mfma, 32 LDS reads, 20 DMAs, wait + barrier per step", 2000, cus);
  r |= run<4, 4, true, false, 4>("LDS reads only", 8000, cus);
  r |= run<4, 4, true, false, 16>("LDS reads only", 8000, cus);
  return r;
}
