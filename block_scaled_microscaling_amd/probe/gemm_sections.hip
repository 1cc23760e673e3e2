// Section timing of the 256 x 256 tile GEMM (csrc/gemm.hip), built as a
// program of its own: this file gives the kernel's SectionTimer hooks a body
// and includes the kernel source, so the kernel timed is the library's, with
// s_memtime reads at its section marks (a few scalar instructions each). Each
// wave sums the cycles of every section and stores its sums once, at the end
// of the launch, into g_sections. The library itself compiles the hooks to
// nothing.
//
// For each workload: operands of random code bytes and scales 118..130,
// rotated through enough copies to exceed twice the last-level cache; 20
// untimed launches, then one launch whose sums are read back. Prints one JSON
// object per workload: per section the mean cycles per wave and tile (and per
// K step for the loop sections), the engine clock (s_memtime against the 100
// MHz s_memrealtime) and the launch time. Run by `python bench.py --sections`.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

namespace mxfp4 {

constexpr int kMaxTimedWaves = 1024;  // 256 workgroups x 4 waves
constexpr int kSlots = 16;            // per wave: sections, then start and end time stamps

__device__ unsigned long long g_sections[kMaxTimedWaves * kSlots];

struct SectionTimer {
  unsigned long long last;
  unsigned long long t0, r0;
  unsigned long long acc[kSlots - 4];
  __device__ void start() {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    last = t0;
#pragma unroll
    for (int i = 0; i < kSlots - 4; ++i) acc[i] = 0;
  }
  template <int kSec>
  __device__ void mark() {
    static_assert(kSec < kSlots - 4, "section slot");
    const unsigned long long t = __builtin_amdgcn_s_memtime();
    acc[kSec] += t - last;
    last = t;
  }
  __device__ void store(int w) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if ((threadIdx.x & 63) != 0 || w >= kMaxTimedWaves) return;
    unsigned long long* o = g_sections + (size_t)w * kSlots;
#pragma unroll
    for (int i = 0; i < kSlots - 4; ++i) o[i] = acc[i];
    o[kSlots - 4] = t1 - t0;  // cycles of the whole wave
    o[kSlots - 3] = r1 - r0;  // 100 MHz ticks of the whole wave
    o[kSlots - 2] = 0;
    o[kSlots - 1] = 0;
  }
};

}  // namespace mxfp4

#define MXFP4_SECTION_TIMERS
#include "../csrc/gemm.hip"

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)

// Random code bytes, or scale bytes in 118..130.
__global__ void fill_bytes(uint8_t* p, size_t n, uint32_t seed, int scales) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    uint32_t x = (uint32_t)i * 2654435761u ^ seed;
    x ^= x >> 15;
    x *= 2246822519u;
    x ^= x >> 13;
    p[i] = scales ? (uint8_t)(118 + x % 13) : (uint8_t)(x >> 24);
  }
}

static const char* kNames[] = {"tile_wait", "loop",       "data_wait", "barrier",  "loop_end",
                               "epi_head",  "epi_store",  "epi_barrier", "epi_tail"};

struct Shape {
  const char* name;
  int M, N, K;
  bool fp32, swiglu;
};

static int run(const Shape& s) {
  const size_t ac = (size_t)s.M * s.K / 2, as = (size_t)s.M * s.K / 32;
  const size_t bc = (size_t)s.N * s.K / 2, bs = (size_t)s.N * s.K / 32;
  const size_t set_bytes = ac + as + bc + bs;
  const size_t llc = 256u << 20;
  const int copies = (int)std::min<size_t>(16, (2 * llc + set_bytes - 1) / set_bytes + 1);
  std::vector<uint8_t*> sets(copies);
  for (int i = 0; i < copies; ++i) {
    CHECK(hipMalloc(&sets[i], set_bytes));
    hipLaunchKernelGGL(fill_bytes, dim3(1024), dim3(256), 0, 0, sets[i], ac, 11u + i, 0);
    hipLaunchKernelGGL(fill_bytes, dim3(1024), dim3(256), 0, 0, sets[i] + ac, as, 23u + i, 1);
    hipLaunchKernelGGL(fill_bytes, dim3(1024), dim3(256), 0, 0, sets[i] + ac + as, bc, 37u + i, 0);
    hipLaunchKernelGGL(fill_bytes, dim3(1024), dim3(256), 0, 0, sets[i] + ac + as + bc, bs,
                       41u + i, 1);
    CHECK(hipGetLastError());
  }
  void* C = nullptr;
  uint8_t *act_codes = nullptr, *act_scales = nullptr;
  if (s.swiglu) {
    CHECK(hipMalloc(&act_codes, (size_t)s.M * (s.N / 4)));
    CHECK(hipMalloc(&act_scales, (size_t)s.M * (s.N / 64)));
  } else {
    CHECK(hipMalloc(&C, (size_t)s.M * s.N * (s.fp32 ? 4 : 2)));
  }
  auto launch = [&](int i) {
    uint8_t* p = sets[i % copies];
    if (s.swiglu)
      return mxfp4::launch_gemm_swiglu(p, p + ac, p + ac + as, p + ac + as + bc, s.M, s.N, s.K,
                                       act_codes, act_scales, nullptr, 0);
    return mxfp4::launch_gemm(p, p + ac, p + ac + as, p + ac + as + bc, s.M, s.N, s.K, s.fp32,
                              C, 0);
  };
  for (int i = 0; i < 20; ++i) CHECK(launch(i));
  CHECK(hipDeviceSynchronize());
  std::vector<unsigned long long> h(mxfp4::kMaxTimedWaves * mxfp4::kSlots, 0);
  CHECK(hipMemcpyToSymbol(HIP_SYMBOL(mxfp4::g_sections), h.data(),
                          sizeof(unsigned long long) * h.size()));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0, 0));
  CHECK(launch(20));
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipMemcpyFromSymbol(h.data(), HIP_SYMBOL(mxfp4::g_sections),
                            sizeof(unsigned long long) * h.size()));

  int workers = 0;
  CHECK(mxfp4::device_workers(workers));
  const int tiles_m = (s.M + 255) / 256;
  const int tiles_n = s.swiglu ? (s.N / 2 + 127) / 128 : (s.N + 255) / 256;
  const int total = tiles_m * tiles_n;
  const int grid = mxfp4::tile_grid(total, workers);
  const int ksteps = s.K / 256;
  double sum[mxfp4::kSlots] = {0};
  double tiles = 0;
  int waves = 0;
  for (int b = 0; b < grid && b < mxfp4::kMaxTimedWaves / 4; ++b) {
    const int nt = (total - b + grid - 1) / grid;
    for (int w = 0; w < 4; ++w) {
      const unsigned long long* o = h.data() + (size_t)(b * 4 + w) * mxfp4::kSlots;
      for (int i = 0; i < mxfp4::kSlots; ++i) sum[i] += (double)o[i];
      tiles += nt;
      ++waves;
    }
  }
  const double total_cyc = sum[mxfp4::kSlots - 4];
  const double mhz = total_cyc / (sum[mxfp4::kSlots - 3] / 100.0);
  printf("{\"workload\": \"%s\", \"M\": %d, \"N\": %d, \"K\": %d, \"out\": \"%s\", "
         "\"tiles\": %d, \"workgroups\": %d, \"launch_us\": %.2f, \"clock_mhz\": %.1f, "
         "\"cycles_per_wave\": %.0f, \"sections\": {",
         s.name, s.M, s.N, s.K, s.swiglu ? "swiglu+mxfp4" : (s.fp32 ? "fp32" : "bf16"), total,
         grid, ms * 1000.0, mhz, total_cyc / waves);
  for (int i = 0; i < mxfp4::kNumSections; ++i) {
    const bool per_step = i >= mxfp4::kSecLoop && i <= mxfp4::kSecBarrier;
    printf("%s\"%s\": {\"cycles_per_tile\": %.0f, \"share\": %.4f%s", i ? ", " : "", kNames[i],
           sum[i] / tiles, sum[i] / total_cyc, per_step ? ", \"cycles_per_k_step\": " : "");
    if (per_step) printf("%.0f", sum[i] / (tiles * ksteps));
    printf("}");
  }
  printf("}}\n");
  fflush(stdout);
  for (auto p : sets) CHECK(hipFree(p));
  if (C) CHECK(hipFree(C));
  if (act_codes) CHECK(hipFree(act_codes));
  if (act_scales) CHECK(hipFree(act_scales));
  return 0;
}

int main() {
  const Shape shapes[] = {
      {"square", 8192, 8192, 8192, false, false},
      {"mlp_gate_up", 16384, 28672, 4096, false, false},
      {"mlp_down", 16384, 4096, 14336, false, false},
      {"ragged", 4128, 6176, 7936, true, false},
      {"swiglu_gate_up", 16384, 28672, 4096, false, true},
  };
  int r = 0;
  for (const Shape& s : shapes) r |= run(s);
  return r;
}
