// Pre-shuffle of an MXFP4 weight B [N, K] for the tile GEMM, on gfx950.
//
// The a4w4 path of "Integrate MXFP4 hipblaslt GEMM support" (#697, Changes
// list) and the call site reviewed on "Initial integration of a4w4 GEMM"
// (#663) take the weight pre-shuffled, with swizzled scales, so that the GEMM
// moves it without address arithmetic. The layout here is this library's
// own: the exact byte order in which gemm_tile_kernel lands B in LDS.
//   Codes: one 32 KiB block per (256-row tile nt, 256-K step ks) at
//   (nt * KS + ks) * 32768; row x of the tile at x * 128, its physical
//   16-byte chunk p holding logical chunk p ^ swz(x), swz as chunk_swizzle.
//   Scales: one 8 KiB block per (tile nt, 1024-K chunk ch) at
//   (nt * NC + ch) * 8192; the 4-byte word of row 128 h + 32 t + r and
//   half-step s (128 K) at 128 (32 h + r) + 16 (s ^ ((r >> 1) & 7)) + 4 t.
// Rows past N and half-steps past K are written as zeros, so the GEMM reads
// whole blocks without clamping.
// Work mapping: one thread per 16-byte code chunk (a wave writes 1 KiB
// contiguously and reads 8 rows x 128 bytes, whole lines) and one thread
// per scale word (a wave writes 256 bytes contiguously).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950.h"
#include "kernels.h"

namespace mxfp4 {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void shuffle_codes_kernel(const uint8_t* __restrict__ codes,
                                                                 int N, int K,
                                                                 uint4* __restrict__ out,
                                                                 int64_t nchunks16) {
  const int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (o >= nchunks16) return;
  const int ks_n = K / 256;
  const int64_t blk = o >> 11;  // 2048 chunks of 16 bytes per 32 KiB block
  const int within = (int)(o & 2047);
  const int x = within >> 3, p = within & 7;
  const int nt = (int)(blk / ks_n), ks = (int)(blk % ks_n);
  const int row = 256 * nt + x;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < N) {
    const int c = p ^ chunk_swizzle(x);
    v = *reinterpret_cast<const uint4*>(codes + (int64_t)row * (K / 2) + 128 * ks + 16 * c);
  }
  out[o] = v;
}

__global__ __launch_bounds__(kThreads) void shuffle_scales_kernel(const uint8_t* __restrict__ scales,
                                                                  int N, int K,
                                                                  uint32_t* __restrict__ out,
                                                                  int64_t nwords) {
  const int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (w >= nwords) return;
  const int nc = (K + 1023) / 1024;
  const int64_t blk = w >> 11;  // 2048 words per 8 KiB block
  const int within = (int)(w & 2047);
  const int hr = within >> 5;  // 32 h + r
  const int h = hr >> 5, r = hr & 31;
  const int sp = (within >> 2) & 7, t = within & 3;
  const int s = sp ^ ((r >> 1) & 7);
  const int nt = (int)(blk / nc), ch = (int)(blk % nc);
  const int row = 256 * nt + 128 * h + 32 * t + r;
  const int hs = 8 * ch + s;  // half-step of the row
  uint32_t v = 0;
  if (row < N && hs < K / 128)
    v = *reinterpret_cast<const uint32_t*>(scales + (int64_t)row * (K / 32) + 4 * hs);
  out[w] = v;
}

// Fragment order (the skinny register-ring GEMM's operand order): one thread
// per 16-byte code chunk o of the output: block o / 256 = t KS + s, slice
// q = (o / 64) % 4, lane l = o % 64 holding row 32 t + l % 32 and block
// 4 (l / 32) + q of step s; and one thread per 4-byte scale word w: block
// w / 64, lane w % 64, scale bytes 8 s + 4 (l / 32) .. + 3 of its row.
__global__ __launch_bounds__(kThreads) void frag_codes_kernel(const uint8_t* __restrict__ codes,
                                                              int K, uint4* __restrict__ out,
                                                              int64_t nchunks16) {
  const int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (o >= nchunks16) return;
  const int64_t ks_n = K / 256;
  const int64_t blk = o >> 8;
  const int64_t t = blk / ks_n, s = blk - t * ks_n;
  const int q = (int)(o >> 6) & 3, l = (int)o & 63;
  const int64_t row = 32 * t + (l & 31);
  out[o] = *reinterpret_cast<const uint4*>(codes + row * (K / 2) + 128 * s + 16 * (4 * (l >> 5) + q));
}

__global__ __launch_bounds__(kThreads) void frag_scales_kernel(const uint8_t* __restrict__ scales,
                                                               int K, uint32_t* __restrict__ out,
                                                               int64_t nwords) {
  const int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (w >= nwords) return;
  const int64_t ks_n = K / 256;
  const int64_t blk = w >> 6;
  const int64_t t = blk / ks_n, s = blk - t * ks_n;
  const int l = (int)w & 63;
  const int64_t row = 32 * t + (l & 31);
  out[w] = *reinterpret_cast<const uint32_t*>(scales + row * (K / 32) + 8 * s + 4 * (l >> 5));
}

}  // namespace

hipError_t launch_to_frag(const void* codes, const void* scales, int64_t R, int64_t K,
                          void* codes_f, void* scales_f, hipStream_t stream) {
  const int64_t n16 = R * K / 32, nw = R * K / 128;
  hipLaunchKernelGGL(frag_codes_kernel, dim3((unsigned)((n16 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(codes), (int)K,
                     static_cast<uint4*>(codes_f), n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(frag_scales_kernel, dim3((unsigned)((nw + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(scales), (int)K,
                     static_cast<uint32_t*>(scales_f), nw);
  return hipGetLastError();
}

void shuffled_b_sizes(int64_t N, int64_t K, int64_t* code_bytes, int64_t* scale_bytes) {
  const int64_t nt = (N + 255) / 256;
  *code_bytes = nt * (K / 256) * 32768;
  *scale_bytes = nt * ((K + 1023) / 1024) * 8192;
}

hipError_t launch_shuffle_b(const void* codes, const void* scales, int N, int K, void* codes_sh,
                            void* scales_sh, hipStream_t stream) {
  int64_t cb = 0, sb = 0;
  shuffled_b_sizes(N, K, &cb, &sb);
  const int64_t n16 = cb / 16, nw = sb / 4;
  hipLaunchKernelGGL(shuffle_codes_kernel, dim3((unsigned)((n16 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(codes), N, K,
                     static_cast<uint4*>(codes_sh), n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shuffle_scales_kernel, dim3((unsigned)((nw + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(scales), N, K,
                     static_cast<uint32_t*>(scales_sh), nw);
  return hipGetLastError();
}

}  // namespace mxfp4
