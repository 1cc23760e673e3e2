// Row-wise BF16 -> MXFP4 quantize with stochastic rounding, for gfx950.
//
// Same block arithmetic as quantize.hip for the scale (integer amax of the
// BF16 bits, scale byte = max(E_field(amax) - 2, 0)); the codes round
// stochastically with one Philox4x32-10 draw per 16-element half block,
// keyed by (block column, row, direction 0, half) as stochastic.h describes;
// the row is global: the input may be rows row0 .. of a larger one.
//
// Work mapping: as quantize.hip, four consecutive lanes own one 32-element
// block (16 bytes each) and every load instruction of a wave covers 1 KiB of
// input, fully coalesced. A half block spans two lanes, and each lane needs
// 8 of its draw's 16 bytes. Loads go in pairs: in pair g, the even lane of
// each lane pair computes the draw of its half block in load 2g and the odd
// lane the one in load 2g + 1; one swap between the two lanes (DPP
// quad_perm [1,0,3,2]) then hands each lane the two words it lacks. Every
// draw is computed once, with no idle lanes.
//
// Block coordinates come from the flat block index by one division by the
// number of blocks per row, done in float64 with one correction step (the
// product's error is far below one).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "stochastic.h"

namespace mxfp4 {
namespace {

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
// Loads per lane, in pairs. One pair: the kernel is partly bound by its
// arithmetic (Philox), and more waves in flight beat more loads per wave
// (8192 x 8192: 30.3-30.9 us against 31.4-31.6 us with two pairs).
constexpr int kUnroll = 2;

__device__ __forceinline__ u16x2_t abs_pair(uint32_t w) {
  return __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
}

__device__ __forceinline__ uint32_t quarter_absmax(u32x4_t q) {
  u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(abs_pair(q[0]), abs_pair(q[1])),
                                        __builtin_elementwise_max(abs_pair(q[2]), abs_pair(q[3])));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  v = max(v, o);  // quad_perm [1,0,3,2]
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  return max(v, o);  // quad_perm [2,3,0,1]
}

__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

// (row, block column) of flat block `blk` with `nb` blocks per row.
__device__ __forceinline__ void block_coords(int64_t blk, int64_t nb, double inv_nb, uint32_t& row,
                                             uint32_t& col) {
  int64_t q = (int64_t)((double)blk * inv_nb);
  int64_t rem = blk - q * nb;
  if (rem < 0) {
    --q;
    rem += nb;
  } else if (rem >= nb) {
    ++q;
    rem -= nb;
  }
  row = (uint32_t)q;
  col = (uint32_t)rem;
}

__global__ __launch_bounds__(kThreads) void quantize_sr_kernel(
    const u32x4_t* __restrict__ x, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
    int64_t nquarters, int64_t nb, double inv_nb, uint32_t row0, uint32_t key0, uint32_t key1) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t base = wave * (64 * kUnroll) + lane;
  const int odd = lane & 1;
  const uint32_t half = (lane >> 1) & 1;

  u32x4_t v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t q = base + (int64_t)u * 64;
    v[u] = q < nquarters ? __builtin_nontemporal_load(&x[q]) : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int g = 0; g < kUnroll / 2; ++g) {
    // This lane's draw: its half block in load 2g + odd.
    uint32_t row, col;
    block_coords((base + (int64_t)(2 * g + odd) * 64) >> 2, nb, inv_nb, row, col);
    const Draw d = philox4x32_10(col, row0 + row, kDirRowwise, half, key0, key1);
    // The even lane holds bytes 0..7 of its half in load 2g and needs bytes
    // 0..7 of load 2g + 1 (the odd lane's draw); the odd lane the reverse.
    const uint32_t got0 = swap_pair(odd ? d.w[0] : d.w[2]);
    const uint32_t got1 = swap_pair(odd ? d.w[1] : d.w[3]);
    uint32_t rnd[2][2];
    rnd[0][0] = odd ? got0 : d.w[0];
    rnd[0][1] = odd ? got1 : d.w[1];
    rnd[1][0] = odd ? d.w[2] : got0;
    rnd[1][1] = odd ? d.w[3] : got1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int u = 2 * g + s;
      const int64_t q = base + (int64_t)u * 64;
      // All 64 lanes take part in the DPP moves; a block's four lanes are
      // either all in range or all out (nquarters is a multiple of 4).
      const uint32_t amax = quad_max(quarter_absmax(v[u]));
      const int byte = max((int)(amax >> 7) - 2, 0);
      const uint32_t c =
          sr_encode8(v[u][0], v[u][1], v[u][2], v[u][3], 1 - byte, rnd[s][0], rnd[s][1]);
      if (q < nquarters) {
        codes[q] = c;
        if ((lane & 3) == 0) scales[q >> 2] = (uint8_t)byte;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize_sr(const void* x_bf16, int64_t M, int64_t K, int64_t row0,
                              uint64_t seed, void* codes, void* scales, hipStream_t stream) {
  const int64_t nb = K / 32;
  const int64_t nquarters = M * nb * 4;
  const int64_t per_block = (int64_t)kThreads * kUnroll;  // quarters per workgroup
  const int64_t grid = (nquarters + per_block - 1) / per_block;
  hipLaunchKernelGGL(quantize_sr_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(x_bf16), static_cast<uint32_t*>(codes),
                     static_cast<uint8_t*>(scales), nquarters, nb, 1.0 / (double)nb,
                     (uint32_t)row0, (uint32_t)seed, (uint32_t)(seed >> 32));
  return hipGetLastError();
}

}  // namespace mxfp4
