// Bidimensional BF16 -> MXFP4 quantize for gfx950: one pass over X [M, K]
// writes both the row-wise MXFP4 form (blocks of 32 along K, as
// quantize.hip) and the column-wise form, i.e. the row-wise MXFP4 form of
// X^T (blocks of 32 along M), as [K, M/2] codes and [K, M/32] scales.
//
// The column-wise operand is what a GEMM contracting over M needs (the
// weight-gradient product of a linear layer). The single-pass design (row
// blocks encoded straight from registers, only the transposed direction
// staged through on-chip memory) is the bidimensional quantize kernel
// described on NVIDIA/TransformerEngine #3809 (description); the block
// arithmetic is the one of quantize.hip (integer amax of |bits|, scale byte
// = max(E_field(amax) - 2, 0), v_cvt_scalef32_pk_fp4_bf16 for RNE E2M1).
//
// Work mapping: a workgroup of 4 C threads handles one 256-row x C-column
// tile at a time (C = 128). For round to nearest the grid is persistent
// (two workgroups per CU) and each workgroup loads its next tile into
// registers while it finishes the last; the stochastic variant launches one
// workgroup per tile.
//   Row phase: load i of thread t reads the 16-byte chunk t % (C / 8) of row
//   32 i + t / (C / 8): C / 8 lanes per 2C-byte row segment, so each wave
//   load fetches whole lines; four consecutive lanes hold one MX block
//   (amax finished with two quad DPP moves), and a row's codes of the tile
//   are C / 2 bytes (half a 128-byte line). The tile is parked in LDS
//   with rows padded by 16 bytes.
//   Column phase: thread t takes columns 2 (t % (C / 2)), +1 and row block
//   t / (C / 2): 32 dword reads (both columns at once), an integer amax per column, byte permutes pairing consecutive
//   rows, 16 conversions per column block. The column codes and scales are
//   parked in LDS again and written with 8 lanes per 128-byte column
//   segment: whole cache lines per store.
// Edge tiles (M or K not multiples of the tile) mask whole 32-element blocks.
//
// The stochastic-rounding variant (kSR) keeps the mapping and replaces only
// the element rounding (stochastic.h). Row phase: loads go in pairs and the
// two lanes of a half block split the draws as in quantize_sr.hip (the even
// lane draws for load 2g, the odd lane for 2g + 1, one DPP swap). Column
// phase: each thread owns whole column blocks and takes both draws of each,
// keyed with direction 1, the column of X as the row and the block index
// along M as the block column. Both directions key by global coordinates:
// the input may be rows row0 .. row0 + M - 1 of a larger X (row0 % 32 == 0),
// whose rows and row blocks the draws then take, so that a row shard's
// outputs are the corresponding part of the whole input's.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "stochastic.h"

namespace mxfp4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRows = 256;
// Tile width kC (128 columns) and its workgroup: kRB row blocks per thread
// in the column phase, so 4 kC / kRB threads (256 or 512).
template <int kC, int kRB>
struct Geom {
  static constexpr int kThreads = 4 * kC / kRB;
  static constexpr int kSeg = kC / 8;              // lanes per row segment (16 bytes each)
  static constexpr int kRowsPerLoad = kThreads / kSeg;
  static constexpr int kLoads = kRows / kRowsPerLoad;
  static constexpr int kLdsRow = 2 * kC + 16;      // padded LDS row, bytes
};

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
__device__ __forceinline__ uint32_t encode8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                            float scale) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w0), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w1), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w2), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w3), scale, 3);
  return r;
}
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  v = max(v, o);
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  return max(v, o);
}

__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

// Loads of one tile into registers: load i covers rows kRowsPerLoad i +
// t / kSeg, 16-byte chunk t % kSeg (zeros outside the matrix).
template <int kC, int kRB>
__device__ __forceinline__ void load_tile(const uint8_t* __restrict__ x, int M, int K, int m0,
                                          int c0, int t, u32x4_t (&v)[Geom<kC, kRB>::kLoads]) {
  using G = Geom<kC, kRB>;
  constexpr int kSeg = G::kSeg;
  const int64_t row_bytes = 2 * (int64_t)K;
  const int col = c0 + 8 * (t % kSeg);
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {
    const int m = m0 + G::kRowsPerLoad * i + t / kSeg;
    v[i] = (m < M && col < K)
               ? __builtin_nontemporal_load(
                     reinterpret_cast<const u32x4_t*>(x + m * row_bytes + 2 * (int64_t)col))
               : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Visit q of the tile sequence -> tile id (row-major over the tile grid),
// or -1 for a visit number that maps past the grid. Workgroups take visits
// g, g + gridDim.x, ... and workgroup g runs on XCD g % 8 (when the grid is
// a multiple of 8). With xcd_regions the tile grid is cut into 4 x 2
// rectangles (row bands x column halves) and XCD x walks rectangle x row by
// row, so the tiles that share lines of the outputs (the two halves of a
// 128-byte row-code line, a row's scale line, a column's scale line) mostly
// run on one XCD and meet in its L2: 8192 x 8192 unchanged (41.3 us), 4128
// x 7936 30.5 -> 28.4 us, against pairing only the row-code half lines.
// Visits run to 8 x the largest rectangle; every tile gets exactly one.
constexpr int kRegionRows = 4, kRegionCols = 2;
__device__ __forceinline__ int tile_of_visit(int q, int total, int tiles_x, bool xcd_regions) {
  if (!xcd_regions) return q < total ? q : -1;
  const int tiles_y = total / tiles_x;
  const int xcd = q & 7, local = q >> 3;
  const int ry = xcd / kRegionCols, rx = xcd % kRegionCols;
  const int y0 = ry * tiles_y / kRegionRows, y1 = (ry + 1) * tiles_y / kRegionRows;
  const int x0 = rx * tiles_x / kRegionCols, x1 = (rx + 1) * tiles_x / kRegionCols;
  const int w = x1 - x0;
  if (w <= 0 || local >= w * (y1 - y0)) return -1;
  return (y0 + local / w) * tiles_x + x0 + local % w;
}
__device__ __forceinline__ int visits_end(int total, int tiles_x, bool xcd_regions) {
  if (!xcd_regions) return total;
  const int tiles_y = total / tiles_x;
  return 8 * ((tiles_y + kRegionRows - 1) / kRegionRows) *
         ((tiles_x + kRegionCols - 1) / kRegionCols);
}

// Persistent: workgroup g takes visits g, g + gridDim.x, ... (tiles by
// tile_of_visit) and issues the next tile's loads as soon as the current
// tile's rows are in LDS, so they are in flight during its column phase and
// stores.
template <bool kSR, int kC, int kRB>
__global__ __launch_bounds__((Geom<kC, kRB>::kThreads)) void quantize_2d_kernel(
    const uint8_t* __restrict__ x, int M, int K, uint8_t* __restrict__ codes_row,
    uint8_t* __restrict__ scales_row, uint8_t* __restrict__ codes_col,
    uint8_t* __restrict__ scales_col, uint32_t row0, uint32_t key0, uint32_t key1,
    bool xcd_regions) {
  using G = Geom<kC, kRB>;
  constexpr int kCols = kC;
  constexpr int kThreads = G::kThreads;
  constexpr int kSeg = G::kSeg;
  constexpr int kLdsRow = G::kLdsRow;
  constexpr int kRpl = G::kRowsPerLoad;
  __shared__ __align__(16) uint8_t tile[kRows * kLdsRow];
  const int t = threadIdx.x;
  const int tiles_x = (K + kCols - 1) / kCols;
  const int total = tiles_x * ((M + kRows - 1) / kRows);
  // Visit order q -> tile p (see tile_of_visit); the loop and
  // its prefetch skip visit numbers that map past the last tile.
  const int qend = visits_end(total, tiles_x, xcd_regions);
  int q = blockIdx.x;
  int p = tile_of_visit(q, total, tiles_x, xcd_regions);
  while (q < qend && p < 0) {
    q += gridDim.x;
    p = tile_of_visit(q, total, tiles_x, xcd_regions);
  }
  if (q >= qend) return;
  u32x4_t v[G::kLoads];
  load_tile<kC, kRB>(x, M, K, (p / tiles_x) * kRows, (p % tiles_x) * kCols, t, v);
  for (;;) {
    const int m0 = (p / tiles_x) * kRows;
    const int c0 = (p % tiles_x) * kCols;
    // Row phase: park the rows in LDS, encode them row-wise.
    {
      const int chunk = t % kSeg;
      const int col = c0 + 8 * chunk;
      const int odd = t & 1;
      uint32_t rnd_next[2] = {0u, 0u};  // kSR: the odd load's bytes of a pair
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) {
        const int r = kRpl * i + t / kSeg;
        *reinterpret_cast<u32x4_t*>(tile + r * kLdsRow + 16 * chunk) = v[i];
        const u32x4_t q = v[i];
        const u16x2_t mx = max2(max2(abs_pair(q[0]), abs_pair(q[1])),
                                max2(abs_pair(q[2]), abs_pair(q[3])));
        const uint32_t amax = quad_max(max((uint32_t)mx.x, (uint32_t)mx.y));
        const uint32_t byte = scale_byte(amax);
        uint32_t c;
        if constexpr (kSR) {
          // Draws for the pair of loads (i, i + 1), taken at the even one.
          uint32_t rnd[2];
          if ((i & 1) == 0) {
            const uint32_t drow = row0 + (uint32_t)(m0 + kRpl * (i + odd) + t / kSeg);
            const Draw d = philox4x32_10((uint32_t)(col / 32), drow, kDirRowwise,
                                         (uint32_t)((t >> 1) & 1), key0, key1);
            const uint32_t got0 = swap_pair(odd ? d.w[0] : d.w[2]);
            const uint32_t got1 = swap_pair(odd ? d.w[1] : d.w[3]);
            rnd[0] = odd ? got0 : d.w[0];
            rnd[1] = odd ? got1 : d.w[1];
            rnd_next[0] = odd ? d.w[2] : got0;
            rnd_next[1] = odd ? d.w[3] : got1;
          } else {
            rnd[0] = rnd_next[0];
            rnd[1] = rnd_next[1];
          }
          c = sr_encode8(q[0], q[1], q[2], q[3], 1 - (int)byte, rnd[0], rnd[1]);
        } else {
          c = encode8(q[0], q[1], q[2], q[3], __uint_as_float(byte << 23));
        }
        const int m = m0 + r;
        if (m < M && col < K) {
          *reinterpret_cast<uint32_t*>(codes_row + (int64_t)m * (K / 2) + col / 2) = c;
          if ((t & 3) == 0) scales_row[(int64_t)m * (K / 32) + col / 32] = (uint8_t)byte;
        }
      }
    }
    // The registers are free again: start the next tile's loads.
    int qn = q + (int)gridDim.x;
    int pn = tile_of_visit(qn, total, tiles_x, xcd_regions);
    while (qn < qend && pn < 0) {
      qn += gridDim.x;
      pn = tile_of_visit(qn, total, tiles_x, xcd_regions);
    }
    if (qn < qend)
      load_tile<kC, kRB>(x, M, K, (pn / tiles_x) * kRows, (pn % tiles_x) * kCols, t, v);
    __syncthreads();

    // Column phase: columns c0 + 2 cp, +1; row blocks 2 bp, 2 bp + 1. The
    // codes and scales are parked in LDS (the tile is dead by then) and
    // written out with whole lines: 8 lanes per 128-byte column segment.
    const int cp = t % (kCols / 2);
    const int bp = t / (kCols / 2);
    u32x4_t out[kRB][2];
    uint32_t sbyte[kRB][2];
#pragma unroll
    for (int rbi = 0; rbi < kRB; ++rbi) {
      const int rb = kRB * bp + rbi;
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
        if constexpr (kSR) {
          // Block (column c0 + 2 cp + e of X, global row block row0 / 32 +
          // m0 / 32 + rb): draw h
          // covers its rows 16 h .. 16 h + 15.
          const uint32_t kcol = (uint32_t)(c0 + 2 * cp + e);
          const uint32_t jblk = row0 / 32 + (uint32_t)(m0 / 32 + rb);
          const Draw d[2] = {philox4x32_10(jblk, kcol, kDirColumnwise, 0u, key0, key1),
                             philox4x32_10(jblk, kcol, kDirColumnwise, 1u, key0, key1)};
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t xs[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
              xs[i] = e == 0 ? w[8 * g + i] << 16 : w[8 * g + i] & 0xFFFF0000u;
            out[rbi][e][g] = sr_encode8_f32(xs, 1 - (int)byte, d[g >> 1].w[2 * (g & 1)],
                                            d[g >> 1].w[2 * (g & 1) + 1]);
          }
        } else {
          const float scale = __uint_as_float(byte << 23);
          const uint32_t sel = e == 0 ? 0x05040100u : 0x07060302u;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 8 * g + 2 * j;
              pr[j] = __builtin_amdgcn_perm(w[i + 1], w[i], sel);
            }
            out[rbi][e][g] = encode8(pr[0], pr[1], pr[2], pr[3], scale);
          }
        }
        sbyte[rbi][e] = byte;
      }
    }
    __syncthreads();
    // Staging: column c's 128 code bytes at c * kColStage, its 8 scale bytes
    // at kScaleStage + 8 c.
    constexpr int kColStage = 144;
    constexpr int kScaleStage = kCols * kColStage;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 2 * cp + e;
#pragma unroll
      for (int rbi = 0; rbi < kRB; ++rbi) {
        const int rb = kRB * bp + rbi;
        *reinterpret_cast<u32x4_t*>(tile + c * kColStage + 16 * rb) = out[rbi][e];
        tile[kScaleStage + 8 * c + rb] = (uint8_t)sbyte[rbi][e];
      }
    }
    __syncthreads();
    const int rows_valid = min(kRows, M - m0);  // multiple of 32
#pragma unroll
    for (int j = 0; j < kCols / (kThreads / 8); ++j) {
      const int c = (kThreads / 8) * j + (t >> 3);
      const int part = t & 7;  // 16-byte part = row block
      const int k = c0 + c;
      if (k < K && 32 * part < rows_valid)
        *reinterpret_cast<u32x4_t*>(codes_col + (int64_t)k * (M / 2) + m0 / 2 + 16 * part) =
            *reinterpret_cast<const u32x4_t*>(tile + c * kColStage + 16 * part);
    }
    if (t < kCols) {
      const int k = c0 + t;
      uint8_t* dst = scales_col + (int64_t)k * (M / 32) + m0 / 32;
      if (k < K) {
        // One 8-byte store when the destination is 8-byte aligned (base and
        // row pitch) and the tile has all 8 row blocks.
        if (rows_valid == kRows && (M / 32) % 8 == 0 &&
            (reinterpret_cast<uintptr_t>(scales_col) & 7) == 0) {
          *reinterpret_cast<uint2*>(dst) =
              *reinterpret_cast<const uint2*>(tile + kScaleStage + 8 * t);
        } else {
#pragma unroll
          for (int rb = 0; rb < 8; ++rb)
            if (32 * rb < rows_valid) dst[rb] = tile[kScaleStage + 8 * t + rb];
        }
      }
    }
    // Every thread's column stores have read the staging area before the
    // next tile's rows overwrite it.
    __syncthreads();
    if (qn >= qend) break;
    q = qn;
    p = pn;
  }
}

}  // namespace

// Round to nearest: a persistent grid of two workgroups per CU (69.6 KiB of
// LDS each), tiles visited by XCD rectangles (tile_of_visit). Measured on
// 8192 x 8192: 41.3 us (43.6 us visiting tiles in plain order); 256 x
// 256 tiles (whole lines of row-wise codes too, 512 threads, 132 KiB of
// LDS, one workgroup per CU) took 46.0 us. Stochastic rounding is bound by its VALU work, where the
// prefetch only adds register pressure (measured 4% slower): one tile per
// workgroup, the loop runs once.
constexpr int kColsRn = 128;
constexpr int kColsSr = 128;
// 512 threads per tile (one row block per thread in the column phase):
// 16 waves per CU instead of 8 hide more latency (8192^2: round to nearest
// 41.5 -> 39.4 us, stochastic 59.8 -> 55.9 us; 16384 x 14336 stochastic
// 196 -> 179 us, round to nearest unchanged).
constexpr int kRbRn = 1;
constexpr int kRbSr = 1;
constexpr int kWorkgroupsPerCu = 2;

static hipError_t grid_2d(int M, int K, int cols, bool persistent, dim3& grid) {
  const int64_t total = (int64_t)((K + cols - 1) / cols) * ((M + kRows - 1) / kRows);
  if (!persistent) {
    grid = dim3((unsigned)total);
    return hipSuccess;
  }
  int workers = 0;
  const hipError_t e = device_workers(workers);
  if (e != hipSuccess) return e;
  const int64_t cap = (int64_t)kWorkgroupsPerCu * workers;
  grid = dim3((unsigned)(total < cap ? total : cap));
  return hipSuccess;
}

hipError_t launch_quantize_2d(const void* x_bf16, int M, int K, void* codes_row, void* scales_row,
                              void* codes_col, void* scales_col, hipStream_t stream) {
  dim3 grid;
  const hipError_t e = grid_2d(M, K, kColsRn, true, grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((quantize_2d_kernel<false, kColsRn, kRbRn>), grid,
                     dim3(Geom<kColsRn, kRbRn>::kThreads), 0,
                     stream, static_cast<const uint8_t*>(x_bf16), M, K,
                     static_cast<uint8_t*>(codes_row), static_cast<uint8_t*>(scales_row),
                     static_cast<uint8_t*>(codes_col), static_cast<uint8_t*>(scales_col), 0u, 0u,
                     0u, true);
  return hipGetLastError();
}

hipError_t launch_quantize_2d_sr(const void* x_bf16, int M, int K, int64_t row0, uint64_t seed,
                                 void* codes_row, void* scales_row, void* codes_col,
                                 void* scales_col, hipStream_t stream) {
  dim3 grid;
  const hipError_t e = grid_2d(M, K, kColsSr, false, grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((quantize_2d_kernel<true, kColsSr, kRbSr>), grid,
                     dim3(Geom<kColsSr, kRbSr>::kThreads), 0,
                     stream, static_cast<const uint8_t*>(x_bf16), M, K,
                     static_cast<uint8_t*>(codes_row), static_cast<uint8_t*>(scales_row),
                     static_cast<uint8_t*>(codes_col), static_cast<uint8_t*>(scales_col),
                     (uint32_t)row0, (uint32_t)seed, (uint32_t)(seed >> 32), false);
  return hipGetLastError();
}

}  // namespace mxfp4
