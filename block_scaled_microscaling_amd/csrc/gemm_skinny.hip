// Block-scaled MXFP4 x MXFP4 GEMM (TN) for few rows of A: decode-shaped
// problems such as M = 32 against a large N x K weight, where the work is
// streaming B from HBM once and the MFMAs are nearly idle. mxfp4_gemm also
// runs it for problems of at most CUs / 8 tiles of 256 x 256, whose 32 x 32
// tiles here spread over the whole chip where the tile kernel would keep
// most CUs idle.
//
// Same contract and arithmetic as the tile kernel (the MXFP4 hipBLASLt path
// of "Integrate MXFP4 hipblaslt GEMM support", ROCm/TransformerEngine #697,
// Changes list: TN, plain UE8M0 block-32 scales, BF16/FP32 out, K % 256,
// M/N % 32, no bias, beta = 0); only the work split differs.
//
// Work split. One workgroup of 8 waves owns a 32 x 32 tile of C (32 rows of
// A, 32 rows of B), so M = 32 already gives N / 32 workgroups. The K range
// is split between the waves (intra-workgroup split-K): wave w takes the K
// steps w, w + 8, w + 16, ... of the K / 256, accumulates a 32 x 32 fp32
// partial with one v_mfma_scale_f32_32x32x64_f8f6f4 per 64-wide K slice, and
// the 8 partials are summed in LDS, in wave order, before the epilogue.
// (Interleaved steps measured 5% faster than one contiguous K range per
// wave at 32 x 8192 x 8192: 11.05 against 11.6 us.)
//
// Data movement, row-major operands (gemm_skinny_kernel). Each wave streams
// its K steps through a private two-slot LDS ring with global_load_lds: per
// 256-wide K step, 32 rows x 128 bytes of A codes and of B codes (four wave
// instructions each, 8 whole cache lines per instruction) and 32 rows x 8
// bytes of A and B scales (one dword instruction each). Two steps are in
// flight per wave (16 KiB), 128 KiB per workgroup: the LDS caps the bytes in
// flight per CU, and with one workgroup per CU that caps the HBM rate
// (10.9 us at 32 x 8192 x 8192, B's loads nontemporal, against 6.3 us for
// a plain 1024-workgroup streaming read of B).
//
// Data movement, fragment-order operands (gemm_frag_kernel). A and B are
// stored so that each MFMA operand is one contiguous 1 KiB; every load is a
// whole-line wave instruction straight into registers, four K steps per
// wave in flight (256 KiB per workgroup) with no LDS ring, B's loads
// nontemporal: 8.4 us on the same problem (9.0 us with cacheable B loads). Loading the fragments of row-major operands straight into
// registers instead was slower (12.9 us): each such load instruction touches
// 32 rows, 32 bytes of each line.
//
// K order inside a step. The MFMA only needs A and B to agree on which K
// block a lane holds, so lane half h of slice s takes block 4 h + s of the
// step's 8 blocks: its scale bytes for the 4 slices are then one dword of
// its row (dword h), byte s picked by op_sel, and its code chunk 4 h + s is
// read from the XOR-swizzled 128-byte LDS row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950.h"
#include "kernels.h"

namespace mxfp4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                             // rows of A and of B per workgroup
constexpr int kStepK = 256;                           // K per ring slot
constexpr int kRowBytes = kStepK / 2;                 // code bytes per row per step
constexpr int kCodeBytes = kTile * kRowBytes;         // 4 KiB per operand per slot
constexpr int kScaleRow = kStepK / 32;                // scale bytes per row per step
constexpr int kScaleBytes = kTile * kScaleRow;        // 256 B per operand per slot
// Slot layout: [A codes][B codes][A scales][B scales].
constexpr int kSlotB = kCodeBytes;
constexpr int kSlotAs = 2 * kCodeBytes;
constexpr int kSlotBs = 2 * kCodeBytes + kScaleBytes;
constexpr int kSlotBytes = 2 * kCodeBytes + 2 * kScaleBytes;
constexpr int kWaveBytes = 2 * kSlotBytes;
constexpr int kLdsBytes = kWaves * kWaveBytes;        // 136 KiB
constexpr int kLoadsPerStep = 10;                     // 4 + 4 code, 2 scale instructions
constexpr int kMaxFragTiles = 3;                      // tiles of A per fragment-order workgroup

static_assert(kWaves * kTile * kTile * 4 <= kLdsBytes, "reduction buffer fits the ring");

// Per-lane global offsets of one wave's loads.
struct Lanes {
  uint32_t code[2];  // code DMA, rows at 0 and 8 mod 16 (swizzle applied at the source)
  uint32_t scale;    // scale DMA: row lane / 2, dword lane % 2
};

// dma16 with the nontemporal hint: for B when a single tile row of A reads
// it, so that each line is used once (32 x 8192 x 8192: 11.2 -> 10.9 us;
// with several tile rows of A the other rows' workgroups then miss, 64 x
// 8192 x 8192: 17.1 -> 19.8 us, so it is kept for one tile row only).
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(g), "s"(lds) : "m0");
}

// Issue the loads of K step `st` into the slot at LDS address `slot`.
// Code instruction q fills tile rows 8 q .. 8 q + 7: lane i lands at row
// 8 q + i / 8, physical chunk i % 8, and so fetches logical chunk
// (i % 8) ^ swizzle(row). The scale instruction lands lane i's dword at
// 4 i: [row][dword 0, 1].
template <bool kNtB>
__device__ __forceinline__ void issue_step(const uint8_t* a, const uint8_t* b, const uint8_t* as,
                                           const uint8_t* bs, int row_bytes, const Lanes& ln,
                                           uint32_t slot, int st) {
  const int kb = st * kRowBytes;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    dma16(a + (int64_t)(8 * q) * row_bytes + kb + ln.code[q & 1], slot + q * 1024);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint8_t* g = b + (int64_t)(8 * q) * row_bytes + kb + ln.code[q & 1];
    if constexpr (kNtB)
      dma16_nt(g, slot + kSlotB + q * 1024);
    else
      dma16(g, slot + kSlotB + q * 1024);
  }
  dma4(as + st * kScaleRow + ln.scale, slot + kSlotAs);
  dma4(bs + st * kScaleRow + ln.scale, slot + kSlotBs);
}

// Split-K reduce and epilogue, shared by both kernels. B is the MFMA's
// first operand, so accumulator register 4 q + t of lane l holds
// C[m0 + l % 32][n0 + 8 q + 4 (l / 32) + t]. Each wave parks its partial in
// `red` (kWaves x 4 KiB of LDS, free for this use), then 256 threads sum the
// partials in wave order and store C.
template <bool kOutFp32>
__device__ __forceinline__ void reduce_store(float* red, const v16f_t& acc, int wave, int lane,
                                             int m0, int n0, int N, void* __restrict__ C) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<float4*>(red + wave * 1024 + q * 256 + lane * 4) =
        make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  __syncthreads();
  if (threadIdx.x < 256) {
    const int q = threadIdx.x >> 6;
    float4 sum = *reinterpret_cast<const float4*>(red + q * 256 + lane * 4);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(red + w * 1024 + q * 256 + lane * 4);
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
    const int m = m0 + (lane & 31);
    const int n = n0 + 8 * q + 4 * (lane >> 5);
    if constexpr (kOutFp32) {
      *reinterpret_cast<float4*>(static_cast<float*>(C) + (int64_t)m * N + n) = sum;
    } else {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + (int64_t)m * N + n) =
          make_uint2(pack_bf16x2(sum.x, sum.y), pack_bf16x2(sum.z, sum.w));
    }
  }
}

template <bool kOutFp32, bool kNtB>
__global__ __launch_bounds__(kThreads) void gemm_skinny_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int N, int K,
    void* __restrict__ C) {
  __shared__ __align__(16) uint8_t lds[kLdsBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r = lane & 31;
  const int h = lane >> 5;
  const int n0 = blockIdx.x * kTile;
  const int m0 = blockIdx.y * kTile;
  const int row_bytes = K / 2;
  const int srow_bytes = K / 32;
  const int steps = K / kStepK;
  // Wave w takes steps w, w + 8, w + 16, ...: at any time the eight waves
  // stream neighbouring 128-byte pieces of the same rows.
  const int nst = (steps - wave + kWaves - 1) / kWaves;

  Lanes ln;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int prow = lane >> 3;
    ln.code[par] =
        (uint32_t)(prow * row_bytes + (((lane & 7) ^ chunk_swizzle(8 * par + prow)) << 4));
  }
  ln.scale = (uint32_t)((lane >> 1) * srow_bytes + 4 * (lane & 1));

  const uint8_t* a = A + (int64_t)m0 * row_bytes;
  const uint8_t* b = B + (int64_t)n0 * row_bytes;
  const uint8_t* as = As + (int64_t)m0 * srow_bytes;
  const uint8_t* bs = Bs + (int64_t)n0 * srow_bytes;
  uint8_t* ring = lds + wave * kWaveBytes;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));

  // Fragment offsets within a slot: logical chunk 4 h + s of row r.
  const int swz = chunk_swizzle(r);
  const int frag_row = r * kRowBytes;
  const int scale_off = r * kScaleRow + 4 * h;

  v16f_t acc = v16f_t{};
  if (nst > 0) issue_step<kNtB>(a, b, as, bs, row_bytes, ln, ring_lds, wave);
  if (nst > 1) issue_step<kNtB>(a, b, as, bs, row_bytes, ln, ring_lds + kSlotBytes, wave + kWaves);
  for (int i = 0; i < nst; ++i) {
    // Step i has landed once at most the next step's loads are outstanding.
    if (i + 1 < nst)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kLoadsPerStep) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint8_t* slot = ring + (i & 1) * kSlotBytes;
    uint4 fa[4], fb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int off = frag_row + (((4 * h + s) ^ swz) << 4);
      fa[s] = *reinterpret_cast<const uint4*>(slot + off);
      fb[s] = *reinterpret_cast<const uint4*>(slot + kSlotB + off);
    }
    const uint32_t sa = *reinterpret_cast<const uint32_t*>(slot + kSlotAs + scale_off);
    const uint32_t sb = *reinterpret_cast<const uint32_t*>(slot + kSlotBs + scale_off);
    if (i + 2 < nst) {
      // The slot is refilled only after every read of it has returned.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue_step<kNtB>(a, b, as, bs, row_bytes, ln, ring_lds + (i & 1) * kSlotBytes,
                 wave + (i + 2) * kWaves);
    }
    acc = mfma_fp4<0, 0>(fb[0], fa[0], acc, sb, sa);
    acc = mfma_fp4<1, 1>(fb[1], fa[1], acc, sb, sa);
    acc = mfma_fp4<2, 2>(fb[2], fa[2], acc, sb, sa);
    acc = mfma_fp4<3, 3>(fb[3], fa[3], acc, sb, sa);
  }

  // Every wave's loads have completed (vmcnt(0) on its last step); the ring
  // is reused for the reduction once all waves are past their LDS reads.
  __syncthreads();
  reduce_store<kOutFp32>(reinterpret_cast<float*>(lds), acc, wave, lane, m0, n0, N, C);
}

// Fragment-order operands (both A and B re-arranged so that each MFMA
// operand is one contiguous 1 KiB: codes block t KS + s holds slice q's
// 16 bytes of lane l at 1024 q + 16 l, scales block t KS + s the lane's
// 4-byte word at 4 l). Same work split, K order, MFMA sequence and
// reduction as gemm_skinny_kernel, so the results are identical bit for
// bit; only the data movement differs. Every load is one whole-line wave
// instruction straight into registers, and kDepth steps per wave are in
// flight (32 KiB per wave, 256 KiB per workgroup) instead of the two
// LDS-bound steps of the row-major kernel. All loads are ordinary
// compiler-visible loads, so the compiler's in-order vmcnt waits are exact;
// loads are unconditional (past the wave's last step they re-read that
// step) so that no branch makes those waits conservative.
// Up to three 32-row tiles of A per workgroup (kMT): the B fragments of a
// step are loaded once and used for every tile of A, and each tile's
// accumulator sees exactly the sequence of MFMAs of a one-tile kernel (same
// bits). Steps in flight per wave: kDepth (4 for one tile; 2 beyond, which
// keeps A's extra fragments within two waves' share of the register file:
// 160 and 218 VGPRs for two and three tiles, no spills; four tiles spilled
// 30 VGPRs).
template <bool kOutFp32, int kMT, int kDepth>
__global__ __launch_bounds__(kThreads) void gemm_frag_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int m_tile0, int N, int K,
    void* __restrict__ C) {
  __shared__ __align__(16) float red[kWaves * 1024];
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int steps = K / kStepK;
  const int nst = (steps - wave + kWaves - 1) / kWaves;
  const int mt0 = m_tile0 + (int)blockIdx.y * kMT;  // first tile of A
  // Blocks of this workgroup's tiles; lane offsets inside a block.
  const u32x4_t* pa = reinterpret_cast<const u32x4_t*>(A) + (int64_t)mt0 * steps * 256 + lane;
  const u32x4_t* pb = reinterpret_cast<const u32x4_t*>(B) + (int64_t)blockIdx.x * steps * 256 + lane;
  const uint32_t* psa = reinterpret_cast<const uint32_t*>(As) + (int64_t)mt0 * steps * 64 + lane;
  const uint32_t* psb = reinterpret_cast<const uint32_t*>(Bs) + (int64_t)blockIdx.x * steps * 64 + lane;
  const int64_t a_tile = (int64_t)steps * 256;  // u32x4 per tile of A codes
  const int64_t s_tile = (int64_t)steps * 64;   // words per tile of A scales

  u32x4_t fa[kDepth][kMT][4], fb[kDepth][4];
  uint32_t sa[kDepth][kMT], sb[kDepth];
  int last = wave + kWaves * (nst > 0 ? nst - 1 : 0);
  last = last < steps ? last : steps - 1;
  auto step_of = [&](int j) {
    const int st = wave + kWaves * j;
    return st < last ? st : last;
  };
  // B is read once: nontemporal loads (8.4 against 9.0 us at 32 x 8192 x
  // 8192). A is re-read by every workgroup and stays cacheable.
  auto load = [&](int d, int st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) fb[d][q] = __builtin_nontemporal_load(pb + (st * 4 + q) * 64);
    sb[d] = __builtin_nontemporal_load(psb + st * 64);
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) fa[d][m][q] = pa[m * a_tile + (st * 4 + q) * 64];
      sa[d][m] = psa[m * s_tile + st * 64];
    }
  };
  v16f_t acc[kMT];
#pragma unroll
  for (int m = 0; m < kMT; ++m) acc[m] = v16f_t{};
  auto compute = [&](int d) {
    uint4 xb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xb[q] = make_uint4(fb[d][q].x, fb[d][q].y, fb[d][q].z, fb[d][q].w);
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      uint4 xa[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xa[q] = make_uint4(fa[d][m][q].x, fa[d][m][q].y, fa[d][m][q].z, fa[d][m][q].w);
      acc[m] = mfma_fp4<0, 0>(xb[0], xa[0], acc[m], sb[d], sa[d][m]);
      acc[m] = mfma_fp4<1, 1>(xb[1], xa[1], acc[m], sb[d], sa[d][m]);
      acc[m] = mfma_fp4<2, 2>(xb[2], xa[2], acc[m], sb[d], sa[d][m]);
      acc[m] = mfma_fp4<3, 3>(xb[3], xa[3], acc[m], sb[d], sa[d][m]);
    }
  };

#pragma unroll
  for (int d = 0; d < kDepth; ++d) load(d, step_of(d));
  int i = 0;
  for (; i + kDepth < nst; i += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      compute(d);
      load(d, step_of(i + d + kDepth));
    }
  }
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (i + d < nst) compute(d);

#pragma unroll
  for (int m = 0; m < kMT; ++m) {
    // The reduction buffer is reused per tile: every wave has read the
    // previous tile's partials before any writes the next one's.
    if (m > 0) __syncthreads();
    reduce_store<kOutFp32>(red, acc[m], wave, lane, (mt0 + m) * kTile, (int)blockIdx.x * kTile,
                           N, C);
  }
}

// `groups` workgroup rows of `mt` tiles of A each, from tile m_tile0 on.
template <bool kOutFp32>
hipError_t launch_frag_tiles(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                             const uint8_t* bs, int m_tile0, int groups, int mt, int N, int K,
                             void* C, hipStream_t stream) {
  const dim3 grid(N / kTile, groups);
  switch (mt) {
    case 1:
      hipLaunchKernelGGL((gemm_frag_kernel<kOutFp32, 1, 4>), grid, dim3(kThreads), 0, stream, a,
                         as, b, bs, m_tile0, N, K, C);
      break;
    case 2:
      hipLaunchKernelGGL((gemm_frag_kernel<kOutFp32, 2, 2>), grid, dim3(kThreads), 0, stream, a,
                         as, b, bs, m_tile0, N, K, C);
      break;
    case 3:
      hipLaunchKernelGGL((gemm_frag_kernel<kOutFp32, 3, 2>), grid, dim3(kThreads), 0, stream, a,
                         as, b, bs, m_tile0, N, K, C);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const void* A, const void* As, const void* B, const void* Bs, int M,
                              int N, int K, bool out_fp32, void* C, hipStream_t stream) {
  const dim3 grid(N / kTile, M / kTile);
  const auto* a = static_cast<const uint8_t*>(A);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* b = static_cast<const uint8_t*>(B);
  const auto* bs = static_cast<const uint8_t*>(Bs);
  // One tile row of A: every line of B is read by one workgroup only. Short
  // K (few steps per wave) measured slower with the hint (32 x 8192 x 1024:
  // 3.50 -> 3.66 us), long K faster (32 x 28672 x 4096: 20.5 -> 20.2 us).
  const bool nt_b = M == kTile && K >= 4096;
  if (out_fp32 && nt_b)
    hipLaunchKernelGGL((gemm_skinny_kernel<true, true>), grid, dim3(kThreads), 0, stream, a, as,
                       b, bs, N, K, C);
  else if (out_fp32)
    hipLaunchKernelGGL((gemm_skinny_kernel<true, false>), grid, dim3(kThreads), 0, stream, a, as,
                       b, bs, N, K, C);
  else if (nt_b)
    hipLaunchKernelGGL((gemm_skinny_kernel<false, true>), grid, dim3(kThreads), 0, stream, a, as,
                       b, bs, N, K, C);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<false, false>), grid, dim3(kThreads), 0, stream, a, as,
                       b, bs, N, K, C);
  return hipGetLastError();
}

// Tiles of A per workgroup: passes over B are what cost (each pass streams
// all of B), so the launch uses the fewest groups of at most 3 tiles,
// ceil(tiles / 3), with sizes as equal as possible: `extra` groups of
// base + 1 tiles and the rest of base tiles, at most two launches. Measured
// at N = K = 8192 (B from HBM), M = 64 / 96 / 128 / 160: 10.7 / 13.0 / 19.5 /
// 23.6 us, against 15.1 / 21.7 / 28.7 / 35.7 us with one tile per
// workgroup; M = 128 as 3 + 1 tiles took 21.6 us, M = 160 as 2 + 2 + 1 28.3.
hipError_t launch_gemm_frag(const void* A, const void* As, const void* B, const void* Bs, int M,
                            int N, int K, bool out_fp32, void* C, hipStream_t stream) {
  const auto* a = static_cast<const uint8_t*>(A);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* b = static_cast<const uint8_t*>(B);
  const auto* bs = static_cast<const uint8_t*>(Bs);
  const int tiles_m = M / kTile;
  const int groups = (tiles_m + kMaxFragTiles - 1) / kMaxFragTiles;
  const int base = tiles_m / groups, extra = tiles_m % groups;
  auto launch = [&](int m_tile0, int count, int mt) {
    return out_fp32 ? launch_frag_tiles<true>(a, as, b, bs, m_tile0, count, mt, N, K, C, stream)
                    : launch_frag_tiles<false>(a, as, b, bs, m_tile0, count, mt, N, K, C, stream);
  };
  if (extra > 0) {
    const hipError_t e = launch(0, extra, base + 1);
    if (e != hipSuccess) return e;
  }
  return launch(extra * (base + 1), groups - extra, base);
}

}  // namespace mxfp4
