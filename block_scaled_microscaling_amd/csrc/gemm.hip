// Block-scaled MXFP4 x MXFP4 GEMM (TN) for gfx950.
//
// Computes C[m, n] = sum_k dq(A[m, k]) * dq(B[n, k]), the FP4 x FP4 ("a4w4")
// GEMM of "Initial integration of a4w4 GEMM" (ROCm/TransformerEngine #663),
// under the contract of the hipBLASLt MXFP4 path on "Integrate MXFP4
// hipblaslt GEMM support" (#697, Changes list): TN, plain E2M1 data and
// plain UE8M0 block-32 scales, BF16/FP32 output, K % 256, M/N % 32, no bias,
// beta = 0.
//
// MFMA. The contraction runs on v_mfma_scale_f32_32x32x64_f8f6f4 with both
// operand formats set to FP4 (cbsz = blgp = 4); on gfx950 it sustains about
// 1.4x the FP4 rate of the 16x16x128 form per instruction stream. Per lane l
// of a wavefront, an operand fragment is the 32 codes (16 bytes) of row
// l % 32 in K block l / 32 of a 64-wide K slice, and the lane's scale byte
// is that same (row, K block)'s UE8M0 scale: one MX block per lane, so plain
// row-major data and scales feed the instruction without any reshuffle.
// Accumulator register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4,
// column l % 32. B's fragment is the instruction's first operand and A's the
// second, so the kernel produces C^T tiles: lane l then holds groups of four
// consecutive columns of one row of C, stored with one 8-byte (BF16) or
// 16-byte (FP32) write each.
//
// Tiling. One workgroup of 8 wavefronts (2 per SIMD) owns a 256 x 256 tile
// of C; wavefront (wy, wx) owns rows 128 wy .. +127 and columns 64 wx .. +63:
// 4 x 2 MFMA tiles of 32 x 32, 128 fp32 accumulators per lane.
//
// Data movement. A K step is 256 wide: 128 bytes of codes per row, four MFMA
// K slices. Code tiles go global -> LDS with global_load_lds_dwordx4, each
// wave instruction filling 8 rows x 128 bytes: whole cache lines, which the
// memory pipeline moves at about twice the rate of the half lines a 128-wide
// step would fetch. LDS holds two K steps (2 x 64 KiB). Scale words (one
// per row per 128 K) are loaded kChunk * 128 K at a time into a separate
// double buffer, so each of those loads also touches few cache lines.
//   Step T, phases p = 0..3 (slice p of step T on the MFMAs):
//     p = 0..2: read the fragments of slice p+1 of step T;
//     barrier after p = 2 (all loads of step T+1 landed, all reads of step T
//     from its slot done);
//     p = 3: read slice 0 and the scales of step T+1 from the other slot.
//   The loads of step T+2 (into step T's slot) are issued in phase 3 of step
//   T and phases 0-1 of step T+1, spread between MFMAs, so the memory
//   pipeline works alongside the MFMAs and has most of a step to finish.
// LDS layouts.
//   * Code rows are 128 bytes; their eight 16-byte chunks are XOR-swizzled
//     by the row, so the 16 lanes reading one chunk column of 16 consecutive
//     rows fall on distinct banks (in groups of 8 and of 16). The swizzle is
//     applied on the global side of the DMA by choosing which chunk a lane
//     fetches.
//   * Scale words are stored so that one 16-byte (A) or 8-byte (B) read gives
//     a lane the words of all its tiles; a byte permute then picks the lane
//     half's K blocks and the MFMA's op_sel picks the byte.
// Tile order. Workgroups are renumbered so that each XCD (every 8th
// workgroup id) walks a contiguous range of tiles, grouped 4 tile-rows at a
// time; the tiles running together on one XCD then share A and B panels in
// its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950.h"
#include "kernels.h"

namespace mxfp4 {
namespace {

constexpr int kThreads = 512;
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kRowBytes = 128;  // 256 FP4 codes of one row per K step
constexpr int kTileBytes = kTileM * kRowBytes;
constexpr int kGroupM = 4;
constexpr int kNumXcd = 8;

// Scale chunks: kChunk half-steps (128 K each) of scale words for the 256
// rows of an operand, laid out A: [half][r][half-step][A tile],
// B: [quarter][r][half-step][B tile] for rows 128 half + 32 tile + r and
// 64 quarter + 32 tile + r.
constexpr int kChunk = 8;                          // half-steps per chunk
constexpr int kChunkSteps = kChunk / 2;            // K steps per chunk
constexpr int kChunkBytes = kTileM * kChunk * 4;   // 8 KiB per operand

struct __align__(16) Slot {
  uint8_t a[kTileBytes];
  uint8_t b[kTileBytes];
};

// Map the hardware workgroup id to a (tile_m, tile_n) pair.
__device__ __forceinline__ void tile_of(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / kNumXcd, rem = total % kNumXcd;
  const int xcd = pid % kNumXcd, idx = pid / kNumXcd;
  const int p = xcd * q + min(xcd, rem) + idx;
  const int width = kGroupM * tiles_n;
  const int group = p / width;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = p - group * width;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Per-lane operands of one MFMA K slice: 4 A and 2 B fragments.
struct SliceFrags {
  uint4 a[4];
  uint4 b[2];
};

// Scale operands of one half-step (two K slices), built per lane from the
// scale words of its rows: a0 holds A tiles 0, 1 and a1 tiles 2, 3, as
// [tile even, tile odd] for the first slice in bytes 0-1 and for the second
// in bytes 2-3; b likewise for B tiles 0, 1. The MFMA's op_sel picks byte
// 2 * (slice % 2) + (tile % 2).
struct HalfScales {
  uint32_t a0, a1, b;
};

// Everything a lane needs to move and read one workgroup tile.
struct Ctx {
  const uint8_t* A;
  const uint8_t* B;
  const uint8_t* As;
  const uint8_t* Bs;
  int row_bytes, scale_row_bytes;
  int row0, col0, M, N;
  int klast;                // last K step
  int hlast;                // last half-step (128 K) of scale words
  uint32_t code_lane[2];    // per-lane code DMA offset for row groups at 16 r, 16 r + 8
  int scale_lane_a, scale_lane_b;  // per-lane row offsets of the scale DMAs
  int scale_t_a, scale_t_b;        // per-lane half-step within a chunk
  int a_base, b_base;       // fragment row offsets (bytes) of this lane
  uint32_t frag_x;          // chunk swizzle of this lane's rows, pre-shifted, with h
  int sa_off, sb_off;       // scale word offsets within a chunk (half-step 0)
  uint32_t s_sel;           // byte-permute selector picking this lane half's bytes
  int wave;
};

// Code load q (0..3) of this wave's share of K step kt: tile rows
// 32 w + 8 q .. +7, 128 bytes each. Lane i lands at row 32 w + 8 q + i / 8,
// physical chunk i % 8, so it fetches logical chunk (i % 8) ^ swizzle(row);
// the swizzle depends on the row mod 16, so a lane needs two offsets. The 8
// rows of one load lie wholly below M (or N) or wholly above it (M % 32 ==
// 0); loads above it re-read the last 8 rows: computed, never stored.
__device__ __forceinline__ const uint8_t* code_src(const Ctx& c, const uint8_t* base, int origin,
                                                   int rows, int q, int kt) {
  const int grow = min(origin + 32 * c.wave + 8 * q, rows - 8);  // wave-uniform
  return base + (int64_t)grow * c.row_bytes + kt * kRowBytes + c.code_lane[q & 1];
}
__device__ __forceinline__ void load_a(const Ctx& c, Slot& s, int q, int kt) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds_addr(s.a) + c.wave * 4096 + q * 1024);
  dma16(code_src(c, c.A, c.row0, c.M, q, kt), l);
}
__device__ __forceinline__ void load_b(const Ctx& c, Slot& s, int q, int kt) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds_addr(s.b) + c.wave * 4096 + q * 1024);
  dma16(code_src(c, c.B, c.col0, c.N, q, kt), l);
}

// Scale part u (0..7) of chunk `chunk` into chunk buffer `buf` (A words in
// the first 8 KiB, B words in the second). Part u covers chunk words
// q = 512 (u % 4) + 64 w + lane of the A (u < 4) or B (u >= 4) layout:
//   A [half][r][half-step][tile]:  row = 128 (u'/2) + 16 (u'%2) + 2 w
//                                      + 32 (lane % 4) + lane / 32,
//                                  half-step = (lane / 4) % 8
//   B [quarter][r][half-step][tile]: row = 64 u' + 4 w + 32 (lane % 2)
//                                      + lane / 16, half-step = (lane / 2) % 8
// with u' = u % 4; the lane-dependent terms are precomputed.
template <int U>
__device__ __forceinline__ void load_scale_part(const Ctx& c, uint8_t* buf, int chunk) {
  constexpr bool kIsA = U < 4;
  constexpr int up = U & 3;
  int row, t;
  const uint8_t* base;
  if constexpr (kIsA) {
    row = min(c.row0 + 128 * (up >> 1) + 16 * (up & 1) + 2 * c.wave + c.scale_lane_a, c.M - 1);
    base = c.As;
    t = c.scale_t_a;
  } else {
    row = min(c.col0 + 64 * up + 4 * c.wave + c.scale_lane_b, c.N - 1);
    base = c.Bs;
    t = c.scale_t_b;
  }
  const int hs = min(kChunk * chunk + t, c.hlast);
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      lds_addr(buf) + (kIsA ? 0 : kChunkBytes) + 4 * (512 * up + 64 * c.wave));
  dma4(base + (int64_t)row * c.scale_row_bytes + hs * 4, dst);
}

// The lane's scale operands of half-step hs from its chunk buffer.
__device__ __forceinline__ void read_half_scales(const Ctx& c, const uint8_t* buf, int t,
                                                 HalfScales& sc) {
  const uint4 wa = *reinterpret_cast<const uint4*>(buf + c.sa_off + 16 * t);
  const uint2 wb = *reinterpret_cast<const uint2*>(buf + kChunkBytes + c.sb_off + 8 * t);
  sc.a0 = __builtin_amdgcn_perm(wa.y, wa.x, c.s_sel);
  sc.a1 = __builtin_amdgcn_perm(wa.w, wa.z, c.s_sel);
  sc.b = __builtin_amdgcn_perm(wb.y, wb.x, c.s_sel);
}

// Fragment of K slice `sl` (chunk 2 sl + h of the lane's row, swizzled).
__device__ __forceinline__ int frag_off(const Ctx& c, int sl) {
  return (int)((uint32_t)(32 * sl) ^ c.frag_x);
}
__device__ __forceinline__ void read_frag_a(const Ctx& c, const Slot& s, int sl, int i, uint4& f) {
  f = *reinterpret_cast<const uint4*>(&s.a[c.a_base + frag_off(c, sl) + i * 32 * kRowBytes]);
}
__device__ __forceinline__ void read_frag_b(const Ctx& c, const Slot& s, int sl, int j, uint4& f) {
  f = *reinterpret_cast<const uint4*>(&s.b[c.b_base + frag_off(c, sl) + j * 32 * kRowBytes]);
}

template <int SLICE, int I>
__device__ __forceinline__ void mma_tile_row(v16f_t (&acc)[4][2], const SliceFrags& f,
                                             const HalfScales& sc) {
  constexpr int KH = SLICE & 1;
  const uint32_t sa = I < 2 ? sc.a0 : sc.a1;
  acc[I][0] = mfma_fp4<2 * KH + 0, 2 * KH + (I & 1)>(f.b[0], f.a[I], acc[I][0], sc.b, sa);
  acc[I][1] = mfma_fp4<2 * KH + 1, 2 * KH + (I & 1)>(f.b[1], f.a[I], acc[I][1], sc.b, sa);
}


// Wait for every load this wave issued and for its LDS reads, then meet the
// other waves. The memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void step_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

#define MXFP4_FENCE() __builtin_amdgcn_sched_barrier(0)

// One K step T, with P = (T + 1) % kChunkSteps: `cur` holds step T, `oth` receives step T+1 (its B half in
// phase 0; the A half arrived during phase 3 of step T-1) and provides step
// T+1's slice 0 in phase 3, when `cur` starts receiving step T+2's A half.
// sc0/sc1: scales of step T's two half-steps, replaced by step T+1's.
template <int P>
__device__ __forceinline__ void k_step(const Ctx& c0, Slot& cur, Slot& oth, uint8_t (*chunks)[2 * kChunkBytes],
                                       v16f_t (&acc)[4][2], SliceFrags& fa, SliceFrags& fb,
                                       HalfScales& sc0, HalfScales& sc1, int T) {
  // Re-derive the per-lane offsets from opaque copies each step, so that the
  // compiler recomputes the addresses built on them instead of holding every
  // one of them in a register across the loop.
  Ctx c = c0;
  asm volatile("" : "+v"(c.code_lane[0]), "+v"(c.code_lane[1]), "+v"(c.scale_lane_a),
               "+v"(c.scale_lane_b), "+v"(c.scale_t_a), "+v"(c.scale_t_b));
  asm volatile("" : "+v"(c.a_base), "+v"(c.b_base), "+v"(c.frag_x), "+v"(c.sa_off),
               "+v"(c.sb_off));
  const int kb = min(T + 1, c.klast);
  // Phase 0: slice 0 of step T; read slice 1; B half of step T+1.
  mma_tile_row<0, 0>(acc, fa, sc0);
  load_b(c, oth, 0, kb);
  read_frag_b(c, cur, 1, 0, fb.b[0]);
  read_frag_b(c, cur, 1, 1, fb.b[1]);
  MXFP4_FENCE();
  mma_tile_row<0, 1>(acc, fa, sc0);
  load_b(c, oth, 1, kb);
  read_frag_a(c, cur, 1, 0, fb.a[0]);
  read_frag_a(c, cur, 1, 1, fb.a[1]);
  MXFP4_FENCE();
  mma_tile_row<0, 2>(acc, fa, sc0);
  load_b(c, oth, 2, kb);
  read_frag_a(c, cur, 1, 2, fb.a[2]);
  read_frag_a(c, cur, 1, 3, fb.a[3]);
  MXFP4_FENCE();
  mma_tile_row<0, 3>(acc, fa, sc0);
  load_b(c, oth, 3, kb);
  MXFP4_FENCE();
  // Phase 1: slice 1; read slice 2.
  mma_tile_row<1, 0>(acc, fb, sc0);
  read_frag_b(c, cur, 2, 0, fa.b[0]);
  read_frag_b(c, cur, 2, 1, fa.b[1]);
  MXFP4_FENCE();
  mma_tile_row<1, 1>(acc, fb, sc0);
  read_frag_a(c, cur, 2, 0, fa.a[0]);
  read_frag_a(c, cur, 2, 1, fa.a[1]);
  MXFP4_FENCE();
  mma_tile_row<1, 2>(acc, fb, sc0);
  read_frag_a(c, cur, 2, 2, fa.a[2]);
  read_frag_a(c, cur, 2, 3, fa.a[3]);
  MXFP4_FENCE();
  mma_tile_row<1, 3>(acc, fb, sc0);
  MXFP4_FENCE();
  // Phase 2: slice 2; read slice 3.
  mma_tile_row<2, 0>(acc, fa, sc1);
  read_frag_b(c, cur, 3, 0, fb.b[0]);
  read_frag_b(c, cur, 3, 1, fb.b[1]);
  MXFP4_FENCE();
  mma_tile_row<2, 1>(acc, fa, sc1);
  read_frag_a(c, cur, 3, 0, fb.a[0]);
  read_frag_a(c, cur, 3, 1, fb.a[1]);
  MXFP4_FENCE();
  mma_tile_row<2, 2>(acc, fa, sc1);
  read_frag_a(c, cur, 3, 2, fb.a[2]);
  read_frag_a(c, cur, 3, 3, fb.a[3]);
  MXFP4_FENCE();
  mma_tile_row<2, 3>(acc, fa, sc1);
  MXFP4_FENCE();
  step_barrier();
  MXFP4_FENCE();
  // Phase 3: slice 3; read slice 0 and the scales of step T+1; A half and
  // two scale parts of step T+2.
  const int ka = min(T + 2, c.klast);
  const int hs = 2 * (T + 1);                 // first half-step of step T+1
  const uint8_t* sbuf = chunks[(hs / kChunk) & 1];
  uint8_t* pbuf = chunks[((T + 1) / kChunkSteps + 1) & 1];
  mma_tile_row<3, 0>(acc, fb, sc1);
  load_a(c, cur, 0, ka);
  load_a(c, cur, 1, ka);
  read_frag_b(c, oth, 0, 0, fa.b[0]);
  read_frag_b(c, oth, 0, 1, fa.b[1]);
  MXFP4_FENCE();
  mma_tile_row<3, 1>(acc, fb, sc1);
  load_a(c, cur, 2, ka);
  load_a(c, cur, 3, ka);
  read_frag_a(c, oth, 0, 0, fa.a[0]);
  read_frag_a(c, oth, 0, 1, fa.a[1]);
  MXFP4_FENCE();
  mma_tile_row<3, 2>(acc, fb, sc1);
  load_scale_part<2 * P>(c, pbuf, (T + 1) / kChunkSteps + 1);
  read_frag_a(c, oth, 0, 2, fa.a[2]);
  read_frag_a(c, oth, 0, 3, fa.a[3]);
  MXFP4_FENCE();
  mma_tile_row<3, 3>(acc, fb, sc1);
  load_scale_part<2 * P + 1>(c, pbuf, (T + 1) / kChunkSteps + 1);
  HalfScales n0, n1;
  read_half_scales(c, sbuf, hs % kChunk, n0);
  read_half_scales(c, sbuf, hs % kChunk + 1, n1);
  MXFP4_FENCE();
  sc0 = n0;
  sc1 = n1;
}

template <bool kOutFp32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tile_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                      const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int M, int N,
                      int K, void* __restrict__ C, int tiles_m, int tiles_n) {
  __shared__ Slot slot0, slot1;
  __shared__ __align__(16) uint8_t chunks[2][2 * kChunkBytes];

  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * kTileM;
  const int col0 = tn * kTileN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wy = wave >> 2;  // 128-row half of the A tile
  const int wx = wave & 3;   // 64-row quarter of the B tile
  const int r = lane & 31;
  const int h = lane >> 5;
  const int ksteps = K / 256;  // >= 1

  Ctx c;
  c.A = A;
  c.B = B;
  c.As = As;
  c.Bs = Bs;
  c.row_bytes = K / 2;
  c.scale_row_bytes = K / 32;
  c.row0 = row0;
  c.col0 = col0;
  c.M = M;
  c.N = N;
  c.klast = ksteps - 1;
  c.hlast = 2 * ksteps - 1;
  c.wave = wave;
  // Code DMA lane offsets for a load whose first row is at 0 or 8 mod 16.
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int prow = lane >> 3;
    const int chunk = (lane & 7) ^ chunk_swizzle(8 * par + prow);
    c.code_lane[par] = (uint32_t)(prow * c.row_bytes + chunk * 16);
  }
  c.scale_lane_a = 32 * (lane & 3) + (lane >> 5);
  c.scale_t_a = (lane >> 2) & 7;
  c.scale_lane_b = 32 * (lane & 1) + (lane >> 4);
  c.scale_t_b = (lane >> 1) & 7;
  // Fragments: row (base + 32 * tile + r), chunk (2 * slice + h) ^ swizzle(r);
  // since 2 * slice is even, that chunk's byte offset is 32 slice ^ frag_x.
  c.a_base = (wy * 128 + r) * kRowBytes;
  c.b_base = (wx * 64 + r) * kRowBytes;
  c.frag_x = (uint32_t)((h ^ chunk_swizzle(r)) << 4);
  // Scale words of the lane's rows within a chunk (half-step 0).
  c.sa_off = 16 * kChunk * (wy * 32 + r);
  c.sb_off = 8 * kChunk * (wx * 32 + r);
  // Bytes [w0.b(h), w1.b(h), w0.b(2+h), w1.b(2+h)] of words w0 (low), w1.
  c.s_sel = (uint32_t)h | (uint32_t)(4 + h) << 8 | (uint32_t)(2 + h) << 16 |
            (uint32_t)(6 + h) << 24;

  v16f_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f_t{};

  // Prologue: step 0 and scale chunk 0; then what phase 3 of step "-1"
  // would have issued: the A half of step 1 and scale parts 0, 1 of chunk 1.
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    load_a(c, slot0, q, 0);
    load_b(c, slot0, q, 0);
  }
  load_scale_part<0>(c, chunks[0], 0);
  load_scale_part<1>(c, chunks[0], 0);
  load_scale_part<2>(c, chunks[0], 0);
  load_scale_part<3>(c, chunks[0], 0);
  load_scale_part<4>(c, chunks[0], 0);
  load_scale_part<5>(c, chunks[0], 0);
  load_scale_part<6>(c, chunks[0], 0);
  load_scale_part<7>(c, chunks[0], 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) load_a(c, slot1, q, min(1, c.klast));
  load_scale_part<0>(c, chunks[1], 1);
  load_scale_part<1>(c, chunks[1], 1);
  asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");

  SliceFrags fa, fb;
  HalfScales sc0, sc1;
#pragma unroll
  for (int j = 0; j < 2; ++j) read_frag_b(c, slot0, 0, j, fa.b[j]);
#pragma unroll
  for (int i = 0; i < 4; ++i) read_frag_a(c, slot0, 0, i, fa.a[i]);
  read_half_scales(c, chunks[0], 0, sc0);
  read_half_scales(c, chunks[0], 1, sc1);

  // Four steps per trip, so that the ring slot and the scale part of every
  // step are compile-time constants.
  int T = 0;
  for (; T + 4 <= ksteps; T += 4) {
    k_step<1>(c, slot0, slot1, chunks, acc, fa, fb, sc0, sc1, T);
    k_step<2>(c, slot1, slot0, chunks, acc, fa, fb, sc0, sc1, T + 1);
    k_step<3>(c, slot0, slot1, chunks, acc, fa, fb, sc0, sc1, T + 2);
    k_step<0>(c, slot1, slot0, chunks, acc, fa, fb, sc0, sc1, T + 3);
  }
  if (T < ksteps) k_step<1>(c, slot0, slot1, chunks, acc, fa, fb, sc0, sc1, T);
  if (T + 1 < ksteps) k_step<2>(c, slot1, slot0, chunks, acc, fa, fb, sc0, sc1, T + 1);
  if (T + 2 < ksteps) k_step<3>(c, slot0, slot1, chunks, acc, fa, fb, sc0, sc1, T + 2);
  // No LDS write may still be in flight when the workgroup ends.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: accumulator register 4q + t of tile (i, j) holds
  // C[row0 + 128 wy + 32 i + r][col0 + 64 wx + 32 j + 8 q + 4 h + t].
  // M and N are multiples of 32, so each 32 x 32 tile is wholly in or out.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m_base = row0 + wy * 128 + i * 32;
    if (m_base >= M) continue;
    const int m = m_base + r;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n_base = col0 + wx * 64 + j * 32;
      if (n_base >= N) continue;
      const v16f_t v = acc[i][j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n_base + 8 * q + 4 * h;
        if constexpr (kOutFp32) {
          float* dst = static_cast<float*>(C) + (int64_t)m * N + n;
          *reinterpret_cast<float4*>(dst) =
              make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        } else {
          uint16_t* dst = static_cast<uint16_t*>(C) + (int64_t)m * N + n;
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[4 * q], v[4 * q + 1]),
                                                      pack_bf16x2(v[4 * q + 2], v[4 * q + 3]));
        }
      }
    }
  }
}

}  // namespace

hipError_t init_kernels_for_current_device() { return hipSuccess; }

hipError_t launch_gemm(const void* A, const void* As, const void* B, const void* Bs, int M, int N,
                       int K, bool out_fp32, void* C, hipStream_t stream) {
  const int tiles_m = (M + kTileM - 1) / kTileM;
  const int tiles_n = (N + kTileN - 1) / kTileN;
  const dim3 grid(tiles_m * tiles_n);
  const auto* a = static_cast<const uint8_t*>(A);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* b = static_cast<const uint8_t*>(B);
  const auto* bs = static_cast<const uint8_t*>(Bs);
  if (out_fp32)
    hipLaunchKernelGGL(gemm_tile_kernel<true>, grid, dim3(kThreads), 0, stream, a, as, b, bs, M, N,
                       K, C, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(gemm_tile_kernel<false>, grid, dim3(kThreads), 0, stream, a, as, b, bs, M,
                       N, K, C, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace mxfp4
