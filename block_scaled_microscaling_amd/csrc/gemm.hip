// Block-scaled MXFP4 x MXFP4 GEMM (TN) for gfx950.
//
// Computes C[m, n] = sum_k dq(A[m, k]) * dq(B[n, k]), the FP4 x FP4 ("a4w4")
// GEMM of "Initial integration of a4w4 GEMM" (ROCm/TransformerEngine #663),
// under the contract of the hipBLASLt MXFP4 path on "Integrate MXFP4
// hipblaslt GEMM support" (#697, Changes list): TN, plain E2M1 data and
// plain UE8M0 block-32 scales, BF16/FP32 output, K % 256, M/N % 32, no bias,
// beta = 0.
//
// The contraction runs on v_mfma_scale_f32_32x32x64_f8f6f4 with both operand
// formats set to FP4 (cbsz = blgp = 4); on gfx950 it sustains about 1.4x the
// FP4 rate of the 16x16x128 form per instruction stream. Per lane l of a
// wavefront, an operand fragment is the 32 codes (16 bytes) of row l % 32 in
// K block l / 32 of a 64-wide K slice, and the lane's scale byte is that same
// (row, K block)'s UE8M0 scale: one MX block per lane, so plain row-major
// data and scales feed the instruction without any reshuffle. Accumulator
// register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4, column l % 32.
//
// The kernel feeds B's fragment as the instruction's first operand and A's
// as the second, so it produces C^T tiles: lane l then holds groups of four
// consecutive columns of one row of C, each stored with one 8-byte (BF16) or
// 16-byte (FP32) write.
//
// Tiling: one workgroup of 8 wavefronts (2 per SIMD) owns a 256 x 256 tile
// of C; wavefront (wy, wx) owns rows 128*wy .. +127 and columns 64*wx .. +63,
// i.e. 4 x 2 MFMA tiles of 32 x 32 and 128 fp32 accumulators per lane.
//
// Pipeline (K step = 128 = two MFMA K slices; 64 bytes of codes per row):
//   * Code tiles go straight from global memory into a 3-slot LDS ring with
//     global_load_lds_dwordx4 (no register staging): each wave instruction
//     fills 16 rows x 64 bytes of LDS, lane i at byte 16 i; the chunk
//     swizzle is applied on the global side by choosing which 16-byte chunk
//     lane i fetches. Scale words take a register hop because their LDS
//     layout is a byte transpose.
//   * Step t, with slots cur = t % 3, next = (t+1) % 3, fill = (t+2) % 3:
//       issue loads of step t+2 into `fill`;
//       phase 0: MFMAs of K slice 0 of step t, while the slice-1 fragments
//                of step t are read from `cur`;
//       store step t+2's scale bytes; barrier (own loads of step t+1 done);
//       phase 1: MFMAs of K slice 1 of step t, while the slice-0 fragments
//                and scales of step t+1 are read from `next`.
//     No MFMA waits on an LDS read and the global loads have a step and a
//     half to land. The three slots are three distinct LDS arrays and the
//     loop is unrolled three times, so every access names its slot at
//     compile time and the compiler only waits for loads into the slot read.
//   * LDS rows are 64 bytes; their four 16-byte chunks are XOR-swizzled by
//     bits 1-3 of the row, so the 16 lanes that read one chunk column of 16
//     consecutive rows fall on distinct banks (in groups of 8 and of 16).
//   * Scale tiles are stored in LDS transposed, so one 8-byte (A) or 4-byte
//     (B) read gives a lane the scale bytes of all its MFMA tiles and both K
//     slices; the instruction's op_sel picks the byte.
//   * Workgroups are renumbered so that each XCD (every 8th workgroup id)
//     walks a contiguous range of tiles, grouped 4 tile-rows at a time; the
//     tiles running together on one XCD then share A and B panels in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "kernels.h"

namespace mxfp4 {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kStepBytes = 64;  // 128 FP4 codes of one row per K step
constexpr int kTileBytes = kTileM * kStepBytes;
constexpr int kScaleBytes = kTileM * 4;  // 4 scale bytes per row per K step
constexpr int kGroupM = 4;
constexpr int kNumXcd = 8;

// One ring slot: the A and B code tiles of one K step.
struct __align__(16) Slot {
  uint8_t a[kTileBytes];
  uint8_t b[kTileBytes];
};

// Scale words of kChunk consecutive K steps for all 256 rows of an operand
// (one 4-byte word = the row's 4 block scales of one step), in the order
//   A: [128-row half][r][step][A tile]   B: [64-row quarter][r][step][B tile]
// for rows 128 half + 32 tile + r and 64 quarter + 32 tile + r, so that one
// 16-byte (A) or 8-byte (B) read gives a lane the words of all its tiles.
constexpr int kChunk = 8;
constexpr int kChunkBytes = kTileM * kChunk * 4;  // 8 KiB per operand

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// XOR swizzle of the 16-byte chunk index within a 64-byte LDS row.
__device__ __forceinline__ int chunk_swizzle(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

template <int SEL_X, int SEL_Y>
__device__ __forceinline__ v16f_t mfma_fp4(const uint4& x, const uint4& y, v16f_t c, uint32_t sx,
                                           uint32_t sy) {
  const v8i_t xv = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  const v8i_t yv = {(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xv, yv, c, 4, 4, SEL_X, (int)sx, SEL_Y,
                                                         (int)sy);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 l = (__bf16)lo;
  const __bf16 h = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) |
         ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

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

// Scale operands of one K step, built per lane from the scale words of its
// rows: a0 holds A tiles 0, 1 and a1 tiles 2, 3, as [tile even, tile odd]
// for K slice 0 in bytes 0-1 and for K slice 1 in bytes 2-3; b likewise for
// B tiles 0, 1. The MFMA's op_sel picks byte 2 * slice + (tile % 2).
struct StepScales {
  uint32_t a0, a1, b;
};

// Everything a lane needs to move and read one workgroup tile.
struct Ctx {
  const uint8_t* a_src[2];  // code DMA sources of this lane: row groups 2w, 2w+1
  const uint8_t* b_src[2];
  const uint8_t* As;        // scale matrices and tile origin, for the chunk loads
  const uint8_t* Bs;
  int64_t scale_row_bytes;
  int row0, col0, M, N, klast;
  int a_off[2], b_off[2];   // fragment offsets per K slice
  int sa_off, sb_off;       // scale word offsets within a chunk (step 0)
  uint32_t s_sel;           // v_perm selector picking this lane half's bytes
  int wave, lane;
};

// Global -> LDS copies. lds is the wave-uniform LDS byte address of the
// destination; lane i's bytes land at lds + size * i. Written as inline
// assembly so that the compiler, which cannot tell the ring slots apart,
// adds no wait for them before LDS reads: every wait on these loads is the
// explicit one in ring_barrier.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds) : "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds) : "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Code-tile loads of K step kt into slot s: the two 1 KiB A (or B) row
// groups of this wave.
__device__ __forceinline__ void issue_a_loads(const Ctx& c, Slot& s, int kt) {
  const int64_t koff = (int64_t)kt * kStepBytes;
  const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr(s.a) + c.wave * 2048);
  dma16(c.a_src[0] + koff, la);
  dma16(c.a_src[1] + koff, la + 1024);
}
__device__ __forceinline__ void issue_b_loads(const Ctx& c, Slot& s, int kt) {
  const int64_t koff = (int64_t)kt * kStepBytes;
  const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(s.b) + c.wave * 2048);
  dma16(c.b_src[0] + koff, lb);
  dma16(c.b_src[1] + koff, lb + 1024);
}

// Part u (0..7) of scale chunk `chunk` (steps kChunk*chunk ..): one 4-byte
// DMA per wave; parts 0-3 fill the A chunk, parts 4-7 the B chunk. Lane
// `lane` of wave w fills word q = 512 (u % 4) + 64 w + lane of the chunk.
__device__ __forceinline__ void issue_scale_part(const Ctx& c, uint8_t* sa_buf, uint8_t* sb_buf,
                                                 int chunk, int u) {
  const bool is_a = u < 4;
  const int q = 512 * (u & 3) + 64 * c.wave + c.lane;
  int row, t;
  if (is_a) {  // [half][r][step][tile], tile = 2 bits
    row = 128 * (q >> 10) + 32 * (q & 3) + ((q >> 5) & 31);
    t = (q >> 2) & 7;
  } else {     // [quarter][r][step][tile], tile = 1 bit
    row = 64 * (q >> 9) + 32 * (q & 1) + ((q >> 4) & 31);
    t = (q >> 1) & 7;
  }
  const int kt = min(kChunk * chunk + t, c.klast);
  const uint8_t* src = is_a ? c.As + (int64_t)min(c.row0 + row, c.M - 1) * c.scale_row_bytes
                            : c.Bs + (int64_t)min(c.col0 + row, c.N - 1) * c.scale_row_bytes;
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      lds_addr(is_a ? sa_buf : sb_buf) + 4 * (512 * (u & 3) + 64 * c.wave));
  dma4(src + kt * 4, dst);
}

__device__ __forceinline__ void read_frag_a(const Ctx& c, const Slot& s, int kh, int i, uint4& f) {
  f = *reinterpret_cast<const uint4*>(&s.a[c.a_off[kh] + i * 32 * kStepBytes]);
}
__device__ __forceinline__ void read_frag_b(const Ctx& c, const Slot& s, int kh, int j, uint4& f) {
  f = *reinterpret_cast<const uint4*>(&s.b[c.b_off[kh] + j * 32 * kStepBytes]);
}

template <int KH, int I>
__device__ __forceinline__ void mma_tile_row(v16f_t (&acc)[4][2], const SliceFrags& f,
                                             const StepScales& sc) {
  const uint32_t sa = I < 2 ? sc.a0 : sc.a1;
  acc[I][0] = mfma_fp4<2 * KH + 0, 2 * KH + (I & 1)>(f.b[0], f.a[I], acc[I][0], sc.b, sa);
  acc[I][1] = mfma_fp4<2 * KH + 1, 2 * KH + (I & 1)>(f.b[1], f.a[I], acc[I][1], sc.b, sa);
}

// Wait until this wave's LDS reads are done and all but its newest four
// global loads (the code tiles of step t+2) have landed, then meet the other
// waves. The memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

#define MXFP4_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// One K step t (see the pipeline notes at the top of the file). `cur` holds
// step t, `next` step t+1, `fill` receives step t+2 (B half here; its A
// half was issued in the previous step); `cur` receives step t+3's A half
// in phase 1. sa_cur/sb_cur hold the scale chunk of step t+1.
__device__ __forceinline__ void k_step(const Ctx& c, Slot& cur, const Slot& next, Slot& fill,
                                       const uint8_t* sa_next, const uint8_t* sb_next,
                                       uint8_t* sa_buf2, uint8_t* sb_buf2, v16f_t (&acc)[4][2],
                                       SliceFrags& f0, SliceFrags& f1, StepScales& sc, int t) {
  // Phase 0: slice-0 MFMAs of step t; slice-1 fragments of step t; B half
  // of step t+2.
  issue_b_loads(c, fill, min(t + 2, c.klast));
  read_frag_b(c, cur, 1, 0, f1.b[0]);
  read_frag_b(c, cur, 1, 1, f1.b[1]);
  mma_tile_row<0, 0>(acc, f0, sc);
  MXFP4_SCHED_FENCE();
  read_frag_a(c, cur, 1, 0, f1.a[0]);
  read_frag_a(c, cur, 1, 1, f1.a[1]);
  mma_tile_row<0, 1>(acc, f0, sc);
  MXFP4_SCHED_FENCE();
  read_frag_a(c, cur, 1, 2, f1.a[2]);
  read_frag_a(c, cur, 1, 3, f1.a[3]);
  mma_tile_row<0, 2>(acc, f0, sc);
  MXFP4_SCHED_FENCE();
  mma_tile_row<0, 3>(acc, f0, sc);
  MXFP4_SCHED_FENCE();
  ring_barrier();
  MXFP4_SCHED_FENCE();
  // Phase 1: slice-1 MFMAs of step t; scales and slice-0 fragments of step
  // t+1; one part of a later scale chunk; A half of step t+3.
  {
    const int nt = t + 1;                       // scale part (nt % 8) of chunk nt / 8 + 1
    issue_scale_part(c, sa_buf2, sb_buf2, nt / kChunk + 1, nt % kChunk);
  }
  const int tt = (t + 1) % kChunk;
  const uint4 wa = *reinterpret_cast<const uint4*>(sa_next + c.sa_off + 16 * tt);
  const uint2 wb = *reinterpret_cast<const uint2*>(sb_next + c.sb_off + 8 * tt);
  mma_tile_row<1, 0>(acc, f1, sc);
  MXFP4_SCHED_FENCE();
  issue_a_loads(c, cur, min(t + 3, c.klast));
  read_frag_b(c, next, 0, 0, f0.b[0]);
  read_frag_b(c, next, 0, 1, f0.b[1]);
  mma_tile_row<1, 1>(acc, f1, sc);
  MXFP4_SCHED_FENCE();
  read_frag_a(c, next, 0, 0, f0.a[0]);
  read_frag_a(c, next, 0, 1, f0.a[1]);
  mma_tile_row<1, 2>(acc, f1, sc);
  MXFP4_SCHED_FENCE();
  read_frag_a(c, next, 0, 2, f0.a[2]);
  read_frag_a(c, next, 0, 3, f0.a[3]);
  mma_tile_row<1, 3>(acc, f1, sc);
  MXFP4_SCHED_FENCE();
  sc.a0 = __builtin_amdgcn_perm(wa.y, wa.x, c.s_sel);
  sc.a1 = __builtin_amdgcn_perm(wa.w, wa.z, c.s_sel);
  sc.b = __builtin_amdgcn_perm(wb.y, wb.x, c.s_sel);
}

template <bool kOutFp32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tile_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                      const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int M, int N,
                      int K, void* __restrict__ C, int tiles_m, int tiles_n) {
  __shared__ Slot slot0, slot1, slot2;
  __shared__ __align__(16) uint8_t sa_chunk[2][kChunkBytes];
  __shared__ __align__(16) uint8_t sb_chunk[2][kChunkBytes];

  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * kTileM;
  const int col0 = tn * kTileN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave >> 2;  // 128-row half of the A tile
  const int wx = wave & 3;   // 64-row quarter of the B tile
  const int r = lane & 31;
  const int h = lane >> 5;

  const int64_t row_bytes = K / 2;
  const int ksteps = K / 128;  // >= 2

  Ctx c;
  c.wave = wave;
  c.lane = lane;
  c.As = As;
  c.Bs = Bs;
  c.scale_row_bytes = K / 32;
  c.row0 = row0;
  c.col0 = col0;
  c.M = M;
  c.N = N;
  c.klast = ksteps - 1;
  // Code loads: wave w fills row groups 2w and 2w+1 (16 rows each) of A and
  // of B; lane i lands at row 16 g + i / 4, physical chunk i % 4, so it
  // fetches logical chunk (i % 4) ^ swizzle(row). Rows past M or N are
  // clamped to the last row: computed, never stored.
  {
    const int prow = lane >> 2;
    const int lchunk = ((lane & 3) ^ chunk_swizzle(prow)) << 4;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int trow = (2 * wave + q) * 16 + prow;
      c.a_src[q] = A + (int64_t)min(row0 + trow, M - 1) * row_bytes + lchunk;
      c.b_src[q] = B + (int64_t)min(col0 + trow, N - 1) * row_bytes + lchunk;
    }
  }
  // Fragment offsets: row (base + 32 * tile + r), chunk 2 * slice + h; the
  // scale words of the lane's rows within a chunk (step 0).
  {
    const int a_row = wy * 128 + r, b_row = wx * 64 + r;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      c.a_off[kh] = a_row * kStepBytes + (((2 * kh + h) ^ chunk_swizzle(r)) << 4);
      c.b_off[kh] = b_row * kStepBytes + (((2 * kh + h) ^ chunk_swizzle(r)) << 4);
    }
    c.sa_off = 16 * kChunk * (wy * 32 + r);
    c.sb_off = 8 * kChunk * (wx * 32 + r);
    // Bytes [w0.b(h), w1.b(h), w0.b(2+h), w1.b(2+h)] of words w0 (low), w1.
    c.s_sel = (uint32_t)h | (uint32_t)(4 + h) << 8 | (uint32_t)(2 + h) << 16 |
              (uint32_t)(6 + h) << 24;
  }

  v16f_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f_t{};

  // Prologue: scale chunk 0, code steps 0 and 1, then what step "-1" would
  // have issued: part 0 of scale chunk 1 and the A half of step 2.
#pragma unroll
  for (int u = 0; u < kChunk; ++u) issue_scale_part(c, sa_chunk[0], sb_chunk[0], 0, u);
  issue_a_loads(c, slot0, 0);
  issue_b_loads(c, slot0, 0);
  issue_a_loads(c, slot1, 1);
  issue_b_loads(c, slot1, 1);
  issue_scale_part(c, sa_chunk[1], sb_chunk[1], 1, 0);
  issue_a_loads(c, slot2, min(2, c.klast));
  asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");

  SliceFrags f0, f1;
  StepScales sc;
  {
    const uint4 wa = *reinterpret_cast<const uint4*>(sa_chunk[0] + c.sa_off);
    const uint2 wb = *reinterpret_cast<const uint2*>(sb_chunk[0] + c.sb_off);
    sc.a0 = __builtin_amdgcn_perm(wa.y, wa.x, c.s_sel);
    sc.a1 = __builtin_amdgcn_perm(wa.w, wa.z, c.s_sel);
    sc.b = __builtin_amdgcn_perm(wb.y, wb.x, c.s_sel);
#pragma unroll
    for (int j = 0; j < 2; ++j) read_frag_b(c, slot0, 0, j, f0.b[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) read_frag_a(c, slot0, 0, i, f0.a[i]);
  }

  // Steps t, t+1, t+2 per trip; the scale chunk of step t+1 is in buffer
  // ((t+1) / kChunk) % 2, its successor's in the other one.
#define MXFP4_STEP(CUR, NEXT, FILL, T)                                                    \
  do {                                                                                    \
    const int nb_ = ((T) + 1) / kChunk & 1;                                                \
    k_step(c, CUR, NEXT, FILL, sa_chunk[nb_], sb_chunk[nb_], sa_chunk[nb_ ^ 1],            \
           sb_chunk[nb_ ^ 1], acc, f0, f1, sc, (T));                                       \
  } while (0)
  int kt = 0;
  for (; kt + 3 <= ksteps; kt += 3) {
    MXFP4_STEP(slot0, slot1, slot2, kt);
    MXFP4_STEP(slot1, slot2, slot0, kt + 1);
    MXFP4_STEP(slot2, slot0, slot1, kt + 2);
  }
  if (kt < ksteps) MXFP4_STEP(slot0, slot1, slot2, kt);
  if (kt + 1 < ksteps) MXFP4_STEP(slot1, slot2, slot0, kt + 1);
#undef MXFP4_STEP
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
