// Block-scaled MXFP4 x MXFP4 GEMM (TN) for gfx950 on 256 x 256 tiles: what
// mxfp4_gemm runs for M > 128 with more than CUs / 8 tiles, and what
// mxfp4_gemm_tile runs for any shape.
//
// Computes C[m, n] = sum_k dq(A[m, k]) * dq(B[n, k]), the FP4 x FP4 ("a4w4")
// GEMM of "Initial integration of a4w4 GEMM" (ROCm/TransformerEngine #663),
// under the contract of the hipBLASLt MXFP4 path on "Integrate MXFP4
// hipblaslt GEMM support" (#697, Changes list): TN, plain E2M1 data and
// plain UE8M0 block-32 scales, BF16/FP32 output, K % 256, M/N % 32, no bias,
// beta = 0.
//
// MFMA. v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4 (see
// gfx950.h for the lane layout). B's fragment is the first operand and A's
// the second, so each lane ends with four consecutive columns of one row of
// C.
//
// Tiling. One workgroup of 4 waves (one per SIMD) owns a 256 x 256 tile of
// C; wave (wy, wx) owns rows 128 wy .. +127 and columns 128 wx .. +127: 4 x 4
// MFMA tiles of 32 x 32, whose 256 fp32 accumulators per lane live in the
// accumulation registers. Per 64-wide K slice a wave reads 4 A and 4 B
// fragments from LDS for 16 MFMAs (half the LDS reads per MFMA of a 128 x 64
// wave tile). The kernel is persistent: a grid of (CU count rounded down to
// a multiple of 8) workgroups walks the tiles, each starting the next tile's
// loads while its stores of the last tile drain.
//
// Data movement. A K step is 256 wide: 128 bytes of codes per row (one
// cache line), four MFMA K slices. Code tiles go global -> LDS with
// global_load_lds_dwordx4, each wave instruction filling 8 rows x 128 bytes,
// issued in pairs from a wave-uniform SGPR base and per-lane offsets
// prepared once per tile. Every non-MFMA instruction in the K loop costs
// MFMA issue time once there are more than about two per MFMA, so the loop
// keeps address arithmetic out: fragment reads use a per-lane register plus
// an immediate offset, and DMA addresses need no per-lane arithmetic.
// LDS holds two K steps (2 x 64 KiB) and a double buffer of scale words (one
// word per row per 128 K, 8 half-steps per chunk, 2 x 16 KiB): 160 KiB.
//   Step T, phases p = 0..3 (slice p of step T on the MFMAs):
//     p = 0..2: read the fragments of slice p+1 of step T;
//     barrier after p = 2 (all loads of step T+1 landed, all reads of step T
//     from its slot done);
//     p = 3: read slice 0 and the scales of step T+1 from the other slot.
//   Loads of step T+1 are issued in phase 3 of step T-1 and phases 0-1 of
//   step T, spread between MFMAs; within each group of four MFMAs the
//   fragment reads go one after each of the first two (group_end).
// LDS layouts.
//   * Code rows are 128 bytes; their eight 16-byte chunks are XOR-swizzled
//     by the row (chunk_swizzle), so the fragment reads of 16 rows fall on
//     distinct banks. The swizzle is applied on the global side of the DMA
//     by choosing which chunk a lane fetches.
//   * Scale words are stored so that one 16-byte read gives a lane the words
//     of its 4 tiles; a byte permute then picks the lane half's K blocks and
//     the MFMA's op_sel picks the byte. The half-step index is XOR-swizzled
//     by the row so that these reads are conflict-free too.
// Epilogue. The next tile's first loads are issued before C is written, so
// that they do not queue behind its stores. C is parked in the second K-step
// slot (BF16 in two rounds of 64 rows, FP32 in four of 32) and written with
// whole cache lines per buffer store instruction, lanes past M or N masked
// by the store resource.
// Tile order. Tile ids are renumbered so that each XCD (every 8th workgroup)
// walks a contiguous range of tiles, grouped 4 tile-rows at a time; the
// tiles running together on one XCD then share A and B panels in its L2.
// Variants (template parameters of gemm_tile_kernel):
//   kEpi = kEpiSwiglu: the gate+up GEMM of a SwiGLU MLP with the activation
//     and its MXFP4 requantize in the epilogue (store_tile_swiglu); B rows
//     follow b_row's gate/up interleave.
//   kShufB: B pre-shuffled by shuffle.hip into this kernel's LDS order, so
//     every B DMA reads one contiguous 1 KiB piece of a 32 KiB block.
//   kFull: K % 1024 == 0 (every scale chunk whole, no tail steps).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gfx950.h"
#include "kernels.h"

namespace mxfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kRowBytes = 128;  // 256 FP4 codes of one row per K step
constexpr int kTileBytes = kTileM * kRowBytes;
constexpr int kGroupM = 4;
constexpr int kNumXcd = 8;

// Epilogue modes: C in BF16 or FP32, or the fused SwiGLU + MXFP4 requantize
// of a gate+up GEMM (see store_tile_swiglu).
constexpr int kEpiBf16 = 0;
constexpr int kEpiFp32 = 1;
constexpr int kEpiSwiglu = 2;

// Section timers. In the library SectionTimer does nothing and its calls
// compile to no code. A profiling build (probe/gemm_sections.hip) defines
// MXFP4_SECTION_TIMERS and its own SectionTimer before including this file:
// each wave then adds the s_memtime cycles since its previous mark to the
// section a mark ends, and stores its sums once at the end of the kernel.
enum Section {
  kSecTileWait,     // a tile's first wait: its head loads landed, all waves met
  kSecLoop,         // K loop: MFMAs, fragment reads and load issue, up to each step's wait
  kSecDataWait,     // a step's wait for its next step's loads (and LDS reads)
  kSecBarrier,      // a step's barrier after that wait
  kSecLoopEnd,      // the last step's phase 3 and the wait after the loop
  kSecEpiHead,      // next tile's context and head loads
  kSecEpiStore,     // C (or the SwiGLU activation) parked and stored
  kSecEpiBarrier,   // the wait and barrier after the stores
  kSecEpiTail,      // next tile's tail loads
  kNumSections
};
#ifndef MXFP4_SECTION_TIMERS
struct SectionTimer {
  __device__ void start() {}
  template <int kSec>
  __device__ void mark() {}
  __device__ void store(int) {}
};
#endif

// Scale chunks: kChunk half-steps (128 K each) of scale words for the 256
// rows of an operand, laid out [half][r][half-step'][tile] for row
// 128 half + 32 tile + r, where half-step' = half-step ^ ((r >> 1) & 7): the
// XOR spreads the 16-byte reads of one half-step by lanes r = 0..31 over all
// LDS banks.
constexpr int kChunk = 8;
constexpr int kChunkSteps = kChunk / 2;
constexpr int kChunkBytes = kTileM * kChunk * 4;  // 8 KiB per operand

// The two K-step slots of each operand: a[S] and b[S] for S = 0, 1. Keeping
// both A slots within 64 KiB lets every fragment read use a per-lane
// register plus an immediate offset (slot, tile).
struct __align__(16) Tiles {
  uint8_t a[2][kTileBytes];
  uint8_t b[2][kTileBytes];
};

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

// Per-lane MFMA operands of one K slice: 4 A and 4 B fragments.
struct Frags {
  uint4 a[4];
  uint4 b[4];
};

// a0: A tiles 0, 1; a1: A tiles 2, 3; b0, b1 likewise; bytes
// [tile even, tile odd] for the first slice, then for the second.
struct HalfScales {
  uint32_t a0, a1, b0, b1;
};

// Everything a lane needs to move and read one workgroup tile.
struct Ctx {
  const uint8_t* A;
  const uint8_t* B;
  const uint8_t* As;
  const uint8_t* Bs;
  int row_bytes, scale_row_bytes;
  int row0, col0, M, N;
  int Nh;                 // SwiGLU: activation columns (B rows per half)
  int ksteps, nchunks;    // pre-shuffled B: K steps and 1024-K scale chunks
  int b_scale_blk;        // pre-shuffled B: first scale block of this tile
  uint32_t lane16;        // 16 * lane
  int klast, hlast;
  int rot, rot_chunks;    // K rotation of this tile: K steps (multiple of 4), chunks
  int rot_xcd;            // K rotation of this workgroup's XCD (-1: none)
  uint32_t code_lane[2];  // per-lane code DMA offset for row groups at 16 r, 16 r + 8
  const uint8_t* tile_a;  // wave-uniform code bases of this tile, less kDmaBias
  const uint8_t* tile_b;
  uint32_t off_a[8];      // per-lane offsets of code loads q = 0..7 from those bases
  uint32_t off_b[8];
  int scale_lane;          // 32 (lane % 4) + lane / 32
  int scale_t;             // (lane / 4) % 8: the scale DMA lane's stored half-step
  int a_base, b_base;      // fragment row offsets (bytes) of this lane
  uint32_t fa_off[4];      // a_base + (32 sl ^ frag_x) for slices sl = 0..3
  uint32_t fb_off[4];      // b_base + (32 sl ^ frag_x)
  uint32_t soff[2][4][2];  // scale DMA pair (operand, pair p): per-lane offsets of parts 2p, 2p+1
  uint32_t frag_x;         // chunk swizzle of this lane's rows, pre-shifted, with h
  int s_off, sb_off;       // the lane's scale words in a chunk: 128 (32 wy + r), 128 (32 wx + r)
  int s_x;                 // half-step XOR key of the lane's scale rows: (r >> 1) & 7
  uint32_t s_sel;          // byte-permute selector picking this lane half's bytes
  int wave;
  bool interior;           // off_a, off_b, soff hold the offsets of a tile with no clamped row
};

// Logical K step T (and 1024-K scale chunk) -> the step (chunk) loaded: the
// K loop of a tile starts rot steps into K and wraps around. rot is its XCD's
// offset (XCD x starts x K / 8 in): the 8 XCDs running tiles of one B panel
// row then read different parts of it at any moment, so each part comes from
// HBM for the first XCD only and from the last-level cache for the other
// seven, instead of all eight waiting on HBM together. Plain GEMM tiles add 4
// steps where tile row + tile column is odd: of the tiles sharing an A or B
// panel on one XCD, half then run 4 steps behind the others and find the
// panel's lines in L2 (8192^3: the step's wait for its loads 180 -> 158
// cycles, the epilogue 14.1k -> 12.0k cycles per tile, 2.3% faster; the
// SwiGLU tiles, whose B rows come in gate/up halves, gained nothing and keep
// the XCD offset alone). rot is 0 unless K % 1024 == 0, and a multiple of 4
// steps, so scale chunks stay whole.
__device__ __forceinline__ int phys_step(const Ctx& c, int t) {
  const int p = t + c.rot;
  return p >= c.ksteps ? p - c.ksteps : p;
}
__device__ __forceinline__ int phys_chunk(const Ctx& c, int ch) {
  const int p = ch + c.rot_chunks;
  return p >= c.nchunks ? p - c.nchunks : p;
}

// Global B row of B-tile row t (0..255), clamped into B. With kGlu the tile
// covers activation columns col0 .. col0 + 127 of a stacked [W_gate; W_up]
// weight (Nh rows each): tile row t = 128 wx + 32 i + rr (wave column wx,
// MFMA tile i) is gate row j for even i and up row Nh + j for odd i, where
// j = col0 + 64 wx + 32 (i / 2) + rr. Each wave then holds the gate and up
// sums of the same 64 activation columns in matching accumulators. Nh is a
// multiple of 128, so no row needs clamping, and every per-lane offset built
// on this map stays an affine function of the lane (per-row clamps cost the
// K loop about 30 registers, which then spilled around the epilogue).
template <bool kGlu>
__device__ __forceinline__ int b_row(const Ctx& c, int t) {
  if constexpr (kGlu) {
    return c.col0 + 64 * (t >> 7) + 32 * ((t >> 6) & 1) + (t & 31) + ((t >> 5) & 1) * c.Nh;
  } else {
    return min(c.col0 + t, c.N - 1);
  }
}

// First global row of the 8-row code group at B-tile rows t .. t + 7
// (t % 8 == 0), clamped within B (the kGlu map needs no clamp).
template <bool kGlu>
__device__ __forceinline__ int b_group_row(const Ctx& c, int t) {
  if constexpr (kGlu) {
    return c.col0 + 64 * (t >> 7) + 32 * ((t >> 6) & 1) + (t & 31) + ((t >> 5) & 1) * c.Nh;
  } else {
    return min(c.col0 + t, c.N - 8);
  }
}

// Code load q (0..7) of this wave's share of K step kt: tile rows
// 64 w + 8 q .. +7. Lane i lands at row 64 w + 8 q + i / 8, physical chunk
// i % 8, so it fetches logical chunk (i % 8) ^ swizzle(row); the swizzle
// depends on the row mod 16, so a lane needs two offsets. The 8 rows of one
// load lie wholly below M (or N) or wholly above it (M % 32 == 0); loads
// above it re-read the last 8 rows: computed, never stored.
// Code loads go in pairs q, q + 1 (q even) of one operand: a wave-uniform
// base in SGPRs, a per-lane 32-bit offset, and M0 = the LDS address of load
// 4 (q / 4); the instruction's immediate offset (q % 4) * 1024 moves both the
// global and the LDS address. The per-lane offsets carry kDmaBias to stay
// non-negative after the immediate is taken off.
constexpr int kDmaBias = 3072;

template <int Q0>
__device__ __forceinline__ void dma_pair(const uint8_t* base, uint32_t off0, uint32_t off1,
                                         uint32_t m0) {
  asm volatile(
      "s_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %2 offset:%4\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:%5"
      :: "v"(off0), "v"(off1), "s"(sgpr_ptr(base)), "s"(m0), "n"((Q0 % 4) * 1024),
         "n"(((Q0 + 1) % 4) * 1024)
      : "m0");
}
template <int Q0, int S>
__device__ __forceinline__ void load_a2(const Ctx& c, Tiles& t, int kt) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane(lds_addr(t.a[S]) + c.wave * 8192 + (Q0 / 4) * 4096);
  dma_pair<Q0>(c.tile_a + kt * kRowBytes, c.off_a[Q0], c.off_a[Q0 + 1], m0);
}
// A pre-shuffled B keeps each (tile, K step) as one 32 KiB block in LDS
// order, so a K step advances the base by a block instead of a row chunk.
template <bool kShufB, int Q0, int S>
__device__ __forceinline__ void load_b2(const Ctx& c, Tiles& t, int kt) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane(lds_addr(t.b[S]) + c.wave * 8192 + (Q0 / 4) * 4096);
  dma_pair<Q0>(c.tile_b + kt * (kShufB ? kTileBytes : kRowBytes), c.off_b[Q0], c.off_b[Q0 + 1],
               m0);
}

// Scale part u (0..7) of operand X (0 = A, 1 = B) of a chunk is its words
// q = 256 u + 64 w + lane: tile = lane % 4, half-step' = (lane / 4) % 8,
// r = 8 (u % 4) + 2 w + lane / 32, half = u / 4, so the lane's row is
// 128 (u / 4) + 32 (lane % 4) + 8 (u % 4) + 2 w + lane / 32 and the XOR key
// (r >> 1) & 7 = 4 (u % 2) + w. Parts 2p, 2p + 1 go as one DMA pair: their
// words sit 1024 bytes apart in the chunk buffer, and their per-lane offsets
// (prepared per tile, with kScaleBias) are relative to part 2p's clamped
// base row. kClampK (K not a multiple of 1024): the last chunk ends past K.
constexpr int kScaleBias = 1024;
template <bool kGlu, bool kShufB, int X, int PP, bool kClampK>
__device__ __forceinline__ void load_scale_pair(const Ctx& c, uint8_t* buf, int chunk) {
  const uint8_t* base = X == 0 ? c.As : c.Bs;
  // The last steps prefetch chunks past the end of K: those re-read the last
  // chunk (never used) instead of running past the scale rows.
  const int chunk_c = phys_chunk(c, min(chunk, c.hlast / kChunk));
  const uint8_t* sbase;
  if constexpr (kShufB && X == 1) {
    // Parts 2 PP, 2 PP + 1 of wave w: bytes 2048 PP + 256 w (+ 1024) of the
    // shuffled block, the same offsets as in LDS.
    sbase = base + (int64_t)(c.b_scale_blk + chunk_c) * kChunkBytes + 2048 * PP +
            256 * c.wave - kScaleBias;
  } else {
    const int t_row = 128 * (PP / 2) + 16 * (PP % 2) + 2 * c.wave;
    const int row_c = X == 0 ? min(c.row0 + t_row, c.M - 1) : b_row<kGlu>(c, t_row);
    sbase = base + (int64_t)row_c * c.scale_row_bytes + kChunk * 4 * chunk_c - kScaleBias;
  }
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(buf) + X * kChunkBytes +
                                                     4 * (256 * (2 * PP) + 64 * c.wave));
  uint32_t o0 = c.soff[X][PP][0], o1 = c.soff[X][PP][1];
  if constexpr (kClampK) {
    // The chunk may end past K: a lane whose half-step t lies past the last
    // one (tl) reads half-step tl instead (4 (t - tl) bytes back), so no
    // lane reads past its row, and past the scale array at its last row.
    const int tl = c.hlast - kChunk * chunk_c;
    o0 -= 4u * (uint32_t)max((c.scale_t ^ c.wave) - tl, 0);
    o1 -= 4u * (uint32_t)max((c.scale_t ^ (4 + c.wave)) - tl, 0);
  }
  asm volatile(
      "s_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dword %0, %2\n\t"
      "global_load_lds_dword %1, %2 offset:1024"
      :: "v"(o0), "v"(o1), "s"(sgpr_ptr(sbase)), "s"(m0)
      : "m0");
}

// kFull: K is a multiple of 1024, so every chunk is whole.
template <bool kFull, bool kGlu, bool kShufB, int X, int PP>
__device__ __forceinline__ void load_scales2(const Ctx& c, uint8_t* buf, int chunk) {
  // Shuffled B scales are padded to whole chunks, so they need no clamp.
  load_scale_pair<kGlu, kShufB, X, PP, !kFull && !(kShufB && X == 1)>(c, buf, chunk);
}

// The lane's scale operands of half-step t (0..7) of a chunk buffer.
__device__ __forceinline__ void read_half_scales(const Ctx& c, const uint8_t* buf, int t,
                                                 HalfScales& sc) {
  const int tx = 16 * (t ^ c.s_x);
  const uint4 wa = *reinterpret_cast<const uint4*>(buf + c.s_off + tx);
  const uint4 wb = *reinterpret_cast<const uint4*>(buf + kChunkBytes + c.sb_off + tx);
  sc.a0 = __builtin_amdgcn_perm(wa.y, wa.x, c.s_sel);
  sc.a1 = __builtin_amdgcn_perm(wa.w, wa.z, c.s_sel);
  sc.b0 = __builtin_amdgcn_perm(wb.y, wb.x, c.s_sel);
  sc.b1 = __builtin_amdgcn_perm(wb.w, wb.z, c.s_sel);
}

// Fragment of K slice `sl` (chunk 2 sl + h of the lane's row, swizzled):
// since 2 sl is even, its byte offset is 32 sl ^ frag_x.
__device__ __forceinline__ int frag_off(const Ctx& c, int sl) {
  return (int)((uint32_t)(32 * sl) ^ c.frag_x);
}
template <int S>
__device__ __forceinline__ void read_frag_a(const Ctx& c, const Tiles& t, int sl, int i, uint4& f) {
  f = *reinterpret_cast<const uint4*>(&t.a[0][0] + c.fa_off[sl] + S * kTileBytes +
                                      i * 32 * kRowBytes);
}
template <int S>
__device__ __forceinline__ void read_frag_b(const Ctx& c, const Tiles& t, int sl, int j, uint4& f) {
  f = *reinterpret_cast<const uint4*>(&t.b[0][0] + c.fb_off[sl] + S * kTileBytes +
                                      j * 32 * kRowBytes);
}

// The four MFMAs of A tile row I of one K slice.
template <int SLICE, int I>
__device__ __forceinline__ void mma_row(v16f_t (&acc)[4][4], const Frags& f, const HalfScales& sc) {
  constexpr int KH = SLICE & 1;
  const uint32_t sa = I < 2 ? sc.a0 : sc.a1;
  acc[I][0] = mfma_fp4<2 * KH + 0, 2 * KH + (I & 1)>(f.b[0], f.a[I], acc[I][0], sc.b0, sa);
  acc[I][1] = mfma_fp4<2 * KH + 1, 2 * KH + (I & 1)>(f.b[1], f.a[I], acc[I][1], sc.b0, sa);
  acc[I][2] = mfma_fp4<2 * KH + 0, 2 * KH + (I & 1)>(f.b[2], f.a[I], acc[I][2], sc.b1, sa);
  acc[I][3] = mfma_fp4<2 * KH + 1, 2 * KH + (I & 1)>(f.b[3], f.a[I], acc[I][3], sc.b1, sa);
}

// Wait for every load this wave issued and for its LDS reads, then meet the
// other waves. The memory clobber keeps LDS accesses on their side.
// The profiling build times the wait and the barrier apart (two asm
// statements); in the library they stay one statement, as scheduled.
__device__ __forceinline__ void step_barrier(SectionTimer& st) {
#ifdef MXFP4_SECTION_TIMERS
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  st.mark<kSecDataWait>();
  asm volatile("s_barrier" ::: "memory");
  st.mark<kSecBarrier>();
#else
  (void)st;
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
}

#define MXFP4_FENCE() __builtin_amdgcn_sched_barrier(0)

// End of one MFMA group of the K step (one A tile row: four MFMAs) and the
// LDS reads issued beside it: one read after each of the first R MFMAs (the
// group's two fragment reads after its first two MFMAs; the last group's six
// reads after its four). In a probe of 8 ds_read_b128 per 16 FP4 MFMAs (one
// wave per SIMD) the MFMAs kept 95% of their issue rate with single reads
// between them, against 86% with the reads in pairs and 88% in the
// compiler's own order; in this kernel the order gains 0.5-0.9% (8192^3
// 242.8 -> 241.2 us, 16384 x 28672 x 4096 911 -> 905 us).
template <int R>
__device__ __forceinline__ void group_end() {
#pragma unroll
  for (int i = 0; i < (R < 4 ? R : 4); ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  if constexpr (R < 4) __builtin_amdgcn_sched_group_barrier(0x008, 4 - R, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// One K step T, P = (T + 1) % 4. `cur` holds step T; `oth` receives step
// T+1: A rows of loads 4..7 and all of B in phases 0-1 (A loads 0..3 came in
// phase 3 of step T-1). Phase 3 issues step T+2's A loads 0..3 into `cur`
// and scale parts 2P, 2P+1 of both operands for chunk (T+1)/4 + 1.
template <bool kFull, bool kGlu, bool kShufB, int P, int S>
__device__ __forceinline__ void k_step(const Ctx& c0, Tiles& tl,
                                       uint8_t (*chunks)[2 * kChunkBytes], v16f_t (&acc)[4][4],
                                       Frags& fa, Frags& fb, HalfScales& sc0, HalfScales& sc1,
                                       int T, SectionTimer& st) {
  // The per-lane offsets and the addresses built on them stay in registers
  // across the loop (161-217 VGPRs beside the 256 accumulation registers,
  // no spills). Re-deriving them each step from opaque copies, which saved
  // registers in an earlier layout, cost 10 more VALU instructions per step
  // and 0.4-1.2% on every tile-GEMM workload.
  const Ctx& c = c0;
  const int kb = phys_step(c, min(T + 1, c.klast));
  // Phase 0: slice 0; read slice 1.
  mma_row<0, 0>(acc, fa, sc0);
  read_frag_b<S>(c, tl, 1, 0, fb.b[0]);
  read_frag_b<S>(c, tl, 1, 1, fb.b[1]);
  load_a2<4, 1 - S>(c, tl, kb);
  group_end<2>();
  mma_row<0, 1>(acc, fa, sc0);
  read_frag_b<S>(c, tl, 1, 2, fb.b[2]);
  read_frag_b<S>(c, tl, 1, 3, fb.b[3]);
  load_a2<6, 1 - S>(c, tl, kb);
  group_end<2>();
  mma_row<0, 2>(acc, fa, sc0);
  read_frag_a<S>(c, tl, 1, 0, fb.a[0]);
  read_frag_a<S>(c, tl, 1, 1, fb.a[1]);
  load_b2<kShufB, 0, 1 - S>(c, tl, kb);
  group_end<2>();
  mma_row<0, 3>(acc, fa, sc0);
  read_frag_a<S>(c, tl, 1, 2, fb.a[2]);
  read_frag_a<S>(c, tl, 1, 3, fb.a[3]);
  load_b2<kShufB, 2, 1 - S>(c, tl, kb);
  group_end<2>();
  // Phase 1: slice 1; read slice 2.
  mma_row<1, 0>(acc, fb, sc0);
  read_frag_b<S>(c, tl, 2, 0, fa.b[0]);
  read_frag_b<S>(c, tl, 2, 1, fa.b[1]);
  load_b2<kShufB, 4, 1 - S>(c, tl, kb);
  group_end<2>();
  mma_row<1, 1>(acc, fb, sc0);
  read_frag_b<S>(c, tl, 2, 2, fa.b[2]);
  read_frag_b<S>(c, tl, 2, 3, fa.b[3]);
  group_end<2>();
  mma_row<1, 2>(acc, fb, sc0);
  read_frag_a<S>(c, tl, 2, 0, fa.a[0]);
  read_frag_a<S>(c, tl, 2, 1, fa.a[1]);
  load_b2<kShufB, 6, 1 - S>(c, tl, kb);
  group_end<2>();
  mma_row<1, 3>(acc, fb, sc0);
  read_frag_a<S>(c, tl, 2, 2, fa.a[2]);
  read_frag_a<S>(c, tl, 2, 3, fa.a[3]);
  group_end<2>();
  // Phase 2: slice 2; read slice 3.
  mma_row<2, 0>(acc, fa, sc1);
  read_frag_b<S>(c, tl, 3, 0, fb.b[0]);
  read_frag_b<S>(c, tl, 3, 1, fb.b[1]);
  group_end<2>();
  mma_row<2, 1>(acc, fa, sc1);
  read_frag_b<S>(c, tl, 3, 2, fb.b[2]);
  read_frag_b<S>(c, tl, 3, 3, fb.b[3]);
  group_end<2>();
  mma_row<2, 2>(acc, fa, sc1);
  read_frag_a<S>(c, tl, 3, 0, fb.a[0]);
  read_frag_a<S>(c, tl, 3, 1, fb.a[1]);
  group_end<2>();
  mma_row<2, 3>(acc, fa, sc1);
  read_frag_a<S>(c, tl, 3, 2, fb.a[2]);
  read_frag_a<S>(c, tl, 3, 3, fb.a[3]);
  group_end<2>();
  st.mark<kSecLoop>();
  step_barrier(st);
  MXFP4_FENCE();
  // Phase 3: slice 3; read slice 0 and the scales of step T+1.
  const int ka = phys_step(c, min(T + 2, c.klast));
  const int hs = 2 * (T + 1);
  const uint8_t* sbuf = chunks[(hs / kChunk) & 1];
  const int pchunk = (T + 1) / kChunkSteps + 1;
  uint8_t* pbuf = chunks[pchunk & 1];
  mma_row<3, 0>(acc, fb, sc1);
  read_frag_b<1 - S>(c, tl, 0, 0, fa.b[0]);
  read_frag_b<1 - S>(c, tl, 0, 1, fa.b[1]);
  load_a2<0, S>(c, tl, ka);
  load_scales2<kFull, kGlu, kShufB, 0, P>(c, pbuf, pchunk);
  group_end<2>();
  mma_row<3, 1>(acc, fb, sc1);
  read_frag_b<1 - S>(c, tl, 0, 2, fa.b[2]);
  read_frag_b<1 - S>(c, tl, 0, 3, fa.b[3]);
  load_scales2<kFull, kGlu, kShufB, 1, P>(c, pbuf, pchunk);
  group_end<2>();
  mma_row<3, 2>(acc, fb, sc1);
  read_frag_a<1 - S>(c, tl, 0, 0, fa.a[0]);
  read_frag_a<1 - S>(c, tl, 0, 1, fa.a[1]);
  load_a2<2, S>(c, tl, ka);
  group_end<2>();
  mma_row<3, 3>(acc, fb, sc1);
  read_frag_a<1 - S>(c, tl, 0, 2, fa.a[2]);
  read_frag_a<1 - S>(c, tl, 0, 3, fa.a[3]);
  HalfScales n0, n1;
  read_half_scales(c, sbuf, hs % kChunk, n0);
  read_half_scales(c, sbuf, hs % kChunk + 1, n1);
  group_end<4>();
  sc0 = n0;
  sc1 = n1;
}

// Issue the loads that start a tile: K step 0 and scale chunk 0 into slot 0
// and chunks[0]. With whole chunks (kFull) the scale words go as the K
// loop's DMA pairs, whose per-lane offsets are prepared per tile.
template <bool kFull, bool kGlu, bool kShufB>
__device__ __forceinline__ void issue_tile_head(const Ctx& c0, Tiles& tl,
                                                uint8_t (*chunks)[2 * kChunkBytes]) {
  Ctx c = c0;
  asm volatile("" : "+v"(c.scale_lane), "+v"(c.scale_t));
  const int k0 = c.rot;
  load_a2<0, 0>(c, tl, k0);
  load_a2<2, 0>(c, tl, k0);
  load_a2<4, 0>(c, tl, k0);
  load_a2<6, 0>(c, tl, k0);
  load_b2<kShufB, 0, 0>(c, tl, k0);
  load_b2<kShufB, 2, 0>(c, tl, k0);
  load_b2<kShufB, 4, 0>(c, tl, k0);
  load_b2<kShufB, 6, 0>(c, tl, k0);
  load_scales2<kFull, kGlu, kShufB, 0, 0>(c, chunks[0], 0);
  load_scales2<kFull, kGlu, kShufB, 0, 1>(c, chunks[0], 0);
  load_scales2<kFull, kGlu, kShufB, 0, 2>(c, chunks[0], 0);
  load_scales2<kFull, kGlu, kShufB, 0, 3>(c, chunks[0], 0);
  load_scales2<kFull, kGlu, kShufB, 1, 0>(c, chunks[0], 0);
  load_scales2<kFull, kGlu, kShufB, 1, 1>(c, chunks[0], 0);
  load_scales2<kFull, kGlu, kShufB, 1, 2>(c, chunks[0], 0);
  load_scales2<kFull, kGlu, kShufB, 1, 3>(c, chunks[0], 0);
}

// What phase 3 of step "-1" would have issued: A loads 0..3 of step 1 and
// parts 0, 1 of chunk 1. Exactly 8 loads: the tile's first wait is vmcnt(8).
template <bool kFull, bool kGlu, bool kShufB>
__device__ __forceinline__ void issue_tile_tail(const Ctx& c0, Tiles& tl,
                                                uint8_t (*chunks)[2 * kChunkBytes]) {
  Ctx c = c0;
  asm volatile("" : "+v"(c.scale_lane), "+v"(c.scale_t));
  load_a2<0, 1>(c, tl, phys_step(c, min(1, c.klast)));
  load_a2<2, 1>(c, tl, phys_step(c, min(1, c.klast)));
  load_scales2<kFull, kGlu, kShufB, 0, 0>(c, chunks[1], 1);
  load_scales2<kFull, kGlu, kShufB, 1, 0>(c, chunks[1], 1);
}

// Point the context at tile id p (XCD-aware order). A SwiGLU tile spans
// 128 activation columns (256 B rows: 128 gate, 128 up).
template <bool kGlu, bool kShufB>
__device__ __forceinline__ void set_tile(Ctx& c, int p, int tiles_m, int tiles_n) {
  int tm, tn;
  tile_of(p, tiles_m, tiles_n, tm, tn);
  if constexpr (!kGlu) {
    if (c.rot_xcd >= 0) {
      int r = c.rot_xcd + 4 * ((tm + tn) & 1);
      if (r >= c.ksteps) r -= c.ksteps;
      c.rot = r;
      c.rot_chunks = r / kChunkSteps;
    }
  }
  c.row0 = tm * kTileM;
  c.col0 = tn * (kGlu ? kTileN / 2 : kTileN);
  // Wave's first code row, clamped like the rows of its loads: rows past M
  // (or N) re-read the last 8 rows, computed but never stored.
  const int ra = min(c.row0 + 64 * c.wave, c.M - 8);
  const int rb = b_group_row<kGlu>(c, 64 * c.wave);
  c.tile_a = c.A + (int64_t)ra * c.row_bytes - kDmaBias;
  if constexpr (kShufB) {
    // Block (tile, step 0) of the shuffled B; this wave's rows start 8 KiB in.
    c.tile_b = c.B + (int64_t)tn * c.ksteps * kTileBytes + 8192 * c.wave - kDmaBias;
    c.b_scale_blk = tn * c.nchunks;
  } else {
    c.tile_b = c.B + (int64_t)rb * c.row_bytes - kDmaBias;
  }
  // The per-lane offsets below are relative to the wave's first rows, so
  // they are the same for every tile that lies wholly inside A and B (no
  // clamped row): keep them when both this tile and the last are such.
  const bool interior = c.row0 + kTileM <= c.M && (kGlu || c.col0 + kTileN <= c.N);
  if (interior && c.interior) return;
  c.interior = interior;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int ga = min(c.row0 + 64 * c.wave + 8 * q, c.M - 8) - ra;
    const int gb = b_group_row<kGlu>(c, 64 * c.wave + 8 * q) - rb;
    c.off_a[q] = (uint32_t)(ga * c.row_bytes) + c.code_lane[q & 1] + kDmaBias - (q % 4) * 1024;
    c.off_b[q] = kShufB ? c.lane16 + 4096 * (q / 4) + kDmaBias
                        : (uint32_t)(gb * c.row_bytes) + c.code_lane[q & 1] + kDmaBias -
                              (q % 4) * 1024;
  }
  // Scale pairs: part U = 2p + e of operand X reads tile row
  // 128 (U / 4) + 8 (U % 4) + 2 w + scale_lane (its global row clamped),
  // half-step scale_t ^ (4 e + w); offsets relative to the global row of
  // part 2p's first tile row (the smallest the pair reads).
#pragma unroll
  for (int x = 0; x < 2; ++x) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int tb = 128 * (pp / 2) + 16 * (pp % 2) + 2 * c.wave;
      const int row_c = x == 0 ? min(c.row0 + tb, c.M - 1) : b_row<kGlu>(c, tb);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tr = tb + 8 * e + c.scale_lane;
        const int lane_row = (x == 0 ? min(c.row0 + tr, c.M - 1) : b_row<kGlu>(c, tr)) - row_c;
        if (kShufB && x == 1) {
          c.soff[x][pp][e] = (c.lane16 >> 2) + kScaleBias;
          continue;
        }
        const int t = c.scale_t ^ (4 * e + c.wave);
        c.soff[x][pp][e] =
            (uint32_t)(lane_row * c.scale_row_bytes + 4 * t + kScaleBias - 1024 * e);
      }
    }
  }
}

// Read-back half of the BF16 epilogue: lane l copies rows x = 4 k + l / 16
// (k = 0..15), 16-byte chunk l % 16, of a parked 64-row block to C, four
// reads in flight. With four rows per read the swizzle key
// x % 16 = 4 (k % 4) + l / 16 and the half swap (k / 4) % 2 are constants,
// so each read is one of four per-lane bases plus an immediate. Each store
// is a buffer store without a branch: its resource starts at the first of
// its four rows and covers them (8 N <= 2^31 bytes), lane l's offset is
// (l / 16) 2 N + 16 (l % 16), and a lane whose row lies at or past rows_left
// or whose columns lie past N (n_ok false) gets offset 2^31, past the
// resource, so the hardware drops its store.
__device__ __forceinline__ void copy_parked_rows(const uint8_t* region, int lane, uint8_t* cbase,
                                                 int N, bool n_ok, int rows_left) {
  const int l4 = lane >> 4, cc = lane & 15;
  const uint8_t* rb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) rb[kk] = region + l4 * 256 + (((cc ^ l4) << 4) ^ (64 * kk));
  const uint32_t row4 = 8u * (uint32_t)N;
  const uint32_t lane_off = n_ok ? (uint32_t)(l4 * 2 * N + 16 * cc) : 0x80000000u;
#pragma unroll 1
  for (int g2 = 0; g2 < 2; ++g2) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      uint4 w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = *reinterpret_cast<const uint4*>(rb[k] + 1024 * (8 * g2 + 4 * e + k));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int kr = 8 * g2 + 4 * e + k;
        uint4 x = w[k];
        if (e) x = make_uint4(x.z, x.w, x.x, x.y);
        const u32x4_t o = {x.x, x.y, x.z, x.w};
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            cbase + (int64_t)kr * row4, 0, (int)row4, kBufferWord3);
        const uint32_t voff = 4 * kr + l4 < rows_left ? lane_off : 0x80000000u;
        // Whole lines, written once: stream them past L2 (8% faster when C
        // is large, as in a 16384 x 28672 GEMM).
        __builtin_amdgcn_raw_buffer_store_b128(o, rsrc, (int)voff, 0, kBufferNt);
      }
    }
  }
}

// BF16 epilogue through LDS, in two rounds of 64 rows (MFMA tile rows i =
// 0, 1, then 2, 3): each wave parks a 64 x 128 BF16 block in a 16 KiB
// region (256-byte rows; 16-byte chunk c of row x at c ^ (x % 16), and its
// two 8-byte halves swapped when (x / 16) % 2 = 1, so both the 8-byte writes
// of 32 rows and the 16-byte reads of one row are conflict-free), then
// writes it to C with 16 lanes per 256-byte row: 4 rows, 8 whole cache
// lines per store instruction. A wave whose block lies inside C issues
// exactly 32 stores.
__device__ __forceinline__ void store_tile_bf16_lds(const Ctx& c, v16f_t (&acc)[4][4], int wy,
                                                    int wx, int lane, uint8_t* region,
                                                    void* __restrict__ C) {
  int r = lane & 31, h = lane >> 5;
  asm volatile("" : "+v"(r), "+v"(h));
  const int swz = r & 15;
  const int half = 8 * (h ^ ((r >> 4) & 1));
  const int mrow = c.row0 + wy * 128;  // first row and column of the wave's block
  const int ncol = c.col0 + wx * 128;
  const int cc = lane & 15;
  uint8_t* cbase = static_cast<uint8_t*>(C) + ((int64_t)mrow * c.N + ncol) * 2;
  const int64_t row4_bytes = (int64_t)c.N * 8;
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v16f_t v = acc[2 * rd + ii][j];
        asm volatile("" : "+v"(v));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int off = (32 * ii + r) * 256 + (((4 * j + q) ^ swz) << 4) + half;
          *reinterpret_cast<uint2*>(region + off) = make_uint2(
              pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3]));
        }
        MXFP4_FENCE();
      }
    }
    copy_parked_rows(region, lane, cbase + 16 * rd * row4_bytes, c.N, ncol + 8 * cc < c.N,
                     c.M - mrow - 64 * rd);
    MXFP4_FENCE();
  }
}

// SwiGLU + MXFP4 epilogue through the wave's 16 KiB LDS region. Tiles
// (i, 2 b) and (i, 2 b + 1) of a wave hold the gate and up sums of the same
// 32 x 32 block of activations act = silu(g) * u (rows
// row0 + 128 wy + 32 i + r, columns col0 + 64 wx + 32 b + 8 q + 4 h + t for
// register 4 q + t), lane for lane.
// Pass 1: act in fp32 straight from the accumulators, one tile pair at a
// time, rounded to BF16 and parked: the wave's 128 x 64 BF16 block, row R
// at 128 R, 16-byte chunk k (columns 8 k .. 8 k + 7) at chunk
// k ^ ((R >> 1) & 7), so that the 8-byte writes of 32 rows and the 16-byte
// reads of 8 rows both spread over all banks.
// Pass 2: item n of lane l is row (64 n + l) / 8 and columns
// 8 ((64 n + l) % 8) .. + 7: four lanes holding one MX block of 32
// activations quantize it exactly as the row-wise quantize kernel does.
// Codes go to act_codes [M, Nh/2] (32 bytes per row per wave), scale bytes
// to act_scales [M, Nh/32] and, when act is given, the BF16 rows to
// act [M, Nh] (16 bytes per lane, whole 128-byte lines per 8 lanes).
__device__ __forceinline__ uint32_t swiglu_park_offset(int R, int k) {
  return (uint32_t)(128 * R + 16 * (k ^ ((R >> 1) & 7)));
}

// FP32 epilogue through LDS, in four rounds of 32 rows (MFMA tile row i):
// each wave parks its 32 x 128 fp32 block in its 16 KiB region (512-byte
// rows; 16-byte chunk c = 8 j + 2 q + h of row r, i.e. columns
// 32 j + 8 q + 4 h .. + 3, at chunk c ^ (r % 16), so that the writes of 16
// rows and the reads of one row spread over all banks), then copies it out
// with 32 lanes per 512-byte row segment: two rows, 8 whole cache lines per
// store instruction, against 32 partial lines per instruction stored
// straight from the accumulators. Stores are buffer stores as in
// copy_parked_rows: one resource per two rows of C (8 N <= 2^31 bytes), a
// masked lane's offset 2^31 past it. A wave issues exactly 64 stores.
__device__ __forceinline__ void store_tile_f32_lds(const Ctx& c, v16f_t (&acc)[4][4], int wy,
                                                   int wx, int lane, uint8_t* region,
                                                   void* __restrict__ C) {
  int r = lane & 31, h = lane >> 5;
  asm volatile("" : "+v"(r), "+v"(h));
  const int mrow = c.row0 + wy * 128;  // first row and column of the wave's block
  const int ncol = c.col0 + wx * 128;
  const int k = lane & 31, x1 = lane >> 5;  // read-back: chunk k of row 2 g + x1
  const uint32_t row2 = 8u * (uint32_t)c.N;
  const uint32_t lane_off = ncol + 32 * (k >> 3) < c.N ? x1 * 4u * (uint32_t)c.N + 16u * k
                                                         : 0x80000000u;
  uint8_t* cbase = static_cast<uint8_t*>(C) + ((int64_t)mrow * c.N + ncol) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v16f_t v = acc[i][j];
      asm volatile("" : "+v"(v));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int chunk = 8 * j + 2 * q + h;
        *reinterpret_cast<float4*>(region + r * 512 + 16 * (chunk ^ (r & 15))) =
            make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
      MXFP4_FENCE();
    }
    const int rows_left = c.M - mrow - 32 * i;
    uint8_t* rbase = cbase + (int64_t)(32 * i) * c.N * 4;
#pragma unroll 1
    for (int g0 = 0; g0 < 16; g0 += 4) {
      uint4 w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = 2 * (g0 + e) + x1;
        w[e] = *reinterpret_cast<const uint4*>(region + x * 512 + 16 * (k ^ (x & 15)));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int g = g0 + e;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            rbase + (int64_t)g * row2, 0, (int)row2, kBufferWord3);
        const uint32_t voff = 2 * g + x1 < rows_left ? lane_off : 0x80000000u;
        const u32x4_t o = {w[e].x, w[e].y, w[e].z, w[e].w};
        __builtin_amdgcn_raw_buffer_store_b128(o, rsrc, (int)voff, 0, 0);
      }
    }
    // This round's reads are done before the next round overwrites the region.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    MXFP4_FENCE();
  }
}

__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ void store_tile_swiglu(const int row0, const int col0, const int M,
                                                  const int Nh, v16f_t (&acc)[4][4], int wy,
                                                  int wx, int lane, uint8_t* region,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales,
                                                  uint16_t* __restrict__ act) {
  int r = lane & 31, h = lane >> 5;
  asm volatile("" : "+v"(r), "+v"(h));
  const int ncol = col0 + 64 * wx;  // first activation column of the wave
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      v16f_t g = acc[i][2 * b];
      v16f_t u = acc[i][2 * b + 1];
      asm volatile("" : "+v"(g), "+v"(u));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint2 w = make_uint2(pack_bf16x2(silu(g[4 * q]) * u[4 * q],
                                               silu(g[4 * q + 1]) * u[4 * q + 1]),
                                   pack_bf16x2(silu(g[4 * q + 2]) * u[4 * q + 2],
                                               silu(g[4 * q + 3]) * u[4 * q + 3]));
        *reinterpret_cast<uint2*>(region + swiglu_park_offset(32 * i + r, 4 * b + q) + 8 * h) = w;
      }
      MXFP4_FENCE();
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const int mrow = row0 + 128 * wy;
#pragma unroll 1
  for (int n0 = 0; n0 < 16; n0 += 4) {
    u32x4_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int item = 64 * (n0 + k) + lane;
      w[k] = *reinterpret_cast<const u32x4_t*>(region + swiglu_park_offset(item >> 3, item & 7));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int item = 64 * (n0 + k) + lane;
      const int R = item >> 3, cg = item & 7;
      const uint32_t byte = scale_byte_of(quad_max(block_quarter_absmax(w[k])));
      const uint32_t c = encode8(w[k], __uint_as_float(byte << 23));
      const int m = mrow + R;
      if (m < M) {
        *reinterpret_cast<uint32_t*>(codes + (int64_t)m * (Nh / 2) + ncol / 2 + 4 * cg) = c;
        if ((lane & 3) == 0) scales[(int64_t)m * (Nh / 32) + ncol / 32 + (cg >> 2)] = (uint8_t)byte;
        if (act != nullptr)
          *reinterpret_cast<u32x4_t*>(act + (int64_t)m * Nh + ncol + 8 * cg) = w[k];
      }
    }
  }
}

template <int kEpi, bool kFull, bool kShufB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tile_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                      const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int M, int N,
                      int K, void* __restrict__ C, int tiles_m, int tiles_n,
                      uint8_t* __restrict__ act_codes, uint8_t* __restrict__ act_scales, int Nh) {
  constexpr bool kGlu = kEpi == kEpiSwiglu;
  constexpr bool kOutFp32 = kEpi == kEpiFp32;
  __shared__ Tiles tl;
  __shared__ __align__(16) uint8_t chunks[2][2 * kChunkBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wy = wave >> 1;
  const int wx = wave & 1;
  const int r = lane & 31;
  const int h = lane >> 5;
  const int ksteps = K / 256;
  const int total = tiles_m * tiles_n;

  Ctx c;
  c.A = A;
  c.B = B;
  c.As = As;
  c.Bs = Bs;
  c.row_bytes = K / 2;
  c.scale_row_bytes = K / 32;
  c.M = M;
  c.N = N;
  c.Nh = Nh;
  c.ksteps = ksteps;
  c.nchunks = (K + 1023) / 1024;
  c.lane16 = 16u * (uint32_t)lane;
  c.klast = ksteps - 1;
  c.hlast = 2 * ksteps - 1;
  c.rot = kFull ? (((int)(blockIdx.x % kNumXcd) * ksteps) / kNumXcd) & ~3 : 0;
  c.rot_chunks = c.rot / kChunkSteps;
  c.rot_xcd = kFull ? c.rot : -1;
  c.wave = wave;
  c.interior = false;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int prow = lane >> 3;
    const int chunk = (lane & 7) ^ chunk_swizzle(8 * par + prow);
    c.code_lane[par] = (uint32_t)(prow * c.row_bytes + chunk * 16);
  }
  c.scale_lane = 32 * (lane & 3) + (lane >> 5);
  c.scale_t = (lane >> 2) & 7;
  c.a_base = (wy * 128 + r) * kRowBytes;
  c.b_base = (wx * 128 + r) * kRowBytes;
  c.frag_x = (uint32_t)((h ^ chunk_swizzle(r)) << 4);
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    c.fa_off[sl] = (uint32_t)c.a_base + ((uint32_t)(32 * sl) ^ c.frag_x);
    c.fb_off[sl] = (uint32_t)c.b_base + ((uint32_t)(32 * sl) ^ c.frag_x);
  }
  c.s_off = 16 * kChunk * (wy * 32 + r);
  c.sb_off = 16 * kChunk * (wx * 32 + r);
  c.s_x = (r >> 1) & 7;
  c.s_sel = (uint32_t)h | (uint32_t)(4 + h) << 8 | (uint32_t)(2 + h) << 16 |
            (uint32_t)(6 + h) << 24;

  // Persistent: this workgroup takes tiles blockIdx.x, + gridDim.x, ...; the
  // grid is a multiple of 8, so every tile id keeps its workgroup's XCD.
  int p = blockIdx.x;
  set_tile<kGlu, kShufB>(c, p, tiles_m, tiles_n);
  issue_tile_head<kFull, kGlu, kShufB>(c, tl, chunks);
  issue_tile_tail<kFull, kGlu, kShufB>(c, tl, chunks);
  // A previous tile's epilogue issued all its stores (32 for BF16, 64 for
  // FP32, masked lanes dropped by the store resource) between the head and
  // the tail loads of this tile.
  bool whole_prev = false;
  SectionTimer st;
  st.start();
  for (; p < total; p += gridDim.x) {
    // Wait for the head loads (vector memory operations complete in issue
    // order): outstanding may remain the 8 tail loads and, after a previous
    // tile, the stores issued between head and tail. The counter holds at
    // most 63, so after an FP32 block the oldest 9 of its 64 stores are
    // waited for too.
    if (kEpi == kEpiBf16 && whole_prev)
      asm volatile("s_waitcnt vmcnt(40)\n\ts_barrier" ::: "memory");
    else if (kOutFp32 && whole_prev)
      asm volatile("s_waitcnt vmcnt(63)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    st.mark<kSecTileWait>();

    v16f_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v16f_t{};
    Frags fa, fb;
    HalfScales sc0, sc1;
#pragma unroll
    for (int j = 0; j < 4; ++j) read_frag_b<0>(c, tl, 0, j, fa.b[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) read_frag_a<0>(c, tl, 0, i, fa.a[i]);
    read_half_scales(c, chunks[0], 0, sc0);
    read_half_scales(c, chunks[0], 1, sc1);

    int T = 0;
    for (; T + 4 <= ksteps; T += 4) {
      k_step<kFull, kGlu, kShufB, 1, 0>(c, tl, chunks, acc, fa, fb, sc0, sc1, T, st);
      k_step<kFull, kGlu, kShufB, 2, 1>(c, tl, chunks, acc, fa, fb, sc0, sc1, T + 1, st);
      k_step<kFull, kGlu, kShufB, 3, 0>(c, tl, chunks, acc, fa, fb, sc0, sc1, T + 2, st);
      k_step<kFull, kGlu, kShufB, 0, 1>(c, tl, chunks, acc, fa, fb, sc0, sc1, T + 3, st);
    }
    if (T < ksteps) k_step<kFull, kGlu, kShufB, 1, 0>(c, tl, chunks, acc, fa, fb, sc0, sc1, T, st);
    if (T + 1 < ksteps) k_step<kFull, kGlu, kShufB, 2, 1>(c, tl, chunks, acc, fa, fb, sc0, sc1, T + 1, st);
    if (T + 2 < ksteps) k_step<kFull, kGlu, kShufB, 3, 0>(c, tl, chunks, acc, fa, fb, sc0, sc1, T + 2, st);
    // Every load of this tile has landed and every LDS read has returned,
    // in all waves, before the next tile's loads reuse the buffers.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    st.mark<kSecLoopEnd>();

    // Start the next tile's loads, then write this tile's C while they fly;
    // the last 8 loads issued are the ones the next wait leaves outstanding.
    const int pn = p + gridDim.x;
    if constexpr (kGlu) {
      // As for BF16 C: the next tile's head loads go first, the activation
      // is parked in slot 1, and the tail loads wait for every wave's pass 2.
      const int row0 = c.row0, col0 = c.col0;
      if (pn < total) {
        set_tile<kGlu, kShufB>(c, pn, tiles_m, tiles_n);
        issue_tile_head<kFull, kGlu, kShufB>(c, tl, chunks);
      }
      st.mark<kSecEpiHead>();
      uint8_t* region = wave < 2 ? tl.a[1] + 16384 * wave : tl.b[1] + 16384 * (wave - 2);
      store_tile_swiglu(row0, col0, M, Nh, acc, wy, wx, lane, region, act_codes, act_scales,
                        static_cast<uint16_t*>(C));
      st.mark<kSecEpiStore>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else if constexpr (kOutFp32) {
      // As for BF16 C: head loads first, C parked in slot 1 four rounds of
      // 32 rows, the tail loads after every wave has read its block back.
      // Every wave issues exactly 64 stores (masked lanes are dropped by the
      // store resource), so the next tile's first wait can count them.
      const Ctx cur_tile = c;
      whole_prev = true;
      if (pn < total) {
        set_tile<kGlu, kShufB>(c, pn, tiles_m, tiles_n);
        issue_tile_head<kFull, kGlu, kShufB>(c, tl, chunks);
      }
      st.mark<kSecEpiHead>();
      uint8_t* region = wave < 2 ? tl.a[1] + 16384 * wave : tl.b[1] + 16384 * (wave - 2);
      store_tile_f32_lds(cur_tile, acc, wy, wx, lane, region, C);
      st.mark<kSecEpiStore>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      // The next tile's head loads (slot 0, chunks[0]) go out before the C
      // stores, so that they do not queue behind them; C is parked in slot 1
      // (waves 0, 1 in A's, waves 2, 3 in B's, 16 KiB each), and the tail
      // loads into slot 1 wait until every wave has read its block back.
      const Ctx cur_tile = c;
      whole_prev = true;  // copy_parked_rows issues 32 stores, masked lanes dropped
      if (pn < total) {
        set_tile<kGlu, kShufB>(c, pn, tiles_m, tiles_n);
        issue_tile_head<kFull, kGlu, kShufB>(c, tl, chunks);
      }
      st.mark<kSecEpiHead>();
      uint8_t* region = wave < 2 ? tl.a[1] + 16384 * wave : tl.b[1] + 16384 * (wave - 2);
      store_tile_bf16_lds(cur_tile, acc, wy, wx, lane, region, C);
      st.mark<kSecEpiStore>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    st.mark<kSecEpiBarrier>();
    if (pn < total) issue_tile_tail<kFull, kGlu, kShufB>(c, tl, chunks);
    st.mark<kSecEpiTail>();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  st.store(blockIdx.x * (kThreads / 64) + wave);
}

}  // namespace

// Workgroups of the persistent grid per device: the CU count rounded down
// to a multiple of the XCD count (0 = not queried yet).
std::atomic<int> g_workers[64];

hipError_t init_kernels_for_current_device() {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  g_workers[dev].store(cus / kNumXcd > 0 ? cus / kNumXcd * kNumXcd : kNumXcd,
                       std::memory_order_release);
  return hipSuccess;
}

hipError_t device_workers(int& workers) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  workers = g_workers[dev].load(std::memory_order_acquire);
  if (workers == 0) {
    e = init_kernels_for_current_device();
    if (e != hipSuccess) return e;
    workers = g_workers[dev].load(std::memory_order_acquire);
  }
  return hipSuccess;
}

// Workgroups of the persistent grid for `total` tiles: one per tile when
// they fit in one round; otherwise one per CU (a multiple of 8), except
// when the last round would leave at least half of them idle: then
// ceil(total / rounds) rounded up to a multiple of 8, the same number of
// rounds with every round nearly full, so that no round runs with the whole
// chip busy at its lower, power-capped clock (K = 8192, BF16 C: 320 tiles
// 108.5-112.1 -> 105.2-107.4 us, 544 tiles 166.4 -> 156.3 us, 384 tiles
// 112.0-118.2 -> 112.0-116.3 us; with the last round two-thirds full, as
// for 4128 x 6176 x 7936 (425 tiles), fewer workgroups measured 4% slower).
inline int tile_grid(int total, int workers) {
  if (total <= workers) return total;
  const int rounds = (total + workers - 1) / workers;
  const int last = total - (rounds - 1) * workers;
  if (2 * last > workers) return workers;
  const int even = ((total + rounds - 1) / rounds + kNumXcd - 1) / kNumXcd * kNumXcd;
  return even < workers ? even : workers;
}

template <int kEpi, bool kShufB = false>
static void launch_tile_kernel(bool full, dim3 grid, hipStream_t stream, const uint8_t* a,
                               const uint8_t* as, const uint8_t* b, const uint8_t* bs, int M,
                               int N, int K, void* C, int tiles_m, int tiles_n,
                               uint8_t* act_codes, uint8_t* act_scales, int Nh) {
  if (full)
    hipLaunchKernelGGL((gemm_tile_kernel<kEpi, true, kShufB>), grid, dim3(kThreads), 0, stream, a,
                       as, b, bs, M, N, K, C, tiles_m, tiles_n, act_codes, act_scales, Nh);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<kEpi, false, kShufB>), grid, dim3(kThreads), 0, stream,
                       a, as, b, bs, M, N, K, C, tiles_m, tiles_n, act_codes, act_scales, Nh);
}

hipError_t launch_gemm(const void* A, const void* As, const void* B, const void* Bs, int M, int N,
                       int K, bool out_fp32, void* C, hipStream_t stream) {
  int workers = 0;
  hipError_t e = device_workers(workers);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + kTileM - 1) / kTileM;
  const int tiles_n = (N + kTileN - 1) / kTileN;
  const int total = tiles_m * tiles_n;
  const dim3 grid(tile_grid(total, workers));
  const auto* a = static_cast<const uint8_t*>(A);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* b = static_cast<const uint8_t*>(B);
  const auto* bs = static_cast<const uint8_t*>(Bs);
  const bool full = K % 1024 == 0;
  if (out_fp32)
    launch_tile_kernel<kEpiFp32>(full, grid, stream, a, as, b, bs, M, N, K, C, tiles_m, tiles_n,
                                 nullptr, nullptr, 0);
  else
    launch_tile_kernel<kEpiBf16>(full, grid, stream, a, as, b, bs, M, N, K, C, tiles_m, tiles_n,
                                 nullptr, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_gemm_bshuffled(const void* A, const void* As, const void* Bsh, const void* Bssh,
                                 int M, int N, int K, bool out_fp32, void* C, hipStream_t stream) {
  int workers = 0;
  hipError_t e = device_workers(workers);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + kTileM - 1) / kTileM;
  const int tiles_n = (N + kTileN - 1) / kTileN;
  const int total = tiles_m * tiles_n;
  const dim3 grid(tile_grid(total, workers));
  const auto* a = static_cast<const uint8_t*>(A);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* b = static_cast<const uint8_t*>(Bsh);
  const auto* bs = static_cast<const uint8_t*>(Bssh);
  const bool full = K % 1024 == 0;
  if (out_fp32)
    launch_tile_kernel<kEpiFp32, true>(full, grid, stream, a, as, b, bs, M, N, K, C, tiles_m,
                                       tiles_n, nullptr, nullptr, 0);
  else
    launch_tile_kernel<kEpiBf16, true>(full, grid, stream, a, as, b, bs, M, N, K, C, tiles_m,
                                       tiles_n, nullptr, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(const void* A, const void* As, const void* B, const void* Bs, int M,
                              int N, int K, void* act_codes, void* act_scales, void* act_bf16,
                              hipStream_t stream) {
  int workers = 0;
  hipError_t e = device_workers(workers);
  if (e != hipSuccess) return e;
  const int Nh = N / 2;
  const int tiles_m = (M + kTileM - 1) / kTileM;
  const int tiles_n = (Nh + kTileN / 2 - 1) / (kTileN / 2);
  const int total = tiles_m * tiles_n;
  const dim3 grid(tile_grid(total, workers));
  launch_tile_kernel<kEpiSwiglu>(K % 1024 == 0, grid, stream, static_cast<const uint8_t*>(A),
                                 static_cast<const uint8_t*>(As), static_cast<const uint8_t*>(B),
                                 static_cast<const uint8_t*>(Bs), M, N, K, act_bf16, tiles_m,
                                 tiles_n, static_cast<uint8_t*>(act_codes),
                                 static_cast<uint8_t*>(act_scales), Nh);
  return hipGetLastError();
}

}  // namespace mxfp4
