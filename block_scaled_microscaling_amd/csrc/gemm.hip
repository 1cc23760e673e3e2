// Block-scaled MXFP4 x MXFP4 GEMM (TN) for gfx950.
//
// Computes C[m, n] = sum_k dq(A[m, k]) * dq(B[n, k]), the FP4 x FP4 ("a4w4")
// GEMM of "Initial integration of a4w4 GEMM" (ROCm/TransformerEngine #663),
// under the contract of the hipBLASLt MXFP4 path on "Integrate MXFP4
// hipblaslt GEMM support" (#697, Changes list): TN, plain E2M1 data and
// plain UE8M0 block-32 scales, BF16/FP32 output, K % 256, M/N % 32, no bias,
// beta = 0.
//
// The contraction runs on v_mfma_scale_f32_16x16x128_f8f6f4 with both
// operand formats set to FP4 (cbsz = blgp = 4). Per lane l of a wavefront,
// an operand fragment is the 32 codes (16 bytes) of row l % 16 in the K block
// l / 16 of a 128-wide K step, and the lane's scale byte is that same
// (row, K block)'s UE8M0 scale: one MX block per lane, so plain row-major
// data and scales feed the instruction without any reshuffle. The
// accumulator of lane l holds rows 4*(l/16) .. +3 of column l % 16.
//
// The kernel feeds B's fragment as the instruction's first operand and A's
// as the second, so it produces C^T tiles: lane l then holds four
// consecutive columns of one row of C, stored with one 8-byte (BF16) or
// 16-byte (FP32) write.
//
// Tiling: one workgroup of 8 wavefronts (2 per SIMD) owns a 256 x 256 tile
// of C; wavefront (wy, wx) owns rows 128*wy .. +127 and columns 64*wx .. +63,
// i.e. 8 x 4 MFMA tiles and 128 fp32 accumulators per lane. Two wavefronts
// per SIMD let one issue MFMAs while the other waits on LDS.
//   * K step = 128 (64 bytes of codes per row). A, B and scale tiles go
//     global -> registers -> LDS. Global loads run two K steps ahead in two
//     alternating register sets; LDS holds two K steps (one being read, one
//     being written); one barrier per step.
//   * LDS rows are 64 bytes; their four 16-byte chunks are XOR-swizzled by
//     bits 1-3 of the row, so the 16 lanes that read one chunk column of 16
//     consecutive rows fall on distinct banks (in groups of 8 and of 16).
//   * Scale tiles are stored in LDS transposed, so one 8-byte (A) or 4-byte
//     (B) read gives a lane the scale bytes of all its MFMA tiles; the
//     instruction's op_sel picks the byte.
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
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kStepBytes = 64;  // 128 FP4 codes of one row per K step
constexpr int kTileBytes = kTileM * kStepBytes;
constexpr int kScaleBytes = kTileM * 4;  // 4 scale bytes per row per K step
constexpr int kGroupM = 4;
constexpr int kNumXcd = 8;

struct __align__(16) Smem {
  uint8_t a[2][kTileBytes];
  uint8_t b[2][kTileBytes];
  uint8_t sa[2][kScaleBytes];
  uint8_t sb[2][kScaleBytes];
};

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
__device__ __forceinline__ v4f_t mfma_fp4(const uint4& x, const uint4& y, v4f_t c, uint32_t sx,
                                          uint32_t sy) {
  const v8i_t xv = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  const v8i_t yv = {(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xv, yv, c, 4, 4, SEL_X, (int)sx, SEL_Y,
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

// A K step staged in registers by one thread: two 16-byte chunks of A, two
// of B, and one 4-byte scale word (of A for threads 0..255, of B for threads
// 256..511).
// Global -> register loads of one K step into the named register set
// (a0_, a1_, b0_, b1_, s_) and register -> LDS stores of such a set into
// slot `slot_`. Macros over named registers keep the staged values out of
// any addressable object, so they stay in VGPRs.
#define MXFP4_LOAD_STAGE(a0_, a1_, b0_, b1_, s_, kt_)                          \
  do {                                                                         \
    const int64_t koff_ = (int64_t)(kt_) * kStepBytes;                         \
    a0_ = *reinterpret_cast<const uint4*>(a_src0 + koff_);                     \
    a1_ = *reinterpret_cast<const uint4*>(a_src1 + koff_);                     \
    b0_ = *reinterpret_cast<const uint4*>(b_src0 + koff_);                     \
    b1_ = *reinterpret_cast<const uint4*>(b_src1 + koff_);                     \
    s_ = *reinterpret_cast<const uint32_t*>(s_src + (kt_) * 4);                \
  } while (0)

#define MXFP4_STORE_STAGE(a0_, a1_, b0_, b1_, s_, slot_)                       \
  do {                                                                         \
    *reinterpret_cast<uint4*>(&sm.a[slot_][st_off]) = a0_;                     \
    *reinterpret_cast<uint4*>(&sm.a[slot_][st_off + 128 * kStepBytes]) = a1_;  \
    *reinterpret_cast<uint4*>(&sm.b[slot_][st_off]) = b0_;                     \
    *reinterpret_cast<uint4*>(&sm.b[slot_][st_off + 128 * kStepBytes]) = b1_;  \
    uint8_t* ls_ = (scale_of_a ? sm.sa[slot_] : sm.sb[slot_]) + s_slot;        \
    ls_[0] = (uint8_t)(s_);                                                    \
    ls_[256] = (uint8_t)((s_) >> 8);                                           \
    ls_[512] = (uint8_t)((s_) >> 16);                                          \
    ls_[768] = (uint8_t)((s_) >> 24);                                          \
  } while (0)

template <bool kOutFp32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tile_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                      const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int M, int N,
                      int K, void* __restrict__ C, int tiles_m, int tiles_n) {
  __shared__ Smem sm;

  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * kTileM;
  const int col0 = tn * kTileN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave >> 2;  // 128-row half of the A tile
  const int wx = wave & 3;   // 64-row quarter of the B tile
  const int r = lane & 15;
  const int g = lane >> 4;

  const int64_t row_bytes = K / 2;
  const int64_t scale_row_bytes = K / 32;

  // Loader roles per K step: chunk q (0, 1) of thread tid covers tile row
  // tid / 4 + 128 q, 16-byte column tid % 4, of A and of B. Thread tid also
  // moves the 4 scale bytes of A row tid (tid < 256) or B row tid - 256.
  // Rows past M or N are clamped to the last row: computed, never stored.
  const int trow = tid >> 2, tcol = tid & 3;
  const uint8_t* a_src0 = A + (int64_t)min(row0 + trow, M - 1) * row_bytes + tcol * 16;
  const uint8_t* a_src1 = A + (int64_t)min(row0 + trow + 128, M - 1) * row_bytes + tcol * 16;
  const uint8_t* b_src0 = B + (int64_t)min(col0 + trow, N - 1) * row_bytes + tcol * 16;
  const uint8_t* b_src1 = B + (int64_t)min(col0 + trow + 128, N - 1) * row_bytes + tcol * 16;
  const int st_off = trow * kStepBytes + ((tcol ^ chunk_swizzle(trow)) << 4);
  const bool scale_of_a = tid < 256;
  const int srow = tid & 255;
  const uint8_t* s_src = scale_of_a
                             ? As + (int64_t)min(row0 + srow, M - 1) * scale_row_bytes
                             : Bs + (int64_t)min(col0 + srow, N - 1) * scale_row_bytes;
  // Transposed scale slots. A: [K block][128-row half][row % 16][A tile 0..7];
  // B: [K block][64-row quarter][row % 16][B tile 0..3]; 256 bytes per K block.
  const int s_slot = scale_of_a ? ((srow >> 7) * 16 + (srow & 15)) * 8 + ((srow >> 4) & 7)
                                : ((srow >> 6) * 16 + (srow & 15)) * 4 + ((srow >> 4) & 3);

  // Fragment offsets of this lane: row (base + 16 * tile + r), chunk g.
  const int a_off = (wy * 128 + r) * kStepBytes + ((g ^ chunk_swizzle(r)) << 4);
  const int b_off = (wx * 64 + r) * kStepBytes + ((g ^ chunk_swizzle(r)) << 4);
  const int sa_off = g * 256 + (wy * 16 + r) * 8;
  const int sb_off = g * 256 + (wx * 16 + r) * 4;

  v4f_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.f, 0.f, 0.f, 0.f};

  // One K step from LDS slot `slot`: scales, then B fragments, then A
  // fragments in the order the MFMAs (A tile outer, B tile inner) use them.
  auto compute = [&](int slot) {
    const uint2 sa = *reinterpret_cast<const uint2*>(&sm.sa[slot][sa_off]);
    const uint32_t sb = *reinterpret_cast<const uint32_t*>(&sm.sb[slot][sb_off]);
    uint4 bf[4], af[8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const uint4*>(&sm.b[slot][b_off + j * 16 * kStepBytes]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      af[i] = *reinterpret_cast<const uint4*>(&sm.a[slot][a_off + i * 16 * kStepBytes]);
    static_for<8>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint32_t sai = (i < 4) ? sa.x : sa.y;
      static_for<4>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        acc[i][j] = mfma_fp4<j, i % 4>(bf[j], af[i], acc[i][j], sb, sai);
      });
    });
  };

  // Step s is loaded into register set s % 2 during step s - 2, written to
  // LDS slot s % 2 at the end of step s - 1, and computed in step s.
  const int ksteps = K / 128;  // even, >= 2
  const int klast = ksteps - 1;
  uint4 xa0, xa1, xb0, xb1, ya0, ya1, yb0, yb1;  // register sets x (even), y (odd)
  uint32_t xs, ys;
  MXFP4_LOAD_STAGE(xa0, xa1, xb0, xb1, xs, 0);
  MXFP4_LOAD_STAGE(ya0, ya1, yb0, yb1, ys, 1);
  MXFP4_STORE_STAGE(xa0, xa1, xb0, xb1, xs, 0);
  __syncthreads();

  for (int kt = 0; kt < ksteps; kt += 2) {
    MXFP4_LOAD_STAGE(xa0, xa1, xb0, xb1, xs, min(kt + 2, klast));
    compute(0);
    MXFP4_STORE_STAGE(ya0, ya1, yb0, yb1, ys, 1);
    __syncthreads();

    MXFP4_LOAD_STAGE(ya0, ya1, yb0, yb1, ys, min(kt + 3, klast));
    compute(1);
    MXFP4_STORE_STAGE(xa0, xa1, xb0, xb1, xs, 0);
    __syncthreads();
  }

  // Epilogue: lane holds C[row0 + wy*128 + 16i + r][col0 + wx*64 + 16j + 4g + 0..3].
  // M and N are multiples of 16, so each 16 x 16 tile is wholly in or out.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m_base = row0 + wy * 128 + i * 16;
    if (m_base >= M) continue;
    const int m = m_base + r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n_base = col0 + wx * 64 + j * 16;
      if (n_base >= N) continue;
      const int n = n_base + 4 * g;
      const v4f_t v = acc[i][j];
      if constexpr (kOutFp32) {
        float* dst = static_cast<float*>(C) + (int64_t)m * N + n;
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        uint16_t* dst = static_cast<uint16_t*>(C) + (int64_t)m * N + n;
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
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
