// Host-side launchers of the gfx950 kernels, called by the C ABI in api.hip.
// Arguments are validated by the caller; the launchers only size the grid,
// enqueue on `stream` and report hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

// Row-wise BF16 -> MXFP4 over the flat [M*K/32] block sequence.
hipError_t launch_quantize(const void* x_bf16, int64_t nblocks, void* codes, void* scales,
                           hipStream_t stream);

// Row-wise and column-wise MXFP4 of X [M, K] in one pass: codes_row [M, K/2],
// scales_row [M, K/32], codes_col [K, M/2], scales_col [K, M/32].
hipError_t launch_quantize_2d(const void* x_bf16, int M, int K, void* codes_row, void* scales_row,
                              void* codes_col, void* scales_col, hipStream_t stream);

// Stochastic-rounding variants (Philox4x32-10 keyed by block coordinates,
// direction and `seed`): row-wise over [M, K], and both forms of X [M, K].
// The input holds rows row0 .. row0 + M - 1 of a larger one; the draws are
// keyed by those global rows (and, column-wise, by the global row block
// row0 / 32 + j; row0 % 32 == 0 there).
hipError_t launch_quantize_sr(const void* x_bf16, int64_t M, int64_t K, int64_t row0,
                              uint64_t seed, void* codes, void* scales, hipStream_t stream);
hipError_t launch_quantize_2d_sr(const void* x_bf16, int M, int K, int64_t row0, uint64_t seed,
                                 void* codes_row, void* scales_row, void* codes_col,
                                 void* scales_col, hipStream_t stream);

// C[M,N] = A[M,K] * B[N,K]^T with block scales; out_fp32 selects FP32 vs BF16.
hipError_t launch_gemm(const void* A, const void* As, const void* B, const void* Bs, int M,
                       int N, int K, bool out_fp32, void* C, hipStream_t stream);

// Gate+up GEMM with the SwiGLU + MXFP4 requantize epilogue: B is the stacked
// [W_gate; W_up] (N rows, N / 2 each, N % 256 == 0); writes act codes [M, N/4], scales
// [M, N/64] and, when act_bf16 is not null, the BF16 act [M, N/2].
hipError_t launch_gemm_swiglu(const void* A, const void* As, const void* B, const void* Bs, int M,
                              int N, int K, void* act_codes, void* act_scales, void* act_bf16,
                              hipStream_t stream);

// Pre-shuffled weights: sizes of the shuffled codes and scales of B [N, K],
// the shuffle itself, and the tile GEMM reading B in that layout.
void shuffled_b_sizes(int64_t N, int64_t K, int64_t* code_bytes, int64_t* scale_bytes);
hipError_t launch_shuffle_b(const void* codes, const void* scales, int N, int K, void* codes_sh,
                            void* scales_sh, hipStream_t stream);
hipError_t launch_gemm_bshuffled(const void* A, const void* As, const void* Bsh, const void* Bssh,
                                 int M, int N, int K, bool out_fp32, void* C, hipStream_t stream);

// Edge of the tile kernel's square tiles of C.
constexpr int kGemmTile = 256;

// Same contract, for M up to kSkinnyMaxM and for problems of few tiles: one
// 32 x 32 tile of C per workgroup, K split between its waves.
constexpr int kSkinnyMaxM = 128;
hipError_t launch_gemm_skinny(const void* A, const void* As, const void* B, const void* Bs,
                              int M, int N, int K, bool out_fp32, void* C, hipStream_t stream);

// Fragment order (the register-ring skinny GEMM's operand order; R % 32 == 0,
// K % 256 == 0): row-wise quantize writing it, the re-layout of plain
// MXFP4 bytes into it, and the GEMM reading both operands in it.
hipError_t launch_quantize_frag(const void* x_bf16, int64_t M, int64_t K, void* codes,
                                void* scales, hipStream_t stream);
hipError_t launch_to_frag(const void* codes, const void* scales, int64_t R, int64_t K,
                          void* codes_f, void* scales_f, hipStream_t stream);
hipError_t launch_gemm_frag(const void* A, const void* As, const void* B, const void* Bs, int M,
                            int N, int K, bool out_fp32, void* C, hipStream_t stream);

// One-time per-device set-up of kernel attributes (large LDS allocations).
hipError_t init_kernels_for_current_device();

// Workgroups of a one-per-CU persistent grid on the current device: the CU
// count rounded down to a multiple of the XCD count (cached per device).
hipError_t device_workers(int& workers);

}  // namespace mxfp4
