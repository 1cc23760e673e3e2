/*
 * mxfp4.h -- C ABI of libmxfp4.so: BF16 -> MXFP4 quantize (row-wise or
 * bidimensional, round-to-nearest or stochastic) and the block-scaled
 * MXFP4 x MXFP4 ("a4w4") GEMM on AMD Instinct gfx950 (MI355X).
 *
 * Format ("Integrate MXFP4 hipblaslt GEMM support", ROCm/TransformerEngine
 * #697, Changes list): an MXFP4 operand is FP4 E2M1 elements with one UE8M0
 * power-of-two scale per 32 consecutive K elements. Layouts used here:
 *   codes   uint8 [rows, K/2]  row-major; element 2i in bits 3:0, 2i+1 in 7:4
 *   scales  uint8 [rows, K/32] row-major; value 2^(byte - 127)
 *   E2M1    bit 3 sign, magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}
 *
 * Ownership and threading, for every entry point below:
 *   - All data pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees, copies or synchronizes; work is enqueued
 *     asynchronously on `stream` (a hipStream_t; NULL = the default stream).
 *   - Every argument is validated before anything is enqueued. A non-zero
 *     return means nothing was enqueued and no output was written.
 *   - The arch check runs once per device; calls are thread-safe.
 *
 * Return codes follow the stub convention reviewed on "Initial integration
 * of a4w4 GEMM" (ROCm/TransformerEngine #663): 0 on success, a distinct
 * negative code per failure class, plus an availability probe.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mxfp4_out_dtype { MXFP4_OUT_BF16 = 0, MXFP4_OUT_FP32 = 1 };

enum mxfp4_status {
  MXFP4_OK = 0,
  MXFP4_EINVAL = -1,       /* a size, pointer or out_dtype is invalid        */
  MXFP4_EUNSUPPORTED = -2, /* current device is not gfx950, or no device    */
  MXFP4_ELAUNCH = -3,      /* the HIP runtime reported an error at launch   */
  MXFP4_EALIGN = -4        /* a pointer lacks the alignment stated below    */
};

/* 1 if the current HIP device is gfx950 and the kernels are loadable, else
 * 0. Never fails; suggested on the a4w4 integration page as the probe a
 * framework checks before routing to this backend. */
int mxfp4_available(void);

/* Static, human-readable text for a return code (never NULL). */
const char* mxfp4_strerror(int rc);

/* Row-wise BF16 -> MXFP4 quantize, one 32-element block at a time: the
 * quantizer role of MXFP4Quantizer on "Integrate MXFP4 hipblaslt GEMM
 * support" (plain, un-shuffled data and scales). For each block:
 *   amax  = max |x| over its 32 BF16 values
 *   e     = clamp(floor(log2 amax) - 2, -127, 127)   (e = -127 if amax == 0)
 *   scale = e + 127
 *   code  = sign(x) | E2M1 magnitude nearest to |x| / 2^e, ties to the even
 *           code, saturating at 6; the sign bit is kept on zero results.
 * x_bf16     [M, K] BF16, row-major, 16-byte aligned
 * codes_out  [M, K/2] uint8, 4-byte aligned
 * scales_out [M, K/32] uint8
 * Requires M >= 1, K >= 32, K % 32 == 0, M * K < 2^40, finite inputs
 * (NaN/Inf in a block give unspecified bytes for that block only).
 * mxfp4_quantize enqueues on the default stream; _async on `stream`. */
int mxfp4_quantize(const void* x_bf16, int64_t M, int64_t K, void* codes_out,
                   void* scales_out);
int mxfp4_quantize_async(const void* x_bf16, int64_t M, int64_t K, void* codes_out,
                         void* scales_out, void* stream);

/* Bidimensional quantize: one pass over X [M, K] writes the row-wise MXFP4
 * form (exactly what mxfp4_quantize writes) and the row-wise MXFP4 form of
 * X^T, i.e. blocks of 32 consecutive rows of each column, the operand of a
 * GEMM that contracts over M (the weight gradient of a linear layer). It is
 * the rowwise + columnwise ("bidimensional") quantize of the NVFP4 kernels
 * on NVIDIA/TransformerEngine #3809 (description), for MXFP4 blocks.
 * x_bf16 [M, K] row-major BF16, 16-byte aligned
 * codes_row [M, K/2], scales_row [M, K/32]: as mxfp4_quantize
 * codes_col [K, M/2]: byte i of row k packs X[2i][k] (low nibble) and
 *   X[2i+1][k]; scales_col [K, M/32]: scale of rows 32j..32j+31 of column k
 * codes_row, codes_col 16-byte aligned; scales byte-addressed
 * Requires M, K >= 32, M % 32 == 0, K % 32 == 0, M * K < 2^40; otherwise
 * MXFP4_EINVAL (MXFP4_EALIGN for alignment) and nothing is launched.
 * Asynchronous on `stream` (a hipStream_t, or NULL for the null stream). */
int mxfp4_quantize_2d(const void* x_bf16, int64_t M, int64_t K, void* codes_row,
                      void* scales_row, void* codes_col, void* scales_col, void* stream);

/* Stochastic-rounding quantize. Scales exactly as mxfp4_quantize; each code
 * rounds |x| / 2^e to one of its two E2M1 neighbours lo <= |x|/2^e < hi at
 * random: with frac = (|x|/2^e - lo) / (hi - lo) and u the element's random
 * byte, the result is hi when floor(256 frac) + u >= 256, else lo (so hi
 * with probability floor(256 frac) / 256, which is frac whenever
 * |x|/2^e >= 1/4); |x|/2^e >= 6 gives 6; the sign bit is kept. The random
 * bytes follow the stochastic-rounding design described on
 * NVIDIA/TransformerEngine #3809 (description): one Philox4x32-10 draw
 * (Salmon et al., SC'11) per 16-element half block h of block j of output
 * row r in direction d (0 = row-wise), counter (j, r, d, h), key (seed low
 * 32 bits, seed high 32 bits); element 16 h + i takes byte i % 4, least
 * significant first, of word i / 4. Equal arguments give equal bytes.
 * Arguments, layouts, requirements and errors as mxfp4_quantize_async. */
int mxfp4_quantize_sr(const void* x_bf16, int64_t M, int64_t K, uint64_t seed,
                      void* codes_out, void* scales_out, void* stream);

/* Bidimensional quantize with stochastic rounding: the row-wise outputs are
 * mxfp4_quantize_sr(x, seed) and the column-wise ones are the row-wise
 * stochastic quantize of X^T with direction d = 1 (output row r = column k
 * of X, j = block index along M). Arguments, layouts, requirements and
 * errors as mxfp4_quantize_2d. */
int mxfp4_quantize_2d_sr(const void* x_bf16, int64_t M, int64_t K, uint64_t seed,
                         void* codes_row, void* scales_row, void* codes_col,
                         void* scales_col, void* stream);

/* Row shards of the two calls above, for a caller that splits a larger X
 * over devices or calls: x_bf16 [M, K] holds rows row0 .. row0 + M - 1 of
 * it, and the random bytes are keyed by those global rows (row-wise output
 * row r of the shard draws as row row0 + r) and, column-wise, by the global
 * row block row0 / 32 + j, so each output is exactly the matching part of
 * the whole input's: rows row0 .. of the row-wise codes and scales, and
 * (column-wise, written as [K, M/2] and [K, M/32] for the shard) columns
 * row0 / 2 .. of its codes and row0 / 32 .. of its scales. row0 = 0 is
 * the plain call. Requires 0 <= row0 and row0 + M <= 2^31 - 1, and for the
 * bidimensional form row0 % 32 == 0; otherwise MXFP4_EINVAL. The rest as
 * the plain calls. */
int mxfp4_quantize_sr_rows(const void* x_bf16, int64_t M, int64_t K, int64_t row0,
                           uint64_t seed, void* codes_out, void* scales_out, void* stream);
int mxfp4_quantize_2d_sr_rows(const void* x_bf16, int64_t M, int64_t K, int64_t row0,
                              uint64_t seed, void* codes_row, void* scales_row,
                              void* codes_col, void* scales_col, void* stream);

/* Block-scaled GEMM, TN: C[m, n] = sum_k dq(A[m, k]) * dq(B[n, k]) with
 * dq(code, scale) = E2M1(code) * 2^(scale - 127), fp32 accumulation; the
 * capability gates of the hipBLASLt MXFP4 path on "Integrate MXFP4 hipblaslt
 * GEMM support" (Changes list) are this function's contract:
 *   K % 256 == 0, M % 32 == 0, N % 32 == 0, M, N, K > 0,
 *   out_dtype MXFP4_OUT_BF16 (round to nearest even) or MXFP4_OUT_FP32,
 *   no bias, alpha = 1, beta = 0 (C is overwritten, never read).
 * A_codes [M, K/2], B_codes [N, K/2]: 16-byte aligned
 * A_scales [M, K/32], B_scales [N, K/32]: 4-byte aligned
 * C [M, N] row-major BF16 or FP32: 16-byte aligned
 * M <= 2^31 - 1, N <= 2^28, K <= 2^24, and each buffer < 2^40 bytes;
 * otherwise MXFP4_EINVAL (or MXFP4_EALIGN for alignment) and nothing is
 * launched.
 * M <= 128, and problems of at most CUs / 8 tiles of 256 x 256 (32 tiles
 * on a 256-CU MI355X), run a split-K kernel (one 32 x 32 tile of C per
 * workgroup, the K range split between its waves and summed in LDS in a
 * fixed order); larger problems run 256 x 256 tiles on a persistent grid of
 * one workgroup per CU. Both give the same results up to fp32 summation
 * order.
 * Accuracy: each 64-wide K slice is one block-scaled MFMA whose sum is added
 * to an fp32 accumulator with one rounding, so the 256 x 256 kernel takes
 * K/64 roundings in a row (the split-K kernel K/512 per wave, then 7). With
 * S = sum_k |dq(a_k) dq(b_k)|, an FP32 result satisfies
 *   |C - C_exact| <= max(1e-5, (K/64 + 2) * 2^-24) * S,
 * i.e. 1e-5 * S up to K = 10688 and a bound growing with K past it (about
 * 6.1e-5 * S at K = 65536); inputs whose first K slices hold a large sum and
 * whose later slices each add half a unit in its last place reach it. BF16
 * output is that fp32 value rounded to nearest even. */
int mxfp4_gemm(const void* A_codes, const void* A_scales, const void* B_codes,
               const void* B_scales, int64_t M, int64_t N, int64_t K, int out_dtype,
               void* C, void* stream);

/* mxfp4_gemm on the 256 x 256 tile kernel whatever the shape: the same
 * operation (the a4w4 GEMM of "Initial integration of a4w4 GEMM",
 * ROCm/TransformerEngine #663, under the gates above), for callers that
 * choose the kernel themselves, e.g. to keep one summation order across
 * shapes. Arguments, layouts, requirements, accuracy bound and errors as
 * mxfp4_gemm; asynchronous on `stream`. */
int mxfp4_gemm_tile(const void* A_codes, const void* A_scales, const void* B_codes,
                    const void* B_scales, int64_t M, int64_t N, int64_t K, int out_dtype,
                    void* C, void* stream);

/* Pre-shuffled weights. The a4w4 path of "Integrate MXFP4 hipblaslt GEMM
 * support" (#697, Changes list) and the call reviewed on "Initial integration
 * of a4w4 GEMM" (#663) take the weight pre-shuffled, with swizzled scales:
 * re-arranged once so that the GEMM moves it without address arithmetic.
 * The pages give no layout; this library's is the byte order in which its
 * tile GEMM lands B in LDS:
 *   codes: one 32 KiB block per (256-row tile nt, 256-K step ks) at
 *     (nt * (K/256) + ks) * 32768; row x of the tile at x * 128, its
 *     16-byte chunk p holding the row's chunk p ^ swz(x) of that step, with
 *     swz(x) = (x & 6) | ((x ^ (x >> 3)) & 1);
 *   scales: one 8 KiB block per (tile nt, 1024-K chunk ch) at
 *     (nt * ceil(K/1024) + ch) * 8192; the 4-byte word (four scale bytes)
 *     of row 128 h + 32 t + r and 128-K half-step s of the chunk at
 *     128 (32 h + r) + 16 (s ^ ((r >> 1) & 7)) + 4 t;
 *   rows past N and half-steps past K are zero.
 * mxfp4_shuffle_b_sizes gives the two buffer sizes (N >= 1, K % 256 == 0,
 * K <= 2^24). mxfp4_shuffle_b writes them from plain codes [N, K/2] and
 * scales [N, K/32] (codes 16-byte aligned, scales 4-byte aligned, both
 * outputs likewise); mxfp4_gemm_bshuffled is mxfp4_gemm with B given in
 * this layout (same requirements, results equal up to fp32 summation order;
 * it always runs the 256 x 256 tile kernel). Errors as mxfp4_gemm. */
int mxfp4_shuffle_b_sizes(int64_t N, int64_t K, int64_t* code_bytes, int64_t* scale_bytes);
int mxfp4_shuffle_b(const void* codes, const void* scales, int64_t N, int64_t K, void* codes_sh,
                    void* scales_sh, void* stream);
int mxfp4_gemm_bshuffled(const void* A_codes, const void* A_scales, const void* Bsh_codes,
                         const void* Bsh_scales, int64_t M, int64_t N, int64_t K, int out_dtype,
                         void* C, void* stream);

/* Gate+up GEMM of a SwiGLU MLP with the activation fused into its epilogue
 * and requantized to MXFP4 for the down projection. B holds the stacked
 * weight [W_gate; W_up]: rows 0 .. N/2 - 1 are W_gate, rows N/2 .. N - 1
 * W_up (Nh = N/2 activation columns). With g = A W_gate^T and u = A W_up^T
 * (the sums of mxfp4_gemm, fp32), the kernel computes
 *   act[m, j] = silu(g[m, j]) * u[m, j],  silu(z) = z / (1 + exp(-z))
 * (SwiGLU: Shazeer, "GLU Variants Improve Transformer", 2020) in fp32,
 * rounds act to BF16 (nearest even) and quantizes it exactly as
 * mxfp4_quantize does, blocks of 32 along j. The MXFP4 GEMM of "Integrate
 * MXFP4 hipblaslt GEMM support" (#697, Changes list) has no activation
 * epilogue; this entry point widens it. C [M, N] is never written.
 * A_codes [M, K/2], B_codes [N, K/2]: 16-byte aligned
 * A_scales [M, K/32], B_scales [N, K/32]: 4-byte aligned
 * act_codes [M, Nh/2] uint8, 16-byte aligned; act_scales [M, Nh/32] uint8
 * act_bf16 [M, Nh] BF16, 16-byte aligned, or NULL to skip writing it
 * Requires K % 256 == 0, M % 32 == 0, N % 256 == 0 (the kernel's tiles
 * cover 128 activation columns and never straddle the gate/up boundary),
 * M, N, K > 0, K <= 2^24,
 * N * K / 2 < 2^31 (B's codes under 2 GiB), M * N < 2^40; otherwise
 * MXFP4_EINVAL (MXFP4_EALIGN for alignment) and nothing is launched. */
int mxfp4_gemm_swiglu(const void* A_codes, const void* A_scales, const void* B_codes,
                      const void* B_scales, int64_t M, int64_t N, int64_t K, void* act_codes,
                      void* act_scales, void* act_bf16, void* stream);

/* Fragment order: an MXFP4 operand re-arranged so that a GEMM keeping its
 * operands in registers loads each block-scaled MFMA operand as one
 * contiguous 1 KiB run (the pre-arranged operands of the a4w4 path on
 * "Integrate MXFP4 hipblaslt GEMM support", #697, Changes list, and
 * "Initial integration of a4w4 GEMM", #663; the pages give no layout, this
 * one is the library's own). For X [R, K] (R % 32 == 0, K % 256 == 0), with
 * tile t = row / 32, r = row % 32, step s = k / 256, KS = K / 256, and block
 * j = 4 h + q (h < 2, q < 4) of the 8 32-element blocks of the row's step,
 * lane l = r + 32 h:
 *   codes  [R * K / 2] bytes: the 16 code bytes of that block at
 *          (t KS + s) * 4096 + 1024 q + 16 l
 *   scales [R * K / 32] bytes: its scale at (t KS + s) * 256 + 4 l + q
 * (same sizes as the plain layout; a permutation of its bytes).
 *
 * mxfp4_quantize_frag: mxfp4_quantize with the outputs in fragment order.
 *   x_bf16 [M, K] row-major BF16 (16-byte aligned); codes_frag 16-byte
 *   aligned. Requires M >= 32, M % 32 == 0, K % 256 == 0, K <= 2^24,
 *   M * K < 2^40.
 * mxfp4_to_frag: plain codes [R, K/2] (16-byte aligned) and scales [R, K/32]
 *   (4-byte aligned) -> fragment order (same alignments). Requires R >= 32,
 *   R % 32 == 0, K % 256 == 0, K <= 2^24, R * K / 2 < 2^40.
 * mxfp4_gemm_frag: mxfp4_gemm with both operands in fragment order (codes
 *   16-byte, scales 4-byte aligned; C as mxfp4_gemm). Built for few rows of
 *   A (decode shapes): each workgroup takes one 32-row tile of B and up to
 *   three 32-row tiles of A, the K steps split between its 8 waves and
 *   summed in a fixed order; every 32 x 32 tile of C gets exactly the
 *   arithmetic of mxfp4_gemm's M <= 128 kernel, so for M <= 128 the two
 *   return identical bits. Requires M % 32 == 0, M <= 6291360 (at most
 *   65535 groups of three tiles), N % 32 == 0, K % 256 == 0, K <= 2^24,
 *   each buffer < 2^40 bytes. May enqueue two kernels.
 * All three: asynchronous on `stream`; errors as mxfp4_gemm. */
int mxfp4_quantize_frag(const void* x_bf16, int64_t M, int64_t K, void* codes_frag,
                        void* scales_frag, void* stream);
int mxfp4_to_frag(const void* codes, const void* scales, int64_t R, int64_t K, void* codes_frag,
                  void* scales_frag, void* stream);
int mxfp4_gemm_frag(const void* A_frag, const void* A_scales_frag, const void* B_frag,
                    const void* B_scales_frag, int64_t M, int64_t N, int64_t K, int out_dtype,
                    void* C, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
