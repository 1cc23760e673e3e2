// C ABI of libmxfp4.so (declared in include/mxfp4.h).
//
// Every entry point validates all of its arguments before enqueuing
// anything, checks once per device that the device is gfx950, and maps HIP
// launch errors to MXFP4_ELAUNCH. The return-code scheme (0 = ok, distinct
// negative codes, an availability probe) follows the review of the stub
// library on "Initial integration of a4w4 GEMM" (ROCm/TransformerEngine
// #663); the per-call checks are the capability gates of the hipBLASLt MXFP4
// path on "Integrate MXFP4 hipblaslt GEMM support" (#697, Changes list); the
// arch check that never falls back to a default follows "feat(ck-tile):
// aquant GEMM TE to dispatcher bridge" (rocm-libraries #9980, summary).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/mxfp4.h"
#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxDim = 2147483647;      // 2^31 - 1
constexpr int64_t kMaxGemmN = 1LL << 28;     // C: the tile epilogue's store resource spans <= 2^31 bytes
constexpr int64_t kMaxBytes = int64_t(1) << 40;
constexpr int64_t kMaxGemmK = int64_t(1) << 24;  // per-lane row offsets of the GEMM kernels are 32-bit
constexpr int64_t kMaxSwigluB = int64_t(1) << 31;

// Per-device state: 0 = not checked yet, 1 = gfx950 and ready, -1 = not usable.
std::atomic<int> g_device_state[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MXFP4_EUNSUPPORTED;
  }
  int state = g_device_state[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    state = -1;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
        strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
        (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':') &&
        mxfp4::init_kernels_for_current_device() == hipSuccess)
      state = 1;
    (void)hipGetLastError();
    g_device_state[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? MXFP4_OK : MXFP4_EUNSUPPORTED;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b * c < kMaxBytes for non-negative factors, without overflowing: a
// product past int64 counts as too large.
bool below_max_bytes(int64_t a, int64_t b, int64_t c = 1) {
  int64_t ab = 0, abc = 0;
  if (__builtin_mul_overflow(a, b, &ab) || __builtin_mul_overflow(ab, c, &abc)) return false;
  return abc < kMaxBytes;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ELAUNCH; }

// Argument checks shared by mxfp4_gemm and mxfp4_gemm_tile (everything but
// the device).
int check_gemm_args(const void* A_codes, const void* A_scales, const void* B_codes,
                    const void* B_scales, int64_t M, int64_t N, int64_t K, int out_dtype,
                    const void* C) {
  if (!A_codes || !A_scales || !B_codes || !B_scales || !C) return MXFP4_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return MXFP4_EINVAL;
  if (K % 256 != 0 || M % 32 != 0 || N % 32 != 0 || K > kMaxGemmK) return MXFP4_EINVAL;
  if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_FP32) return MXFP4_EINVAL;
  if (N > kMaxGemmN) return MXFP4_EINVAL;
  const int64_t out_bytes = out_dtype == MXFP4_OUT_FP32 ? 4 : 2;
  if (!below_max_bytes(M, K / 2) || !below_max_bytes(N, K / 2) ||
      !below_max_bytes(M, N, out_bytes))
    return MXFP4_EINVAL;
  if (!aligned(A_codes, 16) || !aligned(B_codes, 16) || !aligned(A_scales, 4) ||
      !aligned(B_scales, 4) || !aligned(C, 16))
    return MXFP4_EALIGN;
  return MXFP4_OK;
}

// mxfp4_gemm's kernel: the split-K kernel for M <= kSkinnyMaxM and for
// problems whose 256 x 256 tiles would fill at most an eighth of the
// persistent grid (32 tiles on 256 CUs), where one tile per CU leaves most of
// the chip idle (measured on MI355X: 256^3 9.4 -> 2.8 us, 512 x 512 x 8192
// 43 -> 7.3 us, 1024^2 x 8192 49 -> 25 us; at 32 tiles the two kernels take
// about as long, at 64 the tile kernel takes half the time).
bool gemm_uses_split_k(int64_t M, int64_t N, int workers) {
  if (M <= mxfp4::kSkinnyMaxM) return true;
  const int64_t tiles = ((M + mxfp4::kGemmTile - 1) / mxfp4::kGemmTile) *
                        ((N + mxfp4::kGemmTile - 1) / mxfp4::kGemmTile);
  return tiles * 8 <= workers;
}

}  // namespace

extern "C" {

int mxfp4_available(void) { return check_device() == MXFP4_OK ? 1 : 0; }

const char* mxfp4_strerror(int rc) {
  switch (rc) {
    case MXFP4_OK:
      return "success";
    case MXFP4_EINVAL:
      return "invalid argument (size, null pointer or out_dtype)";
    case MXFP4_EUNSUPPORTED:
      return "no usable gfx950 device is current";
    case MXFP4_ELAUNCH:
      return "HIP kernel launch failed";
    case MXFP4_EALIGN:
      return "pointer not aligned as required";
    default:
      return "unknown mxfp4 status";
  }
}

int mxfp4_quantize_async(const void* x_bf16, int64_t M, int64_t K, void* codes_out,
                         void* scales_out, void* stream) {
  if (!x_bf16 || !codes_out || !scales_out) return MXFP4_EINVAL;
  if (M < 1 || K < 32 || K % 32 != 0 || M > kMaxDim || K > kMaxDim) return MXFP4_EINVAL;
  if (M * K >= kMaxBytes) return MXFP4_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(codes_out, 4)) return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_quantize(x_bf16, M * (K / 32), codes_out, scales_out,
                                              static_cast<hipStream_t>(stream)));
}

int mxfp4_quantize(const void* x_bf16, int64_t M, int64_t K, void* codes_out, void* scales_out) {
  return mxfp4_quantize_async(x_bf16, M, K, codes_out, scales_out, nullptr);
}

int mxfp4_quantize_2d(const void* x_bf16, int64_t M, int64_t K, void* codes_row,
                      void* scales_row, void* codes_col, void* scales_col, void* stream) {
  if (!x_bf16 || !codes_row || !scales_row || !codes_col || !scales_col) return MXFP4_EINVAL;
  if (M < 32 || K < 32 || M % 32 != 0 || K % 32 != 0 || M > kMaxDim || K > kMaxDim)
    return MXFP4_EINVAL;
  if (M * K >= kMaxBytes) return MXFP4_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(codes_row, 16) || !aligned(codes_col, 16))
    return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_quantize_2d(x_bf16, (int)M, (int)K, codes_row, scales_row,
                                                 codes_col, scales_col,
                                                 static_cast<hipStream_t>(stream)));
}

int mxfp4_quantize_sr_rows(const void* x_bf16, int64_t M, int64_t K, int64_t row0, uint64_t seed,
                           void* codes_out, void* scales_out, void* stream) {
  if (!x_bf16 || !codes_out || !scales_out) return MXFP4_EINVAL;
  if (M < 1 || K < 32 || K % 32 != 0 || M > kMaxDim || K > kMaxDim) return MXFP4_EINVAL;
  if (row0 < 0 || row0 > kMaxDim - M) return MXFP4_EINVAL;
  if (M * K >= kMaxBytes) return MXFP4_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(codes_out, 4)) return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_quantize_sr(x_bf16, M, K, row0, seed, codes_out,
                                                 scales_out, static_cast<hipStream_t>(stream)));
}

int mxfp4_quantize_sr(const void* x_bf16, int64_t M, int64_t K, uint64_t seed, void* codes_out,
                      void* scales_out, void* stream) {
  return mxfp4_quantize_sr_rows(x_bf16, M, K, 0, seed, codes_out, scales_out, stream);
}

int mxfp4_quantize_2d_sr_rows(const void* x_bf16, int64_t M, int64_t K, int64_t row0,
                              uint64_t seed, void* codes_row, void* scales_row, void* codes_col,
                              void* scales_col, void* stream) {
  if (!x_bf16 || !codes_row || !scales_row || !codes_col || !scales_col) return MXFP4_EINVAL;
  if (M < 32 || K < 32 || M % 32 != 0 || K % 32 != 0 || M > kMaxDim || K > kMaxDim)
    return MXFP4_EINVAL;
  if (row0 < 0 || row0 % 32 != 0 || row0 > kMaxDim - M) return MXFP4_EINVAL;
  if (M * K >= kMaxBytes) return MXFP4_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(codes_row, 16) || !aligned(codes_col, 16))
    return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_quantize_2d_sr(x_bf16, (int)M, (int)K, row0, seed,
                                                    codes_row, scales_row, codes_col, scales_col,
                                                    static_cast<hipStream_t>(stream)));
}

int mxfp4_quantize_2d_sr(const void* x_bf16, int64_t M, int64_t K, uint64_t seed,
                         void* codes_row, void* scales_row, void* codes_col, void* scales_col,
                         void* stream) {
  return mxfp4_quantize_2d_sr_rows(x_bf16, M, K, 0, seed, codes_row, scales_row, codes_col,
                                   scales_col, stream);
}

int mxfp4_gemm(const void* A_codes, const void* A_scales, const void* B_codes,
               const void* B_scales, int64_t M, int64_t N, int64_t K, int out_dtype, void* C,
               void* stream) {
  const int rc = check_gemm_args(A_codes, A_scales, B_codes, B_scales, M, N, K, out_dtype, C);
  if (rc != MXFP4_OK) return rc;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  const bool fp32 = out_dtype == MXFP4_OUT_FP32;
  const auto st = static_cast<hipStream_t>(stream);
  int workers = 0;
  if (mxfp4::device_workers(workers) != hipSuccess) return MXFP4_ELAUNCH;
  if (gemm_uses_split_k(M, N, workers))
    return launch_status(mxfp4::launch_gemm_skinny(A_codes, A_scales, B_codes, B_scales, (int)M,
                                                   (int)N, (int)K, fp32, C, st));
  return launch_status(mxfp4::launch_gemm(A_codes, A_scales, B_codes, B_scales, (int)M, (int)N,
                                          (int)K, fp32, C, st));
}

int mxfp4_gemm_tile(const void* A_codes, const void* A_scales, const void* B_codes,
                    const void* B_scales, int64_t M, int64_t N, int64_t K, int out_dtype, void* C,
                    void* stream) {
  const int rc = check_gemm_args(A_codes, A_scales, B_codes, B_scales, M, N, K, out_dtype, C);
  if (rc != MXFP4_OK) return rc;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_gemm(A_codes, A_scales, B_codes, B_scales, (int)M, (int)N,
                                          (int)K, out_dtype == MXFP4_OUT_FP32, C,
                                          static_cast<hipStream_t>(stream)));
}

int mxfp4_shuffle_b_sizes(int64_t N, int64_t K, int64_t* code_bytes, int64_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return MXFP4_EINVAL;
  if (N < 1 || K < 256 || K % 256 != 0 || N > kMaxDim || K > kMaxGemmK) return MXFP4_EINVAL;
  mxfp4::shuffled_b_sizes(N, K, code_bytes, scale_bytes);
  if (*code_bytes >= kMaxBytes) return MXFP4_EINVAL;
  return MXFP4_OK;
}

int mxfp4_shuffle_b(const void* codes, const void* scales, int64_t N, int64_t K, void* codes_sh,
                    void* scales_sh, void* stream) {
  if (!codes || !scales || !codes_sh || !scales_sh) return MXFP4_EINVAL;
  int64_t cb = 0, sb = 0;
  const int rc = mxfp4_shuffle_b_sizes(N, K, &cb, &sb);
  if (rc != MXFP4_OK) return rc;
  if (!aligned(codes, 16) || !aligned(codes_sh, 16) || !aligned(scales, 4) ||
      !aligned(scales_sh, 4))
    return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_shuffle_b(codes, scales, (int)N, (int)K, codes_sh, scales_sh,
                                               static_cast<hipStream_t>(stream)));
}

int mxfp4_gemm_bshuffled(const void* A_codes, const void* A_scales, const void* Bsh_codes,
                         const void* Bsh_scales, int64_t M, int64_t N, int64_t K, int out_dtype,
                         void* C, void* stream) {
  if (!A_codes || !A_scales || !Bsh_codes || !Bsh_scales || !C) return MXFP4_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return MXFP4_EINVAL;
  if (K % 256 != 0 || M % 32 != 0 || N % 32 != 0 || K > kMaxGemmK) return MXFP4_EINVAL;
  if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_FP32) return MXFP4_EINVAL;
  if (N > kMaxGemmN) return MXFP4_EINVAL;
  const int64_t out_bytes = out_dtype == MXFP4_OUT_FP32 ? 4 : 2;
  int64_t cb = 0, sb = 0;
  mxfp4::shuffled_b_sizes(N, K, &cb, &sb);
  if (!below_max_bytes(M, K / 2) || cb >= kMaxBytes || !below_max_bytes(M, N, out_bytes))
    return MXFP4_EINVAL;
  if (!aligned(A_codes, 16) || !aligned(Bsh_codes, 16) || !aligned(A_scales, 4) ||
      !aligned(Bsh_scales, 4) || !aligned(C, 16))
    return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_gemm_bshuffled(A_codes, A_scales, Bsh_codes, Bsh_scales,
                                                    (int)M, (int)N, (int)K,
                                                    out_dtype == MXFP4_OUT_FP32, C,
                                                    static_cast<hipStream_t>(stream)));
}

int mxfp4_gemm_swiglu(const void* A_codes, const void* A_scales, const void* B_codes,
                      const void* B_scales, int64_t M, int64_t N, int64_t K, void* act_codes,
                      void* act_scales, void* act_bf16, void* stream) {
  if (!A_codes || !A_scales || !B_codes || !B_scales || !act_codes || !act_scales)
    return MXFP4_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return MXFP4_EINVAL;
  if (K % 256 != 0 || M % 32 != 0 || N % 256 != 0 || K > kMaxGemmK) return MXFP4_EINVAL;
  // The per-lane code offsets of the up half are 32-bit: B's codes < 2 GiB.
  if (N * (K / 2) >= kMaxSwigluB || !below_max_bytes(M, K / 2) || !below_max_bytes(M, N))
    return MXFP4_EINVAL;
  if (!aligned(A_codes, 16) || !aligned(B_codes, 16) || !aligned(A_scales, 4) ||
      !aligned(B_scales, 4) || !aligned(act_codes, 16) ||
      (act_bf16 != nullptr && !aligned(act_bf16, 16)))
    return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_gemm_swiglu(A_codes, A_scales, B_codes, B_scales, (int)M,
                                                 (int)N, (int)K, act_codes, act_scales, act_bf16,
                                                 static_cast<hipStream_t>(stream)));
}

int mxfp4_quantize_frag(const void* x_bf16, int64_t M, int64_t K, void* codes_frag,
                        void* scales_frag, void* stream) {
  if (!x_bf16 || !codes_frag || !scales_frag) return MXFP4_EINVAL;
  if (M < 32 || K < 256 || M % 32 != 0 || K % 256 != 0 || M > kMaxDim || K > kMaxGemmK)
    return MXFP4_EINVAL;
  if (M * K >= kMaxBytes) return MXFP4_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(codes_frag, 16)) return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_quantize_frag(x_bf16, M, K, codes_frag, scales_frag,
                                                   static_cast<hipStream_t>(stream)));
}

int mxfp4_to_frag(const void* codes, const void* scales, int64_t R, int64_t K, void* codes_frag,
                  void* scales_frag, void* stream) {
  if (!codes || !scales || !codes_frag || !scales_frag) return MXFP4_EINVAL;
  if (R < 32 || K < 256 || R % 32 != 0 || K % 256 != 0 || R > kMaxDim || K > kMaxGemmK)
    return MXFP4_EINVAL;
  if (R * (K / 2) >= kMaxBytes) return MXFP4_EINVAL;
  if (!aligned(codes, 16) || !aligned(codes_frag, 16) || !aligned(scales, 4) ||
      !aligned(scales_frag, 4))
    return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_to_frag(codes, scales, R, K, codes_frag, scales_frag,
                                             static_cast<hipStream_t>(stream)));
}

int mxfp4_gemm_frag(const void* A_frag, const void* A_scales_frag, const void* B_frag,
                    const void* B_scales_frag, int64_t M, int64_t N, int64_t K, int out_dtype,
                    void* C, void* stream) {
  if (!A_frag || !A_scales_frag || !B_frag || !B_scales_frag || !C) return MXFP4_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK)
    return MXFP4_EINVAL;
  if (K % 256 != 0 || M % 32 != 0 || N % 32 != 0) return MXFP4_EINVAL;
  // Workgroup rows hold up to three 32-row tiles of A; the grid's y extent
  // (groups of tiles) is at most 65535.
  if ((M / 32 + 2) / 3 > 65535) return MXFP4_EINVAL;
  if (out_dtype != MXFP4_OUT_BF16 && out_dtype != MXFP4_OUT_FP32) return MXFP4_EINVAL;
  if (N > kMaxGemmN) return MXFP4_EINVAL;
  const int64_t out_bytes = out_dtype == MXFP4_OUT_FP32 ? 4 : 2;
  if (!below_max_bytes(M, K / 2) || !below_max_bytes(N, K / 2) ||
      !below_max_bytes(M, N, out_bytes))
    return MXFP4_EINVAL;
  if (!aligned(A_frag, 16) || !aligned(B_frag, 16) || !aligned(A_scales_frag, 4) ||
      !aligned(B_scales_frag, 4) || !aligned(C, 16))
    return MXFP4_EALIGN;
  const int dev = check_device();
  if (dev != MXFP4_OK) return dev;
  return launch_status(mxfp4::launch_gemm_frag(A_frag, A_scales_frag, B_frag, B_scales_frag,
                                               (int)M, (int)N, (int)K,
                                               out_dtype == MXFP4_OUT_FP32, C,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
