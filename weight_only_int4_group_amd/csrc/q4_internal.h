// Kernel launchers behind the C ABI.  Arguments are already validated by q4_abi.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

// colscale (optional, fp32 [K], 16-byte aligned): quantize bf16(fl32(W[n, k] * colscale[k])).
hipError_t launch_quantize(const void* W, int64_t N, int64_t K, int g, bool sym, void* packed,
                           void* scales, void* zeros, int num_cus, hipStream_t stream,
                           const float* colscale = nullptr);

// Standalone dequantisation of the packed codes to bf16 (or fp16 when f16_out) [N, K].
hipError_t launch_dequantize(const void* packed, const void* scales, const void* zeros, int64_t N,
                             int64_t K, int g, bool sym, void* out, bool f16_out, int num_cus,
                             hipStream_t stream);

// AWQ-style scaling (awq.hip).  Workspace layout of q4_awq_search: byte offsets of each
// buffer (256-byte aligned) and the total.
struct AwqLayout {
  uint64_t partial, absmean, scales_all, packed, qscales, qzeros, xs, y, err_partial, bytes;
};
AwqLayout awq_layout(int64_t M, int64_t N, int64_t K, int g, int n_alpha);
// a[k] = mean_m |X[m, k]| (fp32), via partial sums in `partial` (64 K floats).
hipError_t launch_absmean(const void* X, int64_t M, int64_t K, void* partial, void* a, hipStream_t stream);
// s_all[i][k] for alpha_i = i / (n_alpha - 1).
hipError_t launch_awq_scales(const void* a, int64_t K, int n_alpha, void* s_all, hipStream_t stream);
// out = bf16(fl32(A * s)) or bf16(fl32(A / s)) per column; cols % 8 == 0.
hipError_t launch_scale_columns(const void* A, int64_t rows, int64_t cols, const void* s, bool divide,
                                void* out, int num_cus, hipStream_t stream);
// *err (fp64) = sum over n bf16 elements of (Yq - Yref)^2.
hipError_t launch_sq_err(const void* Yq, const void* Yref, int64_t n, void* partial, void* err,
                         hipStream_t stream);
// *best = first index of the smallest err; s_out = s_all[best].
hipError_t launch_awq_select(const void* err, int n_alpha, const void* s_all, int64_t K, void* best,
                             void* s_out, hipStream_t stream);

// W8A16: 8-bit group-wise RTN (codes uint8 [N, K], one byte per code) and its matmul.
hipError_t launch_quantize8(const void* W, int64_t N, int64_t K, int g, bool sym, void* codes,
                            void* scales, void* zeros, int num_cus, hipStream_t stream);
// GPTQ (group parameters fixed up front, Cholesky of the reversed Hessian, blocked
// error-feedback sweep).  Workspace layout: R [K, K] fp32, then the accumulated feedback
// [N, K] fp32 (a column's residual replaces its feedback once the column is quantized), then
// the factored 32 x 32 diagonal blocks [K / 32, 32, 32] fp32, each 256-byte aligned.
constexpr int64_t kGptqMaxK = 32768;
struct GptqLayout {
  int64_t R, acc, Ld, bytes;
};
GptqLayout gptq_layout(int64_t N, int64_t K);
hipError_t launch_gptq(const void* X, int64_t M, const void* W, int64_t N, int64_t K, int g, bool sym, float damp,
                       void* workspace, void* packed, void* scales, void* zeros, int* info, int num_cus,
                       hipStream_t stream);
// GEMV for M <= kGemv8MaxM with X staged in LDS as scaled fp16 (gemv8_fits: 2.25 M K bytes fit).
constexpr int64_t kGemv8MaxM = 4;
bool gemv8_fits(int64_t M, int64_t K);
hipError_t launch_gemv8(const void* X, int M, int64_t N, int64_t K, int g, bool sym, const void* codes,
                        const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream);
// MFMA GEMM for any M with 8-bit codes (the general GEMM's tiling).
hipError_t launch_gemm8(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                        const void* codes, const void* scales, const void* zeros, void* Y,
                        int num_cus, hipStream_t stream);

// Decode GEMV: M == 1 with K <= kGemvMaxK, or M == 2 with K <= kGemvMaxK2 (the lane's slice
// of X stays in registers).
constexpr int64_t kGemvMaxK = 16384;
constexpr int64_t kGemvMaxK2 = 4096;
hipError_t launch_gemv(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                       const void* packed, const void* scales, const void* zeros, void* Y,
                       int num_cus, hipStream_t stream);

// Decode on the matrix cores for 1 <= M <= 16: g in {32, 64, 128}; K a whole number of the
// waves' K ranges (512 k at 9 <= M <= 16, 1024 at M <= 8, 2048 at M <= 4, shorter ranges
// when K is small), at most 16 ranges.
bool decode_fits(int64_t M, int64_t N, int64_t K, int g);
hipError_t launch_decode(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                         const void* packed, const void* scales, const void* zeros, void* Y,
                         int num_cus, hipStream_t stream);

// GEMM with X staged in LDS and W dequantised in registers: any M >= kPrefillMinM (rows of a
// tile past M are clamped), K a multiple of 128, g a power of two; bits = 4 (W4A16) or 8
// (W8A16, launch_prefill8).  Below 512 rows it is still 2-3x faster than the general GEMM on
// every shape measured (M = 32 ... 384, N = 4096 ... 28672).
constexpr int64_t kPrefillMinM = 1;
bool prefill_fits(int64_t M, int64_t N, int64_t K, int g, int bits = 4);
hipError_t launch_prefill(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                          const void* packed, const void* scales, const void* zeros, void* Y, int num_cus,
                          hipStream_t stream);
hipError_t launch_prefill8(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                           const void* codes, const void* scales, const void* zeros, void* Y,
                           int num_cus, hipStream_t stream);

// MFMA GEMM for any M >= 1.
hipError_t launch_gemm(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                       const void* packed, const void* scales, const void* zeros, void* Y,
                       int num_cus, hipStream_t stream);

}  // namespace q4
