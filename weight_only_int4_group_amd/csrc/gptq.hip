// GPTQ quantization on the GPU (gfx950), in the library's INT4 group format.
//
// Method ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
// "GPTQ vs AWQ: two ways to choose what error to keep"; "Model Quantization" §2.1 "GPTQ"; "DL S067 ·
// Quantization" §4 "GPTQ intuition"): H = X^T X over calibration rows, dampened on the
// diagonal by damp * mean(diag H); the columns of each weight row are quantized in order and
// each column's rounding error is pushed onto the columns not yet quantized through the
// inverse Hessian.  As in the pages' toy, every group's scale and zero-point are fixed up
// front (RTN's, from the original weights), so GPTQ chooses codes only.
//
// Formulation.  With H = Ut Ut^T, Ut upper triangular (the Cholesky factorisation of H taken
// from the last column backwards), the sequential update is equivalent to error feedback from
// the ORIGINAL weights:
//     w'_i = w_i + sum_{j<i} (w_j - x_hat_j) Ut[j, i] / Ut[i, i],   q_i = code(w'_i),
// because the pages' update coefficient [H_i^-1]_{i, j} / [H_i^-1]_{i, i} (H_i^-1 the inverse
// downdated to columns >= i) equals the corresponding entry of Ut^-1 divided by its diagonal,
// and W - X_hat = E Ut^-1 for the scaled errors E.  No inverse is formed: one Cholesky
// factorisation and one sweep.  Ut is obtained as the ordinary lower Cholesky factor L of the
// index-reversed Hessian R = J H J (R[a][b] = H[K-1-a][K-1-b]): Ut[i][j] = L[K-1-i][K-1-j].
//
// Kernels (all fp32, fixed summation order, no atomics):
//   * gemm_f32_kernel: C = alpha A B + beta C on 64 x 64 tiles of the fp32 matrix cores with
//     arbitrary (signed) strides; it forms R from X with the columns read in reverse, the
//     Cholesky's updates (inside an outer block of kOuter columns, then the trailing matrix
//     with inner dimension kOuter, lower tiles only) and the sweep's feedback updates (inside an
//     outer block after every 32 columns, then all later columns once per outer block);
//   * damp_kernel: one block; mean of the diagonal in a fixed order, then the dampening;
//   * panel_kernel: a 32-column panel, the 32 x 32 diagonal block (one lane per row, in
//     registers, in every workgroup) and the rows below it (one thread per row);
//   * diag_store_kernel: the factored diagonal blocks into R once the panels are done;
//   * colscale_kernel: L[a][b] / L[b][b] below the diagonal (the update coefficients);
//   * sweep_block_kernel: one thread per weight row runs 32 columns in order (error feedback
//     inside the step from LDS, earlier columns through the accumulated updates), writes the
//     16 packed bytes and puts the step's residuals w_j - x_hat_j in place of the feedback it
//     has consumed.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kTile = 64;          // GEMM output tile
constexpr int kStep = 16;          // GEMM inner step
constexpr int kB = 32;             // Cholesky panel and sweep step (K % 32 == 0)
constexpr int kOuter = 256;        // columns per outer block: the width of the big updates
constexpr int kSweepThreads = 256; // weight rows per sweep workgroup (one thread per row)

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);       // bf16 -> fp32, exact
}

// C[m * ldc + n] = alpha * sum_k A(m, k) B(k, n) + beta * C, A(m, k) = A[m sam + k sak],
// B(k, n) = B[k sbk + n sbn], on the fp32 matrix cores (each product exact, fp32 sums).
// tri: only tiles with tile row >= tile column (lower part).  beta == 0 writes C without
// reading it.  PREC loads C before the k loop instead of after it, so that for a short inner
// dimension its latency overlaps the operand loads (it holds 16 more registers per thread).
template <typename TA, typename TB, bool PREC>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const TA* __restrict__ A, int64_t sam, int64_t sak,
                                                       const TB* __restrict__ B, int64_t sbk, int64_t sbn,
                                                       float* __restrict__ C, int64_t ldc, int M, int N, int Kd,
                                                       float alpha, float beta, int tri) {
  const int bm = blockIdx.y, bn = blockIdx.x;
  if (tri && bn > bm) return;
  __shared__ float As[kStep][kTile + 4];
  __shared__ float Bs[kStep][kTile + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;      // the wave's 32 x 32 quarter
  const int m0 = bm * kTile, n0 = bn * kTile;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float cpre[2][2][4];
  if constexpr (PREC) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn + 16 * j + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
          cpre[i][j][r] = (beta != 0.0f && m < M && n < N) ? C[(int64_t)m * ldc + n] : 0.0f;
        }
      }
  }
  // Register prefetch: the global values of step k0 + kStep are loaded while step k0 is
  // multiplied from LDS, so their latency overlaps the matrix instructions.
  float pa[4], pb[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;                 // 1024 = 64 x 16 elements of each operand
      const int am = idx >> 4, ak = idx & 15;        // A: row-major over (m, k)
      const int m = m0 + am, k = k0 + ak;
      pa[e] = (m < M && k < Kd) ? ld_f32(A, (int64_t)m * sam + (int64_t)k * sak) : 0.0f;
      const int bk = idx >> 6, bnn = idx & 63;       // B: row-major over (k, n)
      const int kk = k0 + bk, n = n0 + bnn;
      pb[e] = (kk < Kd && n < N) ? ld_f32(B, (int64_t)kk * sbk + (int64_t)n * sbn) : 0.0f;
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < Kd; k0 += kStep) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;
      As[idx & 15][idx >> 4] = pa[e];
      Bs[idx >> 6][idx & 63] = pb[e];
    }
    __syncthreads();
    if (k0 + kStep < Kd) fetch(k0 + kStep);
    // v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] of a
    // 16 x 4 by 4 x 16 step; the 16 x 16 result sits in lane l as rows 4 (l / 16) + r, column l % 16
#pragma unroll
    for (int k4 = 0; k4 < kStep; k4 += 4) {
      const int kr = k4 + (lane >> 4);
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = As[kr][wm + 16 * i + (lane & 15)];
        b[i] = Bs[kr][wn + 16 * i + (lane & 15)];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
        if (m >= M || n >= N) continue;
        float* c = C + (int64_t)m * ldc + n;
        if (beta == 0.0f)
          *c = alpha * acc[i][j][r];
        else
          *c = __builtin_fmaf(alpha, acc[i][j][r], beta * (PREC ? cpre[i][j][r] : *c));
      }
    }
}

__global__ void zero_info_kernel(int* __restrict__ info) {
  if (threadIdx.x == 0) info[0] = 0;
}

// Dampening: mean of diag(R) summed in a fixed order (per-thread strided partials, then a
// fixed tree), R[a][a] += damp * mean; an all-zero R (no calibration information) becomes I.
__global__ __launch_bounds__(1024) void damp_kernel(float* __restrict__ R, int K, float damp) {
  __shared__ float part[1024];
  float s = 0.0f;
  for (int a = threadIdx.x; a < K; a += 1024) s += R[(int64_t)a * K + a];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const float mean = part[0] / (float)K;
  for (int a = threadIdx.x; a < K; a += 1024) {
    float* d = R + (int64_t)a * K + a;
    *d = mean == 0.0f ? 1.0f : *d + damp * mean;
  }
}

// One 32-column panel of the Cholesky factorisation at column k0.
//  * The diagonal block: wave 0 of every workgroup factors the 32 x 32 block at (k0, k0) from
//    R, which no thread writes during this launch.  Lane i holds row i in registers; the
//    column loop is unrolled, so every pivot and every l_kj is a lane read with a constant
//    index.  Workgroup 0 stores the factor to Ld[k0 * 32 ...] (row-major 32 x 32; it reaches
//    R's diagonal block through diag_store_kernel once the factorisation is done) and records
//    a non-positive pivot as info = column + 1 (first failure only).  Such a pivot is replaced
//    by 1e-30 so the factorisation completes.
//  * The rows below: one thread per row r >= k0 + 32 solves L[r, k0:k0+32] = R[r, k0:k0+32]
//    L_kk^-T by forward substitution, multiplying by the reciprocals of the diagonal (taken
//    once per workgroup) so no division sits on the chain.  The row is loaded before the
//    factorisation so its latency overlaps that work.
__global__ __launch_bounds__(256) void panel_kernel(float* __restrict__ R, int K, int k0, float* __restrict__ Ld,
                                                    int* __restrict__ info) {
  __shared__ float l[kB][kB + 1];
  __shared__ float linv[kB];
  const int64_t r = (int64_t)k0 + kB + (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool has_row = r < K;
  float x[kB];
  if (has_row) {
    const float4* rp = reinterpret_cast<const float4*>(R + r * K + k0);
#pragma unroll
    for (int v = 0; v < kB / 4; ++v) {
      const float4 t = rp[v];
      x[4 * v] = t.x;
      x[4 * v + 1] = t.y;
      x[4 * v + 2] = t.z;
      x[4 * v + 3] = t.w;
    }
  }
  if (threadIdx.x < 64) {
    const int i = threadIdx.x & 31;
    const bool own = threadIdx.x < kB;
    const float* row = R + (int64_t)(k0 + i) * K + k0;
    float a[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) a[j] = (own && j <= i) ? row[j] : 0.0f;
    int bad = 0;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[j]), j));
      if (!(d > 0.0f)) {
        if (bad == 0) bad = j + 1;
        d = 1e-30f;
      }
      d = sqrtf(d);
      a[j] = i == j ? d : (i > j ? a[j] / d : a[j]);
#pragma unroll
      for (int k = j + 1; k < kB; ++k) {     // entries above the diagonal (k > i) are never used
        const float lkj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[j]), k));
        a[k] = __builtin_fmaf(-a[j], lkj, a[k]);
      }
    }
    if (own) {
#pragma unroll
      for (int j = 0; j < kB; ++j) l[i][j] = j <= i ? a[j] : 0.0f;
      linv[i] = 1.0f / a[i];
    }
    if (blockIdx.x == 0) {
      if (own) {
        float4* lp = reinterpret_cast<float4*>(Ld + (int64_t)k0 * kB + i * kB);
#pragma unroll
        for (int v = 0; v < kB / 4; ++v)
          lp[v] = float4{4 * v <= i ? a[4 * v] : 0.0f, 4 * v + 1 <= i ? a[4 * v + 1] : 0.0f,
                         4 * v + 2 <= i ? a[4 * v + 2] : 0.0f, 4 * v + 3 <= i ? a[4 * v + 3] : 0.0f};
      }
      if (bad != 0 && threadIdx.x == 0 && info[0] == 0) info[0] = k0 + bad;
    }
  }
  __syncthreads();
  if (!has_row) return;
#pragma unroll
  for (int j = 0; j < kB; ++j) {
    float v = x[j];
#pragma unroll
    for (int t = 0; t < j; ++t) v = __builtin_fmaf(-x[t], l[j][t], v);
    x[j] = v * linv[j];
  }
  float4* wp = reinterpret_cast<float4*>(R + r * K + k0);
#pragma unroll
  for (int v = 0; v < kB / 4; ++v) wp[v] = float4{x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
}

// The factored diagonal blocks from Ld into R's diagonal blocks (lower part), one workgroup
// per block.
__global__ __launch_bounds__(256) void diag_store_kernel(float* __restrict__ R, int K, const float* __restrict__ Ld) {
  const int64_t b0 = (int64_t)blockIdx.x * kB;
  for (int e = threadIdx.x; e < kB * kB; e += 256) {
    const int i = e / kB, j = e % kB;
    if (j <= i) R[(b0 + i) * K + b0 + j] = Ld[b0 * kB + e];
  }
}

// L[a][b] / L[b][b] for a > b: the error-feedback coefficients (in reversed indices).
__global__ __launch_bounds__(256) void colscale_kernel(float* __restrict__ R, int K) {
  const int64_t a = blockIdx.y;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < a; b += (int64_t)gridDim.x * 256)
    R[a * K + b] /= R[b * K + b];
}

// One step of 32 columns [i1, i1 + 32) for every weight row (one thread per row).  The step
// lies inside one group.  Cb[j][i] = Ut[i1 + j][i1 + i] / Ut[i1 + i][i1 + i] for j < i.
// acc[n][i1 .. i1 + 31] holds the feedback of the earlier columns (not read when i1 == 0); the
// thread reads it, then overwrites the same 32 floats with the residuals w_j - x_hat_j, which
// the later feedback updates read from there.  Also writes the step's 16 packed bytes.
template <bool SYM>
__global__ __launch_bounds__(kSweepThreads) void sweep_block_kernel(const uint16_t* __restrict__ W, int64_t N, int K, int g,
                                                          const float* __restrict__ Lc, float* __restrict__ acc,
                                                          int i1, const uint16_t* __restrict__ scales,
                                                          const uint8_t* __restrict__ zeros,
                                                          uint8_t* __restrict__ packed) {
  __shared__ float Cb[kB][kB + 1];
  for (int e = threadIdx.x; e < kB * kB; e += kSweepThreads) {
    const int j = e / kB, i = e % kB;
    Cb[j][i] = j < i ? Lc[(int64_t)(K - 1 - i1 - j) * K + (K - 1 - i1 - i)] : 0.0f;
  }
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * kSweepThreads + threadIdx.x;
  if (n >= N) return;
  const int G = K / g;
  const int grp = i1 / g;
  const float s = (float)__builtin_bit_cast(_Float16, scales[n * G + grp]);
  const float zf = SYM ? 0.0f : (float)zeros[n * G + grp];
  constexpr float qlo = SYM ? -8.0f : 0.0f, qhi = SYM ? 7.0f : 15.0f;

  const u32x4* wp = reinterpret_cast<const u32x4*>(W + n * (int64_t)K + i1);
  float w[kB], f[kB], d[kB];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const u32x4 p = wp[v];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      w[8 * v + 2 * t] = bf16_lo(p[t]);
      w[8 * v + 2 * t + 1] = bf16_hi(p[t]);
    }
  }
  if (i1 > 0) {
    const float4* ap = reinterpret_cast<const float4*>(acc + n * (int64_t)K + i1);
#pragma unroll
    for (int v = 0; v < kB / 4; ++v) {
      const float4 a4 = ap[v];
      f[4 * v] = a4.x;
      f[4 * v + 1] = a4.y;
      f[4 * v + 2] = a4.z;
      f[4 * v + 3] = a4.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kB; ++i) f[i] = 0.0f;
  }
  uint32_t nib[kB / 8] = {};
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    float v = w[i] + f[i];
#pragma unroll
    for (int j = 0; j < i; ++j) v = __builtin_fmaf(d[j], Cb[j][i], v);
    const float c = fminf(fmaxf(rintf(v / s) + zf, qlo), qhi);       // IEEE quotient, as RTN
    d[i] = w[i] - s * (c - zf);
    nib[i / 8] |= ((uint32_t)(int)c & 0xFu) << (4 * (i % 8));
  }
  *reinterpret_cast<u32x4*>(packed + n * (int64_t)(K / 2) + i1 / 2) = u32x4{nib[0], nib[1], nib[2], nib[3]};
  float4* dp = reinterpret_cast<float4*>(acc + n * (int64_t)K + i1);
#pragma unroll
  for (int v = 0; v < kB / 4; ++v) dp[v] = float4{d[4 * v], d[4 * v + 1], d[4 * v + 2], d[4 * v + 3]};
}

template <typename TA, typename TB>
hipError_t gemm(const TA* A, int64_t sam, int64_t sak, const TB* B, int64_t sbk, int64_t sbn, float* C,
                int64_t ldc, int M, int N, int Kd, float alpha, float beta, bool tri, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const dim3 grid((unsigned)((N + kTile - 1) / kTile), (unsigned)((M + kTile - 1) / kTile));
  if (beta != 0.0f && Kd <= 2 * kStep)
    hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, true>), grid, dim3(256), 0, stream, A, sam, sak, B, sbk, sbn, C, ldc, M,
                       N, Kd, alpha, beta, tri ? 1 : 0);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, false>), grid, dim3(256), 0, stream, A, sam, sak, B, sbk, sbn, C, ldc,
                       M, N, Kd, alpha, beta, tri ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

GptqLayout gptq_layout(int64_t N, int64_t K) {
  GptqLayout L;
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  L.R = 0;
  L.acc = up(L.R + 4 * K * K);
  L.Ld = up(L.acc + 4 * N * K);
  L.bytes = up(L.Ld + 4 * K * kB);
  return L;
}

hipError_t launch_gptq(const void* X, int64_t M, const void* W, int64_t N, int64_t K, int g, bool sym, float damp,
                       void* workspace, void* packed, void* scales, void* zeros, int* info, int num_cus,
                       hipStream_t stream) {
  const GptqLayout L = gptq_layout(N, K);
  char* base = static_cast<char*>(workspace);
  float* R = reinterpret_cast<float*>(base + L.R);
  float* acc = reinterpret_cast<float*>(base + L.acc);
  float* Ld = reinterpret_cast<float*>(base + L.Ld);
  const int Ki = (int)K;
  const uint16_t* Xh = static_cast<const uint16_t*>(X);

  // 1. group parameters fixed up front: RTN of the original weights (its codes are replaced)
  hipError_t e = launch_quantize(W, N, K, g, sym, packed, scales, zeros, num_cus, stream);
  if (e != hipSuccess) return e;
  // 2. R = J X^T X J (columns of X read backwards), lower tiles; then the dampening
  hipLaunchKernelGGL(zero_info_kernel, dim3(1), dim3(64), 0, stream, info);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // R[a][b] = sum_t X[t][K-1-a] X[t][K-1-b]: A(a, t) and B(t, b) read the bf16 rows backwards
  const uint16_t* Xr = Xh + (K - 1);
  e = gemm<uint16_t, uint16_t>(Xr, -1, K, Xr, K, -1, R, K, Ki, Ki, (int)M, 1.0f, 0.0f, true, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(1024), 0, stream, R, Ki, damp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. blocked lower Cholesky of R, in place.  Outer blocks of kOuter columns [o1, o2): 32-column
  //    panels (diagonal block, the rows below, the update of the outer block's remaining
  //    columns), then one update of the trailing matrix with inner dimension o2 - o1.
  for (int o1 = 0; o1 < Ki; o1 += kOuter) {
    const int o2 = o1 + kOuter < Ki ? o1 + kOuter : Ki;
    for (int k0 = o1; k0 < o2; k0 += kB) {
      const int rest = Ki - k0 - kB;
      hipLaunchKernelGGL(panel_kernel, dim3(rest > 0 ? (unsigned)((rest + 255) / 256) : 1u), dim3(256), 0, stream, R,
                         Ki, k0, Ld, info);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (rest <= 0) continue;
      const int cols = o2 - k0 - kB;                       // the outer block's columns still to factor
      if (cols > 0) {
        float* P = R + (int64_t)(k0 + kB) * K + k0;        // the panel, rest x 32
        e = gemm<float, float>(P, K, 1, P, 1, K, R + (int64_t)(k0 + kB) * K + (k0 + kB), K, rest, cols, kB, -1.0f,
                               1.0f, false, stream);
        if (e != hipSuccess) return e;
      }
    }
    const int rest = Ki - o2;
    if (rest > 0) {
      float* P = R + (int64_t)o2 * K + o1;                 // rest x (o2 - o1)
      e = gemm<float, float>(P, K, 1, P, 1, K, R + (int64_t)o2 * K + o2, K, rest, rest, o2 - o1, -1.0f, 1.0f, true,
                             stream);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(diag_store_kernel, dim3((unsigned)(K / kB)), dim3(256), 0, stream, R, Ki, Ld);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colscale_kernel, dim3((unsigned)((K + 255) / 256 < 64 ? (K + 255) / 256 : 64), (unsigned)K),
                     dim3(256), 0, stream, R, Ki);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 4. the sweep: outer blocks of kOuter columns [s1, s2), 32 columns per step.  After a step
  //    its residuals feed the outer block's later columns (a small update); after the outer
  //    block its residuals feed every later column (one update with inner dimension s2 - s1).
  //    acc[:, i] = sum over earlier columns j of D_j C[j][i], C[j][i] = Lc[K-1-j][K-1-i], where
  //    the residuals D_j sit in acc[:, j] once column j is quantized; the first update to reach
  //    a column writes it (beta = 0), later ones add.  The updates read residual columns
  //    [s1, s2) and write columns >= s2 (or the step's later columns), never the same ones.
  const unsigned rows_grid = (unsigned)((N + kSweepThreads - 1) / kSweepThreads);
  auto coef = [&](int j0, int i0) { return R + (int64_t)(Ki - 1 - j0) * K + (Ki - 1 - i0); };
  for (int s1 = 0; s1 < Ki; s1 += kOuter) {
    const int s2 = s1 + kOuter < Ki ? s1 + kOuter : Ki;
    for (int i1 = s1; i1 < s2; i1 += kB) {
      if (sym)
        hipLaunchKernelGGL(sweep_block_kernel<true>, dim3(rows_grid), dim3(kSweepThreads), 0, stream,
                           static_cast<const uint16_t*>(W), N, Ki, g, R, acc, i1,
                           static_cast<const uint16_t*>(scales), static_cast<const uint8_t*>(zeros),
                           static_cast<uint8_t*>(packed));
      else
        hipLaunchKernelGGL(sweep_block_kernel<false>, dim3(rows_grid), dim3(kSweepThreads), 0, stream,
                           static_cast<const uint16_t*>(W), N, Ki, g, R, acc, i1,
                           static_cast<const uint16_t*>(scales), static_cast<const uint8_t*>(zeros),
                           static_cast<uint8_t*>(packed));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int i2 = i1 + kB;
      if (i2 < s2) {
        e = gemm<float, float>(acc + i1, K, 1, coef(i1, i2), -K, -1, acc + i2, K, (int)N, s2 - i2, kB, 1.0f,
                               (s1 == 0 && i1 == 0) ? 0.0f : 1.0f, false, stream);
        if (e != hipSuccess) return e;
      }
    }
    if (s2 < Ki) {
      e = gemm<float, float>(acc + s1, K, 1, coef(s1, s2), -K, -1, acc + s2, K, (int)N, Ki - s2, s2 - s1, 1.0f,
                             s1 == 0 ? 0.0f : 1.0f, false, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace q4
