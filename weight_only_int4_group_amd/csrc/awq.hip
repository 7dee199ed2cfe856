// AWQ-style activation-aware scaling before RTN (gfx950): the calibration statistics, the
// scale grid, column scaling of activations, the output-error reduction and the choice of
// the exponent, all on the GPU.
//
// Method ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
// "GPTQ vs AWQ" and its toy; "DL S067 · Quantization", §5 "AWQ intuition"): a per input
// channel activation magnitude a_j = mean |X[m, j]| over calibration rows; for an exponent
// alpha on a grid of [0, 1], s = a^alpha normalised by sqrt(max s * min s); the weights
// W * s are quantized with the plain RTN kernel and 1/s is folded onto the activations; the
// alpha whose layer output on the calibration rows is closest to the unquantized output wins.
// The library's formats (the readings the header states): a_j floored at 2^-20 max a, s in
// fp32, scaled weights bf16(fl32(w * s_j)), scaled activations bf16(fl32(x / s_j)), alpha_i =
// i / (n_alpha - 1), error = sum (Y_alpha - Y_ref)^2, the first smallest error winning.
//
// Every reduction runs in a fixed order (partial sums per fixed slice, then a single pass
// over the slices), so the scales, and hence the quantized weights, are the same on every run.
#include <algorithm>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kAbsSlices = 64;        // row slices of the activation-magnitude reduction
constexpr int kErrBlocks = 1024;      // blocks of the squared-error reduction
constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ---- a_j = mean_m |X[m, j]|: thread t of column block b sums columns 8 (256 b + t) .. + 7
// over the rows of slice y; partial[y][k] -> a[k] = (sum over y in order) / M.
__global__ __launch_bounds__(256) void absmean_partial_kernel(const u32x4* __restrict__ X, int64_t M,
                                                              int64_t c8, int64_t rows_per_slice,
                                                              float* __restrict__ partial) {
  const int64_t cc = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (cc >= c8) return;
  const int64_t m0 = (int64_t)blockIdx.y * rows_per_slice;
  const int64_t m1 = min(m0 + rows_per_slice, M);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t m = m0; m < m1; ++m) {
    const u32x4 v = X[m * c8 + cc];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += fabsf(bf16_lo(v[i]));
      acc[2 * i + 1] += fabsf(bf16_hi(v[i]));
    }
  }
  float* out = partial + (size_t)blockIdx.y * (size_t)(c8 * 8) + 8 * cc;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = acc[i];
}

__global__ __launch_bounds__(256) void absmean_final_kernel(const float* __restrict__ partial, int64_t K,
                                                            int slices, int64_t M, float* __restrict__ a) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  // the slices are independent loads: fetch them eight at a time, add them in slice order
  float sum = 0.0f;
  int y = 0;
  for (; y + 8 <= slices; y += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[(size_t)(y + u) * K + k];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; y < slices; ++y) sum += partial[(size_t)y * K + k];
  a[k] = sum / (float)M;
}

// ---- s_i[k] = 2^(alpha_i (log2 a_k - (log2 max a + log2 min a) / 2)), a_k floored at
// 2^-20 max a: the pages' a^alpha / sqrt(max a^alpha * min a^alpha).  One block.
__global__ __launch_bounds__(1024) void awq_scales_kernel(const float* __restrict__ a, int64_t K,
                                                          int n_alpha, float* __restrict__ s_all) {
  __shared__ float red[1024 / kWave];
  const int tid = threadIdx.x;
  auto block_reduce = [&](float v, bool is_max) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float w = __shfl_xor(v, o);
      v = is_max ? fmaxf(v, w) : fminf(v, w);
    }
    __syncthreads();
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < 1024 / kWave; ++i) r = is_max ? fmaxf(r, red[i]) : fminf(r, red[i]);
    return r;
  };
  float mx = 0.0f;
  for (int64_t k = tid; k < K; k += 1024) mx = fmaxf(mx, a[k]);
  mx = block_reduce(mx, true);
  if (mx == 0.0f) {
    for (int i = 0; i < n_alpha; ++i)
      for (int64_t k = tid; k < K; k += 1024) s_all[(size_t)i * K + k] = 1.0f;
    return;
  }
  const float floor_v = mx * 0x1p-20f;
  float mn = mx;
  for (int64_t k = tid; k < K; k += 1024) mn = fminf(mn, fmaxf(a[k], floor_v));
  mn = block_reduce(mn, false);
  const float mid = 0.5f * (log2f(mx) + log2f(mn));
  for (int64_t k = tid; k < K; k += 1024) {
    const float d = log2f(fmaxf(a[k], floor_v)) - mid;
    for (int i = 0; i < n_alpha; ++i) {
      const float alpha = n_alpha > 1 ? (float)i / (float)(n_alpha - 1) : 0.0f;
      s_all[(size_t)i * K + k] = i == 0 ? 1.0f : exp2f(alpha * d);
    }
  }
}

// ---- out[r, j] = bf16(fl32(A[r, j] * s_j)) (DIV: / s_j); thread owns one 8-column chunk and
// walks rows_per_block rows, so its scales are read once.
template <bool DIV>
__global__ __launch_bounds__(256) void scale_columns_kernel(const u32x4* __restrict__ A, int64_t rows,
                                                            int64_t c8, int64_t rows_per_block,
                                                            const float* __restrict__ s,
                                                            u32x4* __restrict__ out) {
  const int64_t cc = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (cc >= c8) return;
  const float4* sp = reinterpret_cast<const float4*>(s + 8 * cc);
  const float4 a4 = sp[0], b4 = sp[1];
  const float sv[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(r0 + rows_per_block, rows);
  for (int64_t r = r0; r < r1; ++r) {
    const u32x4 v = A[r * c8 + cc];
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = bf16_lo(v[i]), hi = bf16_hi(v[i]);
      const float plo = DIV ? lo / sv[2 * i] : lo * sv[2 * i];
      const float phi = DIV ? hi / sv[2 * i + 1] : hi * sv[2 * i + 1];
      o[i] = pack_bf16x2(plo, phi);
    }
    out[r * c8 + cc] = o;
  }
}

// ---- sum (Yq - Yref)^2: fixed grid, each thread a fixed strided set of elements, a block
// tree, then one pass over the block sums in fp64.
__global__ __launch_bounds__(256) void sq_err_partial_kernel(const uint16_t* __restrict__ Yq,
                                                             const uint16_t* __restrict__ Yr, int64_t n,
                                                             float* __restrict__ partial) {
  __shared__ float red[256 / kWave];
  const int64_t stride = (int64_t)gridDim.x * 256;
  float acc = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const float d = __uint_as_float((uint32_t)Yq[i] << 16) - __uint_as_float((uint32_t)Yr[i] << 16);
    acc = __builtin_fmaf(d, d, acc);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// One wave: lane l adds the block sums l, l + 64, ... in fp64, then a fixed butterfly.
__global__ __launch_bounds__(64) void sq_err_final_kernel(const float* __restrict__ partial, int nb,
                                                          double* __restrict__ err) {
  double sum = 0.0;
  for (int b = threadIdx.x; b < nb; b += kWave) sum += (double)partial[b];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (threadIdx.x == 0) *err = sum;
}

// ---- first smallest error -> best index, and that alpha's scales -> s_out.
__global__ __launch_bounds__(256) void awq_select_kernel(const double* __restrict__ err, int n_alpha,
                                                         const float* __restrict__ s_all, int64_t K,
                                                         int32_t* __restrict__ best,
                                                         float* __restrict__ s_out) {
  __shared__ int sel;
  if (threadIdx.x < kWave) {
    // lane i holds (err[i], i); a butterfly keeps the smaller error, the smaller index on ties
    const int i = threadIdx.x;
    double e = i < n_alpha ? err[i] : __builtin_huge_val();
    int idx = i;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double oe = __shfl_xor(e, o);
      const int oi = __shfl_xor(idx, o);
      if (oe < e || (oe == e && oi < idx)) {
        e = oe;
        idx = oi;
      }
    }
    if (i == 0) {
      sel = idx;
      *best = idx;
    }
  }
  __syncthreads();
  const float* src = s_all + (size_t)sel * K;
  for (int64_t k = threadIdx.x; k < K; k += 256) s_out[k] = src[k];
}

}  // namespace

AwqLayout awq_layout(int64_t M, int64_t N, int64_t K, int g, int n_alpha) {
  AwqLayout L;
  const uint64_t G = (uint64_t)(K / g);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.partial = take((uint64_t)kAbsSlices * K * 4);
  L.absmean = take((uint64_t)K * 4);
  L.scales_all = take((uint64_t)n_alpha * K * 4);
  L.packed = take((uint64_t)N * K / 2);
  L.qscales = take((uint64_t)N * G * 2);
  L.qzeros = take((uint64_t)N * G);
  L.xs = take((uint64_t)M * K * 2);
  L.y = take((uint64_t)M * N * 2);
  L.err_partial = take((uint64_t)kErrBlocks * 4);
  L.bytes = off;
  return L;
}

hipError_t launch_absmean(const void* X, int64_t M, int64_t K, void* partial, void* a, hipStream_t stream) {
  const int64_t c8 = K / 8;
  const int64_t slices = std::min<int64_t>(kAbsSlices, M);
  const int64_t rps = (M + slices - 1) / slices;
  const int64_t used = (M + rps - 1) / rps;
  hipLaunchKernelGGL(absmean_partial_kernel, dim3((unsigned)((c8 + 255) / 256), (unsigned)used), dim3(256), 0,
                     stream, (const u32x4*)X, M, c8, rps, (float*)partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(absmean_final_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream,
                     (const float*)partial, K, (int)used, M, (float*)a);
  return hipGetLastError();
}

hipError_t launch_awq_scales(const void* a, int64_t K, int n_alpha, void* s_all, hipStream_t stream) {
  hipLaunchKernelGGL(awq_scales_kernel, dim3(1), dim3(1024), 0, stream, (const float*)a, K, n_alpha,
                     (float*)s_all);
  return hipGetLastError();
}

hipError_t launch_scale_columns(const void* A, int64_t rows, int64_t cols, const void* s, bool divide,
                                void* out, int num_cus, hipStream_t stream) {
  const int64_t c8 = cols / 8;
  const int64_t xblocks = (c8 + 255) / 256;
  // enough blocks to fill the device, each block at least 4 rows
  int64_t yblocks = std::max<int64_t>(1, std::min<int64_t>((rows + 3) / 4, ((int64_t)num_cus * 16 + xblocks - 1) / xblocks));
  yblocks = std::min<int64_t>(yblocks, 65535);
  const int64_t rpb = (rows + yblocks - 1) / yblocks;
  yblocks = (rows + rpb - 1) / rpb;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)xblocks, (unsigned)yblocks), dim3(256), 0, stream,
                       (const u32x4*)A, rows, c8, rpb, (const float*)s, (u32x4*)out);
    return hipGetLastError();
  };
  return divide ? go(scale_columns_kernel<true>) : go(scale_columns_kernel<false>);
}

hipError_t launch_sq_err(const void* Yq, const void* Yref, int64_t n, void* partial, void* err,
                         hipStream_t stream) {
  hipLaunchKernelGGL(sq_err_partial_kernel, dim3(kErrBlocks), dim3(256), 0, stream, (const uint16_t*)Yq,
                     (const uint16_t*)Yref, n, (float*)partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sq_err_final_kernel, dim3(1), dim3(64), 0, stream, (const float*)partial, kErrBlocks,
                     (double*)err);
  return hipGetLastError();
}

hipError_t launch_awq_select(const void* err, int n_alpha, const void* s_all, int64_t K, void* best,
                             void* s_out, hipStream_t stream) {
  hipLaunchKernelGGL(awq_select_kernel, dim3(1), dim3(256), 0, stream, (const double*)err, n_alpha,
                     (const float*)s_all, K, (int32_t*)best, (float*)s_out);
  return hipGetLastError();
}

}  // namespace q4
