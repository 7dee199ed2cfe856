// Decode GEMV for W4A16 with M <= 2 (gfx950).
//
// W4A16: the 4-bit weights are dequantised inside the kernel and the products run on 16-bit
// operands ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
// "The vocabulary"); decode is bound by the bytes of the weights ("Overview": every output
// token reads every weight).  Dequantisation is x_hat = scale * (q - z) ("DL S067 ·
// Quantization", §1).
//
// Arithmetic.  Y[m, n] = sum_groups scale * sum_{k in group} x[m, k] * (q[n, k] - z), with
//   * (q - z) formed exactly in fp16: a nibble n is OR-ed into the mantissa of 1024.0
//     (0x6400 | n == 1024 + n) and (1024 + z) is subtracted, two weights per instruction;
//     nibbles in bits 4..7 of a byte give 1024 + 16 n and use 1024 + 16 z;
//   * x converted to fp16 exactly, per (row of X, 32-weight chunk), after scaling by a power
//     of two that puts the chunk's largest |x| in [2^14, 2^15) (positions that carry the
//     factor 16 of the weight use the scale / 16);
//   * products x * (q - z) are exact (11 x 11 bits); they are summed with v_dot2 into fp32,
//     then each chunk sum is multiplied by scale * 2^-e in fp32 and accumulated per lane;
//   * lanes are combined by an fp32 wave reduction, and Y is rounded to bf16 once.
// The only approximations are fp32 summation and the final bf16 rounding (x elements
// smaller than 2^-27 of their chunk's maximum lose low bits in fp16; their contribution
// error is below 2^-39 of that maximum times |x_hat|).
//
// Work split.  A wave owns one output row n at a time; lane l owns the 16-byte packed chunks
// c = l + 64 j (32 weights each), so one load instruction reads 1 KiB of a row contiguously.
// The lane's slice of X is fixed for every row, so after a block-wide conversion through LDS
// it stays in registers.  Rows are grid-strided over a persistent grid, and the next row's
// packed chunks, scales and zeros are loaded before the current row is reduced.
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kBlock = 512;

template <int MT, int J, bool SYM>
__global__ __launch_bounds__(kBlock) void gemv_kernel(
    const uint16_t* __restrict__ X, int M, int64_t N, int K, int g,
    const u32x4* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y) {
  extern __shared__ uint32_t lds[];
  const int C = K >> 5;                       // 32-weight chunks per row
  const int G = K / g;
  const int cpg = g >> 5;                     // chunks per group

  // ---- X -> fp16 pairs, 16 dwords per (m, chunk), plus 2^-e per (m, chunk) ----
  uint32_t* xs = lds;
  float* fs = reinterpret_cast<float*>(lds + (size_t)M * C * 16);
  for (int idx = threadIdx.x; idx < M * C; idx += blockDim.x) {
    const int m = idx / C;
    const int c = idx - m * C;
    const u32x4* xp = reinterpret_cast<const u32x4*>(X + (size_t)m * K + (size_t)c * 32);
    float x[32];
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      const u32x4 v = xp[o];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * o + 2 * i] = bf16_lo(v[i]);
        x[8 * o + 2 * i + 1] = bf16_hi(v[i]);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    int e = 0;
    if (amax > 0.0f) {
      int E;
      frexpf(amax, &E);                       // amax = f * 2^E, f in [0.5, 1)
      e = min(15 - E, 100);
    }
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      const float* y = x + 8 * o;
      f16x2 p0 = {(_Float16)ldexpf(y[0], e), (_Float16)ldexpf(y[4], e)};
      f16x2 p1 = {(_Float16)ldexpf(y[1], e - 4), (_Float16)ldexpf(y[5], e - 4)};
      f16x2 p2 = {(_Float16)ldexpf(y[2], e), (_Float16)ldexpf(y[6], e)};
      f16x2 p3 = {(_Float16)ldexpf(y[3], e - 4), (_Float16)ldexpf(y[7], e - 4)};
      uint32_t* dst = xs + (size_t)idx * 16 + 4 * o;
      dst[0] = as_u32(p0);
      dst[1] = as_u32(p1);
      dst[2] = as_u32(p2);
      dst[3] = as_u32(p3);
    }
    fs[idx] = ldexpf(1.0f, -e);
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  uint32_t xr[MT][J][16];
  float fr[MT][J];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + kWave * j;
      const bool ok = m < M && c < C;
#pragma unroll
      for (int t = 0; t < 16; ++t) xr[m][j][t] = ok ? xs[((size_t)m * C + c) * 16 + t] : 0u;
      fr[m][j] = ok ? fs[(size_t)m * C + c] : 0.0f;
    }
  }

  const int64_t waves_per_block = blockDim.x / kWave;
  const int64_t nw = (int64_t)gridDim.x * waves_per_block;
  int64_t n = (int64_t)blockIdx.x * waves_per_block + (threadIdx.x / kWave);

  u32x4 wc[J];
  uint16_t sc[J];
  uint8_t zc[J];
  auto load_row = [&](int64_t row, u32x4 (&w)[J], uint16_t (&s)[J], uint8_t (&z)[J]) {
    const u32x4* pr = packed + (size_t)row * C;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + kWave * j;
      if (c < C) {
        w[j] = __builtin_nontemporal_load(pr + c);
        const size_t gi = (size_t)row * G + c / cpg;
        s[j] = scales[gi];
        z[j] = SYM ? (uint8_t)8 : zeros[gi];
      } else {
        w[j] = u32x4{0u, 0u, 0u, 0u};
        s[j] = 0;
        z[j] = 0;
      }
    }
  };
  if (n < N) load_row(n, wc, sc, zc);

  for (; n < N; n += nw) {
    u32x4 wn[J];
    uint16_t sn[J];
    uint8_t zn[J];
    const int64_t nn = n + nw;
    if (nn < N) load_row(nn, wn, sn, zn);

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t z = zc[j];
      const f16x2 b1 = as_f16x2((0x6400u + z) * 0x00010001u);        // (1024 + z) x2
      const f16x2 b16 = as_f16x2((0x6400u + 16u * z) * 0x00010001u); // (1024 + 16 z) x2
      float d[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) d[m] = 0.0f;
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        uint32_t dw = wc[j][o];
        if (SYM) dw ^= 0x88888888u;          // two's complement nibble -> q + 8
        const uint32_t d8 = dw >> 8;
        const f16x2 h0 = as_f16x2((dw & 0x000F000Fu) | 0x64006400u) - b1;   // k0, k4
        const f16x2 h1 = as_f16x2((dw & 0x00F000F0u) | 0x64006400u) - b16;  // k1, k5 (x16)
        const f16x2 h2 = as_f16x2((d8 & 0x000F000Fu) | 0x64006400u) - b1;   // k2, k6
        const f16x2 h3 = as_f16x2((d8 & 0x00F000F0u) | 0x64006400u) - b16;  // k3, k7 (x16)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          d[m] = __builtin_amdgcn_fdot2(h0, as_f16x2(xr[m][j][4 * o + 0]), d[m], false);
          d[m] = __builtin_amdgcn_fdot2(h1, as_f16x2(xr[m][j][4 * o + 1]), d[m], false);
          d[m] = __builtin_amdgcn_fdot2(h2, as_f16x2(xr[m][j][4 * o + 2]), d[m], false);
          d[m] = __builtin_amdgcn_fdot2(h3, as_f16x2(xr[m][j][4 * o + 3]), d[m], false);
        }
      }
      const float s = (float)__builtin_bit_cast(_Float16, sc[j]);
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = __builtin_fmaf(d[m], s * fr[m][j], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float tot = wave_sum(acc[m]);
      if (lane == m && m < M) Y[(size_t)m * N + n] = f32_to_bf16_bits(tot);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      wc[j] = wn[j];
      sc[j] = sn[j];
      zc[j] = zn[j];
    }
  }
}

template <int MT, int J>
hipError_t launch_mtj(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                      const void* packed, const void* scales, const void* zeros, void* Y,
                      int num_cus, hipStream_t stream) {
  const int C = (int)(K >> 5);
  const size_t lds = (size_t)M * C * 16 * 4 + (size_t)M * C * 4;
  const int64_t waves_per_block = kBlock / kWave;
  int64_t blocks = (N + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)num_cus * 2;
  if (blocks > cap) blocks = cap;
  if (sym) {
    hipLaunchKernelGGL((gemv_kernel<MT, J, true>), dim3((unsigned)blocks), dim3(kBlock), lds, stream,
                       (const uint16_t*)X, M, N, (int)K, g, (const u32x4*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y);
  } else {
    hipLaunchKernelGGL((gemv_kernel<MT, J, false>), dim3((unsigned)blocks), dim3(kBlock), lds, stream,
                       (const uint16_t*)X, M, N, (int)K, g, (const u32x4*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y);
  }
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                     const void* packed, const void* scales, const void* zeros, void* Y,
                     int num_cus, hipStream_t stream) {
  if (K <= 2048) return launch_mtj<MT, 1>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
  if (K <= 4096) return launch_mtj<MT, 2>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
  if constexpr (MT == 1) {
    if (K <= 8192) return launch_mtj<1, 4>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
    if (K <= 16384) return launch_mtj<1, 8>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                       const void* packed, const void* scales, const void* zeros, void* Y,
                       int num_cus, hipStream_t stream) {
  if (M == 1) return launch_mt<1>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
  return launch_mt<2>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
}

}  // namespace q4
