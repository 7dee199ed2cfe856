// W8A16 decode GEMV for M <= 4 (gfx950): 8-bit group-wise weights ("LLM Weight Quantization -
// GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs", "Granularity and outliers": W8A16,
// INT8 weights with 16-bit activations; "DL S067 · Quantization", §1 for the INT8 ranges and
// x_hat = scale * (q - z)).  Decode reads every weight once, so the kernel is HBM bound.
//
// Arithmetic.  Y[m, n] = sum over 16-weight chunks of scale * sum_k x[m, k] (q[n, k] - z), a chunk
// never straddling a group (g % 32 == 0).
//   * q - z is formed exactly in fp16, two weights per instruction pair: a code byte placed
//     under the exponent byte 0x64 is the fp16 1024 + q (one v_perm_b32 builds two), and a
//     packed fp16 subtraction of 1024 + z leaves the integer q - z (|q - z| <= 255).
//     Symmetric codes (int8) are offset by 128 (XOR of the sign bit) and taken with z = 128.
//   * x is staged in LDS as fp16 after scaling each (row, 16-weight chunk) by the power of two
//     2^e that puts its largest |x| in [2^14, 2^15): exact for every x down to 2^-31 of that
//     largest value (2^-17 in fp16, subnormals included);
//   * v_dot2_f32_f16 takes exact products with fp32 sums; each chunk's dot is multiplied by
//     scale * 2^-e and accumulated in fp32; the row total is rounded once to bf16;
//   * X with a smaller nonzero element in some chunk (whose fp16 conversion would lose bits)
//     takes an exact fp32 path instead: (q - z) and x converted to fp32, one fma per weight.
//     The choice is one flag for the whole launch (every block stages the same X).
//
// Work split.  Persistent blocks of 4 waves; a wave owns whole rows (rows w, w + waves, ...).
// Lane l owns the 16-byte chunks c = l + 64 u of a row; a row is walked in segments of four
// chunks per lane (4 KiB of codes), and the next segment's loads are issued before the current
// one is computed.  X is converted into LDS once per block.
#include <atomic>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kBlock = 256;
constexpr int kSeg = 4;                  // chunks per lane per segment
constexpr size_t kLdsMax = 160 * 1024;

// fp16 x [M][K], one fp32 2^-e per (row, chunk) [M][K / 16] and one flag word per wave
size_t gemv8_lds(int64_t M, int64_t K) {
  return (size_t)M * (size_t)K * 2 + (size_t)M * (size_t)(K / 16) * 4 + (kBlock / kWave) * 4;
}

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}
__device__ __forceinline__ float wave_total(float v) {
  v = row_sum16(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

__device__ __forceinline__ float dot2(uint32_t x, h2_t w, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, x), w, acc, false);
}

// Bytes 0, 1 (sel 0x04010400) or 2, 3 (sel 0x04030402) of dw, each under the fp16 exponent
// byte 0x64: the pair (1024 + q_lo, 1024 + q_hi).
__device__ __forceinline__ h2_t biased_pair(uint32_t dw, uint32_t sel) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, dw, sel));
}

struct Seg {
  u32x4 w[kSeg];
  uint32_t s[kSeg];    // fp16 scale bits
  uint32_t z[kSeg];    // zero-point
};

// POW2: g is a power of two and the group of a chunk is a shift (gsh = log2 g); else a division.
template <int MT, bool SYM, bool POW2>
__global__ __launch_bounds__(kBlock) void gemv8_kernel(const u32x4* __restrict__ X, int64_t N, int K, int g,
                                                       int gsh, const uint8_t* __restrict__ codes,
                                                       const uint16_t* __restrict__ scales,
                                                       const uint8_t* __restrict__ zeros,
                                                       uint16_t* __restrict__ Y) {
  extern __shared__ u32x4 lds8[];
  const int C = K >> 4;                        // 16-weight chunks per row
  const int G = K / g;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nw = (int64_t)gridDim.x * (kBlock / kWave);
  const int64_t w0 = (int64_t)blockIdx.x * (kBlock / kWave) +
                     __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int S = (C + kSeg * kWave - 1) / (kSeg * kWave);     // segments per row

  // Loads are unconditional: a row past N gets empty buffer resources and chunks past the row
  // end lie past the resource's end, so both read 0 (and contribute 0: code 0 with zero-point 0,
  // or 0 ^ 0x80 = 128 with 128) without touching memory.
  auto load = [&](Seg& b, int64_t row, int seg) {
    const bool live = row < N;
    const size_t r = live ? (size_t)row : 0;
    const auto rw = buffer_over(codes + r * (size_t)K, live ? (uint32_t)K : 0u);
    const auto rs = buffer_over(scales + r * (size_t)G, live ? (uint32_t)G * 2u : 0u);
    const auto rz = buffer_over(zeros + r * (size_t)G, (live && !SYM) ? (uint32_t)G : 0u);
#pragma unroll
    for (int u = 0; u < kSeg; ++u) {
      const uint32_t c = (uint32_t)(seg * kSeg * kWave + u * kWave + lane);
      const uint32_t grp = POW2 ? (16u * c) >> gsh : (16u * c) / (uint32_t)g;
      b.w[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, 16 * c, 0, kBufferNT));
      b.s[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * grp, 0, 0);
      b.z[u] = SYM ? 128u : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, grp, 0, 0);
    }
  };

  int64_t row = w0;
  int seg = 0;
  Seg a, b;
  if (row < N) load(a, row, seg);

  // ---- X -> LDS: per (row, chunk) i, x 2^e as fp16 and 2^-e ----
  u32x4* xh = lds8;                                                     // [MT * C][2]
  float* xe = reinterpret_cast<float*>(lds8 + 2 * (size_t)MT * C);      // [MT * C]
  int lossy = 0;
  for (int i = threadIdx.x; i < MT * C; i += kBlock) {
    const u32x4 p0 = X[2 * i], p1 = X[2 * i + 1];
    float v[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[2 * d] = bf16_lo(p0[d]);
      v[2 * d + 1] = bf16_hi(p0[d]);
      v[8 + 2 * d] = bf16_lo(p1[d]);
      v[8 + 2 * d + 1] = bf16_hi(p1[d]);
    }
    float mx = 0.0f, mn = __builtin_inff();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float a = fabsf(v[e]);
      mx = fmaxf(mx, a);
      mn = fminf(mn, a > 0.0f ? a : __builtin_inff());
    }
    const int e = mx > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;   // mx 2^e in [2^14, 2^15)
    // x 2^e holds its 8 significant bits in fp16 (subnormals included) while |x| 2^e >= 2^-17
    lossy |= (int)(mn < __builtin_inff() && __builtin_ldexpf(mn, e) < 0x1p-17f);
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const h2_t hv = h2_t{(_Float16)__builtin_ldexpf(v[2 * j], e), (_Float16)__builtin_ldexpf(v[2 * j + 1], e)};
      h[j] = __builtin_bit_cast(uint32_t, hv);
    }
    xh[2 * i] = u32x4{h[0], h[1], h[2], h[3]};
    xh[2 * i + 1] = u32x4{h[4], h[5], h[6], h[7]};
    xe[i] = __builtin_ldexpf(1.0f, -e);
  }
  // one flag for the launch: every block stages the same X.  Each wave writes its own flag word
  // (so none needs clearing first); the block's OR is read after the barrier.  The exact path
  // reads the raw bf16 X from the same LDS words (bf16 is as wide as fp16).
  uint32_t* wflag = reinterpret_cast<uint32_t*>(xe + (size_t)MT * C);   // [kBlock / kWave]
  const uint64_t wl = __builtin_amdgcn_ballot_w64(lossy != 0);
  if (lane == 0) wflag[threadIdx.x / kWave] = wl != 0 ? 1u : 0u;
  __syncthreads();
  uint32_t any = 0;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) any |= wflag[w];
  const bool exact = any != 0;
  if (exact) {
    for (int i = threadIdx.x; i < MT * C; i += kBlock) {
      xh[2 * i] = X[2 * i];
      xh[2 * i + 1] = X[2 * i + 1];
    }
    __syncthreads();
  }
  if (row >= N) return;

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

  // Exact path (X whose fp16 conversion would lose bits): (q - z) and x in fp32, one fma per
  // weight, x the raw bf16 X from LDS.
  auto compute_exact = [&](const Seg& sg, int sgi) {
#pragma unroll
    for (int u = 0; u < kSeg; ++u) {
      const int c = sgi * kSeg * kWave + u * kWave + lane;
      const int cc = c < C ? c : C - 1;                 // LDS index clamp (the codes are 0 there)
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sg.s[u]);
      const float zf = (float)sg.z[u];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const size_t i = (size_t)m * C + cc;
        const u32x4 xv[2] = {xh[2 * i], xh[2 * i + 1]};
        float part = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t dw = SYM ? sg.w[u][d] ^ 0x80808080u : sg.w[u][d];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int k = 4 * d + b;                    // element k of the chunk: dword k / 2 of X
            const uint32_t xd = xv[k >> 3][(k >> 1) & 3];
            const float x = (k & 1) ? bf16_hi(xd) : bf16_lo(xd);
            part = __builtin_fmaf(x, (float)((dw >> (8 * b)) & 0xffu) - zf, part);
          }
        }
        acc[m] = __builtin_fmaf(part, s, acc[m]);
      }
    }
  };

  auto compute_fast = [&](const Seg& sg, int sgi) {
#pragma unroll
    for (int u = 0; u < kSeg; ++u) {
      const int c = sgi * kSeg * kWave + u * kWave + lane;
      const int cc = c < C ? c : C - 1;                 // LDS index clamp (the codes are 0 there)
      const _Float16 bz = (_Float16)(float)(1024u + sg.z[u]);
      const h2_t bzz = h2_t{bz, bz};
      h2_t wq[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t dw = SYM ? sg.w[u][d] ^ 0x80808080u : sg.w[u][d];
        wq[2 * d] = biased_pair(dw, 0x04010400u) - bzz;
        wq[2 * d + 1] = biased_pair(dw, 0x04030402u) - bzz;
      }
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sg.s[u]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const size_t i = (size_t)m * C + cc;
        const u32x4 xa = xh[2 * i], xb = xh[2 * i + 1];
        float t0 = dot2(xa[0], wq[0], 0.0f), t1 = dot2(xb[0], wq[4], 0.0f);
        t0 = dot2(xa[1], wq[1], t0);
        t1 = dot2(xb[1], wq[5], t1);
        t0 = dot2(xa[2], wq[2], t0);
        t1 = dot2(xb[2], wq[6], t1);
        t0 = dot2(xa[3], wq[3], t0);
        t1 = dot2(xb[3], wq[7], t1);
        acc[m] = __builtin_fmaf(t0 + t1, s * xe[i], acc[m]);
      }
    }
  };
  auto compute = [&](const Seg& sg, int sgi) {
    if (exact) compute_exact(sg, sgi);            // block-uniform
    else compute_fast(sg, sgi);
  };
  auto finish_row = [&](int64_t r) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float tot = wave_total(acc[m]);
      if (lane == m) Y[(size_t)m * N + r] = f32_to_bf16_bits(tot);
      acc[m] = 0.0f;
    }
  };

  // Two register sets alternate: the next segment's loads are issued before the current one is
  // computed.  The walk ends once the row passes N (the last loads then read nothing).
  while (true) {
    int64_t nrow = row;
    int nseg = seg + 1;
    if (nseg == S) {
      nseg = 0;
      nrow += nw;
    }
    load(b, nrow, nseg);
    __builtin_amdgcn_sched_barrier(0);
    compute(a, seg);
    if (nseg == 0) finish_row(row);
    __builtin_amdgcn_sched_barrier(0);
    row = nrow;
    seg = nseg;
    if (row >= N) break;

    nrow = row;
    nseg = seg + 1;
    if (nseg == S) {
      nseg = 0;
      nrow += nw;
    }
    load(a, nrow, nseg);
    __builtin_amdgcn_sched_barrier(0);
    compute(b, seg);
    if (nseg == 0) finish_row(row);
    __builtin_amdgcn_sched_barrier(0);
    row = nrow;
    seg = nseg;
    if (row >= N) break;
  }
}

// The kernel instance is chosen with MT == M, so every row of X it touches is staged.
template <int MT, bool SYM, bool POW2>
hipError_t launch_mt(const void* X, int M, int64_t N, int64_t K, int g, const void* codes,
                     const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
  // resident blocks per CU for the last LDS size (the grid of a persistent kernel is sized to it)
  static std::atomic<uint64_t> memo{0};
  const auto kernel = gemv8_kernel<MT, SYM, POW2>;
  const size_t lds = gemv8_lds(M, K);
  int nb = 0;
  const uint64_t mv = memo.load(std::memory_order_relaxed);
  if (mv != 0 && (mv >> 8) == lds) {
    nb = (int)(mv & 0xff);
  } else {
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
      if (e != hipSuccess) return e;
    }
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kBlock, lds) != hipSuccess) {
      (void)hipGetLastError();
      nb = 1;
    }
    nb = nb < 1 ? 1 : (nb > 255 ? 255 : nb);
    memo.store(((uint64_t)lds << 8) | (uint64_t)nb, std::memory_order_relaxed);
  }
  const int64_t wpb = kBlock / kWave;
  int64_t blocks = (N + wpb - 1) / wpb;
  const int64_t cap = (int64_t)num_cus * nb;
  if (blocks > cap) blocks = cap;
  const int gsh = POW2 ? __builtin_ctz((unsigned)g) : 0;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kBlock), lds, stream, (const u32x4*)X, N, (int)K, g,
                     gsh, (const uint8_t*)codes, (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y);
  return hipGetLastError();
}

template <bool SYM, bool POW2>
hipError_t launch_sym(const void* X, int M, int64_t N, int64_t K, int g, const void* codes,
                      const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
  switch (M) {
    case 1: return launch_mt<1, SYM, POW2>(X, M, N, K, g, codes, scales, zeros, Y, num_cus, stream);
    case 2: return launch_mt<2, SYM, POW2>(X, M, N, K, g, codes, scales, zeros, Y, num_cus, stream);
    case 3: return launch_mt<3, SYM, POW2>(X, M, N, K, g, codes, scales, zeros, Y, num_cus, stream);
    case 4: return launch_mt<4, SYM, POW2>(X, M, N, K, g, codes, scales, zeros, Y, num_cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gemv8_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= kGemv8MaxM && gemv8_lds(M, K) <= kLdsMax && K <= (int64_t)1 << 26;
}

hipError_t launch_gemv8(const void* X, int M, int64_t N, int64_t K, int g, bool sym, const void* codes,
                        const void* scales, const void* zeros, void* Y, int num_cus, hipStream_t stream) {
  const bool pow2 = (g & (g - 1)) == 0;
  if (sym)
    return pow2 ? launch_sym<true, true>(X, M, N, K, g, codes, scales, zeros, Y, num_cus, stream)
                : launch_sym<true, false>(X, M, N, K, g, codes, scales, zeros, Y, num_cus, stream);
  return pow2 ? launch_sym<false, true>(X, M, N, K, g, codes, scales, zeros, Y, num_cus, stream)
              : launch_sym<false, false>(X, M, N, K, g, codes, scales, zeros, Y, num_cus, stream);
}

}  // namespace q4
