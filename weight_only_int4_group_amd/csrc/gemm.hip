// W4A16 GEMM on the bf16 matrix cores of gfx950 (v_mfma_f32_16x16x32_bf16).
//
// W4A16: the 4-bit weights are dequantised inside the kernel and the product runs on 16-bit
// operands ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
// "The vocabulary"; prefill stays 16-bit math, "format notes" of the same page).  The
// dequantised weight is x_hat = scale * (q - z) ("DL S067 · Quantization", §1).
//
// Dequantisation.  s * (q - z) is formed exactly in fp32 with one mixed-precision fma per
// weight: a nibble OR-ed into the mantissa of fp16 1024.0 is 1024 + q, and
// fma(1024 + q, s, -s (1024 + z)) = s (q - z) with an exactly representable addend (fp16
// scale x 11-bit integer).  It is then rounded once to bf16 (round to nearest even), which
// is the only rounding besides fp32 accumulation and the bf16 output.
//
// Tiling.  A 256-thread block owns a BM x BN tile of Y (BM rows of X, BN rows of W) and walks
// K in steps of 64.  Per step the block dequantises its BN x 64 weight tile into LDS once
// (double-buffered, one barrier per step); each wave reads weight fragments from LDS and its
// own activation fragments straight from global memory (each X row is private to one wave
// row of the block).  The MFMA computes D[n][m] = sum_k W[n][k] X[m][k], so a lane's four
// accumulators are four consecutive n of one m: an 8-byte store into the row-major Y.
// Inside a step the k order is permuted (lane group q takes k = 16 q .. 16 q + 15 for both
// operands) so every lane loads 32 contiguous bytes of X; the sum is unchanged.
// Blocks are numbered so that consecutive tiles (same X rows) land on the same XCD.
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kBK = 64;
constexpr int kLdsK = kBK + 8;   // bf16 per weight-tile row in LDS (144 bytes, 16-byte aligned)

template <bool SYM>
__device__ __forceinline__ u32x4 dequant8(uint32_t dw, float s, float s16th, float c1, float c16) {
  if (SYM) dw ^= 0x88888888u;                     // two's complement nibble -> q + 8, z = 8
  const uint32_t d8 = dw >> 8;
  const f16x2 q0 = as_f16x2((dw & 0x000F000Fu) | 0x64006400u);   // 1024 + q_k0, q_k4
  const f16x2 q1 = as_f16x2((dw & 0x00F000F0u) | 0x64006400u);   // 1024 + 16 q_k1, q_k5
  const f16x2 q2 = as_f16x2((d8 & 0x000F000Fu) | 0x64006400u);   // k2, k6
  const f16x2 q3 = as_f16x2((d8 & 0x00F000F0u) | 0x64006400u);   // k3, k7 (x16)
  const float w0 = __builtin_fmaf((float)q0[0], s, c1);
  const float w4 = __builtin_fmaf((float)q0[1], s, c1);
  const float w1 = __builtin_fmaf((float)q1[0], s16th, c16);
  const float w5 = __builtin_fmaf((float)q1[1], s16th, c16);
  const float w2 = __builtin_fmaf((float)q2[0], s, c1);
  const float w6 = __builtin_fmaf((float)q2[1], s, c1);
  const float w3 = __builtin_fmaf((float)q3[0], s16th, c16);
  const float w7 = __builtin_fmaf((float)q3[1], s16th, c16);
  return u32x4{pack_bf16x2(w0, w1), pack_bf16x2(w2, w3), pack_bf16x2(w4, w5), pack_bf16x2(w6, w7)};
}

// W8A16: eight 8-bit codes (two dwords, code i in byte i) -> 8 bf16 operand values, each
// fma(q, s, -s z) exact in fp32 (fp16 scale x integer <= 255) and rounded once to bf16.
// Symmetric codes (int8 two's complement) are offset by 128 (XOR 0x80), with z = 128.
template <bool SYM>
__device__ __forceinline__ u32x4 dequant8_bytes(uint32_t d0, uint32_t d1, float s, float sz) {
  if (SYM) {
    d0 ^= 0x80808080u;
    d1 ^= 0x80808080u;
  }
  float w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] = __builtin_fmaf((float)((d0 >> (8 * i)) & 0xFFu), s, -sz);
    w[i + 4] = __builtin_fmaf((float)((d1 >> (8 * i)) & 0xFFu), s, -sz);
  }
  return u32x4{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
               pack_bf16x2(w[6], w[7])};
}

// B: code width, 4 (W4A16, two codes per byte) or 8 (W8A16, one code per byte).
template <int BM, int BN, int WM, int WN, bool SYM, int B = 4>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, int g,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y, int tiles_m, int tiles_n,
    int vec_store) {
  static_assert(WM * WN == 4, "four waves per block");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  static_assert(MB >= 1 && NB >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  constexpr int TASKS = BN * 2;                  // (row, 32-weight half) per K step
  constexpr int TPT = (TASKS + 255) / 256;

  __shared__ __attribute__((aligned(16))) uint16_t wt[2][BN * kLdsK];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int li = lane & 15, lq = lane >> 4;

  const int tiles = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int t = (tiles & 7) == 0 ? (b & 7) * (tiles >> 3) + (b >> 3) : b;
  const int bm = t / tiles_n, bn = t - bm * tiles_n;
  const int m0 = bm * BM, n0 = bn * BN;
  const int G = K / g;
  const size_t rowbytes = B == 8 ? (size_t)K : (size_t)K / 2;
  const int KT = (K + kBK - 1) / kBK;

  f32x4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int CW = B / 4;                      // 16-byte code loads per 32 weights
  u32x4 pw[TPT][CW];
  uint16_t ps[TPT];
  uint8_t pz[TPT];
  auto load_w = [&](int kt) {
    const int kvalid = K - kt * kBK;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int task = tid + 256 * i;
#pragma unroll
      for (int c = 0; c < CW; ++c) pw[i][c] = u32x4{0u, 0u, 0u, 0u};
      ps[i] = 0;
      pz[i] = 0;
      if (task < TASKS) {
        const int r = task >> 1, h = task & 1;
        const int n = n0 + r;
        if (n < N && 32 * h < kvalid) {
          const uint8_t* src = packed + (size_t)n * rowbytes + (size_t)kt * (kBK * B / 8) + 16 * CW * h;
#pragma unroll
          for (int c = 0; c < CW; ++c) pw[i][c] = *reinterpret_cast<const u32x4*>(src + 16 * c);
          const size_t gi = (size_t)n * G + (kt * kBK + 32 * h) / g;
          ps[i] = scales[gi];
          pz[i] = SYM ? (uint8_t)(B == 8 ? 128 : 8) : zeros[gi];
        }
      }
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int task = tid + 256 * i;
      if (task < TASKS) {
        const int r = task >> 1, h = task & 1;
        const float s = (float)__builtin_bit_cast(_Float16, ps[i]);
        const float zf = (float)pz[i];
        u32x4* dst = reinterpret_cast<u32x4*>(&wt[buf][r * kLdsK + 32 * h]);
        if constexpr (B == 8) {
          const float sz = s * zf;
#pragma unroll
          for (int o = 0; o < 4; ++o)
            dst[o] = dequant8_bytes<SYM>(pw[i][o / 2][2 * (o % 2)], pw[i][o / 2][2 * (o % 2) + 1], s, sz);
        } else {
          const float c1 = -s * (1024.0f + zf);
          const float c16 = -s * (64.0f + zf);
          const float s16th = s * 0.0625f;
#pragma unroll
          for (int o = 0; o < 4; ++o) dst[o] = dequant8<SYM>(pw[i][0][o], s, s16th, c1, c16);
        }
      }
    }
  };

  u32x4 xa[MB][2], xb[MB][2];
  auto load_x = [&](int kt, u32x4 (&dst)[MB][2]) {
    const int kvalid = K - kt * kBK;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + wm * WTM + mb * 16 + li;
      if (m < M && 16 * lq < kvalid) {
        const u32x4* p = reinterpret_cast<const u32x4*>(X + (size_t)m * K + (size_t)kt * kBK + 16 * lq);
        dst[mb][0] = p[0];
        dst[mb][1] = p[1];
      } else {
        dst[mb][0] = u32x4{0u, 0u, 0u, 0u};
        dst[mb][1] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  load_w(0);
  load_x(0, xa);
  store_w(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      load_w(kt + 1);
      load_x(kt + 1, xb);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* base = &wt[cur][(wn * WTN + nb * 16 + li) * kLdsK + 16 * lq];
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(base);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(base + 8);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a0, __builtin_bit_cast(bf16x8, xa[mb][0]), acc[nb][mb], 0, 0, 0);
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a1, __builtin_bit_cast(bf16x8, xa[mb][1]), acc[nb][mb], 0, 0, 0);
      }
    }
    if (more) store_w(cur ^ 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        xa[mb][0] = xb[mb][0];
        xa[mb][1] = xb[mb][1];
      }
    }
  }

  // D[n][m]: lane (li, lq) holds n = 4 lq + e (e = 0..3) of column m = li.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + wm * WTM + mb * 16 + li;
      const int nbase = n0 + wn * WTN + nb * 16 + 4 * lq;
      if (m < M) {
        const f32x4 v = acc[nb][mb];
        uint16_t* yrow = Y + (size_t)m * N;
        if (vec_store && nbase + 3 < N) {
          *reinterpret_cast<u32x2*>(yrow + nbase) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nbase + e < N) yrow[nbase + e] = f32_to_bf16_bits(v[e]);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int B = 4>
hipError_t launch_cfg(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                      const void* packed, const void* scales, const void* zeros, void* Y,
                      hipStream_t stream) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int64_t blocks = (int64_t)tiles_m * tiles_n;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(Y) & 7) == 0);
  if (sym) {
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, true, B>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)X, (int)M, (int)N, (int)K, g, (const uint8_t*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y, tiles_m, tiles_n, vec);
  } else {
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, false, B>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)X, (int)M, (int)N, (int)K, g, (const uint8_t*)packed,
                       (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y, tiles_m, tiles_n, vec);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                       const void* packed, const void* scales, const void* zeros, void* Y,
                       int num_cus, hipStream_t stream) {
  (void)num_cus;
  if (M <= 16) return launch_cfg<16, 64, 1, 4>(X, M, N, K, g, sym, packed, scales, zeros, Y, stream);
  if (M <= 32) return launch_cfg<32, 64, 1, 4>(X, M, N, K, g, sym, packed, scales, zeros, Y, stream);
  if (M <= 64) return launch_cfg<64, 64, 1, 4>(X, M, N, K, g, sym, packed, scales, zeros, Y, stream);
  if (M <= 128) return launch_cfg<128, 128, 2, 2>(X, M, N, K, g, sym, packed, scales, zeros, Y, stream);
  return launch_cfg<256, 128, 4, 1>(X, M, N, K, g, sym, packed, scales, zeros, Y, stream);
}

hipError_t launch_gemm8(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                        const void* codes, const void* scales, const void* zeros, void* Y,
                        int num_cus, hipStream_t stream) {
  (void)num_cus;
  if (M <= 16) return launch_cfg<16, 64, 1, 4, 8>(X, M, N, K, g, sym, codes, scales, zeros, Y, stream);
  if (M <= 32) return launch_cfg<32, 64, 1, 4, 8>(X, M, N, K, g, sym, codes, scales, zeros, Y, stream);
  if (M <= 64) return launch_cfg<64, 64, 1, 4, 8>(X, M, N, K, g, sym, codes, scales, zeros, Y, stream);
  if (M <= 128) return launch_cfg<128, 128, 2, 2, 8>(X, M, N, K, g, sym, codes, scales, zeros, Y, stream);
  return launch_cfg<256, 128, 4, 1, 8>(X, M, N, K, g, sym, codes, scales, zeros, Y, stream);
}

}  // namespace q4
