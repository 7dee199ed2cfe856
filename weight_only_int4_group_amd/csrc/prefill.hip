// W4A16 prefill GEMM for large M on the bf16 matrix cores of gfx950 (v_mfma_f32_16x16x32_bf16).
//
// The weights stay 4-bit in HBM and are dequantised inside the kernel; the product runs on
// 16-bit operands ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8
// Trade-offs", "The vocabulary" and "format notes").  The dequantised weight is
// x_hat = scale * (q - z) ("DL S067 · Quantization", §1), formed exactly in fp32 by one
// mixed-precision fma per weight and rounded once to bf16.
//
// Block = 4 waves, tile = 256 rows of X x 256 rows of W, k walked in steps of 128.
//   * X: the block's 256 x 128 bf16 slice of each step is copied global -> LDS by the
//     direct-to-LDS loads of gfx950 (no registers), double-buffered: the copy for step s + 1
//     is issued at the start of step s.  Rows are XOR-swizzled in 16-byte chunks so that the
//     MFMA fragment reads hit 16 different bank groups.
//   * W: each wave owns 64 W rows; a lane loads the 32 codes (16 bytes) it needs per row and
//     step, one step ahead, and dequantises them in registers straight into MFMA operands, so
//     every weight of the tile is dequantised exactly once per block.
//   * One barrier per step, after the step's loads have landed.
// The k order inside a step is permuted identically for both operands (lane group q takes the
// 32 contiguous k of its codes), which leaves each output sum unchanged.
// MFMA: D[n][m] = sum_k W[n][k] X[m][k]; a lane's four accumulators are four consecutive n of
// one m, written as one 8-byte store into row-major Y.  Blocks are numbered so the tiles that
// share X rows land on one XCD (one L2).
#include <type_traits>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {
namespace {

constexpr int kStepK = 128;                            // k per step
constexpr int kTileM = 128;                            // X rows per block
constexpr int kTileN = 256;                            // W rows per block (64 per wave)
constexpr uint32_t kRowBytes = kStepK * 2;             // one X row of a step in LDS
constexpr uint32_t kStageBytes = kTileM * kRowBytes;   // 32 KiB
constexpr uint32_t kWaveDma = kStageBytes / 4;         // bytes each wave copies per step
constexpr int kDmaOps = kWaveDma / 1024;               // 1 KiB copy instructions per wave

template <bool SYM>
__device__ __forceinline__ u32x4 dequant8(uint32_t dw, float s, float s16th, float c1, float c16) {
  if (SYM) dw ^= 0x88888888u;                     // two's complement nibble -> q + 8, z = 8
  const uint32_t d8 = dw >> 8;
  // fp16 1024 + n for the nibbles at bits 0/16 (k0, k4) and 8/24 (k2, k6); the nibbles at
  // bits 4/20 and 12/28 land 4 bits up, i.e. 1024 + 16 n, and use s/16 and -s (64 + z).
  const f16x2 q0 = as_f16x2((dw & 0x000F000Fu) | 0x64006400u);
  const f16x2 q1 = as_f16x2((dw & 0x00F000F0u) | 0x64006400u);
  const f16x2 q2 = as_f16x2((d8 & 0x000F000Fu) | 0x64006400u);
  const f16x2 q3 = as_f16x2((d8 & 0x00F000F0u) | 0x64006400u);
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

// 16 bytes per lane, global -> LDS: lane i writes LDS bytes [lds + 16 i, lds + 16 i + 16).
// `base` and `lds` are wave-uniform; the instruction has no register result.
__device__ __forceinline__ void copy_to_lds(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Wait for every load of this wave (the LDS copies included) and for its LDS traffic, then
// meet the other waves.
__device__ __forceinline__ void step_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int R>
using Slot = std::integral_constant<int, R>;

template <bool SYM>
__global__ __launch_bounds__(256, 2) void prefill_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, int lg,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y, int tiles_m, int tiles_n,
    int vec_store) {
  constexpr int MB = kTileM / 16;    // 16-row blocks of X
  constexpr int NB = 4;              // 16-row blocks of W per wave

  __shared__ __attribute__((aligned(1024))) uint8_t xl[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, lq = lane >> 4;

  const int tiles = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int t = (tiles & 7) == 0 ? (b & 7) * (tiles >> 3) + (b >> 3) : b;
  const int bm = t / tiles_n, bn = t - bm * tiles_n;
  const int m0 = bm * kTileM, n0 = bn * kTileN;
  const int KT = K / kStepK;
  const int G = K >> lg;
  const uint32_t xrow_bytes = (uint32_t)K * 2u;

  // X copy: this wave's instruction i fills LDS rows r = R wave + 4 i + lane / 16 (R = rows per
  // wave) at chunk
  // position lane % 16, which holds chunk (lane % 16) ^ (r % 16) of the row.  Rows past M copy
  // row M - 1 (their outputs are dropped).
  const uint16_t* xblk = X + (size_t)m0 * K;
  uint32_t dma_off[kDmaOps];
#pragma unroll
  for (int i = 0; i < kDmaOps; ++i) {
    const int r = (kTileM / 4) * wave + 4 * i + (lane >> 4);
    const int rr = min(m0 + r, M - 1) - m0;
    const int c = (lane & 15) ^ (r & 15);
    dma_off[i] = (uint32_t)rr * xrow_bytes + 16u * (uint32_t)c;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)xl;
  const uint32_t lds_wave = lds_base + (uint32_t)wave * kWaveDma;

  // B fragment of k-chunk (4 lq + ks) of row 16 mb + li sits at chunk position (4 lq + ks) ^ li.
  uint32_t rd_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) rd_off[ks] = (uint32_t)li * kRowBytes + 16u * (uint32_t)((4 * lq + ks) ^ li);

  // W rows of this lane (clamped: rows past N load valid memory, their outputs are dropped).
  const uint8_t* pblk = packed + (size_t)n0 * (size_t)(K / 2);
  const uint16_t* sblk = scales + (size_t)n0 * G;
  const uint8_t* zblk = zeros + (size_t)n0 * G;
  uint32_t wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wrow[nb] = (uint32_t)(min(n0 + 64 * wave + 16 * nb + li, N - 1) - n0);

  f32x4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wq[2][NB];                  // codes: k = 32 lq .. 32 lq + 31 of the step, per W row
  uint32_t ws[2][NB], wz[2][NB];    // raw scale bits / zero point of that 32-k chunk

  auto copy_x = [&](int buf, int kt) {
    const uint16_t* src = xblk + (size_t)min(kt, KT - 1) * kStepK;
    const uint32_t dst = lds_wave + (uint32_t)buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < kDmaOps; ++i) copy_to_lds(src, dma_off[i], dst + 1024u * i);
  };
  auto load_w = [&](auto S, int kt) {
    constexpr int R = decltype(S)::value;
    const int ktc = min(kt, KT - 1);
    const uint8_t* pb = pblk + (size_t)ktc * (kStepK / 2) + 16 * lq;
    const uint32_t gi = (uint32_t)((ktc * kStepK + 32 * lq) >> lg);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      wq[R][nb] = *reinterpret_cast<const u32x4*>(pb + wrow[nb] * (uint32_t)(K / 2));
      ws[R][nb] = sblk[wrow[nb] * (uint32_t)G + gi];
      wz[R][nb] = SYM ? 8u : (uint32_t)zblk[wrow[nb] * (uint32_t)G + gi];
    }
  };

  // One step: copy X of step kt + 1 into the other buffer, load W codes of step kt + 1 into
  // the other slot, multiply step kt.
  auto step = [&](auto S, int kt) {
    constexpr int R = decltype(S)::value;
    // The previous barrier already waited for these registers; naming them here, before any
    // new load is issued, keeps the compiler's own wait for them from covering the new loads.
    asm volatile("" ::"v"(wq[R][0]), "v"(wq[R][1]), "v"(wq[R][2]), "v"(wq[R][3]));
    asm volatile("" ::"v"(ws[R][0]), "v"(ws[R][1]), "v"(ws[R][2]), "v"(ws[R][3]));
    if (!SYM) asm volatile("" ::"v"(wz[R][0]), "v"(wz[R][1]), "v"(wz[R][2]), "v"(wz[R][3]));
    copy_x(R ^ 1, kt + 1);
    load_w(Slot<R ^ 1>{}, kt + 1);

    float s[NB], s16[NB], c1[NB], c16[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s[nb] = (float)__builtin_bit_cast(_Float16, (uint16_t)ws[R][nb]);
      const float zf = (float)wz[R][nb];
      s16[nb] = s[nb] * 0.0625f;
      c1[nb] = -s[nb] * (1024.0f + zf);
      c16[nb] = -s[nb] * (64.0f + zf);
    }
    const uint8_t* xs = xl + (uint32_t)R * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        a[nb] = __builtin_bit_cast(bf16x8, dequant8<SYM>(wq[R][nb][ks], s[nb], s16[nb], c1[nb], c16[nb]));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 bx = *reinterpret_cast<const bf16x8*>(xs + mb * 16 * kRowBytes + rd_off[ks]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[nb], bx, acc[nb][mb], 0, 0, 0);
      }
    }
    step_barrier();
  };

  copy_x(0, 0);
  load_w(Slot<0>{}, 0);
  step_barrier();

  // Straight-line body of two steps (one per buffer / register slot); an odd last step follows.
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    step(Slot<0>{}, kt);
    step(Slot<1>{}, kt + 1);
  }
  if (kt < KT) step(Slot<0>{}, kt);

  // D[n][m]: lane (li, lq) holds n = 4 lq + e (e = 0..3) of column m = li.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + li;
      const int nbase = n0 + 64 * wave + nb * 16 + 4 * lq;
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

template <bool SYM>
hipError_t launch_sym(const void* X, int64_t M, int64_t N, int64_t K, int lg, const void* packed,
                      const void* scales, const void* zeros, void* Y, hipStream_t stream) {
  const int tiles_m = (int)((M + kTileM - 1) / kTileM);
  const int tiles_n = (int)((N + kTileN - 1) / kTileN);
  const int64_t blocks = (int64_t)tiles_m * tiles_n;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(Y) & 7) == 0);
  hipLaunchKernelGGL((prefill_kernel<SYM>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t*)X, (int)M, (int)N, (int)K, lg, (const uint8_t*)packed,
                     (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y, tiles_m, tiles_n, vec);
  return hipGetLastError();
}

}  // namespace

bool prefill_fits(int64_t M, int64_t N, int64_t K, int g) {
  (void)N;
  // 32-bit in-tile offsets: 256 rows of X (bf16) and of W (codes) must span < 4 GiB.
  return M >= kPrefillMinM && K % kStepK == 0 && g >= 32 && (g & (g - 1)) == 0 &&
         (int64_t)kTileM * K * 2 < (int64_t(1) << 32);
}

hipError_t launch_prefill(const void* X, int64_t M, int64_t N, int64_t K, int g, bool sym,
                          const void* packed, const void* scales, const void* zeros, void* Y,
                          hipStream_t stream) {
  int lg = 0;
  while ((1 << lg) < g) ++lg;
  return sym ? launch_sym<true>(X, M, N, K, lg, packed, scales, zeros, Y, stream)
             : launch_sym<false>(X, M, N, K, lg, packed, scales, zeros, Y, stream);
}

}  // namespace q4
