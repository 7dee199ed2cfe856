// Decode GEMV for W4A16 with M <= 2 (gfx950).
//
// W4A16: the 4-bit weights are dequantised inside the kernel and the products run on 16-bit
// operands ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
// "The vocabulary"); decode is bound by the bytes of the weights ("Overview": every output
// token reads every weight).  Dequantisation is x_hat = scale * (q - z) ("DL S067 ·
// Quantization", §1).
//
// Arithmetic.  Y[m, n] = sum_chunks scale * (sum_{k in chunk} x[m, k] q[n, k] - z sum_k x[m, k]),
// chunks of 32 weights never straddling a group, with
//   * the codes q used as exact fp16 subnormals: a nibble masked into the low bits of a 16-bit
//     half is the fp16 value q * 2^-24 (a nibble in bits 4..7 gives 16 q * 2^-24), two weights
//     per instruction and no bias to remove;
//   * x converted to fp16 exactly, per (row of X, chunk), after scaling by a power of two 2^e
//     that puts the chunk's largest |x| in [2^14, 2^15) (positions that meet a 16 q weight carry
//     2^(e-4)); the chunk sums of the scaled x are precomputed once per block;
//   * products x q are exact; v_dot2 sums them in fp32; the zero-point enters as one fma per
//     chunk (sum x q - z sum x), the chunk result is multiplied by 2^24, 2^-e and the scale in
//     fp32 and accumulated per lane; lanes are combined by an fp32 wave reduction and Y is rounded to
//     bf16 once.
// Beyond fp32 summation and the bf16 output, the rounding of the two chunk sums adds at most
// about 2^-24 * 30 * scale * sum|x| per chunk (the q and z terms are each at most 15 sum|x|);
// x elements smaller than 2^-27 of their chunk's maximum lose low bits in fp16.
//
// Work split.  A wave owns one output row n at a time; lane l owns the 16-byte packed chunks
// c = l + 64 j (32 weights each), so one load instruction reads 1 KiB of a row contiguously.
// One persistent block of 16 waves per compute unit converts X once into LDS (laid out in
// four planes so that a lane's 16-byte reads of consecutive chunks hit distinct banks).
// Each wave keeps three rows in flight: the loads of rows n + nw and n + 2 nw are issued
// before row n is computed, and the first three rows are requested before the conversion of
// X, so HBM latency overlaps it.  Row sums are reduced with DPP row operations and lane reads.
#include "q4_device.h"
#include "q4_internal.h"

#include <atomic>

namespace q4 {
namespace {

// Sum over the 64 lanes of a wave, returned uniformly.
__device__ __forceinline__ float dpp_row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)); // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)); // row_mirror
  return v;   // every lane of a 16-lane row holds that row's sum
}
__device__ __forceinline__ float wave_total(float v) {
  v = dpp_row_sum(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Loaded values stay untouched until use, so the loads of later rows remain in flight.
// SHARE (a row has at most 64 groups): lane l loads the scale and zero of group l only, and a
// lane reads the values of its chunks' groups from the owning lanes (ds_bpermute), i.e. two
// coalesced loads per row instead of two per chunk.  The rows of a wave are processed with all
// 64 lanes active, so every source lane of the exchange holds its value.
template <int J, bool SHARE>
struct RowBuf {
  u32x4 w[J];
  uint32_t s[SHARE ? 1 : J];      // fp16 scale bits
  uint32_t z[SHARE ? 1 : J];      // zero-point
};

template <int MT, int J, bool SYM, int BLOCK, bool FULL, bool SHARE, int RING>
__global__ __launch_bounds__(BLOCK) void gemv_kernel(
    const uint16_t* __restrict__ X, int M, int64_t N, int K, int g,
    const u32x4* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y) {
  extern __shared__ u32x4 lds4[];
  const int C = K >> 5;                       // 32-weight chunks per row
  const int G = K / g;
  const int cpg = g >> 5;                     // chunks per group
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wpb = BLOCK / kWave;
  const int64_t nw = (int64_t)gridDim.x * wpb;
  const int64_t n0 = (int64_t)blockIdx.x * wpb +
                    __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));   // wave-uniform

  int goff[J];
  bool cval[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = lane + kWave * j;
    cval[j] = FULL || c < C;
    goff[j] = (cval[j] ? c : C - 1) / cpg;
  }

  // Loads are unconditional, from clamped (always valid) chunks: a load under a branch makes the
  // compiler wait for every load in flight, prefetched rows included, before the next use.  A
  // row past the end gets an empty buffer resource, so its loads read no memory and return 0;
  // chunks past the row end are skipped when computed and rows past N are not stored.
  const int gown = min(lane, G - 1);           // SHARE: the group this lane loads
  auto load = [&](RowBuf<J, SHARE>& b, int64_t row) {
    const bool live = row < N;                  // wave-uniform
    const size_t r = live ? (size_t)row : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_over(packed + r * C, live ? (uint32_t)C * 16u : 0u);
    const __amdgpu_buffer_rsrc_t rs = buffer_over(scales + r * G, live ? (uint32_t)G * 2u : 0u);
    const __amdgpu_buffer_rsrc_t rz = buffer_over(zeros + r * G, live ? (uint32_t)G : 0u);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = FULL ? lane + kWave * j : min(lane + kWave * j, C - 1);
      b.w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, 16 * c, 0, kBufferNT));
      if (!SHARE) {
        b.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * goff[j], 0, 0);
        if (!SYM) b.z[j] = __builtin_amdgcn_raw_buffer_load_b8(rz, goff[j], 0, 0);
      }
    }
    if (SHARE) {
      b.s[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * gown, 0, 0);
      if (!SYM) b.z[0] = __builtin_amdgcn_raw_buffer_load_b8(rz, gown, 0, 0);
    }
  };

  static_assert(RING == 2 || RING == 3, "two or three rows in flight");
  RowBuf<J, SHARE> b0, b1, b2;
  load(b0, n0);
  load(b1, n0 + nw);
  if constexpr (RING == 3) load(b2, n0 + 2 * nw);

  // ---- X -> LDS: fp16 pairs scaled by 2^e per (m, chunk), four planes of 16 bytes ----
  // plane t of chunk c of row m holds (x0,x4), (x1,x5)/16, (x2,x6), (x3,x7)/16 of octet t;
  // fs holds 2^-e and sx the chunk sum of the scaled x times 2^-24.
  u32x4* xs = lds4;                                           // [M][4][C]
  float* fs = reinterpret_cast<float*>(lds4 + (size_t)M * 4 * C);   // [M][C]
  float* sx = fs + (size_t)M * C;                                   // [M][C]
  for (int idx = threadIdx.x; idx < M * C; idx += BLOCK) {
    const int m = idx / C;
    const int c = idx - m * C;
    const u32x4* xp = reinterpret_cast<const u32x4*>(X + (size_t)m * K + (size_t)c * 32);
    u32x4 v[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) v[o] = xp[o];
    float amax = 0.0f;
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[o][i])), fabsf(bf16_hi(v[o][i]))));
    int e = 0;
    if (amax > 0.0f) {
      int E;
      frexpf(amax, &E);                       // amax = f * 2^E, f in [0.5, 1)
      e = min(15 - E, 100);                   // amax * 2^e in [2^14, 2^15)
    }
    float sum = 0.0f;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      // octet o: x0..x7 = lo/hi halves of v[o][0..3]
      const u32x4 q = v[o];
      const f16x2 p0 = {(_Float16)ldexpf(bf16_lo(q[0]), e), (_Float16)ldexpf(bf16_lo(q[2]), e)};
      const f16x2 p1 = {(_Float16)ldexpf(bf16_hi(q[0]), e - 4), (_Float16)ldexpf(bf16_hi(q[2]), e - 4)};
      const f16x2 p2 = {(_Float16)ldexpf(bf16_lo(q[1]), e), (_Float16)ldexpf(bf16_lo(q[3]), e)};
      const f16x2 p3 = {(_Float16)ldexpf(bf16_hi(q[1]), e - 4), (_Float16)ldexpf(bf16_hi(q[3]), e - 4)};
      xs[((size_t)m * 4 + o) * C + c] = u32x4{as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
      // sum of the scaled x as the dot products see them (the x16 positions count 16 times)
      sum += (float)p0[0] + (float)p0[1] + (float)p2[0] + (float)p2[1] +
             16.0f * ((float)p1[0] + (float)p1[1] + (float)p3[0] + (float)p3[1]);
    }
    fs[idx] = ldexpf(1.0f, -e);
    sx[idx] = ldexpf(sum, -24);
  }
  __syncthreads();

  // XREG (one row of X): a lane meets the same J chunks of X in every row of W, so it copies
  // them, with their factors, from LDS into registers once and reads no LDS per row.
  constexpr bool XREG = MT == 1 && (J <= 2 || (J == 4 && (BLOCK <= 768 || RING <= 2)));   // register budget
  u32x4 xr[XREG ? J : 1][4];
  float xf[XREG ? J : 1], xsum[XREG ? J : 1];
  if constexpr (XREG) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = FULL ? lane + kWave * j : min(lane + kWave * j, C - 1);
#pragma unroll
      for (int o = 0; o < 4; ++o) xr[j][o] = xs[(size_t)o * C + c];
      xf[j] = fs[c];
      xsum[j] = sx[c];
    }
  }

  auto process = [&](const RowBuf<J, SHARE>& b, int64_t row) {
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    // SHARE: every lane takes part in the exchange (all 64 lanes active), before any branch.
    uint32_t shared[SHARE ? J : 1];
    if (SHARE) {
      const uint32_t sz = SYM ? b.s[0] : (b.s[0] | (b.z[0] << 16));   // one word per group
#pragma unroll
      for (int j = 0; j < J; ++j) shared[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * goff[j], (int)sz);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (cval[j]) {
        const int c = lane + kWave * j;
        uint32_t sbits, zbits;
        if (SHARE) {
          sbits = shared[j] & 0xffffu;
          zbits = shared[j] >> 16;
        } else {
          sbits = b.s[j];
          zbits = SYM ? 8u : b.z[j];
        }
        const float zf = SYM ? 8.0f : (float)zbits;
        // four independent partial sums per row of X (one per dword) keep the dot2 chains short
        float d[MT][4];
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          uint32_t dw = b.w[j][o];
          if (SYM) dw ^= 0x88888888u;          // two's complement nibble -> q + 8
          const uint32_t d8 = dw >> 8;
          const f16x2 h0 = as_f16x2(dw & 0x000F000Fu);   // q k0, k4   (x 2^-24)
          const f16x2 h1 = as_f16x2(dw & 0x00F000F0u);   // 16 q k1, k5
          const f16x2 h2 = as_f16x2(d8 & 0x000F000Fu);   // q k2, k6
          const f16x2 h3 = as_f16x2(d8 & 0x00F000F0u);   // 16 q k3, k7
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4 xv = XREG ? xr[XREG ? j : 0][o] : xs[((size_t)m * 4 + o) * C + c];
            float t = __builtin_amdgcn_fdot2(h0, as_f16x2(xv[0]), 0.0f, false);
            t = __builtin_amdgcn_fdot2(h1, as_f16x2(xv[1]), t, false);
            t = __builtin_amdgcn_fdot2(h2, as_f16x2(xv[2]), t, false);
            d[m][o] = __builtin_amdgcn_fdot2(h3, as_f16x2(xv[3]), t, false);
          }
        }
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float sxv = XREG ? xsum[XREG ? j : 0] : sx[m * C + c];
          const float fsv = XREG ? xf[XREG ? j : 0] : fs[m * C + c];
          const float r = __builtin_fmaf(-zf, sxv, (d[m][0] + d[m][1]) + (d[m][2] + d[m][3]));
          // 2^24 and 2^-e applied as two exact power-of-two products: no overflow unless the
          // chunk's dot product itself overflows
          acc[m] = __builtin_fmaf((r * 16777216.0f) * fsv, s, acc[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float tot = wave_total(acc[m]);
      if (lane == m && m < M) Y[(size_t)m * N + row] = f32_to_bf16_bits(tot);
    }
  };

  // sched_barrier keeps the compiler from hoisting one row's work into another's, which would
  // keep more than RING rows of registers live.  The slots are named, not an array: indexed
  // slots made the compiler wait for a later row's loads before computing an earlier one.
  const int64_t step = RING * nw;
  for (int64_t n = n0; n < N; n += step) {
    process(b0, n);
    __builtin_amdgcn_sched_barrier(0);
    load(b0, n + step);
    __builtin_amdgcn_sched_barrier(0);
    if (n + nw < N) process(b1, n + nw);
    __builtin_amdgcn_sched_barrier(0);
    load(b1, n + nw + step);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RING == 3) {
      if (n + 2 * nw < N) process(b2, n + 2 * nw);
      __builtin_amdgcn_sched_barrier(0);
      load(b2, n + 2 * nw + step);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Blocks of one kernel that fit on a compute unit at once (from its register and LDS use),
// remembered per LDS size: the grid of a persistent kernel is sized to what is resident.
template <typename Kernel>
int64_t resident_blocks(Kernel kernel, int block, size_t lds, std::atomic<uint64_t>& memo) {
  const uint64_t m = memo.load(std::memory_order_relaxed);
  if (m != 0 && (m >> 8) == lds) return (int64_t)(m & 0xff);
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, block, lds) != hipSuccess) {
    (void)hipGetLastError();
    nb = 1;
  }
  nb = nb < 1 ? 1 : (nb > 255 ? 255 : nb);
  memo.store(((uint64_t)lds << 8) | (uint64_t)nb, std::memory_order_relaxed);
  return nb;
}

template <int MT, int J, bool SYM, int BLOCK, bool FULL, bool SHARE, int RING>
hipError_t launch_one(const void* X, int M, int64_t N, int64_t K, int g, const void* packed,
                      const void* scales, const void* zeros, void* Y, int num_cus,
                      hipStream_t stream) {
  static std::atomic<uint64_t> memo{0};
  const auto kernel = gemv_kernel<MT, J, SYM, BLOCK, FULL, SHARE, RING>;
  const int64_t C = K >> 5;
  const size_t lds = (size_t)M * C * 64 + (size_t)M * C * 8;
  const int64_t wpb = BLOCK / kWave;
  int64_t blocks = (N + wpb - 1) / wpb;
  const int64_t cap = (int64_t)num_cus * resident_blocks(kernel, BLOCK, lds, memo);
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(BLOCK), lds, stream,
                     (const uint16_t*)X, M, N, (int)K, g, (const u32x4*)packed,
                     (const uint16_t*)scales, (const uint8_t*)zeros, (uint16_t*)Y);
  return hipGetLastError();
}

template <int MT, int J, int BLOCK, int RING>
hipError_t launch_mtj(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                      const void* packed, const void* scales, const void* zeros, void* Y,
                      int num_cus, hipStream_t stream) {
  const bool full = (K >> 5) == kWave * J;
  const bool share = K / g <= kWave;
#define Q4_GEMV_ONE(SYMV, FULLV, SHAREV)                                                     \
  return launch_one<MT, J, SYMV, BLOCK, FULLV, SHAREV, RING>(X, M, N, K, g, packed, scales, \
                                                             zeros, Y, num_cus, stream)
#define Q4_GEMV_SHARE(SYMV, FULLV)                                                           \
  if (share) { Q4_GEMV_ONE(SYMV, FULLV, true); } else { Q4_GEMV_ONE(SYMV, FULLV, false); }
  if (sym) {
    if (full) { Q4_GEMV_SHARE(true, true); } else { Q4_GEMV_SHARE(true, false); }
  } else {
    if (full) { Q4_GEMV_SHARE(false, true); } else { Q4_GEMV_SHARE(false, false); }
  }
#undef Q4_GEMV_SHARE
#undef Q4_GEMV_ONE
}

template <int MT>
hipError_t launch_mt(const void* X, int M, int64_t N, int64_t K, int g, bool sym,
                     const void* packed, const void* scales, const void* zeros, void* Y,
                     int num_cus, hipStream_t stream) {
  if (K <= 2048) return launch_mtj<MT, 1, 1024, 3>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
  if (K <= 4096) return launch_mtj<MT, 2, (MT == 1 ? 1024 : 768), 3>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
  if constexpr (MT == 1) {
    if (K <= 8192) {
      // Whole rows per wave, X held in registers: 12 waves per compute unit with three rows in
      // flight, or 16 waves with two when that spreads the rows more evenly (it minimises
      // (rows of the busiest wave) x (waves per unit)).  The 16-wave form fits its registers
      // only with shared scale loads (at most 64 groups) on full 8192-wide rows.
      auto cost = [&](int64_t w) { return ((N + (int64_t)num_cus * w - 1) / ((int64_t)num_cus * w)) * w; };
      const bool lean = K == 8192 && K / g <= kWave;
      if (lean && cost(16) < cost(12))
        return launch_mtj<1, 4, 1024, 2>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
      return launch_mtj<1, 4, 768, 3>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
    }
    if (K <= 16384) return launch_mtj<1, 8, 512, 3>(X, M, N, K, g, sym, packed, scales, zeros, Y, num_cus, stream);
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
