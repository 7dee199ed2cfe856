// Decode GEMV for W4A16 with M <= 2 (gfx950).
//
// W4A16: the 4-bit weights are dequantised inside the kernel and the products run on 16-bit
// operands ("LLM Weight Quantization - GPTQ, AWQ, SmoothQuant, FP8 & INT4/INT8 Trade-offs",
// "The vocabulary"); decode is bound by the bytes of the weights ("Overview": every output
// token reads every weight).  Dequantisation is x_hat = scale * (q - z) ("DL S067 ·
// Quantization", §1), with one scale and zero-point per group of g weights along K ("Model
// Quantization", §1).
//
// Work split.  A wave owns one output row n at a time.  Each 1 KiB of the row's codes is one
// load instruction (64 lanes x 16 bytes, contiguous); lane l = kq * 16 + n reads the 16-byte
// chunk 4 n + kq of it (32 weights), so the four lanes n, n + 16, n + 32, n + 48 together hold
// 128 consecutive weights.  One persistent block of 12 or 16 waves per compute unit converts X
// once into LDS; with M = 1 a lane meets the same chunks of X in every row, so it keeps them
// in registers.  Each wave keeps two or three rows in flight: the loads of the next rows are
// issued before a row is computed, and the first rows are requested before the conversion of
// X, so HBM latency overlaps it.
//
// Arithmetic (every product exact, sums in fp32, Y rounded once to bf16):
//   * (q - z) is formed exactly in fp16: the nibble OR-ed into the mantissa of 1024.0, minus
//     1024 + z (nibbles in bits 4..7 give 16 (q - z));
//   * x is converted to fp16 exactly after scaling each (row of X, 128-weight block) by a
//     power of two 2^e that puts its largest |x| in [2^14, 2^15); the positions that meet a
//     16 (q - z) weight carry 2^(e - 4);
//   * g a multiple of 128: one v_mfma_f32_16x16x32_f16 per dword of codes, with each lane's A
//     operand the x of its own weights: the diagonal D[n][n] sums the exact products of the
//     four lanes of a 128-weight block (one group), and the other entries are not used; the
//     block's sum is multiplied by its scale and 2^-e and accumulated in fp32;
//   * other g (32, 64, 96): v_dot2_f32_f16 of the same exact operands per 32-weight chunk;
//   * X whose fp16 conversion would lose a bit (a nonzero |x| 2^(e-4) below 2^-14, fp16's
//     smallest normal: a dynamic range above about 2^24 inside one 128-weight block) takes an
//     exact fp32 path instead: (q - z) and x converted to fp32, one fma per weight.  The
//     choice is one flag for the whole launch (every block stages the same X).
#include "q4_device.h"
#include "q4_internal.h"

#include <atomic>

namespace q4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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

// Max (or min) over each aligned quad of lanes, returned to every lane of the quad.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
}
__device__ __forceinline__ float quad_min(float v) {
  v = fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  return fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
}

// Four fp16 pairs (q - z) of one dword of codes (8 nibbles): nibble OR-ed into 1024.0 minus
// 1024 + z (1024 + 16 z for the nibbles in bits 4..7).  Slot order (k0, k4, k1, k5, k2, k6,
// k3, k7); the odd k carry 16 (q - z).
template <bool SYM>
__device__ __forceinline__ f16x8 dequant(uint32_t dw, uint32_t bias, f16x2 b1, f16x2 b16) {
  if (SYM) dw ^= 0x88888888u;                         // two's complement nibble -> q + 8
  const uint32_t d8 = dw >> 8;
  const f16x2 h0 = as_f16x2((dw & 0x000F000Fu) | bias) - b1;
  const f16x2 h1 = as_f16x2((dw & 0x00F000F0u) | bias) - b16;
  const f16x2 h2 = as_f16x2((d8 & 0x000F000Fu) | bias) - b1;
  const f16x2 h3 = as_f16x2((d8 & 0x00F000F0u) | bias) - b16;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
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

// DIAG: g is a multiple of 128 (the matrix-core diagonal form); else v_dot2 per chunk.
template <int MT, int J, bool SYM, int BLOCK, bool FULL, bool SHARE, int RING, bool DIAG>
__global__ __launch_bounds__(BLOCK) void gemv_kernel(
    const uint16_t* __restrict__ X, int M, int64_t N, int K, int g,
    const u32x4* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, uint16_t* __restrict__ Y) {
  extern __shared__ u32x4 lds4[];
  const int C = K >> 5;                       // 32-weight chunks per row
  const int G = K / g;
  const int cpg = g >> 5;                     // chunks per group
  const int lane = threadIdx.x & (kWave - 1);
  const int pi = 4 * (lane & 15) + (lane >> 4);   // this lane's chunk inside each 1 KiB
  const int64_t wpb = BLOCK / kWave;
  const int64_t nw = (int64_t)gridDim.x * wpb;
  const int64_t n0 = (int64_t)blockIdx.x * wpb +
                    __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));   // wave-uniform

  int goff[J];
  bool cval[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = pi + kWave * j;
    cval[j] = FULL || c < C;
    goff[j] = (cval[j] ? c : C - 1) / cpg;
  }

  // Loads are unconditional.  A row past the end gets an empty buffer resource, so its loads
  // read no memory and return 0; chunks past the row end lie past the resource's end (read 0
  // and meet x = 0), and rows past N are not stored.
  const int gown = min(lane, G - 1);           // SHARE: the group this lane loads
  auto load = [&](RowBuf<J, SHARE>& b, int64_t row) {
    const bool live = row < N;                  // wave-uniform
    const size_t r = live ? (size_t)row : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_over(packed + r * C, live ? (uint32_t)C * 16u : 0u);
    const __amdgpu_buffer_rsrc_t rs = buffer_over(scales + r * G, live ? (uint32_t)G * 2u : 0u);
    const __amdgpu_buffer_rsrc_t rz = buffer_over(zeros + r * G, live ? (uint32_t)G : 0u);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = pi + kWave * j;
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

  // ---- X -> LDS: fp16 pairs scaled by 2^e per (m, 128-weight block), four planes ----
  // plane t of chunk c of row m holds (x0,x4), (x1,x5)/16, (x2,x6), (x3,x7)/16 of octet t; fs
  // holds 2^-e per chunk (the same for the four chunks of a block).  One thread per chunk; the
  // four chunks of a block are an aligned quad of lanes (C is a multiple of 4 or the block is
  // the row's last), so the block's range is a quad reduction.
  u32x4* xs = lds4;                                                 // [M][4][C]
  float* fs = reinterpret_cast<float*>(lds4 + (size_t)M * 4 * C);   // [M][C]
  int lossy = 0;
  const int total = M * C;
  const int trips = (total + BLOCK - 1) / BLOCK;
  for (int it = 0; it < trips; ++it) {          // all lanes take part in every quad reduction
    const int idx = it * BLOCK + (int)threadIdx.x;
    const bool act = idx < total;
    const int m = act ? idx / C : 0;
    const int c = act ? idx - m * C : 0;
    u32x4 v[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) v[o] = act ? reinterpret_cast<const u32x4*>(X + (size_t)m * K + (size_t)c * 32)[o]
                                           : u32x4{0u, 0u, 0u, 0u};
    float amax = 0.0f, amin = __builtin_inff();
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = fabsf(bf16_lo(v[o][i])), bb = fabsf(bf16_hi(v[o][i]));
        amax = fmaxf(amax, fmaxf(a, bb));
        amin = fminf(amin, fminf(a > 0.0f ? a : __builtin_inff(), bb > 0.0f ? bb : __builtin_inff()));
      }
    // the block of chunk c is chunks 4 (c / 4) .. + 3 of the same row m: lanes 4 (idx / 4) .. + 3
    // when C is a multiple of 4 (the rows then start on quad boundaries); otherwise per chunk
    if ((C & 3) == 0) {
      amax = quad_max(amax);
      amin = quad_min(amin);
    }
    int e = 0;
    if (amax > 0.0f) e = min(15 - __builtin_amdgcn_frexp_expf(amax), 126);   // amax 2^e in [2^14, 2^15)
    lossy |= (int)(act && amin < __builtin_inff() && __builtin_ldexpf(amin, e) < 0x1p-10f);
    if (act) {
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        const u32x4 q = v[o];
        const f16x2 p0 = {(_Float16)__builtin_ldexpf(bf16_lo(q[0]), e), (_Float16)__builtin_ldexpf(bf16_lo(q[2]), e)};
        const f16x2 p1 = {(_Float16)__builtin_ldexpf(bf16_hi(q[0]), e - 4), (_Float16)__builtin_ldexpf(bf16_hi(q[2]), e - 4)};
        const f16x2 p2 = {(_Float16)__builtin_ldexpf(bf16_lo(q[1]), e), (_Float16)__builtin_ldexpf(bf16_lo(q[3]), e)};
        const f16x2 p3 = {(_Float16)__builtin_ldexpf(bf16_hi(q[1]), e - 4), (_Float16)__builtin_ldexpf(bf16_hi(q[3]), e - 4)};
        xs[((size_t)m * 4 + o) * C + c] = u32x4{as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
      }
      fs[idx] = __builtin_ldexpf(1.0f, -e);
    }
  }
  // one flag for the launch: every block stages the same X
  const bool exact = __syncthreads_or(lossy) != 0;

  // XREG (one row of X): a lane meets the same J chunks of X in every row of W, so it copies
  // them, with their factors, from LDS into registers once and reads no LDS per row.  Chunks
  // past the row end are 0.
  constexpr bool XREG = MT == 1 && (J <= 2 || (J == 4 && (BLOCK <= 768 || RING <= 2)));   // register budget
  u32x4 xr[XREG ? J : 1][4];
  float xf[XREG ? J : 1];
  if constexpr (XREG) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = FULL ? pi + kWave * j : min(pi + kWave * j, C - 1);
#pragma unroll
      for (int o = 0; o < 4; ++o) xr[j][o] = cval[j] ? xs[(size_t)o * C + c] : u32x4{0u, 0u, 0u, 0u};
      xf[j] = fs[c];
    }
  }
  uint32_t bias = 0x64006400u;
  asm volatile("" : "+v"(bias));   // keep in a VGPR: (x & mask) | bias -> one v_and_or_b32
  // the lanes whose D fragment holds a diagonal entry D[n][n]: rows 4 (l / 16) .. + 3 of column
  // l % 16 contain n when l / 16 == (l % 16) / 4; the entry is element (l % 16) % 4
  const bool diag_lane = (lane >> 4) == ((lane & 15) >> 2);

  auto group_sz = [&](const RowBuf<J, SHARE>& b, uint32_t (&sb)[J], uint32_t (&zb)[J]) {
    if (SHARE) {
      const uint32_t sz = SYM ? b.s[0] : (b.s[0] | (b.z[0] << 16));   // one word per group
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * goff[j], (int)sz);
        sb[j] = w & 0xffffu;
        zb[j] = SYM ? 8u : w >> 16;
      }
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        sb[j] = b.s[j];
        zb[j] = SYM ? 8u : b.z[j];
      }
    }
  };

  auto process_fast = [&](const RowBuf<J, SHARE>& b, int64_t row) {
    uint32_t sb[J], zb[J];
    group_sz(b, sb, zb);
    float tot[MT];
    if constexpr (DIAG) {
      f32x4 acc[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = FULL ? pi + kWave * j : min(pi + kWave * j, C - 1);
        const f16x2 b1 = as_f16x2((0x6400u + zb[j]) * 0x00010001u);
        const f16x2 b16 = as_f16x2((0x6400u + 16u * zb[j]) * 0x00010001u);
        f32x4 pacc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) pacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          const f16x8 bw = dequant<SYM>(b.w[j][o], bias, b1, b16);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4 xv = XREG ? xr[XREG ? j : 0][o]
                                  : (cval[j] ? xs[((size_t)m * 4 + o) * C + c] : u32x4{0u, 0u, 0u, 0u});
            pacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, xv), bw, pacc[m], 0, 0, 0);
          }
        }
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sb[j]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float f = s * (XREG ? xf[XREG ? j : 0] : fs[m * C + c]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[m][r] = __builtin_fmaf(pacc[m][r], f, acc[m][r]);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int el = lane & 3;
        const float dv = el == 0 ? acc[m][0] : (el == 1 ? acc[m][1] : (el == 2 ? acc[m][2] : acc[m][3]));
        tot[m] = wave_total(diag_lane ? dv : 0.0f);
      }
    } else {
      float acc[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = FULL ? pi + kWave * j : min(pi + kWave * j, C - 1);
        const f16x2 b1 = as_f16x2((0x6400u + zb[j]) * 0x00010001u);
        const f16x2 b16 = as_f16x2((0x6400u + 16u * zb[j]) * 0x00010001u);
        // four independent partial sums per row of X (one per dword) keep the dot2 chains short
        float d[MT][4];
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          const f16x8 bw = dequant<SYM>(b.w[j][o], bias, b1, b16);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const u32x4 xv = XREG ? xr[XREG ? j : 0][o]
                                  : (cval[j] ? xs[((size_t)m * 4 + o) * C + c] : u32x4{0u, 0u, 0u, 0u});
            float t = __builtin_amdgcn_fdot2(f16x2{bw[0], bw[1]}, as_f16x2(xv[0]), 0.0f, false);
            t = __builtin_amdgcn_fdot2(f16x2{bw[2], bw[3]}, as_f16x2(xv[1]), t, false);
            t = __builtin_amdgcn_fdot2(f16x2{bw[4], bw[5]}, as_f16x2(xv[2]), t, false);
            d[m][o] = __builtin_amdgcn_fdot2(f16x2{bw[6], bw[7]}, as_f16x2(xv[3]), t, false);
          }
        }
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sb[j]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float f = s * (XREG ? xf[XREG ? j : 0] : fs[m * C + c]);
          acc[m] = __builtin_fmaf((d[m][0] + d[m][1]) + (d[m][2] + d[m][3]), f, acc[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) tot[m] = wave_total(acc[m]);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (lane == m && m < M) Y[(size_t)m * N + row] = f32_to_bf16_bits(tot[m]);
  };

  // Exact path: (q - z) and x in fp32, one fma per weight (exact products), x read from X.
  const __amdgpu_buffer_rsrc_t rx = buffer_over(X, (uint32_t)M * (uint32_t)K * 2u);
  auto process_exact = [&](const RowBuf<J, SHARE>& b, int64_t row) {
    uint32_t sb[J], zb[J];
    group_sz(b, sb, zb);
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = pi + kWave * j;
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sb[j]);
      const float zf = (float)zb[j];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float part = 0.0f;
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          uint32_t dw = b.w[j][o];
          if (SYM) dw ^= 0x88888888u;
          // chunks past the row end lie past the resource's end (X row m, or beyond M rows): 0
          const uint32_t off = cval[j] ? 2u * ((uint32_t)m * (uint32_t)K + (uint32_t)c * 32u + 8u * (uint32_t)o)
                                       : 0xffffffc0u;
          const u32x4 xv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float q = (float)((dw >> (4 * i)) & 15u);
            const float x = (i & 1) ? bf16_hi(xv[i >> 1]) : bf16_lo(xv[i >> 1]);
            part = __builtin_fmaf(x, q - zf, part);
          }
        }
        acc[m] = __builtin_fmaf(part, s, acc[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float tot = wave_total(acc[m]);
      if (lane == m && m < M) Y[(size_t)m * N + row] = f32_to_bf16_bits(tot);
    }
  };

  auto process = [&](const RowBuf<J, SHARE>& b, int64_t row) {
    if (exact) process_exact(b, row);           // block-uniform
    else process_fast(b, row);
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

template <int MT, int J, bool SYM, int BLOCK, bool FULL, bool SHARE, int RING, bool DIAG>
hipError_t launch_one(const void* X, int M, int64_t N, int64_t K, int g, const void* packed,
                      const void* scales, const void* zeros, void* Y, int num_cus,
                      hipStream_t stream) {
  static std::atomic<uint64_t> memo{0};
  const auto kernel = gemv_kernel<MT, J, SYM, BLOCK, FULL, SHARE, RING, DIAG>;
  const int64_t C = K >> 5;
  const size_t lds = (size_t)M * C * 64 + (size_t)M * C * 4;
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
  const bool diag = g % 128 == 0;
#define Q4_GEMV_ONE(SYMV, FULLV, SHAREV)                                                            \
  if (diag) return launch_one<MT, J, SYMV, BLOCK, FULLV, SHAREV, RING, true>(X, M, N, K, g, packed, \
                                                                            scales, zeros, Y,       \
                                                                            num_cus, stream);       \
  return launch_one<MT, J, SYMV, BLOCK, FULLV, SHAREV, RING, false>(X, M, N, K, g, packed, scales,  \
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
