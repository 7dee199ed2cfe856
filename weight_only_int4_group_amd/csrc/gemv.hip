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
// load instruction (64 lanes x 16 bytes, contiguous): lane l reads chunk l of it (32 weights).
// One persistent block of 12 or 16 waves per compute unit converts X once into LDS; with M = 1
// a lane meets the same chunks of X in every row, so it keeps them in registers.  Each wave
// keeps two or three rows in flight: the loads of the next rows are issued before a row is
// computed, and its first row is requested before the conversion of X, so HBM latency
// overlaps it.
//
// Scales and zero-points.  A row has at most 64 groups in the common case, and then lane l
// reads group l's scale and zero-point and the lanes exchange them.  Read per row, they are two
// small requests beside the row's 4 KiB of codes (about 9 % of the time of a 28672 x 8192
// layer).  When a wave owns at least four rows, it owns a contiguous range of them instead and
// copies the range's scales and zero-points into its own LDS area once (global -> LDS copies,
// 256 bytes per instruction); each row then reads its pair from LDS.
//
// Arithmetic (every product exact, sums in fp32, Y rounded once to bf16):
//   * (q - z) is formed exactly in fp16: the nibble OR-ed into the mantissa of 1024.0, minus
//     1024 + z (nibbles in bits 4..7 give 16 (q - z));
//   * x is converted to fp16 exactly after scaling each (row of X, 32-weight chunk) by a power
//     of two 2^e that puts its largest |x| in [2^14, 2^15); the positions that meet a
//     16 (q - z) weight carry 2^(e - 4);
//   * the products and their sums run on the matrix cores, whose pipe is separate from the
//     vector ALU that forms (q - z): one v_mfma_f32_4x4x4_16b_f16 per four weights, each lane
//     supplying its own x and (q - z), so that one diagonal entry of its result is its own
//     four-term dot product in fp32 (the matrix cores flush fp16 subnormals, so the staging
//     keeps every nonzero operand normal); each 32-weight chunk's sum is multiplied by its
//     scale and 2^-e and accumulated in fp32;
//   * X whose fp16 conversion would lose a bit (a nonzero |x| 2^(e-4) below 2^-14, fp16's
//     smallest normal: a dynamic range above about 2^24 inside one 32-weight chunk) takes an
//     exact fp32 path instead: (q - z) and x converted to fp32, one fma per weight.  The
//     choice is one flag for the whole launch (every block stages the same X).
#include "q4_device.h"
#include "q4_internal.h"

#include <atomic>

namespace q4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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

// Raw-buffer descriptor words, for inline asm (the format of buffer_over).
__device__ __forceinline__ u32x4 buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), (uint32_t)kBufferFlags};
}

// Global -> LDS copy of 4 bytes per lane: lane i's dword at byte voff of the resource lands at
// LDS byte lds + 4 i.  The asm is taken to touch the memory of dep (a pointer the later loads
// read through), so that the compiler moves no such load across it: a counted wait for the
// copy relies on which loads were issued after it.
__device__ __forceinline__ void copy_dword_to_lds(u32x4 rsrc, uint32_t voff, uint32_t lds, const void* dep) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds), "s"(dep) : "memory");
}

// Bytes of one wave's LDS copy of the scales and zero-points of rows rows (G groups a row).
__host__ __device__ inline uint32_t stage_bytes(uint32_t rows, uint32_t G, bool sym) {
  return ((rows * G * 2u + 255u) & ~255u) + (sym ? 0u : ((rows * G + 255u) & ~255u));
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
// 64 lanes active, so every source lane of the exchange holds its value.  With the LDS copy
// (STAGE), s and z are read from LDS instead of memory.
template <int J, bool SHARE>
struct RowBuf {
  u32x4 w[J];
  uint32_t s[SHARE ? 1 : J];      // fp16 scale bits
  uint32_t z[SHARE ? 1 : J];      // zero-point
};

template <int MT, int J, bool SYM, int BLOCK, bool FULL, bool SHARE, bool STAGE, int RING>
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
  const int wib = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));   // wave in block
  const int64_t n0 = (int64_t)blockIdx.x * wpb + wib;                            // wave-uniform
  static_assert(!STAGE || SHARE, "the LDS copy holds one scale and zero-point per lane and row");

  // The wave's rows: rbase, rbase + rstride, ... below rend.  STAGE: a contiguous range, the
  // waves' counts differing by at most one (N < 2^31, checked at launch); otherwise every nw-th
  // row from n0.
  int64_t rbase = n0, rstride = nw, rend = N;
  uint32_t rmax = 0;                           // STAGE: rows of the busiest wave
  if constexpr (STAGE) {
    const uint32_t q = (uint32_t)N / (uint32_t)nw, r = (uint32_t)N - q * (uint32_t)nw;
    const uint32_t w = (uint32_t)n0;
    rbase = (int64_t)(w * q + min(w, r));
    rstride = 1;
    rend = rbase + (int64_t)(q + (w < r ? 1u : 0u));
    rmax = q + (r != 0u ? 1u : 0u);
  }

  int goff[J];
  bool cval[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = lane + kWave * j;
    cval[j] = FULL || c < C;
    goff[j] = (cval[j] ? c : C - 1) / cpg;
  }
  // SHARE with at most four chunks per lane: the exchange addresses 4 goff[j] (below 256, as a
  // row has at most 64 groups) packed one per byte, a register instead of J
  constexpr bool PACK = SHARE && J <= 4;
  uint32_t gpack = 0;
  if constexpr (PACK) {
#pragma unroll
    for (int j = 0; j < J; ++j) gpack |= (uint32_t)(4 * goff[j]) << (8 * j);
  }

  // Loads are unconditional.  A row past the end gets an empty buffer resource, so its loads
  // read no memory and return 0; chunks past the row end lie past the resource's end (read 0
  // and meet x = 0), and rows past N are not stored.
  const int gown = min(lane, G - 1);           // SHARE: the group this lane loads
  auto load = [&](RowBuf<J, SHARE>& b, int64_t row) __attribute__((always_inline)) {
    const bool live = row < rend;               // wave-uniform
    const size_t r = live ? (size_t)row : 0;
    const __amdgpu_buffer_rsrc_t rw = buffer_over(packed + r * C, live ? (uint32_t)C * 16u : 0u);
    const __amdgpu_buffer_rsrc_t rs = buffer_over(scales + r * G, live ? (uint32_t)G * 2u : 0u);
    const __amdgpu_buffer_rsrc_t rz = buffer_over(zeros + r * G, live ? (uint32_t)G : 0u);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + kWave * j;
      b.w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, 16 * c, 0, kBufferNT));
      if (!SHARE) {
        b.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * goff[j], 0, 0);
        if (!SYM) b.z[j] = __builtin_amdgcn_raw_buffer_load_b8(rz, goff[j], 0, 0);
      }
    }
    if (SHARE && !STAGE) {
      b.s[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * gown, 0, 0);
      if (!SYM) b.z[0] = __builtin_amdgcn_raw_buffer_load_b8(rz, gown, 0, 0);
    }
  };

  // STAGE: the wave's LDS area, after X's: its rows' scales (rmax G fp16) then zero-points
  // (rmax G bytes), each padded to 256 bytes; ldsz reads local row k's pair for group gown
  // (rows past the wave's end read row 0's, never used).
  const uint32_t x_lds = ((uint32_t)(M * C * 68) + 15u) & ~15u;
  const uint32_t s_bytes = ((rmax * (uint32_t)G * 2u + 255u) & ~255u);
  const uint32_t sz_lds = x_lds + (uint32_t)wib * stage_bytes(rmax, (uint32_t)G, SYM);
  const uint32_t nrows = (uint32_t)(rend - rbase);
  auto ldsz = [&](RowBuf<J, SHARE>& b, int64_t k) __attribute__((always_inline)) {
    if constexpr (STAGE) {
      const uint8_t* a = reinterpret_cast<const uint8_t*>(lds4) + sz_lds;
      const uint32_t kk = ((uint32_t)k < nrows ? (uint32_t)k : 0u) * (uint32_t)G + (uint32_t)gown;
      b.s[0] = *reinterpret_cast<const uint16_t*>(a + 2u * kk);
      if (!SYM) b.z[0] = a[s_bytes + kk];
    }
  };

  static_assert(RING == 2 || RING == 3, "two or three rows in flight");
  // ---- X -> LDS: fp16 pairs scaled by 2^e per (m, chunk), four planes ----
  // plane t of chunk c of row m holds (x0,x4), (x1,x5)/16, (x2,x6), (x3,x7)/16 of octet t; fs
  // holds 2^-e.  One thread per chunk (M C <= BLOCK, checked at launch).  X is requested
  // before the first rows of W, so that it arrives first and the rows compute as they land.
  // The range of |x| is taken on the bf16 bit patterns (their order as unsigned 16-bit integers
  // is the order of the values), two at a time; the smallest nonzero one as the smallest of
  // bits - 1 (zero wraps to the largest).
  const int idx = threadIdx.x;
  const bool stager = idx < M * C;
  const int m_x = stager ? idx / C : 0;
  const int c_x = stager ? idx - m_x * C : 0;
  u32x4 v[4];
  if (stager) {
#pragma unroll
    for (int o = 0; o < 4; ++o) v[o] = reinterpret_cast<const u32x4*>(X + (size_t)m_x * K + (size_t)c_x * 32)[o];
  }

  // One row per wave is requested before X is staged, the others after: X's request does not
  // then queue behind the whole first round of rows (the Llama-7B up-projection, whose first
  // round is the whole layer: 8.9 -> 7.5 us; the 70B-shaped layer unchanged within noise).
  RowBuf<J, SHARE> b0, b1, b2;
  load(b0, rbase);

  u32x4* xs = lds4;                                                 // [M][4][C]
  float* fs = reinterpret_cast<float*>(lds4 + (size_t)M * 4 * C);   // [M][C]
  int lossy = 0;
  if (stager) {
    const int m = m_x, c = c_x;
    u16x2 hi = {0, 0}, lo = {0xffff, 0xffff};
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u16x2 a = __builtin_bit_cast(u16x2, v[o][i] & 0x7fff7fffu);
        hi = __builtin_elementwise_max(hi, a);
        lo = __builtin_elementwise_min(lo, a - u16x2{1, 1});
      }
    const uint32_t amax_b = hi[0] > hi[1] ? hi[0] : hi[1];
    const uint32_t amin_b1 = lo[0] < lo[1] ? lo[0] : lo[1];          // 0xffff: no nonzero x
    const float amax = __uint_as_float(amax_b << 16);
    int e = 0;
    if (amax > 0.0f) e = min(15 - __builtin_amdgcn_frexp_expf(amax), 126);   // amax 2^e in [2^14, 2^15)
    lossy |= (int)(amin_b1 != 0xffffu && __builtin_ldexpf(__uint_as_float((amin_b1 + 1u) << 16), e) < 0x1p-10f);
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
  // one flag for the launch: every block stages the same X
  const bool exact = __syncthreads_or(lossy) != 0;

  // XREG (one row of X): a lane meets the same J chunks of X in every row of W, so it copies
  // them, with their factors, from LDS into registers once and reads no LDS per row.  Chunks
  // past the row end are 0.
  constexpr bool XREG = MT == 1 && (J <= 2 || (J == 4 && (BLOCK <= 768 || RING <= 2)));   // register budget
  static_assert(!XREG || J <= 4, "one byte of xe per chunk");
  u32x4 xr[XREG ? J : 1][4];
  // the chunks' factors 2^-e, as the exponents -e packed one per byte (J <= 4): one register
  uint32_t xe = 0;
  uint32_t bias = 0x64006400u;
  asm volatile("" : "+v"(bias));   // keep in a VGPR: (x & mask) | bias -> one v_and_or_b32
  // Y[m, row] from lane m, through a resource based at the element (its address is
  // wave-uniform, so it takes no vector registers)
  auto store_y = [&](int m, int64_t row, float v) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = buffer_over(Y + (size_t)m * (size_t)N + (size_t)row, 2u);
    if (lane == m) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(v), r, 0, 0, 0);
  };

  auto group_sz = [&](const RowBuf<J, SHARE>& b, uint32_t (&sb)[J], uint32_t (&zb)[J]) __attribute__((always_inline)) {
    if (SHARE) {
      const uint32_t sz = SYM ? b.s[0] : (b.s[0] | (b.z[0] << 16));   // one word per group
      // opaque to the compiler, so that the bytes are taken apart here rather than once into J
      // registers
      uint32_t gp = gpack;
      asm volatile("" : "+v"(gp));
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int addr = PACK ? (int)((gp >> (8 * j)) & 0xffu) : 4 * goff[j];
        const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)sz);
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

  // One 4x4x4 matrix-core product per half dword of codes: lane l supplies row l % 4 of A (its
  // own four x) and column l % 4 of B (its own four (q - z)) of block l / 4, so the diagonal
  // entry D[l % 4][l % 4], element l % 4 of lane l's result, is the lane's own exact four-term
  // dot product summed in fp32; the other entries are not used.
  auto process_fast = [&](const RowBuf<J, SHARE>& b, int64_t row) __attribute__((always_inline)) {
    uint32_t sb[J], zb[J];
    group_sz(b, sb, zb);
    // opaque to the compiler, so that the bytes are taken apart here rather than once into J
    // registers
    uint32_t xep = xe;
    asm volatile("" : "+v"(xep));
    auto xexp = [&](int j) { return (int)(int8_t)(uint8_t)(xep >> (8 * j)); };
    f32x4 acc4[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc4[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = FULL ? lane + kWave * j : min(lane + kWave * j, C - 1);
      const f16x2 b1 = as_f16x2((0x6400u + zb[j]) * 0x00010001u);
      const f16x2 b16 = as_f16x2((0x6400u + 16u * zb[j]) * 0x00010001u);
      f32x4 pacc[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) pacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        const f16x8 bw = dequant<SYM>(b.w[j][o], bias, b1, b16);
        const f16x4 blo = {bw[0], bw[1], bw[2], bw[3]}, bhi = {bw[4], bw[5], bw[6], bw[7]};
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 xv = XREG ? xr[XREG ? j : 0][o]
                                : (cval[j] ? xs[((size_t)m * 4 + o) * C + c] : u32x4{0u, 0u, 0u, 0u});
          const f16x8 xa = __builtin_bit_cast(f16x8, xv);
          pacc[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(f16x4{xa[0], xa[1], xa[2], xa[3]}, blo, pacc[m], 0, 0, 0);
          pacc[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(f16x4{xa[4], xa[5], xa[6], xa[7]}, bhi, pacc[m], 0, 0, 0);
        }
      }
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sb[j]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float f = XREG ? __builtin_ldexpf(s, xexp(j)) : s * fs[m * C + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc4[m][r] = __builtin_fmaf(pacc[m][r], f, acc4[m][r]);
      }
    }
    const int el = lane & 3;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float dv = el == 0 ? acc4[m][0] : (el == 1 ? acc4[m][1] : (el == 2 ? acc4[m][2] : acc4[m][3]));
      const float tot = wave_total(dv);
      if (m < M) store_y(m, row, tot);
    }
  };

  // Exact path: (q - z) and x in fp32, one fma per weight (exact products), x read from X.
  const __amdgpu_buffer_rsrc_t rx = buffer_over(X, (uint32_t)M * (uint32_t)K * 2u);
  auto process_exact = [&](const RowBuf<J, SHARE>& b, int64_t row) __attribute__((always_inline)) {
    uint32_t sb[J], zb[J];
    group_sz(b, sb, zb);
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + kWave * j;
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
      if (m < M) store_y(m, row, tot);
    }
  };

  // sched_barrier keeps the compiler from hoisting one row's work into another's, which would
  // keep more than RING rows of registers live.  The slots are named, not an array: indexed
  // slots made the compiler wait for a later row's loads before computing an earlier one.  The
  // exact form has a loop of its own (one row at a time), so that the pipelined loop holds no
  // load but its rows' (a load under a branch makes the compiler wait for every load in flight).
  auto run = [&](auto process) __attribute__((always_inline)) {
    const int64_t step = RING * rstride;
    int64_t k = 0;                              // local index of row n
    for (int64_t n = rbase; n < rend; n += step, k += RING) {
      process(b0, n);
      __builtin_amdgcn_sched_barrier(0);
      load(b0, n + step);
      ldsz(b0, k + RING);
      __builtin_amdgcn_sched_barrier(0);
      if (n + rstride < rend) process(b1, n + rstride);
      __builtin_amdgcn_sched_barrier(0);
      load(b1, n + rstride + step);
      ldsz(b1, k + 1 + RING);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (RING == 3) {
        if (n + 2 * rstride < rend) process(b2, n + 2 * rstride);
        __builtin_amdgcn_sched_barrier(0);
        load(b2, n + 2 * rstride + step);
        ldsz(b2, k + 2 + RING);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if constexpr (STAGE) {
    // issued here, after X, like the rows' second round: requested before X, the copies
    // delayed it
    const uint32_t nb = nrows * (uint32_t)G;
    const u32x4 rs = buffer_words(scales + (size_t)rbase * G, nb * 2u);
    const u32x4 rz = buffer_words(zeros + (size_t)rbase * G, nb);
    const uint32_t a = (uint32_t)(uintptr_t)lds4 + sz_lds;
    for (uint32_t i = 0; i < s_bytes; i += 256u) copy_dword_to_lds(rs, i + 4u * lane, a + i, packed);
    if (!SYM) {
      const uint32_t z_bytes = (rmax * (uint32_t)G + 255u) & ~255u;
      for (uint32_t i = 0; i < z_bytes; i += 256u) copy_dword_to_lds(rz, i + 4u * lane, a + s_bytes + i, packed);
    }
  }
  load(b1, rbase + rstride);
  if constexpr (RING == 3) load(b2, rbase + 2 * rstride);
  // STAGE: exactly the (RING - 1) J loads of rows 1 and 2 were issued after the copies (the
  // asm keeps loads through packed on their side of it)
  if constexpr (STAGE) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((RING - 1) * J), "s"(packed) : "memory");
  if (exact) {                                 // block-uniform; rows one at a time
    int64_t k = 0;
    for (int64_t n = rbase; n < rend; n += rstride, ++k) {
      // X is read again for every row (a compiler barrier keeps its loads in the loop rather
      // than hoisted into registers for all rows)
      asm volatile("" ::: "memory");
      load(b0, n);
      ldsz(b0, k);
      process_exact(b0, n);
    }
    return;
  }
  if constexpr (XREG) {   // after the exact loop: its registers are free there
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = FULL ? lane + kWave * j : min(lane + kWave * j, C - 1);
#pragma unroll
      for (int o = 0; o < 4; ++o) xr[j][o] = cval[j] ? xs[(size_t)o * C + c] : u32x4{0u, 0u, 0u, 0u};
      xe |= (uint32_t)((__builtin_amdgcn_frexp_expf(fs[c]) - 1) & 0xff) << (8 * j);   // fs = 2^(exp - 1)
    }
  }
  ldsz(b0, 0);
  ldsz(b1, 1);
  if constexpr (RING == 3) ldsz(b2, 2);
  run(process_fast);
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

// STAGE: hipErrorNotSupported (nothing launched) when a wave would own fewer than kStageRows
// rows, its LDS copy does not fit or the copy's conditions fail; the caller then launches the
// form without it.
constexpr int64_t kStageRows = 4;

template <int MT, int J, bool SYM, int BLOCK, bool FULL, bool SHARE, bool STAGE, int RING>
hipError_t launch_one(const void* X, int M, int64_t N, int64_t K, int g, const void* packed,
                      const void* scales, const void* zeros, void* Y, int num_cus,
                      hipStream_t stream) {
  static std::atomic<uint64_t> memo{0};
  const auto kernel = gemv_kernel<MT, J, SYM, BLOCK, FULL, SHARE, STAGE, RING>;
  const int64_t C = K >> 5;
  if ((int64_t)M * C > BLOCK) return hipErrorInvalidValue;   // one staging thread per chunk of X
  const size_t x_lds = ((size_t)M * C * 68 + 15) & ~(size_t)15;   // X's fp16 planes and factors
  const int64_t wpb = BLOCK / kWave;
  int64_t blocks = (N + wpb - 1) / wpb;
  size_t lds = x_lds;
  // the copies move whole dwords of each wave's range: 4 | G keeps a range's ends on dwords
  if (STAGE && (N >= ((int64_t)1 << 31) || (K / g) % 4 != 0 ||
                (((uintptr_t)scales | (SYM ? (uintptr_t)0 : (uintptr_t)zeros)) & 3) != 0))
    return hipErrorNotSupported;
  // the grid is what is resident; with the copy, the LDS per block grows as the grid shrinks
  for (;;) {
    if (STAGE) {
      const int64_t rmax = (N + blocks * wpb - 1) / (blocks * wpb);
      lds = x_lds + (size_t)wpb * stage_bytes((uint32_t)rmax, (uint32_t)(K / g), SYM);
      if (lds > 160 * 1024) return hipErrorNotSupported;
    }
    const int64_t cap = (int64_t)num_cus * resident_blocks(kernel, BLOCK, lds, memo);
    if (blocks <= cap) break;
    blocks = cap;
  }
  if (STAGE && blocks * wpb * kStageRows > N) return hipErrorNotSupported;
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
#define Q4_GEMV_ONE(SYMV, FULLV, SHAREV, STAGEV)                                                 \
  launch_one<MT, J, SYMV, BLOCK, FULLV, SHAREV, STAGEV, RING>(X, M, N, K, g, packed, scales, zeros, \
                                                              Y, num_cus, stream)
#define Q4_GEMV_SHARE(SYMV, FULLV)                                                       \
  if (share) {                                                                           \
    const hipError_t e = Q4_GEMV_ONE(SYMV, FULLV, true, true);                           \
    return e == hipErrorNotSupported ? Q4_GEMV_ONE(SYMV, FULLV, true, false) : e;        \
  }                                                                                      \
  return Q4_GEMV_ONE(SYMV, FULLV, false, false);
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
